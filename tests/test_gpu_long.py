"""Block-autoregressive long generation at full size: the 30-layer stack over a
32768-token prompt, consecutive blocks each committed to the cache before the
next starts.  Two blocks of the library's loop equal their call-by-call
composition bit for bit (blocks, round counts, the cache the commits
wrote), and the cache grows by one canvas per block; the logits stay
finite with a context of 33 000 keys."""
import pytest
import torch

from discrete_text_diffusion_denoise_amd import binding, synthetic

from helpers import DEV
from test_gpu_layer_full import gpu_weights

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

BLOCKS = 2
ROUNDS = 3


def test_long_context_blocks_are_their_composition():
    shape = synthetic.SHAPES["long"]
    cfg = synthetic.model_config("long")
    P, N, V = shape["prompt"], cfg["canvas"], cfg["vocab"]
    print(f"long context: {cfg['n_layers']} layers, prompt {P}, {BLOCKS} blocks", flush=True)
    W = gpu_weights(cfg, 5)
    g = torch.Generator(device=DEV)
    g.manual_seed(6)
    prompt = torch.randint(0, V, (1, P), generator=g, device=DEV, dtype=torch.int32)
    params = synthetic.default_sampler_params(max_steps=ROUNDS, seed=9, selfcond_on=1)
    cap = P + (BLOCKS + 1) * N
    mg = binding.Model(cfg, W, batch=1, capacity=cap, generate_ws=True)
    mg.encode_prompt(prompt)
    torch.cuda.synchronize()
    print("prompt encoded", flush=True)
    blocks_g, steps_g = [], []
    for k in range(BLOCKS):
        blk = torch.zeros((1, N), dtype=torch.int32, device=DEV)
        steps_g.append(mg.generate_block(params, k, blk)[0])
        blocks_g.append(blk)
        assert mg.kv_length == P + (k + 1) * N
    torch.cuda.synchronize()
    Kg = [t.clone() for t in mg.kv_tensors()]
    del mg
    torch.cuda.empty_cache()
    mc = binding.Model(cfg, W, batch=1, capacity=cap)
    mc.encode_prompt(prompt)
    lg = [torch.empty((1, N, V), dtype=torch.float32, device=DEV) for _ in range(2)]
    st = [torch.empty((1, N, 4), dtype=torch.float32, device=DEV) for _ in range(2)]
    ws = binding.sampler_workspace(1, N)
    for k in range(BLOCKS):
        canvas = torch.zeros((1, N), dtype=torch.int32, device=DEV)
        binding.canvas_init(params["seed"], k, canvas, V)
        argmax = torch.zeros((1, N), dtype=torch.int32, device=DEV)
        lock = torch.zeros((1, N), dtype=torch.uint8, device=DEV)
        stop = torch.zeros(1, dtype=torch.int32, device=DEV)
        prev = prev_st = None
        steps = 0
        for t in range(ROUNDS):
            mc.denoise_step(canvas, lg[t % 2], prev, prev_st)
            binding.sample_update(params, t, lg[t % 2], canvas, argmax, lock, st[t % 2], stop, ws)
            if stop.item():
                steps = t + 1
                break
            prev, prev_st = lg[t % 2], st[t % 2]
        assert torch.isfinite(lg[(steps - 1) % 2]).all()
        mc.commit_block(argmax)
        assert steps == steps_g[k] == ROUNDS
        assert torch.equal(blocks_g[k], argmax)
    torch.cuda.synchronize()
    L = P + BLOCKS * N
    Kc = mc.kv_tensors()
    assert mc.kv_length == L
    assert torch.equal(Kg[0][..., :L, :], Kc[0][..., :L, :])
    assert torch.equal(Kg[1][..., :L, :], Kc[1][..., :L, :])
