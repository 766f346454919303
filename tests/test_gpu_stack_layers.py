"""The 30-layer stack of the full denoise step (30 layers of d 2048, 16 query /
4 KV heads x 128, 128 experts top-8, d_ff 768, vocabulary 262144, prompt
4096, canvas 256, bf16) run as a chain of stage calls: layers 0, 15 and 29
are checked against the float64 oracle on the GPU's own inputs to them (the
hidden state arriving at the layer, the layer's cached prompt K/V, the MoE
with the GPU's route set), every position; the head after the last layer is
checked at every logit; the chain equals dg_denoise_step bit for bit."""
import pytest
import torch

from discrete_text_diffusion_denoise_amd import binding, synthetic

import chain
from helpers import DEV, TOL_BF16
from test_gpu_layer_full import gpu_weights

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

CHECKED = (0, 15, 29)


def test_stack_layers_against_oracle():
    shape = synthetic.SHAPES["stack"]
    cfg = synthetic.model_config("stack")
    P, N, V, d = shape["prompt"], cfg["canvas"], cfg["vocab"], cfg["d_model"]
    print(f"stack: {cfg['n_layers']} layers, prompt {P}", flush=True)
    W = gpu_weights(cfg, 11)
    g = torch.Generator(device=DEV)
    g.manual_seed(12)
    prompt = torch.randint(0, V, (1, P), generator=g, device=DEV, dtype=torch.int32)
    canvas = torch.randint(0, V, (1, N), generator=g, device=DEV, dtype=torch.int32)
    m = binding.Model(cfg, W, batch=1, capacity=P + N)
    m.encode_prompt(prompt)
    logits = torch.empty((1, N, V), dtype=torch.float32, device=DEV)
    m.denoise_step(canvas, logits)
    torch.cuda.synchronize()
    print("step done; chain", flush=True)
    h = torch.empty((N, d), dtype=torch.float32, device=DEV)
    m.stage_input(canvas, h)
    for l in range(cfg["n_layers"]):
        if l in CHECKED:
            lw = chain.layer64(W["layers"][l])
            chain.check_attention(m, cfg, lw, l, h, N, False, TOL_BF16, label="stack")
            chain.check_moe(m, cfg, lw, l, h, TOL_BF16, label="stack")
            del lw
        else:
            m.stage_attention(l, h, N, False)
            m.stage_moe(l, h)
    torch.cuda.synchronize()
    Wk = {"embed": W["embed"].float().cpu().numpy(),
          "final_norm": W["final_norm"].cpu().numpy().astype("float64")}
    lc = chain.check_head(m, cfg, Wk, h, TOL_BF16, label="stack")
    assert torch.equal(lc.view(1, N, V), logits)
