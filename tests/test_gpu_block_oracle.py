"""dg_generate_block against the oracle's block loop (oracle/driver.generate_block).

Report-summary page, sections 1 and 4: a block starts from uniform random
tokens; each round predicts every position, locks confident positions,
re-randomises the rest, and each canvas stops on its own when its mean
entropy falls below the threshold (here without the stability condition, so
the threshold decides); a stopped canvas is left as it is; the block is the
last round's most likely sequence and is committed to the cache.

The library's loop reads each round's stop flags one round late and raises a
device flag once every canvas has stopped, so the round it has already
queued does nothing.  Its rounds are not observable from outside, so the
test runs three things on identical seeded inputs:

  1. dg_generate_block, as dg_generate_block_trace (block, round counts,
     committed cache, and each round's mean entropy and locked count);
  2. the same rounds call by call on the GPU (dg_denoise_step +
     dg_sample_update), recording every round's logits and sampler outputs;
  3. the oracle's loop with its model logits replaced by the GPU's of the
     same round (logits_hook), after checking them against the oracle's own
     on the same canvas and self-conditioning input.

The oracle's canvas, most likely sequence, locks, statistics and stop flags
must equal the GPU's bit for bit in every round, its block and round counts
must equal dg_generate_block's, and its committed cache (float64 encode of
the block) must match the GPU's within the model tolerance.  The head's
output is scaled up (RMSNorm scale of the final norm) so that the random
model is confident at part of the positions and the lock rule acts."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_denoise_amd import binding, synthetic
from oracle import driver
from oracle import model as om
from oracle import sampler as osampler

from helpers import DEV, normwise, route_ambiguous, to_dev, tol_for
from test_gpu_model import MODELS

pytestmark = pytest.mark.gpu

B, P, ROUNDS = 2, 40, 5

# model, final-norm scale, stop variant, sampler overrides
CASES = [
    ("tiny", 8.0, "split", {}),
    ("tiny", 8.0, "all_early", {}),
    ("small_bf16", 4.0, "split", {}),
    ("small_bf16", 6.0, "budget", dict(lock_rule=0, lock_theta=0.9, temp_start=1.0, temp_end=1.0)),
    ("small_bf16", 4.0, "split", dict(top_k=8)),
]


def sampler_run(m, params, V, N):
    """The block's rounds call by call on the GPU; returns the per-round
    records and the rounds each canvas ran, and commits the block."""
    canvas = torch.zeros((B, N), dtype=torch.int32, device=DEV)
    binding.canvas_init(params["seed"], 0, canvas, V)
    argmax = torch.zeros((B, N), dtype=torch.int32, device=DEV)
    lock = torch.zeros((B, N), dtype=torch.uint8, device=DEV)
    stop = torch.zeros(B, dtype=torch.int32, device=DEV)
    lg = [torch.empty((B, N, V), dtype=torch.float32, device=DEV) for _ in range(2)]
    st = [torch.zeros((B, N, 4), dtype=torch.float32, device=DEV) for _ in range(2)]
    ws = binding.sampler_workspace(B, N)
    prev = prev_st = None
    recs, steps = [], [0] * B
    top_k = params.get("top_k", 0)
    for t in range(params["max_steps"]):
        canvas_in = canvas.cpu().numpy()
        m.denoise_step(canvas, lg[t % 2], prev, prev_st, top_k=top_k if prev is not None else 0)
        binding.sample_update(params, t, lg[t % 2], canvas, argmax, lock, st[t % 2], stop, ws)
        torch.cuda.synchronize()
        recs.append(dict(canvas_in=canvas_in, logits=lg[t % 2].cpu().numpy(),
                         canvas=canvas.cpu().numpy(), argmax=argmax.cpu().numpy(),
                         lock=lock.cpu().numpy(), stats=st[t % 2].cpu().numpy(),
                         stop=stop.cpu().numpy()))
        s = recs[-1]["stop"].tolist()
        for b in range(B):
            if steps[b] == 0 and s[b]:
                steps[b] = t + 1
        if all(s):
            break
        prev, prev_st = lg[t % 2], st[t % 2]
    m.commit_block(argmax)
    torch.cuda.synchronize()
    return recs, [s or params["max_steps"] for s in steps]


def mean_entropy(stats_row):
    """The sampler's mean entropy of one canvas: a sequential binary32 sum
    over positions divided by N (only used to place the stop threshold)."""
    acc = np.float32(0.0)
    for v in stats_row[:, 2]:
        acc = np.float32(acc + v)
    return float(np.float32(acc / np.float32(stats_row.shape[0])))


def route_keep(canvas_b, prev_b, W64, cfg, cache, b, top_k, gap):
    """Positions whose oracle route is unambiguous at `gap` in every layer of
    the oracle's own step from this canvas and self-conditioning input."""
    h = om.denoiser_input(canvas_b, W64, prev_b, top_k)
    keep = np.ones(h.shape[0], dtype=bool)
    for li, lw in enumerate(W64["layers"]):
        h, _, _ = om.attn_half(h, lw, cfg, cache.k[li][b], cache.v[li][b], cache.length,
                               causal=False)
        u = om.rmsnorm(h, lw["moe_norm"], cfg["rms_eps"])
        keep &= ~route_ambiguous(u @ lw["w_router"].T, cfg["top_k"], gap)
        h, _, _, _ = om.moe_half(h, lw, cfg)
    return keep


@pytest.mark.parametrize("name,scale,variant,over", CASES)
def test_generate_block_against_oracle_loop(name, scale, variant, over):
    cfg = synthetic.model_config(MODELS[name], n_layers=1)
    W = synthetic.make_weights(cfg, seed=0, std=0.05, random_norms=True)
    W["final_norm"] = (W["final_norm"] * np.float32(scale)).astype(np.float32)
    N, V = cfg["canvas"], cfg["vocab"]
    tol = tol_for(cfg)
    prompt = synthetic.make_tokens(V, (B, P), seed=30)
    params = synthetic.default_sampler_params(max_steps=ROUNDS, seed=5, selfcond_on=1, **over)
    print(f"block loop vs oracle: {name} x{scale} {variant} {over}", flush=True)

    mc = binding.Model(cfg, W, batch=B, capacity=P + 2 * N)
    mc.encode_prompt(to_dev(prompt))
    if variant == "split":
        # a stop threshold between the two canvases' round-0 mean entropies:
        # the surer canvas stops after its first round, the other runs on
        probe, _ = sampler_run(mc, dict(params, max_steps=1), V, N)
        mc.set_kv_length(P)
        h0 = [mean_entropy(probe[0]["stats"][b]) for b in range(B)]
        print(f"round-0 mean entropies {h0}", flush=True)
        assert abs(h0[0] - h0[1]) > 1e-3
        params.update(stop_tau=0.5 * (h0[0] + h0[1]), require_stable=0)
    elif variant == "all_early":
        params.update(stop_tau=1e9, require_stable=0)
    recs, steps_c = sampler_run(mc, params, V, N)

    mg = binding.Model(cfg, W, batch=B, capacity=P + 2 * N, generate_ws=True)
    mg.encode_prompt(to_dev(prompt))
    block = torch.zeros((B, N), dtype=torch.int32, device=DEV)
    trace = torch.full((params["max_steps"], B, 2), -7.0, dtype=torch.float32, device=DEV)
    steps_g = mg.generate_block(params, 0, block, trace=trace)
    torch.cuda.synchronize()
    block_g = block.cpu().numpy()
    trace = trace.cpu().numpy()
    Kg, Vg = [t[0].float().cpu().numpy() for t in mg.kv_tensors()]
    assert steps_g == steps_c
    assert (block_g == recs[-1]["argmax"]).all()
    if variant == "split":
        assert steps_g[0] != steps_g[1]
    elif variant == "all_early":
        assert steps_g == [1, 1]
    else:
        assert steps_g == [ROUNDS, ROUNDS]
    locks = np.stack([r["lock"] for r in recs])
    assert locks.any() and not locks.all(), "the lock rule should lock some positions"

    # the block's starting canvas: Philox counter (block, b, i, 1)
    assert (recs[0]["canvas_in"] == osampler.canvas_init(params["seed"], 0, B, N, V)).all()
    W64 = synthetic.to_float64(W)
    cache = om.KVCache(cfg, B)
    om.encode(prompt, W64, cfg, cache)
    assert normwise(Kg[:, :, :P], cache.k[0]) <= tol and normwise(Vg[:, :, :P], cache.v[0]) <= tol
    top_k = params.get("top_k", 0)
    gap = 1e-4 if cfg["dtype"] == "f32" else 3e-2
    seen = []

    def active_at(t):
        return np.ones(B, bool) if t == 0 else recs[t - 1]["stop"] == 0

    def hook(t, logits_o):
        assert t < len(recs), "the oracle runs more rounds than the GPU"
        r = recs[t]
        for b in np.flatnonzero(active_at(t)):
            assert (r["canvas_in"][b] == (seen[-1]["canvas"][b] if t else
                                          recs[0]["canvas_in"][b])).all()
            prev_b = None if t == 0 else recs[t - 1]["logits"][b].astype(np.float64)
            keep = route_keep(r["canvas_in"][b], prev_b, W64, cfg, cache, b,
                              top_k if t else 0, gap)
            assert keep.mean() >= (0.99 if cfg["dtype"] == "f32" else 0.5)
            err = normwise(r["logits"][b][keep], logits_o[b][keep])
            print(f"round {t} canvas {b}: logits {err:.3e} over {int(keep.sum())} positions",
                  flush=True)
            assert err <= tol
        return r["logits"].astype(np.float64)

    def on_round(t, canvas, argmax, lock, stats, stop):
        r = recs[t]
        act = active_at(t)
        assert (canvas == r["canvas"]).all(), f"round {t}: canvas"
        assert (argmax == r["argmax"]).all(), f"round {t}: argmax"
        assert (stop == r["stop"]).all(), f"round {t}: stop flags"
        assert (lock[act] == r["lock"][act]).all(), f"round {t}: locks"
        assert (stats[act].view(np.uint32) == r["stats"][act].view(np.uint32)).all(), \
            f"round {t}: statistics"
        # dg_generate_block_trace: the mean entropy the stop rule tested and the
        # locked count, for every canvas that ran this round (bit for bit)
        for b in np.flatnonzero(act):
            assert np.float32(trace[t, b, 0]) == np.float32(mean_entropy(stats[b])), \
                f"round {t} canvas {b}: traced mean entropy"
            assert trace[t, b, 1] == float(lock[b].sum()), f"round {t} canvas {b}: locked count"
        seen.append(dict(canvas=canvas.copy()))

    block_o, steps_o = driver.generate_block(W64, cfg, cache, params, 0, B, selfcond=True,
                                             logits_hook=hook, round_hook=on_round)
    assert len(seen) == len(recs)
    assert steps_o.tolist() == steps_g
    # rounds a canvas did not run are not written
    for b in range(B):
        assert (trace[steps_g[b]:, b] == -7.0).all()
    assert (block_o == block_g).all()
    # the committed block: the oracle's float64 encode against the GPU's cache
    assert cache.length == P + N
    assert normwise(Kg[:, :, P:P + N], cache.k[0][:, :, P:P + N]) <= tol
    assert normwise(Vg[:, :, P:P + N], cache.v[0][:, :, P:P + N]) <= tol
