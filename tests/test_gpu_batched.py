"""Batched canvases at full size: eight 256-token canvases with 8192-token
prompts each through one full-size denoiser layer (d 2048, 16 query / 4 KV
heads x 128, 128 experts top-8, d_ff 768, vocabulary 262144, bf16), with the
self-conditioning truncated to each position's 64 largest previous logits
(the high-batch sampler setting), in the launch configuration the benchmark's
batched workload times.  Two canvases, one at each end of the batch, are
checked against the float64 oracle: their slices of the KV cache, and the
logits of sampled positions.  Every canvas of the batch runs in the same
launches, so a canvas that reads another's rows or cache would show here."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_denoise_amd import binding, synthetic
from oracle import model as om

from helpers import DEV, TOL_BF16, normwise, route_ambiguous, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

CHECKED = (0, 7)       # canvases compared with the oracle
SAMPLE_ROWS = 16       # positions per checked canvas
TOP_K = 64
ROUTE_GAP = 3e-2       # see route_gap() in test_gpu_model.py


@pytest.fixture(scope="module")
def batched_run():
    shape = synthetic.SHAPES["batched"]
    cfg = synthetic.model_config("batched", n_layers=1)
    B, P, N, V = shape["batch"], shape["prompt"], cfg["canvas"], cfg["vocab"]
    print(f"generating full-size layer weights; batch {B}, prompt {P}", flush=True)
    W = synthetic.make_weights(cfg, seed=0)
    prompt = synthetic.make_tokens(V, (B, P), seed=1)
    canvas = synthetic.make_tokens(V, (B, N), seed=2)
    m = binding.Model(cfg, W, batch=B, capacity=P + N)
    prev = torch.empty((B, N, V), dtype=torch.float32, device=DEV)
    prev_host = {}
    for b in range(B):
        pb = synthetic.make_logits((1, N, V), seed=100 + b, sigma=2.0)
        prev[b].copy_(torch.from_numpy(pb[0]))
        if b in CHECKED:
            prev_host[b] = pb[0]
    m.encode_prompt(to_dev(prompt))
    logits = torch.empty((B, N, V), dtype=torch.float32, device=DEV)
    m.denoise_step(to_dev(canvas), logits, prev, None, top_k=TOP_K)
    torch.cuda.synchronize()
    K, Vc = m.kv_tensors()
    out = dict(cfg=cfg, W=W, prompt=prompt, canvas=canvas, prev=prev_host, P=P,
               logits={b: logits[b].cpu().numpy() for b in CHECKED},
               K={b: K[0, b, :, :P].float().cpu().numpy() for b in CHECKED},
               V={b: Vc[0, b, :, :P].float().cpu().numpy() for b in CHECKED},
               finite=bool(torch.isfinite(logits).all().item()))
    del m, logits, prev
    torch.cuda.empty_cache()
    lw = {k: np.asarray(v, dtype=np.float64) if k.endswith("norm") or k in ("wq", "wk", "wv", "wo")
          else v for k, v in W["layers"][0].items()}
    out["Wk"] = {"embed": W["embed"], "w_sc": W["w_sc"], "final_norm": W["final_norm"],
                 "layers": [lw]}
    out["cache"] = {}
    for b in CHECKED:
        print(f"oracle encode of canvas {b}'s prompt", flush=True)
        cache = om.KVCache(cfg, 1)
        om.encode(prompt[b:b + 1], out["Wk"], cfg, cache)
        out["cache"][b] = cache
    return out


@pytest.mark.parametrize("b", CHECKED)
def test_batched_prompt_kv(batched_run, b):
    r = batched_run
    c = r["cache"][b]
    assert normwise(r["K"][b], c.k[0][0]) <= TOL_BF16
    assert normwise(r["V"][b], c.v[0][0]) <= TOL_BF16


@pytest.mark.parametrize("b", CHECKED)
def test_batched_topk_selfcond_step_sampled_rows(batched_run, b):
    r = batched_run
    assert r["finite"]
    cfg, Wk, cache = r["cfg"], r["Wk"], r["cache"][b]
    P = cache.length
    print(f"oracle step, canvas {b}", flush=True)
    h = om.denoiser_input(r["canvas"][b], Wk, r["prev"][b], TOP_K)
    lw = Wk["layers"][0]
    h, _, _ = om.attn_half(h, lw, cfg, cache.k[0][0], cache.v[0][0], P, causal=False)
    u = om.rmsnorm(h, lw["moe_norm"], cfg["rms_eps"])
    amb = route_ambiguous(u @ np.asarray(lw["w_router"], np.float64).T, cfg["top_k"], ROUTE_GAP)
    h, _, _, _ = om.moe_half(h, lw, cfg)
    rows = np.flatnonzero(~amb)
    rows = rows[np.linspace(0, rows.size - 1, SAMPLE_ROWS).astype(int)]
    ref = om.head(h[rows], Wk, cfg)
    got = r["logits"][b][rows]
    err = normwise(got, ref)
    print(f"canvas {b}: sampled-row normwise error {err:.3e}; near-tie rows {amb.sum()}",
          flush=True)
    assert err <= TOL_BF16
