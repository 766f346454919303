"""Route-fed stage chain: the library's denoiser stages run one call at a time
(dg_stage_input / dg_stage_attention / dg_stage_moe / dg_stage_head), and the
float64 oracle recomputes every stage from the GPU's own input to it.  In the
MoE the oracle takes the GPU's route set (oracle.model.moe(idx=...)) once the
route has been checked: the chosen experts are distinct, each is within the
tie gap of the k-th largest oracle router logit, the set equals the oracle's
own top-k wherever the oracle's k-th and (k+1)-th logits are further apart
than the gap, and at most 1 % of tokens are that close.  So every position
is compared, none is dropped as a near tie, and a bf16 rounding that moves a
route by one expert cannot turn the comparison of the layers after it into a
comparison of two different computations.

Attention and MoE are compared on their contribution to the residual stream
(output minus input), so the residual cannot hide an error in them; the
canvas K/V the attention stage writes into the cache are compared too.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import model as om

from helpers import DEV, normwise, route_ambiguous, route_is_valid

ROUTE_GAP = 1e-4     # router-logit tie gap on identical inputs (fp32 router on both sides)
MAX_TIES = 0.01      # tokens closer than the gap to a tie: at most 1 % (one on tiny batches)


def layer64(lw: dict) -> dict:
    """A layer's weights for the oracle: norms and attention projections as
    float64, expert matrices kept as float32 (bf16-exact values; numpy widens
    them to float64 inside each product).  Accepts numpy arrays or torch
    tensors."""
    out = {}
    for k, v in lw.items():
        if k.startswith("s_") or k.startswith("x_"):
            continue
        a = v.float().cpu().numpy() if isinstance(v, torch.Tensor) else np.asarray(v)
        if k in ("w_gate", "w_up", "w_down", "w_router"):
            out[k] = np.ascontiguousarray(a, dtype=np.float32)
        else:
            out[k] = np.asarray(a, dtype=np.float64)
    return out


def host64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def check_attention(m, cfg, lw, layer, h, n, causal, tol, label=""):
    """Runs dg_stage_attention on h [B*n, d] (device, modified in place) over
    the cache's current context and checks it against the oracle, per
    sequence, from the same h and the same cached K/V.  Returns the largest
    normwise error of the attention output."""
    B = m.batch
    P = m.kv_length
    h_in = host64(h)
    K, V = m.kv_tensors()
    kctx = host64(K[layer, :, :, :P])
    vctx = host64(V[layer, :, :, :P])
    m.stage_attention(layer, h, n, causal)
    torch.cuda.synchronize()
    h_out = host64(h)
    knew = host64(K[layer, :, :, P:P + n])
    vnew = host64(V[layer, :, :, P:P + n])
    worst = 0.0
    for b in range(B):
        rows = slice(b * n, (b + 1) * n)
        ref, kn, vn = om.attn_half(h_in[rows], lw, cfg, kctx[b], vctx[b], P, causal=causal)
        err = normwise(h_out[rows] - h_in[rows], ref - h_in[rows])
        ek, ev = normwise(knew[b], kn), normwise(vnew[b], vn)
        print(f"{label} attention layer {layer} seq {b}: output {err:.3e}, new K {ek:.3e}, "
              f"new V {ev:.3e}", flush=True)
        assert err <= tol, (label, layer, b, err)
        assert ek <= tol and ev <= tol, (label, layer, b, ek, ev)
        worst = max(worst, err)
    return worst


def check_moe(m, cfg, lw, layer, h, tol, label=""):
    """Runs dg_stage_moe on h [T, d] (device, modified in place) and checks the
    route and the MoE output against the oracle fed the GPU's route set.
    Returns (normwise error, fraction of near-tie tokens)."""
    T = h.shape[0]
    k = cfg["top_k"]
    h_in = host64(h)
    route = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    gates = torch.zeros((T, k), dtype=torch.float32, device=DEV)
    m.stage_moe(layer, h, route, gates)
    torch.cuda.synchronize()
    r = route.cpu().numpy().astype(np.int64)
    g = gates.cpu().numpy()
    d_got = host64(h) - h_in
    u = om.rmsnorm(h_in, lw["moe_norm"], cfg["rms_eps"])
    z = u @ lw["w_router"].T
    amb = route_ambiguous(z, k, ROUTE_GAP)
    assert route_is_valid(z, r, k, ROUTE_GAP), (label, layer)
    assert amb.sum() <= max(1, int(MAX_TIES * T)), (label, layer, int(amb.sum()))
    idx, _ = om.route(z, k)
    same = (np.sort(r, axis=1) == np.sort(idx, axis=1)).all(axis=1)
    assert same[~amb].all(), (label, layer, "route set differs off near ties")
    y, _, gref, _ = om.moe(u, lw, k, idx=r, act_mx8=om.act_mx8(cfg))
    err = normwise(d_got, y)
    eg = normwise(g, gref)
    print(f"{label} MoE layer {layer}: output {err:.3e}, gates {eg:.3e}, near ties "
          f"{int(amb.sum())}/{T}, oracle route kept on {int(same.sum())}/{T}", flush=True)
    assert err <= tol, (label, layer, err)
    assert eg <= tol, (label, layer, eg)
    return err, float(amb.mean())


def check_head(m, cfg, W, h, tol, label="", rows=None):
    """dg_stage_head on h [T, d] against the oracle's head on the same h.
    rows: optional row subset the oracle computes (all by default).  Returns
    the device logits."""
    T = h.shape[0]
    logits = torch.empty((T, cfg["vocab"]), dtype=torch.float32, device=DEV)
    m.stage_head(h, logits)
    torch.cuda.synchronize()
    h64 = host64(h)
    sel = np.arange(T) if rows is None else np.asarray(rows)
    got = logits.cpu().numpy()[sel]
    ref = om.head(h64[sel], W, cfg)
    err = normwise(got, ref)
    print(f"{label} head: logits {err:.3e} over {sel.size} rows x {cfg['vocab']}", flush=True)
    assert err <= tol, (label, err)
    assert np.isfinite(got).all()
    return logits
