"""Quantised experts on the block-scaled MFMA at full size: one layer of the
full-size model (d 2048, 128 experts top-8, d_ff 768) with MXFP4 or E4M3
expert weights, quantised on the GPU by the library's own quantisers
(bit-exact against the oracle's in test_gpu_fp8.py), read back out of their
tiled layout and dequantised for the oracle.  The MoE stage (dg_stage_moe) runs on 256 tokens and is compared with
the oracle's MoE fed the GPU's route set, with its expert inputs rounded to
MXFP8 (oracle.model.moe, act_mx8) -- every token and feature.

Router cases: uniform (about 16 tokens per expert: chunks of one or two
16-token tiles), 48 of the tokens pushed towards eight experts (those take 33
to 64 tokens: chunks of three or four tiles, whose rows 32..63 take the
second token load), and 160 pushed (more than 64: several 64-token chunks,
the last one ragged)."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_denoise_amd import binding, synthetic
from oracle import model as om
from oracle import quant as oq

import chain
from helpers import DEV, TOL_BF16, untile_e4m3, untile_mxfp4

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def router_weights(cfg, seed):
    """Router rows drawn on the host (seeded), rounded to bf16 values, so the
    token counts of each case can be worked out without a GPU."""
    rng = np.random.default_rng(seed)
    r = (rng.standard_normal((cfg["n_experts"], cfg["d_model"])) * 0.02).astype(np.float32)
    return torch.from_numpy(r).to(torch.bfloat16).float().numpy()


def stage_input(cfg, router, pushed):
    """256 token rows: standard normal; the first `pushed` rows also carry a
    shared direction along the router rows of experts 0..7, strong enough to
    put those experts in their top-8, so experts 0..7 take about `pushed`
    tokens plus their share of the rest."""
    T, d = cfg["canvas"], cfg["d_model"]
    rng = np.random.default_rng(pushed + 1)
    h = rng.standard_normal((T, d)).astype(np.float32)
    dirn = router[:8].sum(axis=0).astype(np.float64)
    h[:pushed] += (3.0 * dirn / np.linalg.norm(dirn) * np.sqrt(d)).astype(np.float32)
    return h


def quantised_layer(cfg, seed):
    """Full-size layer weights drawn on the GPU, experts quantised by the
    library; returns (device weights, host float64/float32 weights for the
    oracle)."""
    d, F, E = cfg["d_model"], cfg["d_ff"], cfg["n_experts"]
    Hq, Hkv, dh, V = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["vocab"]
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)

    def draw(*shape):
        return (torch.randn(shape, generator=g, device=DEV, dtype=torch.float32) * 0.02).to(
            torch.bfloat16)

    ones = torch.ones(d, device=DEV, dtype=torch.float32)
    router = router_weights(cfg, seed)
    lw = {"attn_norm": ones, "wq": draw(Hq * dh, d), "wk": draw(Hkv * dh, d),
          "wv": draw(Hkv * dh, d), "wo": draw(d, Hq * dh), "moe_norm": ones,
          "w_router": torch.from_numpy(router).to(DEV).to(torch.bfloat16),
          "w_gate": draw(E, F, d), "w_up": draw(E, F, d), "w_down": draw(E, d, F)}
    host = {"moe_norm": np.ones(d), "w_router": router}
    for k, side in (("w_gate", "gate"), ("w_up", "up"), ("w_down", "down")):
        w = lw[k]
        R, K = w.numel() // w.shape[-1], w.shape[-1]
        if cfg["expert_dtype"] == "mxfp4":
            q = torch.empty(w.shape[:-1] + (K // 2,), dtype=torch.uint8, device=DEV)
            sc = torch.empty(w.numel() // 32, dtype=torch.uint8, device=DEV)
            binding.quantize_mxfp4(w, q, sc)
            lw[k], lw["x_" + side] = q, sc
            packed, scr = untile_mxfp4(q.cpu().numpy().reshape(-1), sc.cpu().numpy(), R, K)
            host[k] = oq.mx_dequantize_rows(oq.mx_unpack(packed), scr).reshape(w.shape).astype(
                np.float32)
        else:
            q = torch.empty(w.shape, dtype=torch.uint8, device=DEV)
            sc = torch.empty(w.shape[:-1], dtype=torch.float32, device=DEV)
            binding.quantize_fp8(w, q, sc)
            lw[k], lw["s_" + side] = q, sc
            host[k] = oq.dequantize_rows(untile_e4m3(q.cpu().numpy().reshape(-1), R, K),
                                         sc.cpu().numpy().reshape(R)).reshape(w.shape).astype(
                                             np.float32)
    torch.cuda.synchronize()
    W = {"embed": draw(V, d), "w_sc": draw(d, d), "final_norm": ones, "layers": [lw]}
    return W, host


@pytest.fixture(scope="module", params=["mxfp4", "fp8"])
def mx_layer(request):
    cfg = synthetic.model_config("layer_" + request.param, n_layers=1)
    print(f"quantising a full-size {request.param} layer on the GPU", flush=True)
    W, host = quantised_layer(cfg, seed=3)
    m = binding.Model(cfg, W, batch=1, capacity=cfg["canvas"] + 64)
    yield cfg, m, host
    del m, W
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pushed", [0, 48, 160])
def test_mx_moe_stage_full_size(mx_layer, pushed):
    cfg, m, host = mx_layer
    k = cfg["top_k"]
    h = stage_input(cfg, host["w_router"], pushed)
    hd = torch.from_numpy(h).to(DEV)
    print(f"{cfg['expert_dtype']} MoE stage, {pushed} tokens pushed", flush=True)
    err, _ = chain.check_moe(m, cfg, host, 0, hd, TOL_BF16,
                             label=f"{cfg['expert_dtype']} pushed {pushed}")
    # the chunk sizes this case exercised
    u = om.rmsnorm(h.astype(np.float64), host["moe_norm"], cfg["rms_eps"])
    idx, _ = om.route(u @ host["w_router"].T.astype(np.float64), k)
    counts = np.bincount(idx.ravel(), minlength=cfg["n_experts"])
    print(f"tokens per expert: max {counts.max()}, experts with > 32: {(counts > 32).sum()}, "
          f"> 64: {(counts > 64).sum()}; error {err:.3e}", flush=True)
    if pushed == 48:
        assert ((counts > 32) & (counts <= 64)).any()
    if pushed == 160:
        assert (counts > 64).any() and (counts % 64 != 0).any()
