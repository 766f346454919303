"""GPU denoiser path through the C ABI against the float64 oracle, on the
tiny fp32 model (1e-4) and small bf16 models (2e-2): prompt encode (KV
cache), each stage of the step with identical synthetic inputs, the whole
step with and without self-conditioning, commit == re-encode, and the block
loop == its own composition of calls."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_denoise_amd import binding, synthetic
from oracle import model as om
from oracle import quant as oq
from oracle import sampler as osampler

import chain
from helpers import (DEV, TOL_F32, normwise, round_model_dtype, route_ambiguous, route_is_valid,
                     tile_e4m3, tile_mxfp4, to_dev, tol_for)

pytestmark = pytest.mark.gpu

TINY = synthetic.SHAPES["tiny"]
# bf16 model with grouped-query attention and 64 experts, small enough for a
# full float64 reference
SMALL_BF16 = dict(n_layers=2, d_model=512, n_heads=8, n_kv_heads=2, head_dim=64, n_experts=64,
                  top_k=8, d_ff=256, vocab=4096, canvas=256, dtype="bf16")
# 128-wide heads, fp32, grouped queries, odd canvas length
F32_GQA = dict(n_layers=2, d_model=256, n_heads=4, n_kv_heads=2, head_dim=128, n_experts=8,
               top_k=2, d_ff=96, vocab=2048, canvas=100, dtype="f32")

# bf16 with enough 256 x 256 tiles in the two vocabulary products to take
# the direct-to-LDS ring kernel; the ragged variant (canvas 200, vocabulary
# not a multiple of 256 or 128) clamps rows in the head and falls back to the
# double-buffered kernel for self-conditioning
VOCAB_BF16 = dict(n_layers=1, d_model=1024, n_heads=8, n_kv_heads=2, head_dim=128, n_experts=16,
                  top_k=2, d_ff=256, vocab=32768, canvas=256, dtype="bf16")
VOCAB_RAGGED = dict(VOCAB_BF16, vocab=32768 + 96, canvas=200)

# the bf16 model with 8-bit (E4M3, per-row scale) expert weights; the oracle
# runs the dequantised weights
SMALL_FP8 = dict(SMALL_BF16, expert_dtype="fp8")
# ... and with MXFP4 expert weights (E2M1 codes, an E8M0 scale per 32)
SMALL_MXFP4 = dict(SMALL_BF16, expert_dtype="mxfp4")

# bf16 with 128-wide heads (the attention kernel of the full-size layer) at
# query-head groups of 1, 2 and 4 per KV head
ATT128 = dict(n_layers=1, d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, n_experts=8, top_k=2,
              d_ff=256, vocab=2048, canvas=256, dtype="bf16")

# the bf16 model with 30 experts (not a multiple of the fused router's groups
# of four) and 3 per token (no fused combine and norm: the separate kernels
# run inside the production step)
SMALL_E30 = dict(SMALL_BF16, n_experts=30, top_k=3)

MODELS = {"small_e30": SMALL_E30, "tiny": TINY, "small_bf16": SMALL_BF16, "f32_gqa": F32_GQA, "vocab_bf16": VOCAB_BF16,
          "vocab_ragged": VOCAB_RAGGED, "small_fp8": SMALL_FP8, "small_mxfp4": SMALL_MXFP4,
          "att128_g4": ATT128, "att128_g2": dict(ATT128, n_heads=4),
          "att128_g1": dict(ATT128, n_heads=4, n_kv_heads=4)}


def device_form(cfg, W):
    """(weights for the library, weights for the oracle).  8-bit and MXFP4
    experts: the oracle's quantiser gives the codes and scales the library
    runs on, and the oracle runs their dequantised values."""
    if cfg.get("expert_dtype") == "mxfp4":
        Wg = dict(W, layers=[dict(lw) for lw in W["layers"]])
        Wo = dict(W, layers=[dict(lw) for lw in W["layers"]])
        for lg, lo in zip(Wg["layers"], Wo["layers"]):
            for k, xk in (("w_gate", "x_gate"), ("w_up", "x_up"), ("w_down", "x_down")):
                w = lg[k]
                K = w.shape[-1]
                codes, sc = oq.mx_quantize_rows(w.reshape(-1, K))
                lg[k], lg[xk] = tile_mxfp4(oq.mx_pack(codes), sc)
                lo[k] = oq.mx_dequantize_rows(codes, sc).reshape(w.shape)
        return Wg, Wo
    if cfg.get("expert_dtype") != "fp8":
        return W, W
    Wg = dict(W, layers=[dict(lw) for lw in W["layers"]])
    Wo = dict(W, layers=[dict(lw) for lw in W["layers"]])
    for lg, lo in zip(Wg["layers"], Wo["layers"]):
        for k, sk in (("w_gate", "s_gate"), ("w_up", "s_up"), ("w_down", "s_down")):
            w = lg[k]
            q, sc = oq.quantize_rows(w.reshape(-1, w.shape[-1]))
            lg[k] = tile_e4m3(q)
            lg[sk] = sc.reshape(w.shape[:-1])
            lo[k] = oq.dequantize_rows(q, sc).reshape(w.shape)
    return Wg, Wo


def setup(name, prompt_len, batch=1, std=0.05, seed=0, capacity_extra=0, **over):
    cfg = synthetic.model_config(MODELS[name], **over)
    W = synthetic.make_weights(cfg, seed=seed, std=std, random_norms=True)
    Wg, W = device_form(cfg, W)
    N = cfg["canvas"]
    m = binding.Model(cfg, Wg, batch=batch, capacity=prompt_len + N + capacity_extra)
    m.src_weights = Wg
    return cfg, W, m


def route_gap(cfg, chained=False):
    """Router-logit gap below which either expert set is a correct top-k.
    The GPU computes router logits in fp32 (|z| ~ 1), so on identical inputs
    only gaps ~1e-6 are ambiguous.  When layers are chained, the MoE input
    already carries the bf16 error of the previous kernels (~0.3% of h),
    which moves z by up to ~0.015: there the gap is 0.03."""
    return 3e-2 if (chained and cfg["dtype"] == "bf16") else 1e-4


def oracle_encode_with_gaps(prompt, W64, cfg, gap):
    """The oracle's encode, also returning per layer the tokens whose route
    is ambiguous at `gap` (after that layer's attention)."""
    B, P = prompt.shape
    cache = om.KVCache(cfg, B)
    amb = np.zeros((cfg["n_layers"], B, P), dtype=bool)
    for b in range(B):
        h = om.embed(prompt[b], W64)
        for li, lw in enumerate(W64["layers"]):
            h, kn, vn = om.attn_half(h, lw, cfg, np.zeros((cfg["n_kv_heads"], 0, cfg["head_dim"])),
                                     np.zeros((cfg["n_kv_heads"], 0, cfg["head_dim"])), 0, True)
            if b == 0:
                cache.k[li] = np.zeros((B, cfg["n_kv_heads"], P, cfg["head_dim"]))
                cache.v[li] = np.zeros((B, cfg["n_kv_heads"], P, cfg["head_dim"]))
            cache.k[li][b] = kn
            cache.v[li][b] = vn
            u = om.rmsnorm(h, lw["moe_norm"], cfg["rms_eps"])
            amb[li, b] = route_ambiguous(u @ lw["w_router"].T, cfg["top_k"], gap)
            if li + 1 < cfg["n_layers"]:
                h, _, _, _ = om.moe_half(h, lw, cfg)
    cache.length = P
    return cache, amb


ENCODE_CASES = [("tiny", 32, 1), ("small_bf16", 300, 2), ("f32_gqa", 77, 2), ("small_fp8", 300, 2),
                ("small_mxfp4", 300, 2)]


def layers64(W):
    return [chain.layer64(lw) for lw in W["layers"]]


@pytest.mark.parametrize("name,P,B", ENCODE_CASES)
def test_encode_prompt_kv_cache(name, P, B):
    """dg_encode_prompt equals the same encode run as a chain of stage calls
    bit for bit, and every stage of that chain matches the oracle on the
    GPU's own inputs (the MoE with the GPU's route set): every prompt
    token's K/V in every layer is compared."""
    print(f"encode {name} P={P} B={B}", flush=True)
    cfg, W, m = setup(name, P, batch=B)
    prompt = synthetic.make_tokens(cfg["vocab"], (B, P), seed=1)
    m.encode_prompt(to_dev(prompt))
    torch.cuda.synchronize()
    assert m.kv_length == P
    K, V = m.kv_tensors()
    mc = binding.Model(cfg, m.src_weights, batch=B, capacity=P + cfg["canvas"])
    h = to_dev(np.asarray(W["embed"], np.float32)[prompt.reshape(-1)])
    lws = layers64(W)
    tol = tol_for(cfg)
    for l in range(cfg["n_layers"]):
        chain.check_attention(mc, cfg, lws[l], l, h, P, True, tol, label=f"encode {name}")
        if l + 1 < cfg["n_layers"]:
            chain.check_moe(mc, cfg, lws[l], l, h, tol, label=f"encode {name}")
    Kc, Vc = mc.kv_tensors()
    assert torch.equal(Kc[..., :P, :], K[..., :P, :]) and torch.equal(Vc[..., :P, :], V[..., :P, :])


@pytest.mark.parametrize("name,P,B", [c for c in ENCODE_CASES if MODELS[c[0]]["dtype"] == "f32"])
def test_encode_prompt_end_to_end_fp32(name, P, B):
    """fp32 models: the encode against the oracle's own encode (its own
    routes); tokens within 1e-4 of a router tie (at most 1 %) are skipped in
    the layers after it."""
    cfg, W, m = setup(name, P, batch=B)
    prompt = synthetic.make_tokens(cfg["vocab"], (B, P), seed=1)
    m.encode_prompt(to_dev(prompt))
    torch.cuda.synchronize()
    W64 = synthetic.to_float64(W)
    cache, amb = oracle_encode_with_gaps(prompt, W64, cfg, route_gap(cfg))
    K, V = m.kv_tensors()
    assert amb.mean() <= 0.01
    for l in range(cfg["n_layers"]):
        keep = ~amb[:l].any(axis=0) if l > 0 else np.ones((B, P), dtype=bool)
        gk = K[l, :, :, :P].float().cpu().numpy().transpose(0, 2, 1, 3)[keep]
        gv = V[l, :, :, :P].float().cpu().numpy().transpose(0, 2, 1, 3)[keep]
        assert normwise(gk, cache.k[l].transpose(0, 2, 1, 3)[keep]) <= TOL_F32
        assert normwise(gv, cache.v[l].transpose(0, 2, 1, 3)[keep]) <= TOL_F32


STEP_CASES = [("tiny", 32, 1, False, 1, 0), ("tiny", 32, 1, True, 1, 0),
              ("small_bf16", 200, 2, False, 2, 0), ("small_bf16", 200, 2, True, 2, 0),
              ("f32_gqa", 64, 2, True, 2, 0), ("f32_gqa", 64, 1, False, 3, 0),
              ("small_fp8", 200, 2, True, 2, 0), ("small_mxfp4", 200, 2, True, 2, 0),
              ("tiny", 32, 1, True, 1, 64), ("small_bf16", 200, 2, True, 2, 8),
              ("vocab_bf16", 100, 1, True, 1, 0), ("vocab_ragged", 100, 1, True, 1, 0),
              ("small_e30", 200, 2, True, 2, 0)]


def prev_and_stats(B, N, V, seed=4):
    prev = synthetic.make_logits((B, N, V), seed=seed, sigma=2.0)
    stats = np.zeros((B, N, 4), dtype=np.float32)
    for b in range(B):
        for i in range(N):
            stats[b, i], _ = osampler.row_stats(prev[b, i])
    return prev, stats


@pytest.mark.parametrize("name,P,B,selfcond,layers,top_k", STEP_CASES)
def test_denoise_step(name, P, B, selfcond, layers, top_k):
    """dg_denoise_step (dg_denoise_step_topk for top_k > 0) equals the chain
    of its stage calls bit for bit, and every stage of that chain matches
    the oracle on the GPU's own inputs: the input (embedding + self-
    conditioning, full or top-k truncated), each layer's attention and MoE
    (with the GPU's route set), and the head, at every position and every
    logit.  Several bf16 layers are chained this way."""
    print(f"denoise {name} P={P} B={B} selfcond={selfcond} layers={layers} top_k={top_k}",
          flush=True)
    cfg, W, m = setup(name, P, batch=B, n_layers=layers)
    N, V, d = cfg["canvas"], cfg["vocab"], cfg["d_model"]
    prompt = synthetic.make_tokens(V, (B, P), seed=2)
    canvas = synthetic.make_tokens(V, (B, N), seed=3)
    prev, stats = prev_and_stats(B, N, V) if selfcond else (None, None)
    m.encode_prompt(to_dev(prompt))
    logits = torch.empty((B, N, V), dtype=torch.float32, device=DEV)
    if selfcond:
        m.denoise_step(to_dev(canvas), logits, to_dev(prev), to_dev(stats), top_k=top_k)
    else:
        m.denoise_step(to_dev(canvas), logits)
    torch.cuda.synchronize()
    assert m.kv_length == P
    W64 = synthetic.to_float64(W)
    lws = layers64(W)
    tol = tol_for(cfg)
    h = torch.empty((B * N, d), dtype=torch.float32, device=DEV)
    if not selfcond:
        m.stage_input(to_dev(canvas), h)
    elif top_k:
        m.stage_input_topk(to_dev(canvas), h, to_dev(prev), top_k)
    else:
        m.stage_input(to_dev(canvas), h, to_dev(prev), to_dev(stats))
    torch.cuda.synchronize()
    ref_in = np.concatenate([om.denoiser_input(canvas[b], W64, None if prev is None else prev[b],
                                               top_k) for b in range(B)])
    err = normwise(h.cpu().numpy(), ref_in)
    print(f"input: {err:.3e}", flush=True)
    assert err <= tol
    for l in range(layers):
        chain.check_attention(m, cfg, lws[l], l, h, N, False, tol, label=name)
        chain.check_moe(m, cfg, lws[l], l, h, tol, label=name)
    lc = chain.check_head(m, cfg, W64, h, tol, label=name)
    assert torch.equal(lc.view(B, N, V), logits)


@pytest.mark.parametrize("name,P,B,selfcond,layers,top_k",
                         [c for c in STEP_CASES if MODELS[c[0]]["dtype"] == "f32"])
def test_denoise_step_end_to_end_fp32(name, P, B, selfcond, layers, top_k):
    """fp32 models: the whole step against the oracle's own step (its own
    encode and routes); positions within 1e-4 of a router tie in any layer
    (at most 1 %) are skipped."""
    cfg, W, m = setup(name, P, batch=B, n_layers=layers)
    N, V = cfg["canvas"], cfg["vocab"]
    prompt = synthetic.make_tokens(V, (B, P), seed=2)
    canvas = synthetic.make_tokens(V, (B, N), seed=3)
    prev, stats = prev_and_stats(B, N, V) if selfcond else (None, None)
    m.encode_prompt(to_dev(prompt))
    logits = torch.empty((B, N, V), dtype=torch.float32, device=DEV)
    if selfcond:
        m.denoise_step(to_dev(canvas), logits, to_dev(prev), to_dev(stats), top_k=top_k)
    else:
        m.denoise_step(to_dev(canvas), logits)
    torch.cuda.synchronize()
    W64 = synthetic.to_float64(W)
    cache = om.KVCache(cfg, B)
    om.encode(prompt, W64, cfg, cache)
    got = logits.cpu().numpy()
    keep = np.ones((B, N), dtype=bool)
    refs = []
    for b in range(B):
        h = om.denoiser_input(canvas[b], W64, None if prev is None else prev[b], top_k)
        for li, lw in enumerate(W64["layers"]):
            h, _, _ = om.attn_half(h, lw, cfg, cache.k[li][b], cache.v[li][b], P, causal=False)
            u = om.rmsnorm(h, lw["moe_norm"], cfg["rms_eps"])
            keep[b] &= ~route_ambiguous(u @ lw["w_router"].T, cfg["top_k"], route_gap(cfg))
            h, _, _, _ = om.moe_half(h, lw, cfg)
        refs.append(om.head(h, W64, cfg))
    ref = np.stack(refs)
    assert keep.mean() >= 0.99
    err = normwise(got[keep], ref[keep])
    print(f"end-to-end normwise error {err:.3e} over {keep.sum()} positions", flush=True)
    assert err <= TOL_F32
    assert np.isfinite(got).all()


@pytest.mark.parametrize("name,causal,P,N", [("tiny", False, 333, 256), ("tiny", True, 333, 256),
                                             ("small_bf16", False, 333, 256),
                                             ("small_bf16", True, 333, 256),
                                             ("f32_gqa", False, 333, 100),
                                             ("att128_g4", False, 333, 256),
                                             ("att128_g4", True, 333, 256),
                                             ("att128_g4", False, 40, 100),
                                             ("att128_g4", True, 0, 300),
                                             ("att128_g2", False, 1000, 256),
                                             ("att128_g2", True, 77, 33),
                                             ("att128_g1", False, 333, 256),
                                             ("att128_g1", True, 5, 1)])
def test_stage_attention_on_synthetic_cache(name, causal, P, N):
    """Attention half-block with the cache filled directly from synthetic
    values (no encode), so attention is checked on its own: key ranges with
    partial tiles and several splits, causal masks on and off the diagonal,
    ragged and single-token canvases, one, two and four query heads per KV
    head."""
    B = 2
    cfg, W, m = setup(name, P, batch=B, std=0.05, canvas=N)
    d, Hkv, dh = cfg["d_model"], cfg["n_kv_heads"], cfg["head_dim"]
    rng = np.random.default_rng(10)
    kctx = round_model_dtype(cfg, rng.standard_normal((B, Hkv, P, dh)).astype(np.float32))
    vctx = round_model_dtype(cfg, rng.standard_normal((B, Hkv, P, dh)).astype(np.float32))
    K, V = m.kv_tensors()
    K[0, :, :, :P] = to_dev(kctx, m.dtype)
    V[0, :, :, :P] = to_dev(vctx, m.dtype)
    m.set_kv_length(P)
    h = to_dev(rng.standard_normal((B * N, d)).astype(np.float32))
    torch.cuda.synchronize()
    chain.check_attention(m, cfg, chain.layer64(W["layers"][0]), 0, h, N, causal, tol_for(cfg),
                          label=f"{name} P={P} N={N} causal={causal}")


@pytest.mark.parametrize("name,T,top_k", [("tiny", 256, None), ("small_bf16", 512, None),
                                         ("small_bf16", 37, None), ("f32_gqa", 1000, None),
                                         ("small_fp8", 512, None), ("small_fp8", 37, None),
                                         ("small_mxfp4", 512, None), ("small_mxfp4", 37, None),
                                         ("small_bf16", 512, 4), ("small_bf16", 300, 3),
                                         ("small_bf16", 129, 1), ("small_bf16", 256, 16),
                                         ("small_mxfp4", 300, 3), ("small_fp8", 129, 1),
                                         ("small_mxfp4", 256, 16), ("small_e30", 512, None),
                                         ("small_e30", 77, None)])
def test_stage_moe(name, T, top_k):
    """The MoE stage on identical synthetic inputs: the route is a valid top-k
    (the oracle's own set off near ties, at most 1 % of tokens within 1e-4
    of a tie) and the output matches the oracle fed the GPU's route set at
    every token.  top_k 1, 3, 4 and 16 run the combine kernels other than
    the 2- and 8-expert ones (with quantised experts too: work items and
    token chunks of other sizes)."""
    over = {} if top_k is None else {"top_k": top_k}
    cfg, W, m = setup(name, 0, **over)
    rng = np.random.default_rng(11)
    h = to_dev(rng.standard_normal((T, cfg["d_model"])).astype(np.float32))
    chain.check_moe(m, cfg, chain.layer64(W["layers"][0]), 0, h, tol_for(cfg),
                    label=f"{name} T={T} k={cfg['top_k']}")


@pytest.mark.parametrize("name", ["tiny", "small_bf16", "vocab_bf16", "vocab_ragged"])
def test_stage_head_and_input(name):
    cfg, W, m = setup(name, 0)
    N, V, d = cfg["canvas"], cfg["vocab"], cfg["d_model"]
    rng = np.random.default_rng(12)
    h = rng.standard_normal((N, d)).astype(np.float32)
    logits = torch.empty((N, V), dtype=torch.float32, device=DEV)
    m.stage_head(to_dev(h), logits)
    W64 = synthetic.to_float64(W)
    ref = om.head(h.astype(np.float64), W64, cfg)
    torch.cuda.synchronize()
    assert normwise(logits.cpu().numpy(), ref) <= tol_for(cfg)
    # denoiser input with self-conditioning
    canvas = synthetic.make_tokens(V, (1, N), seed=13)
    prev = synthetic.make_logits((1, N, V), seed=14, sigma=3.0)
    stats = np.stack([osampler.row_stats(prev[0, i])[0] for i in range(N)])[None]
    hd = torch.empty((N, d), dtype=torch.float32, device=DEV)
    m.stage_input(to_dev(canvas), hd, to_dev(prev), to_dev(stats))
    torch.cuda.synchronize()
    ref_in = om.denoiser_input(canvas[0], W64, prev[0])
    assert normwise(hd.cpu().numpy(), ref_in) <= tol_for(cfg)


@pytest.mark.parametrize("T", [256, 200])
def test_stage_head_rowmax(T):
    """The blocked head's slab maxima: the same logits as dg_stage_head, and
    rowmax[t][j] == max(logits[t][64 j : 64 j + 64]) exactly; also with a
    ragged row count.  Models without the blocked head refuse the call."""
    cfg, W, m = setup("vocab_bf16", 0)
    V, d = cfg["vocab"], cfg["d_model"]
    h = to_dev(np.random.default_rng(15).standard_normal((T, d)).astype(np.float32))
    a = torch.empty((T, V), dtype=torch.float32, device=DEV)
    b = torch.empty_like(a)
    rowmax = torch.full((T, V // 64), float("nan"), dtype=torch.float32, device=DEV)
    m.stage_head(h, a)
    m.stage_head_rowmax(h, b, rowmax)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(rowmax, b.view(T, V // 64, 64).amax(dim=-1))
    cr, _, mr = setup("vocab_ragged", 0)
    lr = torch.empty((200, cr["vocab"]), dtype=torch.float32, device=DEV)
    rr = torch.empty((200, cr["vocab"] // 64 + 1), dtype=torch.float32, device=DEV)
    with pytest.raises(binding.DGError):
        mr.stage_head_rowmax(h[:200].contiguous(), lr, rr)


@pytest.mark.parametrize("T", [1, 7, 16, 17, 130, 256, 300, 700])
def test_blocked_head_row_counts(T):
    """The blocked head at the row counts that pick its kernels: the few-row
    decode-step kernel (T <= 16) and the persistent kernel with one, two and
    three row tiles, ragged ones included.  Logits against the float64
    oracle; slab maxima exactly the maxima of the returned logits."""
    print(f"blocked head T={T}", flush=True)
    # a 700-token canvas: the stage calls' workspace (one canvas) holds 768
    # blocked rows
    cfg, W, m = setup("vocab_bf16", 0, canvas=700)
    V, d = cfg["vocab"], cfg["d_model"]
    h = np.random.default_rng(100 + T).standard_normal((T, d)).astype(np.float32)
    logits = torch.full((T, V), float("nan"), dtype=torch.float32, device=DEV)
    rowmax = torch.full((T, V // 64), float("nan"), dtype=torch.float32, device=DEV)
    m.stage_head_rowmax(to_dev(h), logits, rowmax)
    torch.cuda.synchronize()
    ref = om.head(h.astype(np.float64), synthetic.to_float64(W), cfg)
    assert normwise(logits.cpu().numpy(), ref) <= tol_for(cfg)
    assert torch.equal(rowmax, logits.view(T, V // 64, 64).amax(dim=-1))


def test_commit_equals_encode_of_concatenation():
    cfg, W, m1 = setup("small_bf16", 50, batch=1)
    N, V = cfg["canvas"], cfg["vocab"]
    prompt = synthetic.make_tokens(V, (1, 50), seed=20)
    block = synthetic.make_tokens(V, (1, N), seed=21)
    m1.encode_prompt(to_dev(prompt))
    m1.commit_block(to_dev(block))
    m2 = binding.Model(cfg, m1.src_weights, batch=1, capacity=50 + 2 * N)
    m2.encode_prompt(to_dev(np.concatenate([prompt, block], axis=1)))
    torch.cuda.synchronize()
    assert m1.kv_length == m2.kv_length == 50 + N
    K1, V1 = m1.kv_tensors()
    K2, V2 = m2.kv_tensors()
    L = 50 + N
    assert normwise(K1[..., :L, :].float().cpu().numpy(), K2[..., :L, :].float().cpu().numpy()) < 1e-6
    assert normwise(V1[..., :L, :].float().cpu().numpy(), V2[..., :L, :].float().cpu().numpy()) < 1e-6


@pytest.mark.parametrize("name,B,selfcond,early,top_k", [("tiny", 1, True, False, 0),
                                                         ("small_bf16", 2, True, False, 0),
                                                         ("vocab_bf16", 1, True, False, 0),
                                                         ("small_fp8", 2, True, False, 0),
                                                         ("small_mxfp4", 2, True, False, 0),
                                                         ("small_bf16", 2, False, False, 0),
                                                         ("small_bf16", 2, True, True, 0),
                                                         ("tiny", 1, True, False, 16),
                                                         ("small_bf16", 2, True, False, 64),
                                                         ("vocab_bf16", 1, True, False, 32)])
def test_generate_block_is_its_composition(name, B, selfcond, early, top_k):
    """dg_generate_block == canvas init + (denoise, sample) rounds + commit,
    driven call by call; bitwise identical block, round counts and cache.
    early: every sequence stops after its first round (entropy threshold
    above any entropy, no stability condition), so the loop's look-ahead
    round runs after the stop and must leave the block untouched."""
    P = 40
    cfg, W, m = setup(name, P, batch=B, capacity_extra=0)
    N, V = cfg["canvas"], cfg["vocab"]
    prompt = synthetic.make_tokens(V, (B, P), seed=30)
    if early:
        params = synthetic.default_sampler_params(max_steps=5, seed=5, selfcond_on=int(selfcond),
                                                  stop_tau=1e9, require_stable=0, top_k=top_k)
    else:
        params = synthetic.default_sampler_params(max_steps=3, seed=5, selfcond_on=int(selfcond),
                                                  top_k=top_k)
    # library loop
    mg = binding.Model(cfg, m.src_weights, batch=B, capacity=P + 2 * N, generate_ws=True)
    mg.encode_prompt(to_dev(prompt))
    block = torch.zeros((B, N), dtype=torch.int32, device=DEV)
    steps = mg.generate_block(params, 0, block)
    torch.cuda.synchronize()
    # the same rounds, one call at a time
    mc = binding.Model(cfg, m.src_weights, batch=B, capacity=P + 2 * N)
    mc.encode_prompt(to_dev(prompt))
    canvas = torch.zeros((B, N), dtype=torch.int32, device=DEV)
    binding.canvas_init(params["seed"], 0, canvas, V)
    argmax = torch.zeros((B, N), dtype=torch.int32, device=DEV)
    lock = torch.zeros((B, N), dtype=torch.uint8, device=DEV)
    stop = torch.zeros(B, dtype=torch.int32, device=DEV)
    lg = [torch.empty((B, N, V), dtype=torch.float32, device=DEV) for _ in range(2)]
    st = [torch.empty((B, N, 4), dtype=torch.float32, device=DEV) for _ in range(2)]
    ws = binding.sampler_workspace(B, N)
    prev = prev_st = None
    my_steps = [0] * B
    for t in range(params["max_steps"]):
        mc.denoise_step(canvas, lg[t % 2], prev, prev_st, top_k=top_k if prev is not None else 0)
        binding.sample_update(params, t, lg[t % 2], canvas, argmax, lock, st[t % 2], stop, ws)
        s = stop.cpu().tolist()
        for b in range(B):
            if my_steps[b] == 0 and s[b]:
                my_steps[b] = t + 1
        if all(s):
            break
        if selfcond:
            prev, prev_st = lg[t % 2], st[t % 2]
    mc.commit_block(argmax)
    torch.cuda.synchronize()
    assert steps == my_steps == ([1] * B if early else [3] * B)
    assert (block.cpu().numpy() == argmax.cpu().numpy()).all()
    assert mg.kv_length == mc.kv_length == P + N
    K1, V1 = mg.kv_tensors()
    K2, V2 = mc.kv_tensors()
    L = P + N
    assert torch.equal(K1[..., :L, :], K2[..., :L, :]) and torch.equal(V1[..., :L, :], V2[..., :L, :])


def test_generate_block_reports_nonfinite_logits():
    """A canvas whose logits turn non-finite (here: a NaN planted in canvas
    1's cached prompt V, which only its own attention reads; the output head
    shares the embedding, so a NaN embedding row would reach every canvas's
    logits) stops in that round while canvas 0 runs on; dg_generate_block
    returns DG_ERR_NONFINITE naming canvas 1 and commits nothing."""
    P = 40
    cfg, W, m = setup("tiny", P, batch=2)
    N, V = cfg["canvas"], cfg["vocab"]
    params = synthetic.default_sampler_params(max_steps=3, seed=5)
    prompt = synthetic.make_tokens(V, (2, P), seed=30)
    mg = binding.Model(cfg, W, batch=2, capacity=P + 2 * N, generate_ws=True)
    mg.encode_prompt(to_dev(prompt))
    K, Vc = mg.kv_tensors()
    Vc[0, 1, :, 7] = float("nan")
    torch.cuda.synchronize()
    block = torch.zeros((2, N), dtype=torch.int32, device=DEV)
    with pytest.raises(binding.DGError) as e:
        mg.generate_block(params, 0, block)
    assert e.value.status == 5 and "canvas 1" in str(e.value)
    assert "canvas 0" not in str(e.value)
    assert mg.kv_length == P
    assert torch.isfinite(K[..., :P, :].float()).all()
    assert torch.isfinite(Vc[:, 0, :, :P].float()).all()


def test_step_is_deterministic():
    cfg, W, m = setup("small_bf16", 100, batch=1)
    N, V = cfg["canvas"], cfg["vocab"]
    m.encode_prompt(to_dev(synthetic.make_tokens(V, (1, 100), seed=40)))
    canvas = to_dev(synthetic.make_tokens(V, (1, N), seed=41))
    a = torch.empty((1, N, V), dtype=torch.float32, device=DEV)
    b = torch.empty_like(a)
    m.denoise_step(canvas, a)
    m.denoise_step(canvas, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
