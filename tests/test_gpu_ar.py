"""Retained autoregressive mode on the GPU through the C ABI: the greedy
choice bit-exact against numpy's argmax (ties to the lower index); decode
steps after a prompt encode against the float64 oracle stage by stage on the
GPU's own inputs (the MoE with the GPU's route set; fp32 1e-4, bf16 2e-2),
every sequence, and for fp32 models also end to end against the oracle's own
encode and decode; greedy generation bitwise equal to its own composition of
decode steps and greedy choices; one decode step of the full-size layer
(vocabulary 262144, prompt 2048) against the oracle."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_denoise_amd import binding, synthetic
from oracle import model as om

import chain
from helpers import DEV, TOL_BF16, TOL_F32, normwise, route_ambiguous, to_dev, tol_for

pytestmark = pytest.mark.gpu

from test_gpu_model import MODELS, device_form, route_gap  # noqa: E402


def setup(name, capacity, batch, std=0.05, seed=0, **over):
    cfg = synthetic.model_config(MODELS[name], **over)
    W = synthetic.make_weights(cfg, seed=seed, std=std, random_norms=True)
    Wg, W = device_form(cfg, W)
    m = binding.Model(cfg, Wg, batch=batch, capacity=capacity)
    m.src_weights = Wg
    return cfg, W, m


# ------------------------------------------------------------------ greedy


def argmax_case(kind, R, V, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, V), dtype=np.float32)
    if kind == "ties":
        # the maximum planted twice (and three times in the last row)
        for r in range(R):
            a, b = sorted(rng.choice(V, 2, replace=False))
            x[r, a] = x[r, b] = 9.0
        x[-1, V - 1] = 9.0
    elif kind == "flat":
        x[:] = 0.5
        x[0, :] = -np.inf
        x[1, :] = 0.0
        x[1, ::2] = -0.0
    elif kind == "nan":
        # NaN ranks above every number: the first NaN of a row is its choice
        x[0, 5] = x[0, 3000 % V] = np.nan
        x[1, V - 1] = np.nan
        x[1, 0] = np.inf
        x[2, :] = np.nan
    elif kind == "edges":
        x[0, 0] = 50.0
        x[1, V - 1] = 50.0
        x[2, 63] = x[2, 64] = 50.0
    return x


ARGMAX_CASES = [("normal", 4, 262144), ("ties", 5, 262144), ("flat", 3, 4096),
                ("edges", 3, 1001), ("ties", 3, 4099), ("normal", 1, 1),
                ("nan", 3, 262144), ("nan", 3, 4099)]


@pytest.mark.parametrize("kind,R,V", ARGMAX_CASES)
def test_argmax_rows_bit_exact(kind, R, V):
    print(f"argmax {kind} R={R} V={V}", flush=True)
    x = argmax_case(kind, R, V, seed=R * 7 + V)
    out = torch.full((R,), -1, dtype=torch.int32, device=DEV)
    binding.argmax_rows(to_dev(x), out)
    torch.cuda.synchronize()
    assert out.cpu().numpy().tolist() == np.argmax(x, axis=1).tolist()


# ------------------------------------------------------------------ decode


def oracle_decode_with_gaps(tokens, W, cfg, cache, gap):
    """om.ar_decode_step, also returning per sequence whether any layer's
    route of this token is ambiguous at `gap`."""
    B = tokens.size
    amb = np.zeros(B, dtype=bool)
    # the route check on a copy of the cache, layer by layer, mirrors the
    # step itself
    c2 = cache.copy()
    for b in range(B):
        h = om.embed(tokens[b:b + 1], W)
        for li, lw in enumerate(W["layers"]):
            h, _, _ = om.attn_half(h, lw, cfg, c2.k[li][b][:, :c2.length],
                                   c2.v[li][b][:, :c2.length], c2.length, causal=True)
            u = om.rmsnorm(h, lw["moe_norm"], cfg["rms_eps"])
            amb[b] |= bool(route_ambiguous(u @ np.asarray(lw["w_router"]).T, cfg["top_k"], gap)[0])
            h, _, _, _ = om.moe_half(h, lw, cfg)
    return om.ar_decode_step(tokens, W, cfg, cache), amb


def decode_chain_check(m, cfg, W, tok, logits, tol, label):
    """The decode step just taken (logits of tokens tok [B] at position L0 =
    len - 1) run again as a chain of stage calls over the same cache, each
    stage against the oracle on the GPU's own input to it (the MoE with the
    GPU's route set); the chain's logits equal the step's bit for bit."""
    L0 = m.kv_length - 1
    m.set_kv_length(L0)
    h = to_dev(np.asarray(W["embed"], np.float32)[tok])
    for l, lw in enumerate(W["layers"]):
        lw = chain.layer64(lw)
        chain.check_attention(m, cfg, lw, l, h, 1, True, tol, label=label)
        chain.check_moe(m, cfg, lw, l, h, tol, label=label)
    Wh = {"embed": W["embed"], "final_norm": np.asarray(W["final_norm"], np.float64)}
    lc = chain.check_head(m, cfg, Wh, h, tol, label=label)
    assert torch.equal(lc, logits)
    m.set_kv_length(L0 + 1)


@pytest.mark.parametrize("name,P,B,layers", [("tiny", 20, 2, 2), ("small_bf16", 150, 3, 2),
                                             ("f32_gqa", 33, 3, 2), ("small_fp8", 150, 3, 2),
                                             ("small_mxfp4", 150, 3, 2), ("vocab_bf16", 64, 2, 1)])
def test_ar_decode_steps_match_oracle(name, P, B, layers):
    """Five decode steps after a prompt encode; each step against the oracle
    stage by stage on the GPU's own inputs, every sequence."""
    print(f"ar decode {name} P={P} B={B} layers={layers}", flush=True)
    steps = 5
    cfg, W, m = setup(name, P + steps, B, n_layers=layers)
    V = cfg["vocab"]
    toks = synthetic.make_tokens(V, (B, P + steps - 1), seed=11)
    m.encode_prompt(to_dev(toks[:, :P - 1]))
    logits = torch.empty((B, V), dtype=torch.float32, device=DEV)
    for t in range(steps):
        tok = toks[:, P - 1 + t].copy()
        m.ar_decode_step(to_dev(tok), logits)
        torch.cuda.synchronize()
        decode_chain_check(m, cfg, W, tok, logits, tol_for(cfg), f"ar {name} step {t}")
    assert m.kv_length == P - 1 + steps


@pytest.mark.parametrize("name,P,B,layers", [("tiny", 20, 2, 2), ("f32_gqa", 33, 3, 2)])
def test_ar_decode_end_to_end_fp32(name, P, B, layers):
    """fp32 models: decode steps and the cache against the oracle's own
    encode and decode (its own routes); a decoded token within 1e-4 of a
    router tie is not compared."""
    steps = 5
    cfg, W, m = setup(name, P + steps, B, n_layers=layers)
    W = synthetic.to_float64(W)
    V = cfg["vocab"]
    toks = synthetic.make_tokens(V, (B, P + steps - 1), seed=11)
    m.encode_prompt(to_dev(toks[:, :P - 1]))
    cache = om.KVCache(cfg, B)
    om.encode(toks[:, :P - 1], W, cfg, cache)
    logits = torch.empty((B, V), dtype=torch.float32, device=DEV)
    skipped = 0
    for t in range(steps):
        tok = toks[:, P - 1 + t].copy()
        m.ar_decode_step(to_dev(tok), logits)
        ref, amb = oracle_decode_with_gaps(tok, W, cfg, cache, route_gap(cfg))
        got = logits.cpu().numpy()
        skipped += int(amb.sum())
        for b in np.flatnonzero(~amb):
            err = normwise(got[b], ref[b])
            assert err <= TOL_F32, f"step {t} seq {b}: {err:.3e}"
    assert skipped <= 1
    K, Vc = m.kv_tensors()
    L = P - 1 + steps
    for li in range(layers):
        for b in range(B):
            assert normwise(K[li, b, :, :L].float().cpu().numpy(), cache.k[li][b]) <= TOL_F32
            assert normwise(Vc[li, b, :, :L].float().cpu().numpy(), cache.v[li][b]) <= TOL_F32


def test_ar_decode_rejects_full_cache():
    cfg, W, m = setup("tiny", 8, 1)
    toks = synthetic.make_tokens(cfg["vocab"], (1, 8), seed=3)
    m.encode_prompt(to_dev(toks))
    logits = torch.empty((1, cfg["vocab"]), dtype=torch.float32, device=DEV)
    with pytest.raises(binding.DGError):
        m.ar_decode_step(to_dev(toks[:, 0]), logits)
    out = torch.empty((1, 1), dtype=torch.int32, device=DEV)
    with pytest.raises(binding.DGError):
        m.ar_generate(to_dev(toks[:, 0]), 1, out, logits)


@pytest.mark.parametrize("name,P,B,n_new", [("tiny", 12, 2, 6), ("small_bf16", 100, 2, 5),
                                            ("vocab_bf16", 40, 1, 4), ("small_fp8", 100, 1, 4),
                                            ("small_mxfp4", 100, 2, 4)])
def test_ar_generate_equals_composition(name, P, B, n_new):
    print(f"ar generate {name} P={P} B={B} n={n_new}", flush=True)
    cfg, W, m1 = setup(name, P + n_new, B)
    m2 = binding.Model(cfg, m1.src_weights, batch=B, capacity=P + n_new)
    V = cfg["vocab"]
    prompt = to_dev(synthetic.make_tokens(V, (B, P), seed=5))
    for m in (m1, m2):
        m.encode_prompt(prompt[:, :P - 1].contiguous())
    first = prompt[:, P - 1].contiguous()
    out = torch.full((B, n_new), -1, dtype=torch.int32, device=DEV)
    lg1 = torch.empty((B, V), dtype=torch.float32, device=DEV)
    m1.ar_generate(first, n_new, out, lg1)
    lg2 = torch.empty((B, V), dtype=torch.float32, device=DEV)
    tok = first.clone()
    ref = torch.empty((B, n_new), dtype=torch.int32, device=DEV)
    for t in range(n_new):
        m2.ar_decode_step(tok, lg2)
        nxt = torch.empty((B,), dtype=torch.int32, device=DEV)
        binding.argmax_rows(lg2, nxt)
        ref[:, t] = nxt
        tok = nxt
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(lg1, lg2)
    K1, V1 = m1.kv_tensors()
    K2, V2 = m2.kv_tensors()
    assert torch.equal(K1[:, :, :, :P - 1 + n_new], K2[:, :, :, :P - 1 + n_new])
    assert torch.equal(V1[:, :, :, :P - 1 + n_new], V2[:, :, :, :P - 1 + n_new])
    # the greedy tokens of the last step's logits continue the sequence
    assert out[:, -1].cpu().numpy().tolist() == np.argmax(lg1.cpu().numpy(), axis=1).tolist()


# ------------------------------------------------------------------ full size


def test_ar_decode_full_layer():
    """One decode step of four sequences through the full-size layer
    (vocabulary 262144, prompt 2048), each stage against the oracle on the
    GPU's own inputs, every sequence and logit."""
    cfg = synthetic.model_config("layer")
    P, V = synthetic.SHAPES["layer"]["prompt"], cfg["vocab"]
    B = 4
    print("generating full-size layer weights", flush=True)
    W = synthetic.make_weights(cfg, seed=0)
    toks = synthetic.make_tokens(V, (B, P + 1), seed=1)
    m = binding.Model(cfg, W, batch=B, capacity=P + 2)
    m.encode_prompt(to_dev(toks[:, :P]))
    logits = torch.empty((B, V), dtype=torch.float32, device=DEV)
    m.ar_decode_step(to_dev(toks[:, P].copy()), logits)
    torch.cuda.synchronize()
    decode_chain_check(m, cfg, W, toks[:, P].copy(), logits, TOL_BF16, "ar full layer")
