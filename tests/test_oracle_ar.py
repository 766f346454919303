"""Pins of the oracle's retained autoregressive mode (oracle/model.py, "AR
mode"): token-by-token decoding through the KV cache equals the causal
forward of the whole sequence; a prompt encode followed by one decode step
equals that forward's last row; a one-token sequence matches the closed form
(attention over a single key returns its value) with the MoE computed
densely; later tokens never reach earlier rows; greedy decoding feeds each
chosen token back.  CPU only."""
import numpy as np

from discrete_text_diffusion_denoise_amd import synthetic
from oracle import model


def cfg_and_weights(seed=0, **over):
    shape = dict(n_layers=2, d_model=64, n_heads=4, n_kv_heads=2, head_dim=16, n_experts=6,
                 top_k=2, d_ff=48, vocab=96, canvas=16, dtype="f32")
    shape.update(over)
    cfg = synthetic.model_config(shape)
    W = synthetic.to_float64(synthetic.make_weights(cfg, seed, std=0.2, random_norms=True))
    return cfg, W


def test_decode_by_token_equals_causal_forward():
    cfg, W = cfg_and_weights()
    toks = synthetic.make_tokens(cfg["vocab"], (2, 9), seed=4)
    cache = model.KVCache(cfg, 2)
    rows = [model.ar_decode_step(toks[:, t], W, cfg, cache) for t in range(toks.shape[1])]
    got = np.stack(rows, axis=1)                                  # [B, n, V]
    for b in range(2):
        ref = model.causal_logits(toks[b], W, cfg)
        assert np.allclose(got[b], ref, rtol=1e-10, atol=1e-10)
    assert cache.length == toks.shape[1]


def test_encode_then_decode_equals_causal_forward_last_row():
    cfg, W = cfg_and_weights(seed=1)
    toks = synthetic.make_tokens(cfg["vocab"], (2, 12), seed=5)
    cache = model.KVCache(cfg, 2)
    model.encode(toks[:, :-1], W, cfg, cache)
    got = model.ar_decode_step(toks[:, -1], W, cfg, cache)
    full = model.KVCache(cfg, 2)
    model.encode(toks, W, cfg, full)
    for li in range(cfg["n_layers"]):
        assert np.allclose(cache.k[li], full.k[li], rtol=1e-12, atol=1e-12)
        assert np.allclose(cache.v[li], full.v[li], rtol=1e-12, atol=1e-12)
    for b in range(2):
        ref = model.causal_logits(toks[b], W, cfg)[-1]
        assert np.allclose(got[b], ref, rtol=1e-10, atol=1e-10)


def dense_moe(u, lw, k):
    """Every expert on every token, then the top-k gate mask (softmax over the
    selected router logits)."""
    z = u @ lw["w_router"].T
    E = z.shape[1]
    y = np.zeros_like(u)
    for t in range(u.shape[0]):
        sel = np.argsort(-z[t], kind="stable")[:k]
        g = np.exp(z[t, sel] - z[t, sel].max())
        g = g / g.sum()
        for e in range(E):
            a = u[t] @ lw["w_gate"][e].T
            act = a / (1 + np.exp(-a)) * (u[t] @ lw["w_up"][e].T)
            out = act @ lw["w_down"][e].T
            w = g[list(sel).index(e)] if e in sel else 0.0
            y[t] += w * out
    return y


def test_single_token_forward_closed_form():
    cfg, W = cfg_and_weights(seed=2)
    tok = np.array([17])
    Hq, Hkv, dh = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    h = W["embed"][tok].copy()
    for lw in W["layers"]:
        u = model.rmsnorm(h, lw["attn_norm"], cfg["rms_eps"])
        v = (u @ lw["wv"].T).reshape(Hkv, dh)
        # one visible key: every query head returns its KV head's value
        o = np.concatenate([v[q // (Hq // Hkv)] for q in range(Hq)])[None, :]
        h = h + o @ lw["wo"].T
        u = model.rmsnorm(h, lw["moe_norm"], cfg["rms_eps"])
        h = h + dense_moe(u, lw, cfg["top_k"])
    ref = model.rmsnorm(h, W["final_norm"], cfg["rms_eps"]) @ W["embed"].T
    got = model.causal_logits(tok, W, cfg)
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-10)
    cache = model.KVCache(cfg, 1)
    assert np.allclose(model.ar_decode_step(tok, W, cfg, cache), ref, rtol=1e-10, atol=1e-10)


def test_causal_forward_ignores_later_tokens():
    cfg, W = cfg_and_weights(seed=3)
    a = synthetic.make_tokens(cfg["vocab"], (10,), seed=6)
    b = a.copy()
    b[6:] = (b[6:] + 31) % cfg["vocab"]
    la, lb = model.causal_logits(a, W, cfg), model.causal_logits(b, W, cfg)
    assert np.array_equal(la[:6], lb[:6])
    assert not np.allclose(la[6:], lb[6:])


def test_greedy_token_takes_lower_index_on_ties():
    lg = np.array([[1.0, 3.0, 3.0, -1.0], [0.0, 0.0, 0.0, 0.0], [-5.0, -4.0, -4.5, -4.0]])
    assert model.greedy_token(lg).tolist() == [1, 0, 1]


def test_ar_generate_feeds_back_greedy_tokens():
    cfg, W = cfg_and_weights(seed=4)
    V = cfg["vocab"]
    prompt = synthetic.make_tokens(V, (2, 5), seed=7)
    cache = model.KVCache(cfg, 2)
    model.encode(prompt[:, :-1], W, cfg, cache)
    ref_cache = cache.copy()
    # a hook that puts the maximum at a chosen token, different per sequence
    chosen = np.array([[(7 * t + 3 * b) % V for t in range(4)] for b in range(2)], np.int32)

    def hook(t, lg):
        lg = np.full_like(lg, -1.0)
        lg[np.arange(2), chosen[:, t]] = 2.0
        return lg

    out = model.ar_generate(prompt[:, -1], 4, W, cfg, cache, logits_of=hook)
    assert np.array_equal(out, chosen)
    # the same cache as decoding [last prompt token, chosen_0, chosen_1, chosen_2]
    seq = np.concatenate([prompt[:, -1:], chosen[:, :3]], axis=1)
    for t in range(4):
        model.ar_decode_step(seq[:, t], W, cfg, ref_cache)
    for li in range(cfg["n_layers"]):
        assert np.array_equal(cache.k[li], ref_cache.k[li])
        assert np.array_equal(cache.v[li], ref_cache.v[li])
    # without a hook the tokens are the greedy choices of the oracle's logits
    c2 = model.KVCache(cfg, 2)
    model.encode(prompt[:, :-1], W, cfg, c2)
    c3 = c2.copy()
    out2 = model.ar_generate(prompt[:, -1], 3, W, cfg, c2)
    tok = prompt[:, -1]
    for t in range(3):
        tok = model.greedy_token(model.ar_decode_step(tok, W, cfg, c3))
        assert np.array_equal(out2[:, t], tok)
