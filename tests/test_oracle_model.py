"""Pins of the float64 model oracle (oracle/model.py) against library routines
(torch CPU scaled_dot_product_attention), closed forms, and invariants that any
correct implementation of the pages' method must satisfy: canvas permutation
equivariance, causal == incremental encoding, dense-masked == sparse MoE,
one-hot self-conditioning, commit == re-encode.  CPU only."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_denoise_amd import synthetic
from oracle import driver, model, sampler


def tiny_cfg(**over):
    shape = dict(n_layers=2, d_model=64, n_heads=4, n_kv_heads=2, head_dim=16, n_experts=6,
                 top_k=2, d_ff=48, vocab=96, canvas=16, dtype="f32")
    model_over = {k: over.pop(k) for k in list(over) if k not in shape}
    shape.update(over)
    return synthetic.model_config(shape, **model_over)


def tiny_weights(cfg, seed=0, std=0.2, random_norms=True):
    return synthetic.to_float64(synthetic.make_weights(cfg, seed, std=std, random_norms=random_norms))


# ------------------------------------------------------------------ primitives


def test_rmsnorm_closed_form():
    x = np.full((3, 8), -2.5)
    w = np.arange(1, 9, dtype=np.float64)
    y = model.rmsnorm(x, w, 0.0)
    assert np.allclose(y, -w[None, :])
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64)) * 7
    y = model.rmsnorm(x, np.ones(64), 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0)
    eps = 0.5
    y = model.rmsnorm(np.zeros((1, 4)) + 1.0, np.ones(4), eps)
    assert np.allclose(y, 1.0 / np.sqrt(1.0 + eps))


def test_rope_relative_position_and_norm():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((5, 2, 16))
    k = rng.standard_normal((5, 2, 16))
    pos = np.array([0, 3, 7, 100, 4000])
    qa, ka = model.rope(q, pos, 10000.0), model.rope(k, pos, 10000.0)
    qb, kb = model.rope(q, pos + 123, 10000.0), model.rope(k, pos + 123, 10000.0)
    # scores depend only on position differences
    sa = np.einsum("ihd,jhd->hij", qa, ka)
    sb = np.einsum("ihd,jhd->hij", qb, kb)
    assert np.allclose(sa, sb)
    assert np.allclose(np.linalg.norm(qa, axis=-1), np.linalg.norm(q, axis=-1))
    assert np.allclose(model.rope(q, np.zeros(5), 10000.0), q)
    # the lowest pair rotates by exactly pos radians
    x = np.zeros((1, 1, 16))
    x[0, 0, 0] = 1.0
    y = model.rope(x, np.array([0.7]), 10000.0)
    assert np.isclose(y[0, 0, 0], np.cos(0.7)) and np.isclose(y[0, 0, 8], np.sin(0.7))


@pytest.mark.parametrize("Hq,Hkv,causal", [(4, 4, False), (4, 2, False), (8, 2, True)])
def test_attention_matches_torch_sdpa(Hq, Hkv, causal):
    rng = np.random.default_rng(2)
    n = m = 24
    q = rng.standard_normal((n, Hq, 16))
    k = rng.standard_normal((m, Hkv, 16))
    v = rng.standard_normal((m, Hkv, 16))
    allowed = np.tril(np.ones((n, m), dtype=bool)) if causal else np.ones((n, m), dtype=bool)
    got = model.attention(q, k, v, allowed)
    rep = Hq // Hkv
    kt = torch.from_numpy(np.repeat(k, rep, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, rep, axis=1)).permute(1, 0, 2)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
    assert np.allclose(got, ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 2, 8))
    k = np.repeat(rng.standard_normal((1, 2, 8)), 6, axis=0)   # identical keys
    v = rng.standard_normal((6, 2, 8))
    out = model.attention(q, k, v, np.ones((4, 6), dtype=bool))
    assert np.allclose(out, v.mean(axis=0)[None])
    k2 = rng.standard_normal((6, 2, 8)) * 0.01
    k2[4] = q[0] * 1e3                                          # one dominant key for query 0
    out = model.attention(q[:1], k2, v, np.ones((1, 6), dtype=bool))
    assert np.allclose(out[0], v[4], atol=1e-9)


def test_moe_dense_masked_equals_sparse():
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    lw = W["layers"][0]
    u = np.random.default_rng(4).standard_normal((10, cfg["d_model"]))
    y, idx, g, z = model.moe(u, lw, cfg["top_k"])
    # dense: every expert on every token, then mask to the top-k and renormalise
    E = cfg["n_experts"]
    dense = np.stack([(u @ lw["w_gate"][e].T) / (1 + np.exp(-(u @ lw["w_gate"][e].T)))
                      * (u @ lw["w_up"][e].T) @ lw["w_down"][e].T for e in range(E)], axis=1)
    full = np.exp(z - z.max(axis=1, keepdims=True))
    kth = np.sort(z, axis=1)[:, -cfg["top_k"]][:, None]
    mask = z >= kth
    gates = np.where(mask, full, 0.0)
    gates /= gates.sum(axis=1, keepdims=True)
    ref = np.einsum("te,ted->td", gates, dense)
    assert np.allclose(y, ref)
    assert (np.sort(idx, axis=1) == np.sort(np.argsort(-z, axis=1)[:, :cfg["top_k"]], axis=1)).all()


def test_moe_all_experts_is_full_softmax_mixture_and_single_expert_is_swiglu():
    cfg = tiny_cfg(n_experts=4, top_k=4)
    W = tiny_weights(cfg)
    lw = W["layers"][0]
    u = np.random.default_rng(5).standard_normal((7, cfg["d_model"]))
    y, _, g, z = model.moe(u, lw, 4)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ref = sum(p[:, e:e + 1] * ((lambda a: a / (1 + np.exp(-a)))(u @ lw["w_gate"][e].T)
                               * (u @ lw["w_up"][e].T)) @ lw["w_down"][e].T for e in range(4))
    assert np.allclose(y, ref)
    cfg1 = tiny_cfg(n_experts=1, top_k=1)
    lw1 = tiny_weights(cfg1)["layers"][0]
    y1, _, g1, _ = model.moe(u, lw1, 1)
    assert np.allclose(g1, 1.0)
    a = u @ lw1["w_gate"][0].T
    assert np.allclose(y1, (a * torch.sigmoid(torch.from_numpy(a)).numpy()
                            * (u @ lw1["w_up"][0].T)) @ lw1["w_down"][0].T)


def test_route_ties_take_lower_expert():
    z = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    idx, g = model.route(z, 2)
    assert idx.tolist() == [[1, 2]]
    assert np.allclose(g, 0.5)


# ------------------------------------------------------------------ stack invariants


def test_canvas_permutation_equivariance_without_positions():
    cfg = tiny_cfg(rope_on=0)
    W = tiny_weights(cfg)
    cache = model.KVCache(cfg, 1)
    model.encode(synthetic.make_tokens(cfg["vocab"], (1, 9), seed=1), W, cfg, cache)
    canvas = synthetic.make_tokens(cfg["vocab"], (1, cfg["canvas"]), seed=2)
    perm = np.random.default_rng(6).permutation(cfg["canvas"])
    a = model.denoise_step(canvas, W, cfg, cache)
    b = model.denoise_step(canvas[:, perm], W, cfg, cache)
    assert np.allclose(a[:, perm], b)
    # with positions on, the same permutation changes the result
    cfg_r = tiny_cfg(rope_on=1)
    cache_r = model.KVCache(cfg_r, 1)
    model.encode(synthetic.make_tokens(cfg["vocab"], (1, 9), seed=1), W, cfg_r, cache_r)
    ar = model.denoise_step(canvas, W, cfg_r, cache_r)
    br = model.denoise_step(canvas[:, perm], W, cfg_r, cache_r)
    assert not np.allclose(ar[:, perm], br)


def test_causal_encode_equals_incremental_encode():
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    toks = synthetic.make_tokens(cfg["vocab"], (2, 11), seed=3)
    whole = model.KVCache(cfg, 2)
    model.encode(toks, W, cfg, whole)
    inc = model.KVCache(cfg, 2)
    for i in range(toks.shape[1]):
        model.encode(toks[:, i:i + 1], W, cfg, inc)
    assert whole.length == inc.length == 11
    for li in range(cfg["n_layers"]):
        assert np.allclose(whole.k[li], inc.k[li]) and np.allclose(whole.v[li], inc.v[li])


def test_commit_equals_reencode_from_scratch():
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    prompt = synthetic.make_tokens(cfg["vocab"], (1, 7), seed=4)
    block = synthetic.make_tokens(cfg["vocab"], (1, cfg["canvas"]), seed=5)
    a = model.KVCache(cfg, 1)
    model.encode(prompt, W, cfg, a)
    model.encode(block, W, cfg, a)
    b = model.KVCache(cfg, 1)
    model.encode(np.concatenate([prompt, block], axis=1), W, cfg, b)
    for li in range(cfg["n_layers"]):
        assert np.allclose(a.k[li], b.k[li]) and np.allclose(a.v[li], b.v[li])


def test_canvas_sees_context_and_is_bidirectional():
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    canvas = synthetic.make_tokens(cfg["vocab"], (1, cfg["canvas"]), seed=6)
    c1 = model.KVCache(cfg, 1)
    model.encode(synthetic.make_tokens(cfg["vocab"], (1, 5), seed=7), W, cfg, c1)
    base = model.denoise_step(canvas, W, cfg, c1)
    # changing the last canvas token changes the logits of the first position
    canvas2 = canvas.copy()
    canvas2[0, -1] = (canvas2[0, -1] + 1) % cfg["vocab"]
    assert not np.allclose(base[0, 0], model.denoise_step(canvas2, W, cfg, c1)[0, 0])
    # changing the context changes the canvas logits
    c2 = model.KVCache(cfg, 1)
    model.encode(synthetic.make_tokens(cfg["vocab"], (1, 5), seed=8), W, cfg, c2)
    assert not np.allclose(base, model.denoise_step(canvas, W, cfg, c2))


def test_selfcond_one_hot_is_embedding_row_and_none_is_plain_embedding():
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    V = cfg["vocab"]
    j = np.array([5, 17, 95])
    L = np.full((3, V), -1e4)
    L[np.arange(3), j] = 0.0
    s = model.selfcond_vector(L, W)
    assert np.allclose(s, W["embed"][j])
    # uniform previous logits give the mean embedding
    s_u = model.selfcond_vector(np.zeros((1, V)), W)
    assert np.allclose(s_u[0], W["embed"].mean(axis=0))
    x = np.array([1, 2, 3])
    assert np.allclose(model.denoiser_input(x, W, None), W["embed"][x])
    assert np.allclose(model.denoiser_input(x, W, L), W["embed"][x] + W["embed"][j] @ W["w_sc"].T)


def test_head_is_tied_embedding_product():
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    h = np.random.default_rng(9).standard_normal((4, cfg["d_model"]))
    L = model.head(h, W, cfg)
    u = h / np.sqrt((h * h).mean(axis=1, keepdims=True) + cfg["rms_eps"]) * W["final_norm"]
    for t in range(4):
        for v in (0, 1, cfg["vocab"] - 1):
            assert np.isclose(L[t, v], sum(u[t, i] * W["embed"][v, i] for i in range(cfg["d_model"])))


def test_random_init_logit_spread_gives_near_uniform_entropy():
    # random-init head: logits ~ N(0, sigma^2) with sigma ~ 0.02*sqrt(d) ~ 0.9 at
    # d = 2048; the entropy is then about ln V - sigma^2/2 and no position locks.
    cfg = tiny_cfg(d_model=256, vocab=4096, n_heads=4, n_kv_heads=4, head_dim=64)
    W = synthetic.to_float64(synthetic.make_weights(cfg, 0, std=0.02))
    cache = model.KVCache(cfg, 1)
    model.encode(synthetic.make_tokens(cfg["vocab"], (1, 4)), W, cfg, cache)
    L = model.denoise_step(synthetic.make_tokens(cfg["vocab"], (1, cfg["canvas"])), W, cfg, cache)
    sig = L.std()
    st, _ = sampler.row_stats(L[0, 0].astype(np.float32))
    assert abs(float(st[2]) - (np.log(cfg["vocab"]) - sig ** 2 / 2)) < 0.1


def test_block_driver_peaked_logits_stop_after_two_rounds():
    # Logits that put every position on a fixed token with certainty: round 0
    # locks everything (entropy ~ 0), round 1 sees the same most likely
    # sequence and stops; the block is that sequence and is committed.
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    cache = model.KVCache(cfg, 1)
    model.encode(synthetic.make_tokens(cfg["vocab"], (1, 5)), W, cfg, cache)
    target = synthetic.make_tokens(cfg["vocab"], (1, cfg["canvas"]), seed=42)
    seen = []

    def hook(t, logits):
        seen.append(t)
        out = np.full_like(logits, -50.0)
        np.put_along_axis(out, target[..., None].astype(np.int64), 50.0, axis=2)
        return out

    p = synthetic.default_sampler_params(max_steps=48)
    block, steps = driver.generate_block(W, cfg, cache, p, block_index=0, B=1, logits_hook=hook)
    assert steps[0] == 2 and seen == [0, 1]
    assert (block == target).all()
    assert cache.length == 5 + cfg["canvas"]
    ref = model.KVCache(cfg, 1)
    model.encode(synthetic.make_tokens(cfg["vocab"], (1, 5)), W, cfg, ref)
    model.encode(target, W, cfg, ref)
    assert np.allclose(cache.k[1], ref.k[1])


def test_block_driver_random_model_runs_full_budget():
    cfg = tiny_cfg()
    W = tiny_weights(cfg, std=0.02)
    cache = model.KVCache(cfg, 2)
    model.encode(synthetic.make_tokens(cfg["vocab"], (2, 5)), W, cfg, cache)
    p = synthetic.default_sampler_params(max_steps=3)
    block, steps = driver.generate_block(W, cfg, cache, p, block_index=0, B=2)
    assert steps.tolist() == [3, 3]
    assert cache.length == 5 + cfg["canvas"]


def test_block_driver_one_canvas_stops_the_other_continues():
    # Canvas 0 gets logits certain of a fixed sequence (round 0 locks it,
    # round 1 finds the same most likely sequence and stops); canvas 1 gets
    # flat-ish random logits and never stops.  Each canvas stops on its own
    # (report-summary page, section 4), and a stopped canvas is left as it is.
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    cache = model.KVCache(cfg, 2)
    model.encode(synthetic.make_tokens(cfg["vocab"], (2, 5)), W, cfg, cache)
    N, V = cfg["canvas"], cfg["vocab"]
    target = synthetic.make_tokens(V, (N,), seed=43)
    rng = np.random.default_rng(44)
    seen = []

    def hook(t, logits):
        out = rng.standard_normal(logits.shape) * 0.3
        out[0] = -50.0
        out[0, np.arange(N), target] = 50.0
        return out

    def rec(t, canvas, argmax, lock, stats, stop):
        seen.append((t, canvas.copy(), argmax.copy(), lock.copy(), stop.copy()))

    p = synthetic.default_sampler_params(max_steps=6)
    block, steps = driver.generate_block(W, cfg, cache, p, block_index=0, B=2, logits_hook=hook,
                                         round_hook=rec)
    assert steps.tolist() == [2, 6]
    assert [s[0] for s in seen] == list(range(6))
    assert (block[0] == target).all()
    # canvas 0: every position locked to the certain token in rounds 0 and 1
    assert seen[0][3][0].all() and (seen[0][1][0] == target).all()
    # canvas 1: flat logits give no lock under the 0.1 entropy budget
    assert not seen[0][3][1].any()
    # after its stop (round 1) canvas 0 is frozen while canvas 1 moves on
    for t in range(2, 6):
        assert (seen[t][1][0] == seen[1][1][0]).all() and (seen[t][2][0] == seen[1][2][0]).all()
        assert not (seen[t][1][1] == seen[t - 1][1][1]).all()
    assert seen[1][4].tolist() == [1, 0] and seen[5][4].tolist() == [1, 1]
    assert (block[1] == seen[5][2][1]).all()


def test_block_driver_top1_selfcond_is_the_argmax_embedding():
    # With top-k truncation at K = 1 the truncated distribution of a position
    # is certain of its largest logit, so the next round's self-conditioning
    # input must equal the full-distribution path fed with logits certain of
    # that token (exp(-1e4) is exactly 0 in float64).
    cfg = tiny_cfg(n_layers=1)
    W = tiny_weights(cfg)
    cache = model.KVCache(cfg, 1)
    model.encode(synthetic.make_tokens(cfg["vocab"], (1, 5)), W, cfg, cache)
    seen = {}

    def hook(t, logits):
        seen[t] = logits.copy()
        return logits

    def rec(t, canvas, argmax, lock, stats, stop):
        seen[("canvas", t)] = canvas.copy()

    p = synthetic.default_sampler_params(max_steps=2, top_k=1, require_stable=1)
    driver.generate_block(W, cfg, cache.copy(), p, block_index=0, B=1, logits_hook=hook,
                          round_hook=rec)
    am0 = np.argmax(seen[0].astype(np.float32), axis=-1)
    onehot = np.full(seen[0].shape, -1e4)
    np.put_along_axis(onehot, am0[..., None], 0.0, axis=-1)
    ref = model.denoise_step(seen[("canvas", 0)], W, cfg, cache, onehot, top_k=0)
    assert np.allclose(seen[1], ref, rtol=0, atol=1e-12)
    # and it is not the full distribution's self-conditioning
    full = model.denoise_step(seen[("canvas", 0)], W, cfg, cache, seen[0].astype(np.float32)
                              .astype(np.float64), top_k=0)
    assert not np.allclose(seen[1], full, rtol=0, atol=1e-6)
