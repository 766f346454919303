"""Pins of the oracle's training-side forward: the multinomial corruption
(oracle/sampler.c, ora_corrupt) against numpy's independent Philox, its
rate extremes and replacement frequencies; the binary32 cross-entropy
(ora_xent) against closed forms and the float64 log-sum-exp; the model-level
forward (oracle/model.py, train_forward) against the plain denoising step
and scipy's logsumexp.  CPU only."""
import numpy as np
import pytest
from scipy.special import logsumexp

from discrete_text_diffusion_denoise_amd import synthetic
from oracle import model, sampler


def philox_block(seed, ctr):
    value = sum(int(w) << (64 * i) for i, w in enumerate(ctr))
    value = (value - 1) % 2**256
    start = np.array([(value >> (64 * i)) & (2**64 - 1) for i in range(4)], dtype=np.uint64)
    return np.random.Philox(key=np.array([seed, 0], dtype=np.uint64),
                            counter=start).random_raw(4)


# ------------------------------------------------------------------ corruption


def test_corrupt_rate_extremes_and_numpy_philox():
    seed, step, V = 12345, 7, 5000
    B, N = 3, 40
    clean = synthetic.make_tokens(V, (B, N), seed=1)
    same = sampler.corrupt(seed, step, V, np.zeros(B, np.float32), clean)
    assert np.array_equal(same, clean)
    full = sampler.corrupt(seed, step, V, np.ones(B, np.float32), clean)
    for b in range(B):
        for i in range(N):
            w = philox_block(seed, [step, b, i, 2])
            # uniform_token: the high 64 bits of word1 * V
            assert full[b, i] == (int(w[1]) * V) >> 64
    # a rate between: position replaced iff its uniform (2r + 1) 2^-24 < rate
    rate = np.array([0.25, 0.5, 0.9], np.float32)
    mid = sampler.corrupt(seed, step, V, rate, clean)
    for b in range(B):
        for i in range(N):
            w = philox_block(seed, [step, b, i, 2])
            u = (2 * (int(w[0]) >> 41) + 1) * 2.0 ** -24
            exp = (int(w[1]) * V) >> 64 if u < rate[b] else clean[b, i]
            assert mid[b, i] == exp


def test_corrupt_frequencies():
    V, B, N = 16, 4, 8192
    clean = np.zeros((B, N), np.int32)
    rate = np.array([0.0, 0.1, 0.5, 1.0], np.float32)
    out = sampler.corrupt(3, 0, V, rate, clean)
    # a replacement is a uniform token, so it keeps the clean one with prob 1/V
    for b in range(B):
        p = rate[b] * (1 - 1 / V)
        changed = (out[b] != 0).mean()
        assert abs(changed - p) <= 5 * np.sqrt(max(p * (1 - p), 1e-12) / N) + 1e-12
    # at rate 1 the tokens are uniform over V (chi-squared, 15 dof, p ~ 1e-4)
    counts = np.bincount(out[3], minlength=V)
    chi2 = ((counts - N / V) ** 2 / (N / V)).sum()
    assert chi2 < 42.0
    # different steps draw different corruptions
    assert not np.array_equal(out, sampler.corrupt(3, 1, V, rate, clean))


# ------------------------------------------------------------------ cross-entropy


def test_xent_closed_forms():
    V = 4096
    flat = np.full((1, V), 0.75, np.float32)
    loss, mean = sampler.xent(flat, np.array([17]))
    assert abs(float(loss[0]) - np.log(V)) <= 4 * np.spacing(np.float32(np.log(V)))
    two = np.array([[1.5, -0.25]], np.float32)
    loss, _ = sampler.xent(two, np.array([1]))
    assert abs(float(loss[0]) - np.log1p(np.exp(1.75))) < 2e-6
    loss, _ = sampler.xent(two, np.array([0]))
    assert abs(float(loss[0]) - np.log1p(np.exp(-1.75))) < 2e-6
    # a certain prediction costs (almost) nothing, a wrong one the logit gap
    sharp = np.zeros((2, 100), np.float32)
    sharp[:, 3] = 60.0
    loss, _ = sampler.xent(sharp, np.array([3, 4]))
    assert float(loss[0]) == 0.0
    assert abs(float(loss[1]) - 60.0) < 1e-4


@pytest.mark.parametrize("V", [1000, 65536 + 77, 262144])
def test_xent_against_float64_and_mean_order(V):
    lg = synthetic.make_logits((6, V), seed=V, sigma=2.0)
    tgt = synthetic.make_tokens(V, (6,), seed=V + 1)
    loss, mean = sampler.xent(lg, tgt)
    ref = logsumexp(lg.astype(np.float64), axis=1) - lg[np.arange(6), tgt].astype(np.float64)
    assert np.allclose(loss, ref, rtol=2e-6, atol=2e-6)
    acc = np.float32(0.0)
    for v in loss:
        acc = np.float32(acc + v)
    assert mean == np.float32(acc / np.float32(6))


def test_xent_matches_row_stats():
    # loss = L(S) - (l[x] - m) with the sampler's own m and S
    lg = synthetic.make_logits((1, 3000), seed=9, sigma=1.5)
    st, _ = sampler.row_stats(lg[0])
    loss, _ = sampler.xent(lg, np.array([123]))
    exp = np.float32(sampler.log32(st[1]) - np.float32(lg[0, 123] - st[0]))
    assert loss[0] == exp


# ------------------------------------------------------------------ model level


def tiny():
    shape = dict(n_layers=2, d_model=64, n_heads=4, n_kv_heads=2, head_dim=16, n_experts=6,
                 top_k=2, d_ff=48, vocab=96, canvas=16, dtype="f32")
    cfg = synthetic.model_config(shape)
    W = synthetic.to_float64(synthetic.make_weights(cfg, 0, std=0.2, random_norms=True))
    return cfg, W


def test_train_forward_at_rate_zero_is_the_plain_step():
    cfg, W = tiny()
    B, N, V = 2, cfg["canvas"], cfg["vocab"]
    prompt = synthetic.make_tokens(V, (B, 10), seed=2)
    cache = model.KVCache(cfg, B)
    model.encode(prompt, W, cfg, cache)
    clean = synthetic.make_tokens(V, (B, N), seed=3)
    x, logits, loss, mean = model.train_forward(clean, np.zeros(B), 5, 0, W, cfg, cache)
    assert np.array_equal(x, clean)
    ref = model.denoise_step(clean, W, cfg, cache)
    assert np.array_equal(logits, ref)
    ce = logsumexp(ref, axis=-1) - np.take_along_axis(ref, clean[..., None], axis=-1)[..., 0]
    assert np.allclose(loss, ce, rtol=1e-12, atol=1e-12)
    assert abs(mean - ce.mean()) < 1e-12
    assert cache.length == 10


def test_train_forward_corrupts_then_scores_the_clean_tokens():
    cfg, W = tiny()
    B, N, V = 2, cfg["canvas"], cfg["vocab"]
    cache = model.KVCache(cfg, B)
    model.encode(synthetic.make_tokens(V, (B, 6), seed=4), W, cfg, cache)
    clean = synthetic.make_tokens(V, (B, N), seed=5)
    rate = np.array([1.0, 0.5], np.float32)
    x, logits, loss, _ = model.train_forward(clean, rate, 9, 3, W, cfg, cache)
    assert np.array_equal(x, sampler.corrupt(9, 3, V, rate, clean))
    assert np.array_equal(logits, model.denoise_step(x, W, cfg, cache))
    # the loss scores the clean token, not the corrupted one
    ce = logsumexp(logits, axis=-1) - np.take_along_axis(logits, clean[..., None], axis=-1)[..., 0]
    assert np.allclose(loss, ce, rtol=1e-12, atol=1e-12)
    assert (x != clean).any()
