"""Pins of the sampler oracle (oracle/sampler.c) against independent facts:
an independent Philox implementation, libm, closed forms, float64 brute force,
chi-square frequency tests, hand-worked lock cases and the pages' stop rule.
CPU only."""
import ctypes
import json
import math
import os

import numpy as np
import pytest

from oracle import sampler

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# ------------------------------------------------------------------ Philox


@pytest.mark.parametrize("key,ctr", [
    ([0, 0], [0, 0, 0, 0]),
    ([5, 0], [7, 3, 200, 0]),
    ([0xDEADBEEFCAFEF00D, 0], [47, 7, 255, 1]),
    ([2**64 - 1, 0], [2**64 - 2, 2**63, 12345, 1]),
])
def test_philox_matches_numpy(key, ctr):
    # numpy.random.Philox is Philox4x64-10 and bumps its counter by one
    # *before* producing a block, so starting it at ctr - 1 yields block(ctr).
    value = sum(int(w) << (64 * i) for i, w in enumerate(ctr))
    value = (value - 1) % 2**256
    start = np.array([(value >> (64 * i)) & (2**64 - 1) for i in range(4)], dtype=np.uint64)
    ref = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=start).random_raw(4)
    got = sampler.philox4x64(ctr, key)
    assert [int(x) for x in got] == [int(x) for x in ref]


def test_uniform_open_interval_and_exact():
    assert float(sampler.uniform(0)) == 2.0 ** -24
    assert float(sampler.uniform(2**64 - 1)) == 1.0 - 2.0 ** -24
    r = 0x123456
    assert float(sampler.uniform(r << 41)) == (2 * r + 1) * 2.0 ** -24


def test_uniform_token_power_of_two_is_top_bits():
    rng = np.random.default_rng(0)
    for w in rng.integers(0, 2**63, size=200, dtype=np.uint64):
        w = int(w) * 2 + 1
        assert sampler.uniform_token(w, 1024) == w >> 54
        assert sampler.uniform_token(w, 262144) == w >> 46
        assert 0 <= sampler.uniform_token(w, 262000) < 262000


# ------------------------------------------------------------------ exp / log


def test_exp_against_libm():
    xs = np.concatenate([np.linspace(-87.0, 0.0, 40001, dtype=np.float32),
                         -np.logspace(-8, 0, 2001).astype(np.float32)])
    worst = 0.0
    for x in xs[::7]:
        ref = math.exp(float(x))
        got = float(sampler.exp32(float(x)))
        worst = max(worst, abs(got - ref) / ref)
    assert worst < 4 * 2.0 ** -24, worst   # within ~2 ulp


def test_exp_special_values():
    assert float(sampler.exp32(0.0)) == 1.0
    assert float(sampler.exp32(-87.0)) > 0.0
    assert float(sampler.exp32(-87.0)) >= 2.0 ** -126          # never subnormal
    assert float(sampler.exp32(np.nextafter(np.float32(-87.0), np.float32(-100.0)))) == 0.0
    assert float(sampler.exp32(-np.inf)) == 0.0
    assert float(sampler.exp32(-1000.0)) == 0.0


def test_log_against_libm():
    xs = np.concatenate([np.linspace(1.0, 2.0, 5001), np.logspace(0, 7, 5001)]).astype(np.float32)
    for x in xs[::3]:
        ref = math.log(float(x))
        got = float(sampler.log32(float(x)))
        assert abs(got - ref) <= 4 * 2.0 ** -24 * max(ref, 1.0), (x, got, ref)
    assert float(sampler.log32(1.0)) == 0.0


# ------------------------------------------------------------------ chunk layout

NLANE, NDEPTH, TILE = 1024, 16, 65536


def chunk_members(V, c):
    t, lam = divmod(c, NLANE)
    out = []
    for d in range(NDEPTH):
        for q in range(4):
            k = 4 * (t * NLANE * NDEPTH + d * NLANE + lam) + q
            if k < V:
                out.append(k)
    return out


@pytest.mark.parametrize("V", [1, 7, 1024, 4100, 65536, 70001])
def test_chunk_layout_is_a_partition(V):
    nt = -(-V // TILE)
    seen = np.zeros(V, dtype=np.int32)
    for c in range(nt * NLANE):
        m = chunk_members(V, c)
        assert m == sorted(m)
        seen[m] += 1
    assert (seen == 1).all()


# ------------------------------------------------------------------ row statistics


@pytest.mark.parametrize("V", [1, 1024, 4099, 262144])
def test_stats_uniform_logits(V):
    row = np.full(V, 0.37, dtype=np.float32)
    st, am = sampler.row_stats(row)
    assert am == 0
    assert st[0] == np.float32(0.37)
    assert st[1] == np.float32(V)                 # exact: sum of ones
    assert st[3] == np.float32(1.0) / np.float32(V)
    assert abs(float(st[2]) - math.log(V)) <= 4e-7 * max(1.0, math.log(V))


@pytest.mark.parametrize("V,c,pos", [(1024, 3.0, 17), (262144, 9.5, 200000), (5000, 0.5, 4999)])
def test_stats_one_raised_logit_closed_form(V, c, pos):
    row = np.zeros(V, dtype=np.float32)
    row[pos] = c
    st, am = sampler.row_stats(row)
    ec = math.exp(c)
    Z = ec + (V - 1)
    pmax = ec / Z
    H = math.log(Z) - c * ec / Z
    assert am == pos
    assert abs(float(st[3]) - pmax) <= 2e-6 * pmax
    assert abs(float(st[2]) - H) <= 2e-6 * H
    assert abs(float(st[1]) - Z / ec) <= 2e-6 * Z / ec   # S is relative to the max


@pytest.mark.parametrize("V,sigma,seed", [(1024, 0.9, 0), (262144, 0.9, 1), (70001, 3.0, 2),
                                          (300, 20.0, 3)])
def test_stats_against_float64_brute_force(V, sigma, seed):
    row = (np.random.default_rng(seed).standard_normal(V) * sigma).astype(np.float32)
    st, am = sampler.row_stats(row)
    x = row.astype(np.float64)
    m = x.max()
    e = np.exp(x - m)
    S = e.sum()
    p = e / S
    H = -(p[p > 0] * np.log(p[p > 0])).sum()
    assert am == int(np.argmax(row))
    assert st[0] == row.max()
    assert abs(float(st[1]) - S) <= 1e-5 * S
    assert abs(float(st[3]) - 1 / S) <= 1e-5 / S
    assert abs(float(st[2]) - H) <= 1e-5 * max(H, 1.0)


def test_stats_argmax_ties_take_lowest_index():
    row = np.zeros(200000, dtype=np.float32)
    for k in (150000, 70000, 99999):
        row[k] = 2.0
    st, am = sampler.row_stats(row)
    assert am == 70000


def test_random_init_entropy_is_near_log_v():
    # logits ~ N(0, s^2): H -> ln V - s^2/2 for large V
    V, s = 262144, 0.9
    row = (np.random.default_rng(7).standard_normal(V) * s).astype(np.float32)
    st, _ = sampler.row_stats(row)
    assert abs(float(st[2]) - (math.log(V) - s * s / 2)) < 0.02


# ------------------------------------------------------------------ draw


def _three_level_probs(row, inv_t):
    """float64 probabilities of each level of the draw (superchunk, chunk, entry)."""
    V = row.size
    nt = -(-V // TILE)
    x = row.astype(np.float64) * inv_t
    w = np.exp(x - x.max())
    G = np.zeros(nt * NLANE)
    members = [chunk_members(V, c) for c in range(nt * NLANE)]
    for c, m in enumerate(members):
        G[c] = w[m].sum() if m else 0.0
    return w, G, members


@pytest.mark.parametrize("V,sigma,inv_t", [(8, 1.0, 1.0), (1024, 0.9, 1.25), (70001, 2.0, 2.5)])
def test_draw_against_float64_decisions(V, sigma, inv_t):
    """Each level picks the first index whose running sum exceeds u * total;
    compare with float64, skipping draws whose target is within 1e-5 of a
    boundary (float32 rounding may legitimately go either way there)."""
    row = (np.random.default_rng(V).standard_normal(V) * sigma).astype(np.float32)
    w, G, members = _three_level_probs(row, inv_t)
    nsup = G.size // 64
    W = G.reshape(nsup, 64).sum(axis=1)
    rng = np.random.default_rng(11)
    checked = 0

    def pick(weights, u):
        cs = np.cumsum(weights)
        t = u * cs[-1]
        i = int(np.searchsorted(cs, t, side="right"))
        margin = np.min(np.abs(cs - t)) / cs[-1]
        return i, margin

    for _ in range(300):
        u1, u2, u3 = (rng.integers(0, 2**23, size=3) * 2 + 1) * 2.0 ** -24
        s, m1 = pick(W, u1)
        c, m2 = pick(G[s * 64:(s + 1) * 64], u2)
        c += s * 64
        k, m3 = pick(w[members[c]], u3)
        y = sampler.draw(row, inv_t, u1, u2, u3)
        if min(m1, m2, m3) < 1e-5:
            continue
        assert y == members[c][k]
        checked += 1
    assert checked > 250


def test_draw_frequencies_chi_square():
    V, inv_t = 8, 1.25
    row = np.array([0.0, 1.0, -1.0, 2.0, 0.5, -3.0, 1.5, 0.2], dtype=np.float32)
    p = np.exp(row.astype(np.float64) * inv_t)
    p /= p.sum()
    n = 60000
    rng = np.random.default_rng(3)
    us = (rng.integers(0, 2**23, size=(n, 3)) * 2 + 1) * 2.0 ** -24
    counts = np.zeros(V)
    for u1, u2, u3 in us:
        counts[sampler.draw(row, inv_t, u1, u2, u3)] += 1
    chi2 = ((counts - n * p) ** 2 / (n * p)).sum()
    assert chi2 < 24.3     # 7 dof, p = 0.001


def test_draw_low_temperature_is_argmax():
    row = (np.random.default_rng(5).standard_normal(5000)).astype(np.float32)
    am = int(np.argmax(row))
    row[am] += 1.0          # a clear gap: every other weight underflows at 1/T = 200
    rng = np.random.default_rng(6)
    for _ in range(50):
        u = (rng.integers(0, 2**23, size=3) * 2 + 1) * 2.0 ** -24
        assert sampler.draw(row, 200.0, *u) == am


def test_inverse_temperature_schedule():
    T0, T1, S = 0.8, 0.4, 48
    assert sampler.inv_temperature(T0, T1, 0, S) == np.float32(1.0) / np.float32(0.8)
    assert sampler.inv_temperature(T0, T1, S - 1, S) == np.float32(1.0) / np.float32(0.4)
    Ts = [1.0 / float(sampler.inv_temperature(T0, T1, t, S)) for t in range(S)]
    steps = np.diff(Ts)
    assert np.all(steps < 0) and np.allclose(steps, (T1 - T0) / (S - 1), atol=1e-6)


# ------------------------------------------------------------------ lock / stop


def _lock(rule, theta, H, P):
    L = sampler.lib()
    L.ora_lock_set.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p]
    H = np.ascontiguousarray(H, dtype=np.float32)
    P = np.ascontiguousarray(P, dtype=np.float32)
    out = np.zeros(H.size, dtype=np.uint8)
    L.ora_lock_set(rule, theta, H.size, H.ctypes.data, P.ctypes.data, out.ctypes.data)
    return out.tolist()


def test_lock_rules_hand_cases():
    cases = json.load(open(os.path.join(GOLDEN, "lock_cases.json")))["cases"]
    for c in cases:
        assert _lock(c["rule"], c["theta"], c["H"], c["P"]) == c["lock"], c["why"]


def _params(**kw):
    from discrete_text_diffusion_denoise_amd.synthetic import default_sampler_params
    return default_sampler_params(**kw)


def test_one_hot_logits_lock_everything_and_stop():
    B, N, V = 2, 256, 1024
    tok = np.random.default_rng(0).integers(0, V, size=(B, N))
    logits = np.full((B, N, V), -60.0, dtype=np.float32)
    np.put_along_axis(logits, tok[..., None], 40.0, axis=2)
    for require_stable, stop_step in ((0, 0), (1, 1)):
        canvas = np.zeros((B, N), dtype=np.int32)
        argmax = np.zeros((B, N), dtype=np.int32)
        stop = np.zeros(B, dtype=np.int32)
        p = _params(require_stable=require_stable)
        for t in range(3):
            lock, stats = sampler.sample_update(p, t, logits, canvas, argmax, stop)
            if t == 0:
                assert (lock == 1).all()
                assert (stats[..., 2] == 0).all() and (stats[..., 3] == 1).all()
                assert (canvas == tok).all() and (argmax == tok).all()
            if stop.all():
                assert t == stop_step
                break
        assert stop.all()


def test_random_logits_never_lock_or_stop_early():
    B, N, V = 1, 256, 1024
    logits = (np.random.default_rng(1).standard_normal((B, N, V)) * 0.9).astype(np.float32)
    canvas = np.zeros((B, N), dtype=np.int32)
    argmax = np.zeros((B, N), dtype=np.int32)
    stop = np.zeros(B, dtype=np.int32)
    p = _params(max_steps=3)
    for t in range(3):
        lock, stats = sampler.sample_update(p, t, logits, canvas, argmax, stop)
        assert lock.sum() == 0                 # H ~ ln V - 0.4 >> 0.1
        assert stop[0] == (1 if t == 2 else 0)  # only the round budget stops it


def test_stopped_canvas_is_untouched():
    B, N, V = 2, 256, 1024
    logits = (np.random.default_rng(2).standard_normal((B, N, V))).astype(np.float32)
    canvas = np.arange(B * N, dtype=np.int32).reshape(B, N) % V
    argmax = np.zeros((B, N), dtype=np.int32)
    stop = np.array([1, 0], dtype=np.int32)
    before = canvas.copy()
    sampler.sample_update(_params(), 0, logits, canvas, argmax, stop)
    assert (canvas[0] == before[0]).all() and (argmax[0] == 0).all() and stop[0] == 1
    assert (canvas[1] != before[1]).any()


def test_unlocked_positions_are_renoised_uniformly():
    # All positions unlocked: the new canvas is the Philox renoise stream, which
    # must be uniform over [0, V).
    B, N, V = 8, 256, 1000
    logits = np.zeros((B, N, V), dtype=np.float32)
    canvas = np.zeros((B, N), dtype=np.int32)
    argmax = np.zeros((B, N), dtype=np.int32)
    stop = np.zeros(B, dtype=np.int32)
    counts = np.zeros(10)
    for t in range(5):
        stop[:] = 0
        sampler.sample_update(_params(max_steps=48), t, logits, canvas, argmax, stop)
        counts += np.bincount(canvas.ravel() // 100, minlength=10)
    n = counts.sum()
    chi2 = ((counts - n / 10) ** 2 / (n / 10)).sum()
    assert chi2 < 27.9      # 9 dof, p = 0.001


def test_canvas_init_uniform_and_seeded():
    a = sampler.canvas_init(0, 0, 4, 256, 1024)
    b = sampler.canvas_init(0, 1, 4, 256, 1024)
    c = sampler.canvas_init(1, 0, 4, 256, 1024)
    assert a.min() >= 0 and a.max() < 1024
    assert (a != b).mean() > 0.99 and (a != c).mean() > 0.99
    big = sampler.canvas_init(3, 0, 64, 256, 16)
    counts = np.bincount(big.ravel(), minlength=16)
    n = counts.sum()
    assert ((counts - n / 16) ** 2 / (n / 16)).sum() < 37.7   # 15 dof, p = 0.001


def test_page_facts_are_the_defaults():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    p = _params()
    assert p["lock_theta"] == facts["lock_entropy_budget"]["value"]
    assert p["temp_start"] == facts["temperature_start"]["value"]
    assert p["temp_end"] == facts["temperature_end"]["value"]
    assert p["stop_tau"] == facts["stop_mean_entropy"]["value"]
    assert p["max_steps"] == facts["max_rounds"]["value"]
    from discrete_text_diffusion_denoise_amd.synthetic import SHAPES
    assert SHAPES["layer"]["canvas"] == facts["canvas_tokens"]["value"]
    assert SHAPES["layer"]["n_experts"] == facts["n_experts"]["value"]
    assert SHAPES["layer"]["top_k"] == facts["active_experts"]["value"]


@pytest.mark.parametrize("top_k", [0, 8])
def test_nonfinite_canvas_is_reported_and_left_as_it_was(top_k):
    # A NaN, +inf or -inf logit anywhere in a row makes its entropy NaN
    # under the fixed arithmetic (0 * inf, NaN, or a chunk whose maximum is
    # not finite); the canvas gets stop = 2 and keeps its canvas, argmax and
    # locks; a finite canvas in the same call is updated exactly as it would
    # be alone.  With top-k truncation only the candidates are read; a NaN
    # ranks above every number, so a NaN or +inf always is a candidate and
    # shows, while a -inf below K finite logits is no candidate.
    B, N, V = 5, 16, 64
    rng = np.random.default_rng(7)
    logits = (rng.standard_normal((B, N, V)) * 3.0).astype(np.float32)
    logits[1, 5, 17] = np.nan
    logits[2, 0, 3] = np.inf
    logits[3, 15, 63] = -np.inf
    logits[4, 9, 0] = np.nan        # the first member of its chunk
    canvas = rng.integers(0, V, (B, N)).astype(np.int32)
    argmax = rng.integers(0, V, (B, N)).astype(np.int32)
    stop = np.zeros(B, dtype=np.int32)
    c0, a0 = canvas.copy(), argmax.copy()
    p = _params(max_steps=5, top_k=top_k)
    lock, stats = sampler.sample_update(p, 2, logits, canvas, argmax, stop)
    bad = (1, 2, 3, 4) if top_k == 0 else (1, 2, 4)
    for b in bad:
        assert stop[b] == 2
        assert (canvas[b] == c0[b]).all() and (argmax[b] == a0[b]).all()
        assert not lock[b].any()
    if top_k == 0:
        assert np.isnan(stats[1, 5, 2]) and np.isnan(stats[3, 15, 2]) and np.isnan(stats[4, 9, 2])
    assert np.isnan(stats[2, 0, 2])
    if top_k:
        assert np.isnan(stats[1, 5, 2]) and np.isnan(stats[4, 9, 2])
        assert np.isfinite(stats[3]).all() and stop[3] != 2
    # canvas 0 alone gives the same bits
    c1, a1, s1 = c0[:1].copy(), a0[:1].copy(), np.zeros(1, np.int32)
    lock1, stats1 = sampler.sample_update(p, 2, logits[:1], c1, a1, s1)
    assert stop[0] == s1[0] != 2
    assert (canvas[0] == c1[0]).all() and (argmax[0] == a1[0]).all() and (lock[0] == lock1[0]).all()
    assert (stats[0].view(np.uint32) == stats1[0].view(np.uint32)).all()


def test_locked_token_can_change_later():
    # Report-summary page, section 1 (multinomial rather than masked
    # diffusion, so any position can still be replaced), and the youleyou.com
    # article, "How discrete text diffusion works" (self-correction: when the
    # confidence at a position drops in a later pass, the sampler renoises
    # and replaces it): a lock is decided anew every round, so a token locked
    # in one round is re-drawn, or renoised, when a later round is no longer
    # confident about it.  Round 0: every position of canvas 0 is
    # one-hot on token a (all lock to a); round 1: positions 0..127 are
    # one-hot on another token b (they re-lock to b), positions 128..255 are
    # flat (they unlock and are renoised, so they leave a almost surely).
    B, N, V = 1, 256, 1024
    a, b = 17, 900
    p = _params(lock_rule=1, lock_theta=0.1, require_stable=0, stop_tau=-1.0, max_steps=48)
    canvas = np.zeros((B, N), dtype=np.int32)
    argmax = np.zeros((B, N), dtype=np.int32)
    stop = np.zeros(B, dtype=np.int32)
    l0 = np.full((B, N, V), -60.0, dtype=np.float32)
    l0[..., a] = 40.0
    lock, _ = sampler.sample_update(p, 0, l0, canvas, argmax, stop)
    assert (lock == 1).all() and (canvas == a).all()
    l1 = np.zeros((B, N, V), dtype=np.float32)
    l1[:, :128, :] = -60.0
    l1[:, :128, b] = 40.0
    lock, stats = sampler.sample_update(p, 1, l1, canvas, argmax, stop)
    assert stop[0] == 0
    assert (lock[0, :128] == 1).all() and (canvas[0, :128] == b).all()
    assert (lock[0, 128:] == 0).all()
    assert (canvas[0, 128:] != a).mean() > 0.95
    assert (argmax[0, :128] == b).all()
