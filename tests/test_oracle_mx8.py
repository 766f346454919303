"""Pins of the oracle's MXFP8 activation format (oracle/quant.py mx8_*) and of
where the quantised-expert MoE applies it (oracle/model.py moe, act_mx8).

The element rounding is checked against torch's own float8_e4m3fn
conversion (an independent implementation of OCP E4M3 round-to-nearest-even)
on values inside the finite range; the shared-scale rule of the OCP
microscaling specification (X = 2^(floor(log2 amax) - 8) for E4M3) on
hand-worked blocks, including the specification's saturation of the top of
the range; brute force on small blocks (every dequantised element is a
nearest point of the block's whole value grid); exact representability; the
round trip's error bound; and a loop-written MoE on a tiny layer whose
quantisation is the brute-force grid search.  CPU only."""
import math

import numpy as np
import pytest
import torch

from oracle import model as om
from oracle import quant as q

GRID = np.array(sorted({q.e4m3_decode(c) for c in range(256) if not np.isnan(q.e4m3_decode(c))}))


def test_element_rounding_matches_torch_float8():
    rng = np.random.default_rng(0)
    mags = np.concatenate([rng.uniform(0, 448, 20000), np.exp2(rng.uniform(-12, 8.8, 20000)),
                           GRID[GRID >= 0], (GRID[1:] + GRID[:-1]) / 2])
    mags = mags[mags < 448].astype(np.float32)
    x = np.concatenate([mags, -mags]).astype(np.float64)
    got = np.array([q.e4m3_decode(c) for c in q._e4m3_nearest(x)])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, ref)


def test_shared_scale_worked_blocks():
    b = np.zeros((1, 32))
    b[0, 0] = 1.0                 # floor(log2 1) = 0 -> X = 2^-8, scale code 119; 1 / X = 256
    b[0, 1] = -0.5                # -128 exactly: code 0xF0
    b[0, 2] = 1.0 / 1024          # 1/1024 / X = 2^-2: exponent field 5, code 0x28
    codes, sc = q.mx8_quantize_rows(b)
    assert sc.tolist() == [[119]]
    assert codes[0, :3].tolist() == [0x78, 0xF0, 0x28]
    # amax 1.9: X = 2^-8 and 1.9 / X = 486.4 lies above 448 -> saturates
    # (the specification's rule leaves [448, 512) to saturation)
    b[0, 0] = 1.9
    codes, sc = q.mx8_quantize_rows(b)
    assert sc.tolist() == [[119]] and codes[0, 0] == 0x7E
    assert q.mx8_dequantize_rows(codes, sc)[0, 0] == 448.0 / 256
    # amax 0.75: floor(log2 0.75) = -1 -> X = 2^-9, 0.75 / X = 384 = 1.5 * 2^8: code 0x7C
    b[0, 0] = 0.75
    codes, sc = q.mx8_quantize_rows(b)
    assert sc.tolist() == [[118]] and codes[0, 0] == 0x7C
    # an all-zero block takes scale code 0 and zero codes
    codes, sc = q.mx8_quantize_rows(np.zeros((2, 64)))
    assert sc.tolist() == [[0, 0], [0, 0]] and not codes.any()
    # tiny and huge blocks clamp the scale exponent to [-127, 127]
    codes, sc = q.mx8_quantize_rows(np.full((1, 32), 1e-40))
    assert sc[0, 0] == 0
    codes, sc = q.mx8_quantize_rows(np.full((1, 32), 2.0 ** 140))
    assert sc[0, 0] == 254


def brute_block(v):
    """One 32-element block by enumeration: X from floor(log2 amax) (math
    module), each element the nearest grid value times X, ties to the even
    code (the grid is in code order for non-negative values)."""
    amax = max(abs(float(t)) for t in v)
    ex = -127 if amax == 0 else min(127, max(-127, math.floor(math.log2(amax)) - 8))
    X = 2.0 ** ex
    out = []
    for t in v:
        a = abs(float(t)) / X
        if a >= 448:
            m = 448.0
        else:
            pos = GRID[GRID >= 0]
            d = np.abs(pos - a)
            i = np.flatnonzero(d == d.min())
            m = pos[i[0]] if len(i) == 1 or i[0] % 2 == 0 else pos[i[1]]
        out.append(math.copysign(m * X, float(t)))
    return np.array(out), ex + 127


@pytest.mark.parametrize("seed,sigma", [(1, 1.0), (2, 1e-3), (3, 50.0), (4, 1e-30)])
def test_brute_force_small_blocks(seed, sigma):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((6, 64)) * sigma
    x[0, :32] = 0.0
    x[1, 5] = 0.0
    x[2, 40] = -np.abs(x[2, 32:64]).max()              # a negative block maximum
    codes, sc = q.mx8_quantize_rows(x)
    deq = q.mx8_dequantize_rows(codes, sc)
    for r in range(x.shape[0]):
        for blk in range(2):
            v = x[r, 32 * blk:32 * blk + 32]
            ref, code = brute_block(v)
            assert sc[r, blk] == code
            assert np.array_equal(deq[r, 32 * blk:32 * blk + 32], ref)


def test_representable_round_trip_is_identity():
    # blocks whose largest element has exponent field 15 under X reproduce X
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 0x7F, (4, 96)).astype(np.uint8)
    codes[codes == 0x7F] = 0x10
    codes |= (rng.integers(0, 2, codes.shape) << 7).astype(np.uint8)
    codes[:, ::32] = 0x78 | (codes[:, ::32] & 0x80)      # 256: exponent field 15
    sc = rng.integers(100, 150, (4, 3)).astype(np.uint8)
    x = q.mx8_dequantize_rows(codes, sc)
    c2, s2 = q.mx8_quantize_rows(x)
    assert np.array_equal(s2, sc)
    assert np.array_equal(q.mx8_dequantize_rows(c2, s2), x)


def test_round_trip_error_bound():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 256)) * np.exp2(rng.uniform(-20, 20, (64, 1)))
    r = q.mx8_round(x)
    blocks = np.abs(x).reshape(64, 8, 32).max(axis=2)
    X = np.exp2(np.floor(np.log2(blocks)) - 8).repeat(32, axis=1)
    a = np.abs(x) / X
    err = np.abs(r - x) / X
    normal = (a >= 2.0 ** -6) & (a < 448)
    assert (err[normal] <= a[normal] * 2.0 ** -4 * (1 + 1e-12)).all()    # half a 3-bit ulp
    assert (err[a < 2.0 ** -6] <= 2.0 ** -10 * (1 + 1e-12)).all()          # half a subnormal step
    sat = a >= 448
    assert np.allclose(np.abs(r[sat]) / X[sat], 448.0)
    assert (np.sign(r) == np.sign(x))[np.abs(r) > 0].all()


def test_moe_rounds_both_expert_inputs():
    """A three-expert, top-2 layer written as loops: the token rounded to
    MXFP8 (brute force), gate and up, silu(gate) * up rounded to MXFP8
    (brute force), down, times the routing weight (softmax of the two chosen
    router logits, so rounding after the weight would differ); the router
    sees the unrounded token.  The oracle's moe(act_mx8=True) must agree to
    float64 rounding, and differ from the unrounded MoE by far more."""
    rng = np.random.default_rng(11)
    T, d, F, E = 3, 64, 32, 3
    u = rng.standard_normal((T, d))
    lw = {"w_router": rng.standard_normal((E, d)), "w_gate": rng.standard_normal((E, F, d)) * 0.2,
          "w_up": rng.standard_normal((E, F, d)) * 0.2, "w_down": rng.standard_normal((E, d, F)) * 0.2}
    y, idx, g, z = om.moe(u, lw, 2, act_mx8=True)
    y_plain, idx2, _, z2 = om.moe(u, lw, 2)
    assert np.array_equal(idx, idx2) and np.array_equal(z, z2)
    ref = np.zeros((T, d))
    for t in range(T):
        top = sorted(range(E), key=lambda e: -z[t, e])[:2]
        w = np.exp(z[t, top] - z[t, top].max())
        w = w / w.sum()
        xq = np.concatenate([brute_block(u[t, b:b + 32])[0] for b in range(0, d, 32)])
        for e, we in zip(top, w):
            gate = np.array([sum(lw["w_gate"][e, f, i] * xq[i] for i in range(d)) for f in range(F)])
            up = np.array([sum(lw["w_up"][e, f, i] * xq[i] for i in range(d)) for f in range(F)])
            a = gate / (1 + np.exp(-gate)) * up
            aq = np.concatenate([brute_block(a[b:b + 32])[0] for b in range(0, F, 32)])
            ref[t] += we * np.array([sum(lw["w_down"][e, j, f] * aq[f] for f in range(F))
                                     for j in range(d)])
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()
    assert np.abs(y - y_plain).max() > 1e-3 * np.abs(ref).max()
