"""Pins of the oracle's MXFP4 format (oracle/quant.py): the E2M1 value table
against the format's definition by fields, the encoder's ties, saturation
and sign, the shared-scale rule of the OCP microscaling specification on
hand-worked blocks, exact representability (dequantise then quantise is the
identity), and the error bound of the round trip.  CPU only."""
import numpy as np
import pytest

from oracle import quant as q


def test_e2m1_table_from_fields():
    # value = (-1)^s * (e == 0 ? m/2 : (1 + m/2) * 2^(e - 1)), bias 1
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = (m / 2.0) if e == 0 else (1 + m / 2.0) * 2.0 ** (e - 1)
        assert q.fp4_decode(c) == (-v if s else v)
    assert sorted({abs(q.fp4_decode(c)) for c in range(16)}) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


@pytest.mark.parametrize("x,code", [
    (0.0, 0), (-0.0, 8), (0.25, 0), (0.26, 1), (0.5, 1), (0.75, 2), (1.25, 2), (1.3, 3),
    (1.75, 4), (2.5, 4), (2.6, 5), (3.5, 6), (4.9, 6), (5.0, 6), (5.01, 7), (6.0, 7),
    (7.0, 7), (1e9, 7), (-0.74, 9), (-5.5, 15), (-100.0, 15)])
def test_fp4_encode_ties_saturation_sign(x, code):
    assert q.fp4_encode(x) == code
    assert q.fp4_encode_array(np.array([x]))[0] == code


def test_encode_array_matches_scalar():
    xs = np.concatenate([np.linspace(-8, 8, 3201), q.FP4_MAG, -q.FP4_MAG,
                         (q.FP4_MAG[1:] + q.FP4_MAG[:-1]) / 2])
    assert [int(c) for c in q.fp4_encode_array(xs)] == [q.fp4_encode(x) for x in xs]


def test_shared_scale_worked_blocks():
    # amax 3.0: floor(log2 3) = 1 -> X = 2^(1-2) = 0.5, code 126; 3.0 / 0.5 = 6
    b = np.zeros((1, 32), np.float32)
    b[0, 0] = 3.0
    b[0, 1] = -0.75          # / 0.5 = -1.5 exactly
    b[0, 2] = 0.3            # 0.6 -> 0.5
    codes, sc = q.mx_quantize_rows(b)
    assert sc.tolist() == [[126]]
    assert codes[0, :3].tolist() == [7, 11, 1]
    # amax 7.9 (in [4, 8)): X = 2^0 = 1, 7.9 saturates to 6
    b[0, 0] = 7.9
    codes, sc = q.mx_quantize_rows(b)
    assert sc.tolist() == [[127]] and codes[0, 0] == 7
    # an all-zero block: scale code 0, zero codes
    codes, sc = q.mx_quantize_rows(np.zeros((2, 64), np.float32))
    assert (sc == 0).all() and (codes == 0).all()
    # amax exactly a power of two: 2^-6 -> X = 2^-8, element 4
    b = np.zeros((1, 32), np.float32)
    b[0, 5] = 2.0 ** -6
    codes, sc = q.mx_quantize_rows(b)
    assert sc[0, 0] == 127 - 8 and codes[0, 5] == 6


def test_representable_round_trip_is_identity():
    rng = np.random.default_rng(0)
    R, K = 8, 128
    codes = rng.integers(0, 16, size=(R, K), dtype=np.uint8)
    # keep each block's largest magnitude code at 6 or 7 (4 or 6): that is the
    # scale the rule recovers
    for r in range(R):
        for b in range(K // 32):
            codes[r, 32 * b + 3] = 7
    sc = rng.integers(100, 140, size=(R, K // 32), dtype=np.uint8)
    w = q.mx_dequantize_rows(codes, sc).astype(np.float32)
    c2, s2 = q.mx_quantize_rows(w)
    # -0 and +0 both decode to 0: compare values
    assert np.array_equal(q.mx_dequantize_rows(c2, s2), q.mx_dequantize_rows(codes, sc))
    assert np.array_equal(s2, sc)


def test_round_trip_error_bound_and_packing():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    codes, sc = q.mx_quantize_rows(w)
    d = q.mx_dequantize_rows(codes, sc)
    blocks = np.abs(w.reshape(16, 8, 32)).max(axis=2)
    X = np.ldexp(1.0, sc.astype(np.int64) - 127)
    # below 6X an element is within half a grid step (the largest step is
    # 2X, between 4X and 6X); above it the clamp to 6X costs less than 2X;
    # the block maximum keeps at least 3/4 of its size
    err = np.abs(d - w).reshape(16, 8, 32)
    wb = np.abs(w).reshape(16, 8, 32)
    inside = wb <= 6 * X[..., None]
    assert (err[inside] <= np.broadcast_to(X[..., None], err.shape)[inside]).all()
    assert (err < 2 * X[..., None]).all()
    assert (np.abs(d.reshape(16, 8, 32)).max(axis=2) >= 0.74 * blocks).all()
    packed = q.mx_pack(codes)
    assert packed.shape == (16, 128)
    assert np.array_equal(q.mx_unpack(packed), codes)
    assert packed[0, 0] == (codes[0, 0] | (codes[0, 1] << 4))
