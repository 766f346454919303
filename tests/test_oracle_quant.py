"""Pins of the oracle's 8-bit expert-weight format (oracle/quant.py): values
the OCP E4M3 definition fixes, torch's own float8_e4m3fn conversion as an
independent library routine, round trips and the quantisation invariants."""
import numpy as np
import pytest
import torch

from oracle import quant as oq


def test_decode_closed_forms():
    assert oq.e4m3_decode(0x38) == 1.0
    assert oq.e4m3_decode(0x7E) == 448.0
    assert oq.e4m3_decode(0xFE) == -448.0
    assert oq.e4m3_decode(0x01) == 2.0 ** -9        # smallest subnormal
    assert oq.e4m3_decode(0x07) == 7 * 2.0 ** -9    # largest subnormal
    assert oq.e4m3_decode(0x08) == 2.0 ** -6        # smallest normal
    assert oq.e4m3_decode(0x3F) == 1.875
    assert oq.e4m3_decode(0x80) == 0.0 and np.signbit(oq.e4m3_decode(0x80))
    assert np.isnan(oq.e4m3_decode(0x7F)) and np.isnan(oq.e4m3_decode(0xFF))


def test_decode_matches_torch_for_every_code():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oq.e4m3_decode(c) for c in range(256)])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert ((ref == got) | both_nan).all()


def test_encode_round_trip_and_ties():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oq.e4m3_encode(oq.e4m3_decode(c)) == c
    assert oq.e4m3_encode(1.0625) == 0x38          # between 1 and 1.125: even code
    assert oq.e4m3_encode(1.1875) == 0x3A          # between 1.125 and 1.25: even code
    assert oq.e4m3_encode(2.0 ** -10) == 0x00      # half the smallest subnormal: even (zero)
    assert oq.e4m3_encode(3 * 2.0 ** -11) == 0x01
    assert oq.e4m3_encode(1.05) == 0x38 and oq.e4m3_encode(1.07) == 0x39
    for big in (448.0, 449.0, 464.0, 500.0, 1e6):   # saturation
        assert oq.e4m3_encode(big) == 0x7E and oq.e4m3_encode(-big) == 0xFE
    assert oq.e4m3_encode(-0.0) == 0x80 and oq.e4m3_encode(0.0) == 0x00


def test_encode_matches_torch_conversion():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000) * 40, rng.standard_normal(20000) * 1e-2,
                        rng.uniform(-447, 447, 20000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (oq.e4m3_encode_array(x) == ref).all()


def test_vectorised_encoder_is_the_scalar_one():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(3000) * 100, rng.standard_normal(3000) * 1e-3,
                        np.array([0.0, -0.0, 448.0, 449.0, -1e9, 2.0 ** -10, 1.0625])]).astype(np.float32)
    assert (oq.e4m3_encode_array(x) == np.array([oq.e4m3_encode(v) for v in x])).all()


def test_quantize_rows_invariants():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((16, 300)) * 0.02).astype(np.float32)
    w[3] = 0.0                                      # an all-zero row keeps scale 1
    q, s = oq.quantize_rows(w)
    assert s[3] == 1.0 and (q[3] == 0).all()
    amax = np.abs(w).max(axis=1)
    nz = amax > 0
    assert (s[nz] == (amax[nz] / np.float32(448)).astype(np.float32)).all()
    # the largest entry of each row maps to +-448
    i = np.abs(w).argmax(axis=1)
    assert (q[nz, i[nz]] & 0x7F == 0x7E).all()
    d = oq.dequantize_rows(q, s)
    # three mantissa bits: relative error <= 2^-4 on normal codes, and at
    # most half a subnormal step (2^-10 * scale) below them
    err = np.abs(d - w.astype(np.float64))
    bound = np.maximum(np.abs(w) * 2.0 ** -4, 2.0 ** -10 * s[:, None])
    assert (err <= bound * (1 + 1e-12)).all()
