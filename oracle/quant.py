"""Plain CPU oracle of the 8-bit expert-weight format (numpy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the benchmark's
CPU-baseline leg; never by the product path.  It shares no code with the HIP
library.

Why the format exists: the youleyou.com article ("Deployment") says the model
ships tuned for a 4-bit floating-point weight format on NVIDIA parts, so that
the memory-bound mixture of experts moves fewer bytes.  The MI355X analogue
kept here is the OCP 8-bit floating-point format E4M3 ("e4m3fn"), which
CDNA4 converts in hardware, with one fp32 scale per weight row (per output
feature of each expert's matrix).

E4M3 (OCP 8-bit floating point specification): 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits.  Exponent field 0 holds subnormals m * 2^-9;
fields 1..15 hold (1 + m/8) * 2^(e-7); the one NaN pattern per sign is
exponent 15 with mantissa 7, so the largest finite value is 448 and there is
no infinity.

Quantisation of a row w[0..K) (this library's definition, written out):
  amax  = max_k |w_k|                      (binary32)
  scale = amax / 448 in binary32 (scale = 1 when amax = 0)
  q_k   = E4M3 code of the binary32 quotient w_k / scale, rounded to the
          nearest representable value, ties to the even code, magnitudes at
          or above 448 giving 448 (the sign is kept, -0 gives code 0x80)
  dequantised weight = decode(q_k) * scale.
Every function below follows that text; the encoder is the plain
definition (nearest entry of the value table), not a bit trick.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of an E4M3 byte (NaN for the two NaN patterns)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# value of every non-negative finite code 0x00 .. 0x7E (increasing)
_POS = np.array([e4m3_decode(c) for c in range(0x7F)], dtype=np.float64)


def e4m3_encode(x: float) -> int:
    """E4M3 code of the nearest representable value to the finite x (ties to
    the even code), saturating at 448."""
    x = float(np.float32(x))
    neg = np.signbit(x)
    a = abs(x)
    if a >= E4M3_MAX:
        c = 0x7E
    else:
        d = np.abs(_POS - a)
        best = float(d.min())
        cands = np.nonzero(d == best)[0]
        c = int(cands[0])
        if len(cands) > 1:                        # a tie: the even code
            c = int(cands[0] if cands[0] % 2 == 0 else cands[1])
    return c | (0x80 if neg else 0)


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    """e4m3_encode of every entry (the same nearest-table rule, vectorised:
    the two table neighbours of |x|, the nearer one, ties to the even code)."""
    x = np.asarray(x, dtype=np.float32)
    neg = np.signbit(x)
    a = np.abs(x).astype(np.float64)
    hi = np.clip(np.searchsorted(_POS, a), 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    c = np.where(d_hi < d_lo, hi, lo)
    tie = d_hi == d_lo
    c = np.where(tie, np.where(lo % 2 == 0, lo, hi), c)
    c = np.where(a >= E4M3_MAX, 0x7E, c)
    return (c | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_rows(w: np.ndarray):
    """Rows of w [R, K] (rounded to binary32) -> (codes uint8 [R, K], scales
    float32 [R]) by the definition in the module docstring."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=1).astype(np.float32)
    # binary32 scale per row (1 for an all-zero row), binary32 quotients
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    quo = (w / s[:, None]).astype(np.float32)
    return e4m3_encode_array(quo), s


def dequantize_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """decode(q) * scale per row, in float64 (exact)."""
    table = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(q, dtype=np.uint8)] * np.asarray(s, dtype=np.float64)[:, None]
