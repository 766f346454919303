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

MXFP4 (OCP Microscaling Formats specification, v1.0): blocks of 32
consecutive elements of a row share one E8M0 scale (an 8-bit biased
exponent, X = 2^(code - 127)); each element is an FP4 E2M1 value (1 sign, 2
exponent bits with bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6).  The
specification's scale is X = 2^(floor(log2(max |v|)) - emax), emax = 2 for
E2M1 (6 = 1.5 * 2^2), and each element is v / X rounded to the nearest E2M1
value with ties to the even code, magnitudes above 6 clamped to 6.  Readings
of this library: an all-zero block takes code 0 (X = 2^-127) and zero
elements; the scale exponent is clamped to [-127, 127]; two elements per byte,
the even-indexed one in the low nibble.

MXFP8 activations (same specification, element type E4M3, emax = 8 since
448 = 1.75 * 2^8): the quantised experts multiply 8-bit operands on both
sides, so the activations entering each expert product are rounded to MXFP8
first: per token, blocks of 32 consecutive features share the E8M0 scale
X = 2^(floor(log2(max |v|)) - 8) (clamped to [-127, 127], an all-zero block
taking -127), and each element is v / X rounded to the nearest E4M3 value
(ties to the even code), magnitudes at or above 448 giving 448.  Reading:
the pages name only the 4-bit weight format; the activation format, and that
it applies to both the gate/up input (the normalised token) and the down
input (silu(gate) * up, before the routing weight), is this library's
choice, the plainest one that lets both MFMA operands be 8-bit or narrower.
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


# ---------------------------------------------------------------- MXFP4

FP4_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
FP4_MAX = 6.0
MX_BLOCK = 32


def fp4_decode(code: int) -> float:
    """Value of a 4-bit E2M1 code."""
    code = int(code) & 0xF
    return (-1.0 if code & 8 else 1.0) * FP4_MAG[code & 7]


def fp4_encode(x: float) -> int:
    """E2M1 code of the nearest value to x (ties to the even code), magnitudes
    above 6 giving 6; the sign is kept (-0 gives code 8)."""
    neg = bool(np.signbit(x))
    a = abs(float(x))
    if a >= FP4_MAX:
        c = 7
    else:
        d = np.abs(FP4_MAG - a)
        best = d.min()
        cands = np.nonzero(d == best)[0]
        c = int(cands[0])
        if len(cands) > 1:
            c = int(cands[0] if cands[0] % 2 == 0 else cands[1])
    return c | (8 if neg else 0)


def fp4_encode_array(x: np.ndarray) -> np.ndarray:
    """fp4_encode of every entry (the two table neighbours, the nearer one,
    ties to the even code)."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(FP4_MAG, a), 0, 7)
    lo = np.clip(hi - 1, 0, 7)
    d_lo = a - FP4_MAG[lo]
    d_hi = FP4_MAG[hi] - a
    c = np.where(d_hi < d_lo, hi, lo)
    c = np.where(d_hi == d_lo, np.where(lo % 2 == 0, lo, hi), c)
    c = np.where(a >= FP4_MAX, 7, c)
    return (c | np.where(neg, 8, 0)).astype(np.uint8)


def mx_scale_exponent(amax: np.ndarray, emax: int = 2) -> np.ndarray:
    """floor(log2(amax)) - emax per block (emax 2 for E2M1, 8 for E4M3),
    clamped to [-127, 127]; -127 for an all-zero block."""
    amax = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(amax)                  # amax = m 2^e, m in [0.5, 1)
    ex = (e - 1) - emax
    ex = np.where(amax > 0, ex, -127)
    return np.clip(ex, -127, 127).astype(np.int64)


def mx_quantize_rows(w: np.ndarray):
    """Rows of w [R, K] (K % 32 == 0, values rounded to binary32) -> (codes
    uint8 [R, K], one E2M1 code per element; scale codes uint8 [R, K/32])."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    R, K = w.shape
    blocks = w.reshape(R, K // MX_BLOCK, MX_BLOCK)
    ex = mx_scale_exponent(np.abs(blocks).max(axis=2))
    quo = blocks * np.ldexp(1.0, -ex)[..., None]         # exact: a power of two
    codes = fp4_encode_array(quo).reshape(R, K)
    return codes, (ex + 127).astype(np.uint8)


def mx_pack(codes: np.ndarray) -> np.ndarray:
    """Two E2M1 codes per byte along the last axis, the even one in the low
    nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def mx_unpack(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def mx_dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """decode(code) * 2^(scale - 127) per element, in float64 (exact)."""
    table = np.array([fp4_decode(c) for c in range(16)], dtype=np.float64)
    codes = np.asarray(codes, dtype=np.uint8)
    R, K = codes.shape
    x = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (table[codes].reshape(R, K // MX_BLOCK, MX_BLOCK) * x[..., None]).reshape(R, K)


# ---------------------------------------------------------------- MXFP8

MX8_EMAX = 8


def mx8_quantize_rows(x: np.ndarray):
    """Rows of x [R, K] (K % 32 == 0; float64 or float32 values) -> (E4M3
    codes uint8 [R, K], E8M0 scale codes uint8 [R, K/32]) by the MXFP8 rule
    in the module docstring.  The quotient v / X is exact (X is a power of
    two) and is rounded once, to E4M3."""
    x = np.asarray(x, dtype=np.float64)
    R, K = x.shape
    blocks = x.reshape(R, K // MX_BLOCK, MX_BLOCK)
    ex = mx_scale_exponent(np.abs(blocks).max(axis=2), MX8_EMAX)
    quo = blocks * np.ldexp(1.0, -ex)[..., None]
    codes = _e4m3_nearest(quo).reshape(R, K)
    return codes, (ex + 127).astype(np.uint8)


def _e4m3_nearest(a: np.ndarray) -> np.ndarray:
    """E4M3 code of the nearest value to each float64 entry (ties to the even
    code, saturating at 448, sign kept): the table-neighbour rule of
    e4m3_encode_array without its binary32 rounding of the input."""
    a = np.asarray(a, dtype=np.float64)
    neg = np.signbit(a)
    m = np.abs(a)
    hi = np.clip(np.searchsorted(_POS, m), 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_lo = m - _POS[lo]
    d_hi = _POS[hi] - m
    c = np.where(d_hi < d_lo, hi, lo)
    c = np.where(d_hi == d_lo, np.where(lo % 2 == 0, lo, hi), c)
    c = np.where(m >= E4M3_MAX, 0x7E, c)
    return (c | np.where(neg, 0x80, 0)).astype(np.uint8)


def mx8_dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """decode(code) * 2^(scale - 127) per element, in float64 (exact)."""
    table = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
    codes = np.asarray(codes, dtype=np.uint8)
    R, K = codes.shape
    X = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (table[codes].reshape(R, K // MX_BLOCK, MX_BLOCK) * X[..., None]).reshape(R, K)


def mx8_round(x: np.ndarray) -> np.ndarray:
    """x [..., K] rounded to MXFP8 along its last axis (quantise, then
    dequantise), float64."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1, x.shape[-1])
    c, sc = mx8_quantize_rows(flat)
    return mx8_dequantize_rows(c, sc).reshape(x.shape)
