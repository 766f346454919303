"""Shared helpers of the GPU parity tests (the HIP path through the C ABI
against the CPU oracle on identical seeded inputs)."""
import numpy as np
import torch

from discrete_text_diffusion_denoise_amd import synthetic

# Tolerances on max|gpu - ref| / max|ref| per output tensor.
TOL_F32 = 1e-4      # fp32 model: fp32 arithmetic against float64
TOL_BF16 = 2e-2     # bf16 model: bf16 operands, fp32 accumulation

DEV = "cuda:0"


def normwise(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def tol_for(cfg) -> float:
    return TOL_BF16 if cfg["dtype"] == "bf16" else TOL_F32


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def round_model_dtype(cfg, a):
    """Inputs that the GPU stores in the model dtype must be given to the
    oracle with the same rounding."""
    a = np.asarray(a, dtype=np.float32)
    return synthetic.round_bf16(a) if cfg["dtype"] == "bf16" else a


def route_ambiguous(z: np.ndarray, k: int, gap: float) -> np.ndarray:
    """Tokens whose k-th and (k+1)-th router logits are closer than `gap`:
    either route set is a correct top-k at the GPU's precision."""
    if z.shape[1] <= k:
        return np.zeros(z.shape[0], dtype=bool)
    s = -np.sort(-z, axis=1)
    return (s[:, k - 1] - s[:, k]) < gap


def route_is_valid(z: np.ndarray, chosen: np.ndarray, k: int, gap: float) -> bool:
    """Every chosen expert is within `gap` of the k-th largest logit, and the
    chosen experts are distinct."""
    s = -np.sort(-z, axis=1)
    kth = s[:, k - 1]
    zc = np.take_along_axis(z, chosen.astype(np.int64), axis=1)
    distinct = all(len(set(r)) == k for r in chosen.tolist())
    return bool(distinct and (zc >= kth[:, None] - gap).all())


# ---- the quantised experts' tiled weight layout (include/dg.h,
# dg_quantize_fp8 / dg_quantize_mxfp4): 16-row tiles, one after another; in a
# tile its 128-column steps; a step is MFMA operand order -- chunk 16 g + r
# (16 bytes) holds row r's g-th 16-byte piece of the step (E4M3: per 64-column
# half; MXFP4: the 32-column block g), and for MXFP4 byte 16 g + r of 64 is
# that block's scale code.  Written here from that description (a pure index
# permutation), to compare the library's output with the oracle's row-major
# codes and to hand the oracle's codes to the library.

def tile_e4m3(q: np.ndarray) -> np.ndarray:
    """Row-major E4M3 codes [R, K] -> the tiled byte stream."""
    R, K = q.shape
    t = np.asarray(q, np.uint8).reshape(R // 16, 16, K // 128, 2, 4, 16)   # rt r s h g p
    return np.ascontiguousarray(t.transpose(0, 2, 3, 4, 1, 5)).reshape(-1)


def untile_e4m3(b: np.ndarray, R: int, K: int) -> np.ndarray:
    t = np.asarray(b, np.uint8).reshape(R // 16, K // 128, 2, 4, 16, 16)   # rt s h g r p
    return np.ascontiguousarray(t.transpose(0, 4, 1, 2, 3, 5)).reshape(R, K)


def tile_mxfp4(packed: np.ndarray, scales: np.ndarray):
    """Row-major packed E2M1 codes [R, K/2] and scale codes [R, K/32] -> the
    tiled (code bytes, scale bytes)."""
    R, Kh = packed.shape
    S = 2 * Kh // 128
    c = np.asarray(packed, np.uint8).reshape(R // 16, 16, S, 4, 16)        # rt r s g j
    x = np.asarray(scales, np.uint8).reshape(R // 16, 16, S, 4)            # rt r s g
    return (np.ascontiguousarray(c.transpose(0, 2, 3, 1, 4)).reshape(-1),
            np.ascontiguousarray(x.transpose(0, 2, 3, 1)).reshape(-1))


def untile_mxfp4(codes: np.ndarray, scales: np.ndarray, R: int, K: int):
    S = K // 128
    c = np.asarray(codes, np.uint8).reshape(R // 16, S, 4, 16, 16)         # rt s g r j
    x = np.asarray(scales, np.uint8).reshape(R // 16, S, 4, 16)            # rt s g r
    return (np.ascontiguousarray(c.transpose(0, 3, 1, 2, 4)).reshape(R, K // 2),
            np.ascontiguousarray(x.transpose(0, 3, 1, 2)).reshape(R, K // 32))
