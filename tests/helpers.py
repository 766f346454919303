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
