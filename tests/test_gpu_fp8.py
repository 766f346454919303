"""8-bit expert weights: the library's quantiser (dg_quantize_fp8) against
the oracle's (oracle/quant.py), bit for bit, on fp32 and bf16 sources,
including exact ties, subnormal codes, saturation and an all-zero row.  The
expert kernels on 8-bit weights are checked against the oracle in
test_gpu_model.py (small_fp8)."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_denoise_amd import binding, synthetic
from oracle import quant as oq

from helpers import DEV, to_dev

pytestmark = pytest.mark.gpu


def tie_rows(K: int) -> np.ndarray:
    """Rows whose amax is 448 * 2^j, so the scale is the power of two 2^j and
    every quotient is exact: midpoints between codes (ties), subnormal steps,
    the smallest normal, values that round up into the next binade."""
    vals = np.array([448.0, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -11,
                     7.5 * 2.0 ** -9, 15.5 * 2.0 ** -9, 1.96875, 240.0, 232.0, 0.0, -0.0],
                     dtype=np.float32)
    rows = []
    for j in (-12, -3, 0, 5):
        r = np.resize(vals, K) * np.float32(2.0 ** j)
        rows.append(r)
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_quantize_fp8_bit_exact(src):
    rng = np.random.default_rng(7)
    R, K = 300, 777
    w = (rng.standard_normal((R, K)) * 0.02).astype(np.float32)
    w[5] = 0.0                                     # scale 1, all codes zero
    w[6] *= 1e-30                                  # tiny row: subnormal binary32 inputs
    w[7] *= 1e6
    w[8:12] = tie_rows(K)
    if src == "bf16":
        w = synthetic.round_bf16(w)
        d = to_dev(w, torch.bfloat16)
    else:
        d = to_dev(w)
    q = torch.empty((R, K), dtype=torch.uint8, device=DEV)
    s = torch.empty(R, dtype=torch.float32, device=DEV)
    binding.quantize_fp8(d, q, s)
    torch.cuda.synchronize()
    rq, rs = oq.quantize_rows(w)
    gs = s.cpu().numpy()
    assert (gs.view(np.uint32) == rs.view(np.uint32)).all(), np.argwhere(gs != rs)[:5]
    gq = q.cpu().numpy()
    bad = np.argwhere(gq != rq)
    assert len(bad) == 0, [(int(r), int(c), int(gq[r, c]), int(rq[r, c]), float(w[r, c]))
                           for r, c in bad[:5]]


def test_quantize_fp8_expert_shape():
    """A [E][R][K] expert matrix is rows = E*R: the same codes as row by row."""
    rng = np.random.default_rng(8)
    w = synthetic.round_bf16((rng.standard_normal((3, 64, 512)) * 0.02).astype(np.float32))
    d = to_dev(w, torch.bfloat16)
    q = torch.empty(w.shape, dtype=torch.uint8, device=DEV)
    s = torch.empty(w.shape[:-1], dtype=torch.float32, device=DEV)
    binding.quantize_fp8(d, q, s)
    torch.cuda.synchronize()
    rq, rs = oq.quantize_rows(w.reshape(-1, 512))
    assert (q.cpu().numpy().reshape(-1, 512) == rq).all()
    assert (s.cpu().numpy().reshape(-1) == rs).all()
