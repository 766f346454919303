"""The calibration probes behind bench.py's measured peaks (dg_measure_peaks):
they run, report rates in a plausible range of the published peaks
(8 TB/s HBM, 2.5 PFLOP/s bf16 dense), and reject a buffer below 256 MiB."""
import ctypes

import pytest

from discrete_text_diffusion_denoise_amd import binding

torch = pytest.importorskip("torch")


@pytest.mark.gpu
def test_measure_peaks():
    buf = torch.empty(80 << 20, dtype=torch.float32, device="cuda")   # 320 MiB
    gbs, tflops = binding.measure_peaks(buf)
    print(f"probe: HBM read {gbs:.0f} GB/s, bf16 MFMA {tflops:.0f} TFLOP/s", flush=True)
    assert 1000.0 < gbs < 8000.0 * 1.05
    assert 500.0 < tflops < 2500.0 * 1.05
    small = torch.empty(32 << 20, dtype=torch.float32, device="cuda")  # 128 MiB
    d = ctypes.c_double()
    st = binding.lib().dg_measure_peaks(ctypes.c_void_p(small.data_ptr()),
                                        small.numel() * 4, None, ctypes.byref(d),
                                        ctypes.byref(d))
    assert st == 4   # DG_ERR_CAPACITY
