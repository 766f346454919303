"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):

  * the sampler oracle (oracle/sampler.c) driven by tests/sanitize/
    sampler_checks.c: full and top-k updates over ragged vocabularies,
    non-finite rows, corruption, cross-entropy, canvas initialisation;
  * the library's host-side ABI code (dg_api.cpp compiled with the host
    sanitizers, linked with the regular kernel objects) driven by
    tests/sanitize/host_checks.cpp: argument validation, shape and dtype
    checks, size queries and handles -- every call returns before GPU work.

The sanitizers abort on the first report, so a clean exit is the check."""
import glob
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "discrete_text_diffusion_denoise_amd", "csrc")
BUILD = os.path.join(ROOT, "discrete_text_diffusion_denoise_amd", "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, env=None):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env)
    return r.returncode, r.stdout


def test_sampler_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "sampler_checks")
    rc, out = _run([gcc, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-ffp-contract=off",
                    os.path.join(ROOT, "oracle", "sampler.c"),
                    os.path.join(HERE, "sanitize", "sampler_checks.c"), "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert rc == 0 and "sampler checks ok" in out, out


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm toolchain not available")
    kernels = [o for o in glob.glob(os.path.join(BUILD, "*.o")) if not o.endswith("dg_api.o")]
    if len(kernels) < 5:
        pytest.fail("kernel objects missing: build the library first "
                    "(python -m discrete_text_diffusion_denoise_amd.build)")
    api = str(tmp_path / "dg_api_san.o")
    drv = str(tmp_path / "host_checks.o")
    exe = str(tmp_path / "host_checks")
    # the sanitizers instrument host code only (each -fsanitize behind -Xarch_host)
    rc, out = _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=undefined",
                    "-c", os.path.join(CSRC, "dg_api.cpp"), "-o", api])
    assert rc == 0, out
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    rc, out = _run([CLANG, "-O1", "-g", "-std=c++17", *san, "-fno-omit-frame-pointer",
                    "-I" + os.path.join(ROOT, "include"), "-c",
                    os.path.join(HERE, "sanitize", "host_checks.cpp"), "-o", drv])
    assert rc == 0, out
    rc, out = _run([CLANG, *san, drv, api, *kernels, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert rc == 0 and "host checks ok" in out, out
