"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two native drivers are built here with the sanitizers on host code only and
run on the CPU:

* ``native/oracle_checks.c`` with the oracle's C source (gcc): every oracle
  entry point on small inputs in exact-size heap buffers, plus malformed
  arguments;
* ``native/host_api_checks.cpp`` with the library's host-side entry points
  (``api.hip`` rebuilt with ``-Xarch_host`` sanitizer flags, the rest of the
  library linked from ``libcoli_moe.so``): argument, shape and size checks,
  workspace sizing over the whole token range, status strings, and the
  no-device path.  Device pointers there are fake aligned addresses that
  the host never dereferences, so the driver only runs where no GPU is
  visible.

A memory error, a leak or an undefined operation aborts the driver and fails
the test with the sanitizer's report.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def _env(**extra):
    env = dict(os.environ)
    env.update(ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", **extra)
    return env


def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_checks")
    rc, log = _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(NATIVE, "oracle_checks.c"),
                    os.path.join(ROOT, "oracle", "coli_oracle.c"), "-o", exe, "-lm"])
    assert rc == 0, log
    rc, log = _run([exe], env=_env(OMP_NUM_THREADS="2"))
    assert rc == 0 and "oracle checks ok" in log, log


def _gpu_visible() -> bool:
    import torch
    return torch.cuda.is_available()


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_api_under_asan_ubsan():
    if _gpu_visible():
        pytest.skip("the driver passes fake device pointers; it runs only without a GPU")
    from quantized_moe_coli_amd import build as BLD
    assert os.path.exists(BLD.LIB_PATH), "build the library first"
    os.makedirs(OUT, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    api_o = os.path.join(OUT, "api.san.o")
    rc, log = _run([HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
                    "-I", BLD.INCLUDE, "-I", BLD.CSRC,
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
                    "-c", os.path.join(BLD.CSRC, "api.hip"), "-o", api_o])
    assert rc == 0, log
    drv_o = os.path.join(OUT, "host_api_checks.o")
    rc, log = _run([CLANG, "-O1", "-g", "-std=c++17", "-I", BLD.INCLUDE,
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-c", os.path.join(NATIVE, "host_api_checks.cpp"), "-o", drv_o])
    assert rc == 0, log
    exe = os.path.join(OUT, "host_api_checks")
    pkg = os.path.dirname(BLD.LIB_PATH)
    rc, log = _run([HIPCC, "--offload-arch=gfx950", *san, drv_o, api_o, "-L" + pkg,
                    "-lcoli_moe", "-Wl,-rpath," + pkg, "-o", exe])
    assert rc == 0, log
    rc, log = _run([exe], env=_env(COLI_EXPECT_NO_DEVICE="1"))
    assert rc == 0 and "host api checks ok" in log, log
