"""Host sanitizers (no GPU): AddressSanitizer + UndefinedBehaviorSanitizer
builds of the oracle's C code and of the C ABI's host code, each driven
through its entry points by a small program in tests/sanitize/.

* The oracle (oracle/gemm_oracle.c) with gcc: every decoder over every code,
  the dense, strided, points and block-scaled sums on exactly sized heap
  buffers, threaded and not.
* The C ABI (api.hip) with hipcc, the sanitizers on the host side only,
  linked with the library's kernel objects as built: every validation path,
  grouped offsets of 1 to 257 groups read from exactly sized host arrays,
  the host-side layout maps.  Every call there returns before the library
  touches a GPU.

A sanitizer report aborts the driver (-fno-sanitize-recover), so the test
fails on any.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "_build", "san")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan():
    os.makedirs(SAN, exist_ok=True)
    exe = os.path.join(SAN, "oracle_san")
    _run(["gcc", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-pthread", os.path.join(ROOT, "oracle", "gemm_oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert "clean" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_c_abi_host_code_under_asan_ubsan():
    from dense_gemm_swizzled_amd import _build
    objs = [os.path.join(_build.BUILD, s.replace(".hip", ".o"))
            for s in _build.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        _build.build()
    os.makedirs(SAN, exist_ok=True)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    common = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *host_san,
              "-Xarch_host", "-fno-sanitize-recover=all"]
    api_o, drv_o, exe = (os.path.join(SAN, n) for n in ("api_san.o", "abi_driver.o", "abi_san"))
    _run(common + ["-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   "-I", os.path.join(ROOT, "include"), "-c",
                   os.path.join(ROOT, "dense_gemm_swizzled_amd", "csrc", "api.hip"), "-o", api_o])
    _run(common + ["-c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv_o])
    _run([HIPCC, "--offload-arch=gfx950", *host_san, drv_o, api_o, *objs, "-o", exe])
    # The HIP runtime's own process-lifetime allocations are not this code's
    # leaks; addressing and undefined behaviour are what is checked.
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert "clean" in r.stdout
