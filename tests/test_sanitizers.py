"""Host AddressSanitizer + UndefinedBehaviorSanitizer builds (CPU only).

* The C oracle (oracle/kda_oracle.c) with a driver that runs kdao_prefill on
  small inputs of every kind it accepts, and its argument checks.
* The C ABI's host code (kda_api.cpp) with a driver that runs every export's
  validation, the workspace queries over a range of shapes, the status
  strings and the release path (tests/sanitize/abi_driver.cpp).  The ABI
  translation unit and the driver are instrumented; the kernels' objects come
  from the regular build (their host code is not instrumented).  No call
  reaches a launch, so no GPU is needed.

A sanitizer report aborts the driver (halt_on_error, no recovery), which
fails the test with the report in the message.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(ROOT, "gated_delta_rule_28_amd", "_build")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    _run([gcc, "-std=c99", "-O1", "-g", "-fopenmp", *SAN, "-I", os.path.join(ROOT, "oracle"),
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "all runs passed" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr[-3000:]


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc = _hipcc()
    clang = "/opt/rocm/llvm/bin/clang++"
    kernels = ["kda_backward", "kda_cp", "kda_decode", "kda_prefill", "kda_prefill_split"]
    objs = [os.path.join(BUILD, k + ".hip" + ".o") for k in kernels]
    if hipcc is None or not os.path.exists(clang) or not all(os.path.exists(o) for o in objs):
        pytest.skip("hipcc / the library's build objects not available")
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]  # host code only
    inc = ["-I", os.path.join(ROOT, "include")]
    api_o, drv_o = str(tmp_path / "api.o"), str(tmp_path / "drv.o")
    src_api = os.path.join(ROOT, "gated_delta_rule_28_amd", "csrc", "kda_api.cpp")
    _run([hipcc, "--cuda-host-only", "-std=c++17", "-O1", "-g", "-fPIC", *host_san, *inc, "-c", src_api, "-o", api_o])
    _run([hipcc, "--cuda-host-only", "-std=c++17", "-O1", "-g", "-fPIC", *host_san, *inc, "-c",
          os.path.join(HERE, "abi_driver.cpp"), "-o", drv_o])
    exe = str(tmp_path / "abi_driver")
    _run([clang, *SAN, "-o", exe, api_o, drv_o, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=ENV, timeout=300)
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr[-3000:]
