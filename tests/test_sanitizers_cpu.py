"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

  * The oracle (oracle/*.cpp, g++) driven by tests/sanitize/oracle_driver.cpp: every oracle
    entry point on small random inputs, capacity drops, no shared expert, K = E, the FP8 and
    W8A8 forms, both backward modes and the quantiser's edge rows.
  * The host side of the C ABI (the library's .hip sources, the host pass instrumented, the
    kernels built as usual but never launched) driven by tests/sanitize/abi_driver.cpp: every
    size and layout helper over valid, extreme and invalid shapes, and every entry point on
    arguments its host checks reject.
A sanitizer report aborts the driver, and the test fails with its output.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_moe_layer_softmax_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="3")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-6000:])
    return r


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    srcs = sorted(glob.glob(os.path.join(ROOT, "oracle", "*.cpp")))
    _run(["g++", "-std=c++17", "-O1", "-g", "-fopenmp", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"), *srcs,
          os.path.join(SAN, "oracle_driver.cpp"), "-o", exe])
    r = _run([exe], env=ENV)
    assert "0 failure(s)" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="needs ROCm")
def test_abi_host_checks_under_asan_ubsan(tmp_path):
    import concurrent.futures as cf

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        # each -fsanitize applies to the host pass alone (no instrumented GPU code)
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-g",
              "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
              "-c", src, "-o", obj])
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_driver")
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
          os.path.join(SAN, "abi_driver.cpp"), *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # the HIP runtime (not instrumented) keeps allocations until exit: no leak report
    env = dict(ENV, ASAN_OPTIONS="abort_on_error=1:detect_leaks=0")
    r = _run([exe], env=env)
    assert "0 failure(s)" in r.stdout
