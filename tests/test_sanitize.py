"""Sanitizer builds of the host code, run on the CPU.

* The C oracle (oracle/hif4_oracle.c) with OpenMP, driven by
  oracle/sanitize_check.c over every entry point: strided, empty,
  non-finite and invalid inputs, all three HiGPTQ schemes.
* The host side of the C-ABI (bit_block_float_amd/csrc/api.hip), driven by
  tests/abi_sanitize_check.cpp: argument checks and workspace queries over
  the whole int64 range. Only host code is instrumented (each -fsanitize is
  given to the host pass alone); no call reaches a device.

Both programs run under AddressSanitizer (LeakSanitizer included) and
UndefinedBehaviorSanitizer with recovery off, so any finding fails the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"
    return p


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "abort_on_error=0:halt_on_error=1:detect_leaks=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fsanitize=address,undefined", "-static-libasan", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror",
          os.path.join(ROOT, "oracle", "sanitize_check.c"),
          os.path.join(ROOT, "oracle", "hif4_oracle.c"), "-lm", "-o", exe])
    p = _run([exe], env=_env(), timeout=300)
    assert "sanitize-check OK" in p.stdout


def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not available")
    objdir = os.path.join(ROOT, "bit_block_float_amd", "_build")
    others = [os.path.join(objdir, f + ".o") for f in ("quant", "gemm", "pct", "gptq", "autoround")]
    if not all(os.path.exists(o) for o in others):
        from bit_block_float_amd import build
        build.build()
    inc = os.path.join(ROOT, "include")
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("api_san.o", "drv.o", "abi_sanitize"))
    # the device pass of api.hip is built as usual; the sanitizers go to the host pass only
    _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", inc,
          "-c", os.path.join(ROOT, "bit_block_float_amd", "csrc", "api.hip"), "-o", api_o])
    _run([clang, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I", inc, "-I", os.path.join(ROCM, "include"),
          "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(ROOT, "tests", "abi_sanitize_check.cpp"),
          "-o", drv_o])
    _run([clang, "-fsanitize=address,undefined", drv_o, api_o, *others,
          "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
          "-o", exe])
    p = _run([exe], env=_env(), timeout=300)
    assert "abi-sanitize-check OK" in p.stdout
