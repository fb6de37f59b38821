"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

* the oracle's C routines, driven by tests/sanitize/oracle_check.c with every array allocated
  at exactly its documented size (empty and short sequences, N > 256, conv widths 1 and 64,
  refused arguments), built with gcc;
* the C-ABI library's host code (argument checks, plan and size queries), driven by
  tests/sanitize/abi_check.cpp over sizes at and beyond the documented limits; built with hipcc
  with the sanitizers on the host side only (the device code is compiled as usual and never
  runs: every call is refused before anything is enqueued).
Any sanitizer report aborts the program (-fno-sanitize-recover=all), which fails the test.
"""
from __future__ import annotations

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(map(str, cmd))}\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}"
    return res.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_check"
    _run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-o", str(exe), os.path.join(HERE, "oracle_check.c"), os.path.join(ROOT, "oracle", "mamba_oracle.c"), "-lm"])
    out = _run([str(exe)], env=ENV, timeout=300)
    assert "all ok" in out


def test_abi_host_code_under_sanitizers(tmp_path):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hipcc, clang = os.path.join(rocm, "bin", "hipcc"), os.path.join(rocm, "bin", "amdclang++")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("hipcc not installed")
    inc = os.path.join(ROOT, "include")
    lib_o, drv_o, exe = tmp_path / "mm.o", tmp_path / "abi_check.o", tmp_path / "abi_check"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    _run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san, "-I", inc, "-c",
          os.path.join(ROOT, "selective_state_space_causal_amd", "csrc", "mambamix.hip"), "-o", str(lib_o)])
    _run([clang, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", inc, "-c", os.path.join(HERE, "abi_check.cpp"), "-o", str(drv_o)])
    # link with the clang driver, which adds the HIP runtime (--hip-link) and the sanitizer runtimes
    _run([clang, "--hip-link", "--offload-arch=gfx950", "-fsanitize=address,undefined", str(drv_o), str(lib_o),
          "-o", str(exe)])
    out = _run([str(exe)], env=ENV, timeout=600)
    assert out.strip().endswith("ok")

