"""The oracle, the seeded generators and the C ABI's host code, built for the
CPU with AddressSanitizer and UndefinedBehaviorSanitizer and run on small,
exactly sized buffers (drivers under tests/native/).  The ABI build links
stand-ins for the kernel launches that touch every byte each kernel indexes,
so a workspace region carved past the caller's allocation is reported."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generators_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    _run(["gcc", "-std=c11", "-Wall", "-Wno-unknown-pragmas", *SAN, os.path.join(NATIVE, "oracle_sanitize.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "synth", "synth.c"), "-lm", "-o", exe])
    assert "oracle_sanitize: ok" in _run([exe], env=ENV, timeout=120)


@pytest.mark.skipif(not os.path.exists(CLANGXX), reason="ROCm clang++ not available")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_sanitize")
    csrc = os.path.join(ROOT, "sparse_attention_li_amd", "csrc")
    _run([CLANGXX, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I", os.path.join(ROOT, "include"), "-I", csrc, "-I", NATIVE,
          os.path.join(csrc, "abi.cpp"), os.path.join(csrc, "shapes.cpp"),
          os.path.join(NATIVE, "launch_stubs.cpp"), os.path.join(NATIVE, "abi_sanitize.cpp"), "-o", exe])
    assert "abi_sanitize: ok" in _run([exe], env=ENV, timeout=120)
