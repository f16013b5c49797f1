"""Builds libsparse_li.so (the HIP kernels and the C ABI) in place with hipcc
for gfx950.  Usage: python -m sparse_attention_li_amd.build"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparse_li.so")

SOURCES = ["abi.cpp", "shapes.cpp", "indexer_decode.hip", "indexer_prefill.hip", "sfa.hip", "quant.hip", "noalloc.hip",
           "decode_step.hip", "validate.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# Kernels whose LDS operand reads are issued as instructions of their own and
# awaited by explicit lgkmcnt waits: the compiler does not know such a
# register is still being written until the wait, so the build scans their
# assembly for any use of it in between (lds_hazards.py).
LDS_CHECKED = {"sfa.hip": ("sfa_bf16_kernel", "sfa_f8_kernel"), "indexer_decode.hip": ("li_decode_kernel",),
               "decode_step.hip": ("li_step_kernel",)}


def check_lds_hazards(src: str, inc: list, kernels: tuple) -> None:
    from sparse_attention_li_amd import lds_hazards
    out = os.path.join(HERE, "_build", os.path.splitext(src)[0] + ".gfx950.s")
    cmd = ["hipcc", *HIP_FLAGS, *inc, "-S", "--cuda-device-only", "-x", "hip", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stderr}")
    found = lds_hazards.check_asm(open(out).read(), kernels)
    if found:
        lines = "\n".join(f"  {k}: {t}   ({reg})" for k, t, reg in found[:20])
        raise RuntimeError(f"{src}: registers of in-flight LDS reads are used before their wait:\n{lines}")


def build(verbose: bool = False) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = ["hipcc", *HIP_FLAGS, *inc, "-c", *lang, os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = [l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l]
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
        if src in LDS_CHECKED:
            check_lds_hazards(src, inc, LDS_CHECKED[src])
        if msgs and verbose:
            print("\n".join(msgs))
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
