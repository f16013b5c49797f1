"""Builds libsparse_li.so (the HIP kernels and the C ABI) in place with hipcc
for gfx950.  Usage: python -m sparse_attention_li_amd.build"""
from __future__ import annotations

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparse_li.so")

SOURCES = ["abi.cpp", "indexer_decode.hip", "indexer_prefill.hip", "sfa.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# Kernels whose LDS operand reads are issued as instructions of their own and
# awaited by explicit lgkmcnt waits: the compiler does not know such a register
# is still being written until the wait, so a spill or copy of it in between
# would read it early.  They must compile without any scratch.
NO_SCRATCH = {"sfa.hip": ("sfa_bf16_kernel",)}


def check_no_scratch(src: str, remarks: list, kernels: tuple) -> None:
    name = None
    for line in remarks:
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and any(k in name for k in kernels) and int(m.group(1)) != 0:
            raise RuntimeError(f"{src}: {name} uses {m.group(1)} bytes of scratch per lane; "
                               "its explicitly awaited LDS reads require a spill-free build")


def build(verbose: bool = False) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        usage = ["-Rpass-analysis=kernel-resource-usage"] if src in NO_SCRATCH else []
        cmd = ["hipcc", *HIP_FLAGS, *usage, *inc, "-c", *lang, os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        lines = (r.stderr or "").splitlines()
        msgs = [l for l in lines if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l]
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
        if src in NO_SCRATCH:
            check_no_scratch(src, lines, NO_SCRATCH[src])
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
