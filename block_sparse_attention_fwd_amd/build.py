"""Build libbsattn.so (host planner + C-ABI + gfx950 kernels) in-tree with hipcc.

    python -m block_sparse_attention_fwd_amd.build [--asm]

``--asm`` also writes the gfx950 assembly of the kernels next to the build objects
(``block_sparse_attention_fwd_amd/_build/``) for register and instruction review.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbsattn.so")
BUILD = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["plan.cpp", "api.cpp", "fwd_kernel.hip", "bwd_kernel.hip", "chunk_select.hip", "decode_kernel.hip", "plan_update.hip",
           "mfma_probe.hip"]
# packed-fp32 instructions are kept out of generated code (never emitted by hand either)
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(asm: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmd = [HIPCC] + HIP_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if asm:
        for k in ("fwd_kernel", "bwd_kernel"):
            cmd = [HIPCC] + HIP_FLAGS + ["-I", INCLUDE, "-I", CSRC, "--cuda-device-only", "-S",
                                         os.path.join(CSRC, k + ".hip"), "-o", os.path.join(BUILD, k + ".s")]
            _run(cmd)
    return LIB


if __name__ == "__main__":
    print(build(asm="--asm" in sys.argv, verbose=True))
