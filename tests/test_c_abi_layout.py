"""The Python binding's ctypes structures against the C header (no GPU).

A small C program, compiled with gcc against include/bsattn.h as plain C99, prints sizeof
and offsetof of every struct the binding mirrors; each must equal the ctypes layout, so the
binding and the ABI cannot drift apart.  The same compile checks that the header is valid C.
"""
import ctypes
import os
import shutil
import subprocess
import tempfile

import pytest

import block_sparse_attention_fwd_amd as bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

# C struct name -> ctypes structure of the binding
PAIRS = {
    "bsattn_problem": bs.Problem,
    "bsattn_layout": bs.Layout,
    "bsattn_selection": bs.Selection,
    "bsattn_stats": bs.Stats,
    "bsattn_plan_view": bs.PlanView,
    "bsattn_plan_bwd_view": bs.PlanBwdView,
    "bsattn_chunk_problem": bs.ChunkProblem,
}


def _c_layouts():
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "bsattn.h"', "int main(void) {"]
    for cname, cls in PAIRS.items():
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'  printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "layout.c")
        exe = os.path.join(tmp, "layout")
        with open(src, "w") as f:
            f.write("\n".join(lines) + "\n")
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", INCLUDE, src, "-o", exe], check=True,
                       capture_output=True, text=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return dict(line.rsplit(" ", 1) for line in out.strip().splitlines())


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_ctypes_structures_match_the_c_header():
    got = _c_layouts()
    for cname, cls in PAIRS.items():
        assert int(got[cname]) == ctypes.sizeof(cls), f"sizeof({cname})"
        for fname, _ in cls._fields_:
            assert int(got[f"{cname}.{fname}"]) == getattr(cls, fname).offset, f"offsetof({cname}, {fname})"
