"""Host sanitizer run of the planner and the C ABI (no GPU needed).

    python -m block_sparse_attention_fwd_amd.sanitize

Builds a copy of libbsattn.so whose host code (planner, argument checks, plan export,
launch set-up) is compiled with AddressSanitizer and UndefinedBehaviorSanitizer -- the GPU
code is built as usual -- into ``_build/sanitize/``, then runs the CPU tests of the planner
and of the ABI (``tests/test_host_plan.py``, ``tests/test_c_abi_layout.py``) against it in a
child Python with the ASan runtime preloaded.  Any report aborts the run (non-zero exit).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from . import build as _b

OUT = os.path.join(_b.BUILD, "sanitize")
LIB = os.path.join(OUT, "libbsattn.so")
# host-side sanitizers only: each -fsanitize= applies to the host pass (-Xarch_host)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no clang ASan runtime under /opt/rocm/llvm")
    return hits[-1]


def build_sanitized() -> str:
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in _b.SOURCES:
        obj = os.path.join(OUT, src + ".o")
        _b._run([_b.HIPCC] + _b.HIP_FLAGS + SAN + ["-I", _b.INCLUDE, "-I", _b.CSRC, "-c", os.path.join(_b.CSRC, src),
                                                  "-o", obj])
        objs.append(obj)
    _b._run([_b.HIPCC, f"--offload-arch={_b.ARCH}", "-shared", "-fPIC", "-shared-libasan", "-fsanitize=address",
             "-fsanitize=undefined", "-o", LIB] + objs)
    return LIB


# Run inside the child: point the binding at the sanitized library, then run pytest.
_CHILD = """
import sys
sys.path.insert(0, {root!r})
import block_sparse_attention_fwd_amd as bs
bs.LIB_PATH = {lib!r}
import pytest
# no output capture: a sanitizer report must reach stderr before the abort
sys.exit(pytest.main(["-q", "-m", "not gpu", "-p", "no:cacheprovider", "--capture=no"] + {tests!r}))
"""


def run(tests=None) -> int:
    lib = build_sanitized()
    tests = tests or [os.path.join(_b.ROOT, "tests", "test_host_plan.py"),
                      os.path.join(_b.ROOT, "tests", "test_c_abi_layout.py")]
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    # the Python interpreter itself is not instrumented: its own allocations at exit are not
    # this library's leaks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    code = _CHILD.format(root=_b.ROOT, lib=lib, tests=list(tests))
    return subprocess.run([sys.executable, "-c", code], env=env, cwd=_b.ROOT).returncode


if __name__ == "__main__":
    sys.exit(run(sys.argv[1:] or None))
