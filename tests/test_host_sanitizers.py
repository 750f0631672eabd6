"""Host sanitizers over the planner and the C ABI (CPU only, about a minute and a half).

Builds libbsattn.so with AddressSanitizer and UndefinedBehaviorSanitizer on its host code
(block_sparse_attention_fwd_amd/sanitize.py) and runs the planner and ABI tests against it
in a child process; any report aborts that child.
"""
from block_sparse_attention_fwd_amd import sanitize


def test_planner_and_abi_under_asan_ubsan():
    assert sanitize.run() == 0
