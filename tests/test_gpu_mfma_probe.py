"""GPU check of the dense-MFMA calibration call (bsattn_mfma_probe): it runs, writes its
clock spans, and reports a rate no higher than 256 CUs x 4096 FLOP per clock at the clock it
measured."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import block_sparse_attention_fwd_amd as bs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("random", [True, False])
def test_mfma_probe_plausible(random):
    print(f"[gpu] mfma probe random={random}", flush=True)
    tflops, ghz, ms = bs.mfma_probe(iters=4000, random=random)
    print(f"[gpu] mfma probe random={random}: {tflops:.1f} TFLOP/s at {ghz:.3f} GHz ({ms:.3f} ms)", flush=True)
    assert ms > 0 and 0.3 < ghz < 2.6
    assert 0 < tflops <= 256 * 4096 * ghz * 1e9 / 1e12 * 1.05
