"""Checks of the seeded input generators (CPU only)."""
import numpy as np
import pytest
import torch

import workloads.configs as wc
from tests.oracle_select import oracle_chunk_select


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -0.0, 3.0e38, 1.00390625, 1.01171875, 1e-40], np.float32)])
    ours = wc.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_chunked_draws_equal_one_draw(monkeypatch):
    monkeypatch.setattr(wc, "_CHUNK", 1000)
    a = wc.normal_bf16(np.random.default_rng(5), (7, 333))
    monkeypatch.setattr(wc, "_CHUNK", 1 << 24)
    b = wc.normal_bf16(np.random.default_rng(5), (7, 333))
    assert np.array_equal(a, b)


def test_deterministic():
    a = wc.make(1)
    b = wc.make(1)
    for f in ("q", "k", "v", "sel_kblk", "sel_row_ptr", "q_offsets"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert a.q.shape == (1, 720, 2, 64) and a.scale == 1 / 8


def test_partition_workload_shape():
    w = wc.make(4, with_tensors=False)
    for offs, perm in ((w.q_offsets, w.q_perm), (w.k_offsets, w.k_perm)):
        sz = np.diff(offs)
        assert offs[-1] == 75600 and np.all(sz >= 16) and np.all(sz[:-1] <= 300) and sz[-1] <= 315
        assert np.array_equal(np.sort(perm), np.arange(75600))
    ksz = np.diff(w.k_offsets)
    for r in range(len(w.q_offsets) - 1):
        sel = w.sel_kblk[w.sel_row_ptr[r]:w.sel_row_ptr[r + 1]]
        assert ksz[sel].sum() <= 11340 and len(sel) > 0


def test_chunk_gqa_selection_wiring():
    # a scaled-down long-context GQA case: the generator asks its caller for the selection
    # (here the oracle's) and files row b * Hkv + g under unit (b, g); that row is the top-k
    # of a full sort of the chunk scores
    with pytest.raises(ValueError):
        wc.make(5, with_tensors=True)
    w = wc.make_chunk_gqa("small", 9, B=2, Hq=8, Hkv=2, d=16, Nk=64 * 40, Nq=128, chunk=64, topk=10,
                          chunk_select=oracle_chunk_select)
    assert w.sel_nb == 2 and w.sel_nh == 2 and w.causal and w.q_pos0 == 64 * 40 - 128
    kf = wc.f32_from_bf16_bits(w.k).astype(np.float64)
    qf = wc.f32_from_bf16_bits(w.q).astype(np.float64)
    for b in range(2):
        for g in range(2):
            summ = kf[b, :, g].reshape(40, 64, 16).mean(axis=1)
            iq = qf[b, -1, 4 * g:4 * g + 4].mean(axis=0)
            sc = summ @ iq
            best = sorted(range(40), key=lambda c: (-sc[c], c))[:10]
            sel = w.sel_kblk[w.sel_row_ptr[b * 2 + g]:w.sel_row_ptr[b * 2 + g + 1]]
            assert sel.tolist() == sorted(best)
