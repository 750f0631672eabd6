"""Pins for the float64 masked-attention oracle (CPU only).

Each test checks the oracle against something other than its own code:
  * an all-selected mask over full blocks is dense attention (torch SDPA, float64, CPU);
  * pure-Python brute force on tiny inputs (scalar loops, math.exp);
  * locality: a row depends only on its selected keys (perturbing the others changes
    nothing, bitwise) and equals dense attention over the gathered selected keys;
  * closed forms: Q = 0 gives the mean of the selected V rows and LSE = ln(count);
    one selected key gives that V row and its score; a hand-worked 2-key example
    (tests/golden/hand_two_keys.json);
  * convexity: every output lies in the per-dimension hull of its selected V rows.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import masked_attention, masked_attention_w, brute_force_attention, bf16_to_f64
from workloads.configs import make_random, bf16_bits_from_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa(q, k, v, scale, mask=None):
    """Dense attention via torch (float64, CPU): q [Nq, d], k/v [Nk, d]."""
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(k)[None, None]
    vt = torch.from_numpy(v)[None, None]
    am = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale)[0, 0].numpy()


def _full_selection(w):
    nqb, nkb = w.n_qblocks, w.n_kblocks
    rows = w.sel_nb * w.sel_nh * nqb
    w.sel_row_ptr = (np.arange(rows + 1) * nkb).astype(np.int32)
    w.sel_kblk = np.tile(np.arange(nkb, dtype=np.int32), rows)
    return w


@pytest.mark.parametrize("seed,Hq,Hkv,perm", [(1, 2, 2, False), (2, 4, 2, True), (3, 8, 1, False)])
def test_all_selected_equals_dense_sdpa(seed, Hq, Hkv, perm):
    w = _full_selection(make_random(seed, B=2, Hq=Hq, Hkv=Hkv, Nq=97, Nk=131, d=32, max_qblock=40,
                                    max_kblock=50, use_perm=perm, sel_mode="kv"))
    O, L = masked_attention_w(w)
    for b in range(w.B):
        for h in range(w.Hq):
            g = h // (Hq // Hkv)
            q = bf16_to_f64(w.q[b, :, h]); k = bf16_to_f64(w.k[b, :, g]); v = bf16_to_f64(w.v[b, :, g])
            ref = _sdpa(q, k, v, w.scale)
            np.testing.assert_allclose(O[b, :, h], ref, rtol=0, atol=1e-12)
            s = w.scale * q @ k.T
            lse = torch.logsumexp(torch.from_numpy(s), dim=1).numpy()
            np.testing.assert_allclose(L[b, h], lse, rtol=0, atol=1e-12)


def test_causal_full_selection_equals_sdpa_causal():
    w = _full_selection(make_random(7, B=1, Hq=2, Hkv=1, Nq=50, Nk=50, d=16, max_qblock=20, max_kblock=20,
                                    sel_mode="shared", causal=True, q_pos0=0))
    O, L = masked_attention_w(w)
    for h in range(2):
        q = bf16_to_f64(w.q[0, :, h]); k = bf16_to_f64(w.k[0, :, 0]); v = bf16_to_f64(w.v[0, :, 0])
        qt, kt, vt = (torch.from_numpy(x)[None, None] for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=w.scale)[0, 0]
        np.testing.assert_allclose(O[0, :, h], ref.numpy(), rtol=0, atol=1e-12)


def test_causal_offset_against_explicit_mask():
    # queries are the last Nq positions of an Nk-token sequence
    w = _full_selection(make_random(8, B=1, Hq=1, Hkv=1, Nq=24, Nk=70, d=8, max_qblock=10, max_kblock=16,
                                    sel_mode="shared", causal=True))
    assert w.q_pos0 == 46
    O, _ = masked_attention_w(w)
    q = bf16_to_f64(w.q[0, :, 0]); k = bf16_to_f64(w.k[0, :, 0]); v = bf16_to_f64(w.v[0, :, 0])
    allowed = np.arange(70)[None, :] <= (46 + np.arange(24))[:, None]
    ref = _sdpa(q, k, v, w.scale, mask=allowed)
    np.testing.assert_allclose(O[0, :, 0], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kw", [
    dict(seed=11, B=1, Hq=2, Hkv=2, sel_mode="head"),
    dict(seed=12, B=2, Hq=4, Hkv=2, sel_mode="batch-kv", use_perm=True),
    dict(seed=13, B=1, Hq=2, Hkv=1, sel_mode="shared", causal=True, use_perm=True),
    dict(seed=14, B=1, Hq=2, Hkv=2, sel_mode="kv", allow_empty=True, density=0.3, unsorted=True, dup=True),
])
def test_brute_force_tiny(kw):
    w = make_random(Nq=29, Nk=37, d=6, max_qblock=9, max_kblock=11, **kw)
    O, L = masked_attention_w(w)
    Ob, Lb = brute_force_attention(w.q, w.k, w.v, w.q_offsets, w.q_perm, w.k_offsets, w.k_perm, w.sel_nb,
                                   w.sel_nh, w.sel_row_ptr, w.sel_kblk, w.scale, w.causal, w.q_pos0)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    fin = np.isfinite(Lb)
    assert np.array_equal(fin, np.isfinite(L))
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)
    assert np.all(O[np.transpose(~fin, (0, 2, 1))] == 0.0)


def _gathered_keys(w, b, h, i):
    """Key tokens in the graph for query token i, found without the oracle's helpers."""
    nqb = w.n_qblocks
    qslot = i if w.q_perm is None else int(np.nonzero(w.q_perm == i)[0][0])
    qb = int(np.searchsorted(w.q_offsets, qslot, side="right") - 1)
    g = h // (w.Hq // w.Hkv)
    uh = {w.Hq: h, w.Hkv: g, 1: 0}[w.sel_nh] if w.sel_nh != w.Hq else h
    unit = (b if w.sel_nb == w.B else 0) * w.sel_nh + uh
    row = unit * nqb + qb
    keys = []
    for kb in sorted(set(w.sel_kblk[w.sel_row_ptr[row]:w.sel_row_ptr[row + 1]].tolist())):
        for s in range(w.k_offsets[kb], w.k_offsets[kb + 1]):
            keys.append(s if w.k_perm is None else int(w.k_perm[s]))
    if w.causal:
        keys = [j for j in keys if j <= w.q_pos0 + i]
    return sorted(keys)


@pytest.mark.parametrize("seed,perm", [(21, False), (22, True)])
def test_locality_and_gathered_dense(seed, perm):
    w = make_random(seed, B=1, Hq=2, Hkv=2, Nq=120, Nk=150, d=16, max_qblock=30, max_kblock=30,
                    density=0.35, use_perm=perm, sel_mode="head")
    O, L = masked_attention_w(w)
    rng = np.random.default_rng(seed + 100)
    for h in range(w.Hq):
        for i in rng.choice(w.Nq, 12, replace=False):
            keys = _gathered_keys(w, 0, h, int(i))
            if not keys:
                assert np.all(O[0, i, h] == 0) and L[0, h, i] == -np.inf
                continue
            q = bf16_to_f64(w.q[0, i:i + 1, h]); k = bf16_to_f64(w.k[0, keys, h]); v = bf16_to_f64(w.v[0, keys, h])
            np.testing.assert_allclose(O[0, i, h], _sdpa(q, k, v, w.scale)[0], rtol=0, atol=1e-12)
            # perturb every unselected key and value of this head: the row must not move at all
            w2k, w2v = w.k.copy(), w.v.copy()
            others = np.setdiff1d(np.arange(w.Nk), keys)
            w2k[0, others, h] = bf16_bits_from_f32(rng.standard_normal((others.size, w.d)).astype(np.float32) * 50)
            w2v[0, others, h] = bf16_bits_from_f32(rng.standard_normal((others.size, w.d)).astype(np.float32) * 50)
            # same call shape for both runs, so the only difference is the perturbed data
            args = (w.q_offsets, w.q_perm, w.k_offsets, w.k_perm, w.sel_nb, w.sel_nh, w.sel_row_ptr, w.sel_kblk,
                    w.scale, w.causal, w.q_pos0)
            (o1, l1), = masked_attention(w.q, w.k, w.v, *args, rows=[(0, h, np.array([i]))])
            (o2, l2), = masked_attention(w.q, w2k, w2v, *args, rows=[(0, h, np.array([i]))])
            assert np.array_equal(o2, o1) and np.array_equal(l2, l1)


def test_zero_query_closed_form():
    w = make_random(31, B=1, Hq=2, Hkv=1, Nq=80, Nk=90, d=8, max_qblock=25, max_kblock=25, density=0.4,
                    sel_mode="head", use_perm=True)
    w.q[:] = 0
    O, L = masked_attention_w(w)
    for h in range(2):
        for i in range(w.Nq):
            keys = _gathered_keys(w, 0, h, i)
            if not keys:
                continue
            vsel = bf16_to_f64(w.v[0, keys, 0])
            np.testing.assert_allclose(O[0, i, h], vsel.mean(axis=0), rtol=0, atol=1e-13)
            assert abs(L[0, h, i] - math.log(len(keys))) < 1e-13


def test_single_key_closed_form():
    # one K block of one token selected by every Q block
    w = make_random(32, B=1, Hq=1, Hkv=1, Nq=40, Nk=40, d=8, max_qblock=10, max_kblock=10, sel_mode="shared")
    nk = np.diff(w.k_offsets)
    kb = int(np.nonzero(nk == nk.min())[0][0])
    # force block kb to hold exactly one token by re-cutting the layout: slots [0,1) then the rest
    w.k_offsets = np.array([0, 1, w.Nk], dtype=np.int32)
    w.sel_row_ptr = np.arange(w.n_qblocks + 1, dtype=np.int32)
    w.sel_kblk = np.zeros(w.n_qblocks, dtype=np.int32)
    O, L = masked_attention_w(w)
    v0 = bf16_to_f64(w.v[0, 0, 0]); k0 = bf16_to_f64(w.k[0, 0, 0])
    for i in range(w.Nq):
        np.testing.assert_array_equal(O[0, i, 0], v0)
        assert abs(L[0, 0, i] - w.scale * float(bf16_to_f64(w.q[0, i, 0]) @ k0)) < 1e-14
    del kb


def test_hand_worked_two_key_example():
    with open(os.path.join(GOLDEN, "hand_two_keys.json")) as f:
        g = json.load(f)
    q = bf16_bits_from_f32(np.array(g["q"], np.float32)).reshape(1, 1, 1, -1)
    k = bf16_bits_from_f32(np.array(g["k"], np.float32)).reshape(1, 2, 1, -1)
    v = bf16_bits_from_f32(np.array(g["v"], np.float32)).reshape(1, 2, 1, -1)
    O, L = masked_attention(q, k, v, np.array([0, 1]), None, np.array([0, 1, 2]), None, 1, 1,
                            np.array([0, 2]), np.array([0, 1]), g["scale"])
    np.testing.assert_allclose(O[0, 0, 0], g["o"], rtol=0, atol=1e-15)
    assert abs(L[0, 0, 0] - g["lse"]) < 1e-15
    # selecting only the second block leaves one key: O = V1, LSE = its score
    O, L = masked_attention(q, k, v, np.array([0, 1]), None, np.array([0, 1, 2]), None, 1, 1,
                            np.array([0, 1]), np.array([1]), g["scale"])
    np.testing.assert_allclose(O[0, 0, 0], g["v"][1], rtol=0, atol=0)
    assert L[0, 0, 0] == 0.0


def test_outputs_in_hull_of_selected_values():
    w = make_random(41, B=1, Hq=2, Hkv=2, Nq=100, Nk=100, d=8, max_qblock=30, max_kblock=30, density=0.4,
                    sel_mode="head")
    O, _ = masked_attention_w(w)
    for h in range(2):
        for i in range(0, w.Nq, 7):
            keys = _gathered_keys(w, 0, h, i)
            if not keys:
                continue
            vs = bf16_to_f64(w.v[0, keys, h])
            assert np.all(O[0, i, h] >= vs.min(axis=0) - 1e-12) and np.all(O[0, i, h] <= vs.max(axis=0) + 1e-12)


def test_rows_argument_matches_full():
    w = make_random(51, B=2, Hq=4, Hkv=2, Nq=70, Nk=90, d=8, max_qblock=30, max_kblock=30, sel_mode="batch-kv",
                    causal=True, use_perm=True)
    O, L = masked_attention_w(w)
    toks = np.array([0, 5, 69, 33])
    res = masked_attention_w(w, rows=[(1, 3, toks), (0, 0, toks)])
    np.testing.assert_array_equal(res[0][0], O[1, toks, 3])
    np.testing.assert_array_equal(res[1][1], L[0, 0, toks])


def test_invalid_layout_rejected():
    with pytest.raises(ValueError):
        oracle.token_block_map(np.array([0, 5, 9]), None, 10)
    with pytest.raises(ValueError):
        oracle.token_block_map(np.array([0, 3, 6]), np.array([0, 1, 2, 3, 4, 4]), 6)
