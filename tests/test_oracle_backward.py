"""Pins for the float64 backward oracle (CPU only).

Each test checks the gradients against something other than their own formulas:
  * an all-selected mask is dense attention, whose gradients torch autograd gives
    (float64, CPU), non-causal and causal, with grouped KV heads;
  * central finite differences of the scalar sum(dO * O), with O from the forward
    oracle, on tiny block-sparse problems (permuted layouts, grouped heads, causal,
    rows without keys) -- a dropped term, a sign or a transposed operand fails here;
  * invariants: the key gradients of one head sum to zero (each softmax row's dS sums
    to zero); keys that no query reaches and rows without keys get zero gradients;
  * the sampled forms (selected query rows, selected keys) equal the full arrays.
"""
import numpy as np
import pytest
import torch

from oracle.attention import masked_attention, masked_attention_bwd, bf16_to_f64
from workloads.configs import make_random, draw_dout, normal_bf16


def _full_selection(w):
    rows = w.sel_nb * w.sel_nh * w.n_qblocks
    w.sel_row_ptr = (np.arange(rows + 1) * w.n_kblocks).astype(np.int32)
    w.sel_kblk = np.tile(np.arange(w.n_kblocks, dtype=np.int32), rows)
    return w


def _bwd(w, do, **kw):
    return masked_attention_bwd(w.q, w.k, w.v, do, w.q_offsets, w.q_perm, w.k_offsets, w.k_perm, w.sel_nb,
                                w.sel_nh, w.sel_row_ptr, w.sel_kblk, w.scale, w.causal, w.q_pos0, **kw)


def _fwd(w, q, k, v):
    return masked_attention(q, k, v, w.q_offsets, w.q_perm, w.k_offsets, w.k_perm, w.sel_nb, w.sel_nh,
                            w.sel_row_ptr, w.sel_kblk, w.scale, w.causal, w.q_pos0)[0]


@pytest.mark.parametrize("causal", [False, True])
def test_all_selected_equals_dense_autograd(causal):
    w = _full_selection(make_random(11, B=2, Hq=4, Hkv=2, Nq=45, Nk=45 if causal else 61, d=16, max_qblock=20,
                                    max_kblock=20, use_perm=False, sel_mode="kv", causal=causal, q_pos0=0))
    do = draw_dout(w)
    dQ, dK, dV = _bwd(w, do)
    grp = w.Hq // w.Hkv
    for b in range(w.B):
        q = torch.from_numpy(bf16_to_f64(w.q[b])).permute(1, 0, 2).requires_grad_()    # [Hq, Nq, d]
        k = torch.from_numpy(bf16_to_f64(w.k[b])).permute(1, 0, 2).requires_grad_()    # [Hkv, Nk, d]
        v = torch.from_numpy(bf16_to_f64(w.v[b])).permute(1, 0, 2).requires_grad_()
        g = torch.from_numpy(bf16_to_f64(do[b])).permute(1, 0, 2)
        ke = k.repeat_interleave(grp, dim=0)
        ve = v.repeat_interleave(grp, dim=0)
        s = w.scale * torch.matmul(q, ke.transpose(1, 2))
        if causal:
            allowed = torch.arange(w.Nk)[None, :] <= torch.arange(w.Nq)[:, None]
            s = s.masked_fill(~allowed, float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1), ve)
        (o * g).sum().backward()
        np.testing.assert_allclose(dQ[b], q.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dK[b], k.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dV[b], v.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed,Hq,Hkv,perm,causal,sel", [
    (21, 2, 2, False, False, "head"),
    (22, 4, 2, True, False, "kv"),
    (23, 2, 1, True, True, "head"),
    (24, 4, 1, False, True, "shared"),
])
def test_finite_differences(seed, Hq, Hkv, perm, causal, sel):
    w = make_random(seed, B=1, Hq=Hq, Hkv=Hkv, Nq=14, Nk=17, d=4, max_qblock=5, max_kblock=6, density=0.5,
                    use_perm=perm, sel_mode=sel, causal=causal, allow_empty=True)
    do = draw_dout(w)
    q, k, v = (bf16_to_f64(x) for x in (w.q, w.k, w.v))
    dof = bf16_to_f64(do)
    dQ, dK, dV = _bwd(w, do)

    def loss(qq, kk, vv):
        return float(np.sum(np.nan_to_num(_fwd(w, qq, kk, vv)) * dof))

    eps = 1e-6
    rng = np.random.default_rng(seed)
    for name, base, grad in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        flat = base.reshape(-1)
        for idx in rng.choice(flat.size, size=min(40, flat.size), replace=False):
            plus = flat.copy(); plus[idx] += eps
            minus = flat.copy(); minus[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = plus.reshape(base.shape)
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = minus.reshape(base.shape)
            lm = loss(args["q"], args["k"], args["v"])
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.reshape(-1)[idx]) < 1e-7 * max(1.0, abs(fd)), (name, idx, fd, grad.reshape(-1)[idx])


def test_invariants_zero_sums_and_unreached():
    w = make_random(31, B=2, Hq=3, Hkv=3, Nq=60, Nk=70, d=8, max_qblock=12, max_kblock=10, density=0.4,
                    use_perm=True, sel_mode="head", allow_empty=True)
    do = draw_dout(w)
    dQ, dK, dV = _bwd(w, do)
    # the key gradients of a head (one query head per KV head here) sum to zero
    np.testing.assert_allclose(dK.sum(axis=1), 0.0, atol=1e-12)
    # keys that no (unit, Q block) row selects get no gradient; rows that select nothing get none
    bq = np.zeros(w.Nq, np.int64); bk = np.zeros(w.Nk, np.int64)
    for arr, offs, perm in ((bq, w.q_offsets, w.q_perm), (bk, w.k_offsets, w.k_perm)):
        for blk in range(len(offs) - 1):
            sl = np.arange(offs[blk], offs[blk + 1])
            arr[sl if perm is None else perm[sl]] = blk
    nqb = w.n_qblocks
    for h in range(w.Hq):
        sel = [set(w.sel_kblk[w.sel_row_ptr[h * nqb + qb]:w.sel_row_ptr[h * nqb + qb + 1]].tolist())
               for qb in range(nqb)]
        reached = set().union(*sel)
        for j in range(w.Nk):
            if bk[j] not in reached:
                assert not dK[:, j, h].any() and not dV[:, j, h].any()
        for i in range(w.Nq):
            if not sel[bq[i]]:
                assert not dQ[:, i, h].any()


def test_sampled_rows_and_keys_equal_full():
    w = make_random(41, B=2, Hq=4, Hkv=2, Nq=80, Nk=90, d=8, max_qblock=15, max_kblock=12, density=0.3,
                    use_perm=True, sel_mode="head", causal=True)
    do = draw_dout(w)
    dQ, dK, dV = _bwd(w, do)
    q_rows = [(1, 3, np.array([0, 5, 79])), (0, 0, np.arange(10, 30))]
    k_rows = [(1, 1, np.array([2, 3, 88])), (0, 0, np.arange(40, 52))]
    dq_s, dkv_s = _bwd(w, do, q_rows=q_rows, k_rows=k_rows)
    for (b, h, t), got in zip(q_rows, dq_s):
        np.testing.assert_allclose(got, dQ[b, t, h], rtol=0, atol=1e-13)
    for (b, g, t), (gk, gv) in zip(k_rows, dkv_s):
        np.testing.assert_allclose(gk, dK[b, t, g], rtol=0, atol=1e-13)
        np.testing.assert_allclose(gv, dV[b, t, g], rtol=0, atol=1e-13)


def test_dout_draw_follows_qkv():
    # dO continues the generator after Q, K, V: the same seed gives the same dO
    a = make_random(51, Nq=30, Nk=30, d=8)
    b = make_random(51, Nq=30, Nk=30, d=8)
    np.testing.assert_array_equal(draw_dout(a), draw_dout(b))
    assert draw_dout(a) is draw_dout(a)
    assert draw_dout(a).shape == a.q.shape
