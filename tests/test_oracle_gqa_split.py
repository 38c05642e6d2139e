"""Pins for the oracle's grouped-query, cross-length and split-key functions.

Same rules as test_oracle.py: every check ties the oracle to something other
than itself (closed forms, pure-Python brute force, torch's fp64 attention and
autograd, finite differences, invariants), and the planted-mistake tests at
the end show that a plausible bug in each function is caught.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A

from test_oracle import brute_attention, rnd


def sdpa64(q, k, v, gqa=False):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), enable_gqa=gqa).numpy()


# ------------------------------------------------------------ cross lengths

@pytest.mark.parametrize("nq,nk", [(1, 7), (3, 1), (5, 2), (2, 9)])
def test_cross_length_forward_matches_brute_force(nq, nk):
    q, k, v = rnd((nq, 4), 11), rnd((nk, 4), 12), rnd((nk, 4), 13)
    ref = brute_attention(q.tolist(), k.tolist(), v.tolist())
    o, _, _ = oracle.naive_fwd(q, k, v)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-14)
    o, _, _ = oracle.chunked_fwd(q, k, v, chunk=2)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-14)


def test_cross_length_backward_matches_torch_autograd():
    rng = np.random.default_rng(14)
    q, do = rng.standard_normal((2, 3, 5, 16)), rng.standard_normal((2, 3, 5, 16))
    k, v = rng.standard_normal((2, 3, 37, 16)), rng.standard_normal((2, 3, 37, 16))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).backward(torch.from_numpy(do))
    dq, dk, dv = oracle.naive_bwd(q, k, v, do)
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------ grouped query

@pytest.mark.parametrize("H,H_kv", [(6, 2), (4, 1), (3, 3), (8, 4)])
def test_gqa_head_mapping_closed_form(H, H_kv):
    # V constant per key/value head: every output row of query head h equals the
    # constant of the head it reads, whatever the weights are.
    B, nq, nk, d = 2, 5, 7, 8
    q, k = rnd((B, H, nq, d), 15), rnd((B, H_kv, nk, d), 16)
    const = np.arange(B * H_kv, dtype=np.float64).reshape(B, H_kv) + 1.0
    v = np.broadcast_to(const[:, :, None, None], (B, H_kv, nk, d)).copy()
    o, _, _ = oracle.gqa_fwd(q, k, v)
    G = H // H_kv
    for h in range(H):
        assert oracle.kv_head_of(h, H, H_kv) == h // G  # consecutive heads form a group
        np.testing.assert_allclose(o[:, h], np.broadcast_to(const[:, h // G, None, None], (B, nq, d)),
                                   rtol=0, atol=1e-14)


def test_gqa_forward_matches_brute_force_and_torch():
    B, H, H_kv, nq, nk, d = 1, 4, 2, 3, 5, 4
    q, k, v = rnd((B, H, nq, d), 17), rnd((B, H_kv, nk, d), 18), rnd((B, H_kv, nk, d), 19)
    o, m, l = oracle.gqa_fwd(q, k, v)
    for h in range(H):
        j = h // (H // H_kv)
        ref = brute_attention(q[0, h].tolist(), k[0, j].tolist(), v[0, j].tolist())
        np.testing.assert_allclose(o[0, h], ref, rtol=0, atol=1e-14)
    q, k, v = rnd((2, 8, 33, 16), 20), rnd((2, 2, 41, 16), 21), rnd((2, 2, 41, 16), 22)
    o, _, _ = oracle.gqa_fwd(q, k, v)
    np.testing.assert_allclose(o, sdpa64(q, k, v, gqa=True), rtol=0, atol=1e-13)


def test_gqa_rows_subset_and_stats():
    q, k, v = rnd((1, 4, 20, 8), 23), rnd((1, 2, 9, 8), 24), rnd((1, 2, 9, 8), 25)
    o, m, l = oracle.gqa_fwd(q, k, v)
    rows = np.array([19, 0, 7])
    o2, m2, l2 = oracle.gqa_fwd(q, k, v, rows=rows)
    np.testing.assert_allclose(o2, o[:, :, rows], rtol=0, atol=1e-15)
    kk = np.repeat(k, 2, axis=1)
    mr, lr = oracle.row_stats(q, kk)
    np.testing.assert_allclose(m, mr, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, lr, rtol=1e-14, atol=0)


def _gqa_loss(q, k, v, do):
    o, _, _ = oracle.gqa_fwd(q, k, v)
    return float((o * do).sum())


def test_gqa_backward_central_finite_differences():
    rng = np.random.default_rng(26)
    B, H, H_kv, nq, nk, d = 1, 4, 2, 3, 4, 3
    q, do = rng.standard_normal((B, H, nq, d)), rng.standard_normal((B, H, nq, d))
    k, v = rng.standard_normal((B, H_kv, nk, d)), rng.standard_normal((B, H_kv, nk, d))
    dq, dk, dv = oracle.gqa_bwd(q, k, v, do)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a_p = {"q": q, "k": k, "v": v}
            a_m = dict(a_p)
            a_p[name], a_m[name] = xp, xm
            num[idx] = (_gqa_loss(a_p["q"], a_p["k"], a_p["v"], do)
                        - _gqa_loss(a_m["q"], a_m["k"], a_m["v"], do)) / (2 * h)
        assert np.abs(num - g).max() / max(1.0, np.abs(g).max()) <= 1e-6, name


def test_gqa_backward_matches_torch_autograd():
    rng = np.random.default_rng(27)
    q, do = rng.standard_normal((2, 6, 11, 16)), rng.standard_normal((2, 6, 11, 16))
    k, v = rng.standard_normal((2, 3, 19, 16)), rng.standard_normal((2, 3, 19, 16))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True).backward(
        torch.from_numpy(do))
    dq, dk, dv = oracle.gqa_bwd(q, k, v, do, rows=np.arange(11), cols=np.array([0, 18, 5]))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy()[:, :, [0, 18, 5]], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy()[:, :, [0, 18, 5]], rtol=0, atol=1e-12)


def test_kv_head_of_rejects_bad_groups():
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 6, 4)
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 6, 0)


# --------------------------------------------------------------- split keys

def test_one_key_block_summary_closed_form():
    # a block of one key: m = its score, l = 1, u = its value row
    q, k, v = rnd((3, 8), 30), rnd((1, 8), 31), rnd((1, 8), 32)
    m, l, u = oracle.block_summary(q, k, v)
    np.testing.assert_allclose(m, (q @ k[0]) / math.sqrt(8), rtol=0, atol=1e-15)
    assert np.all(l == 1.0)
    np.testing.assert_array_equal(u, np.repeat(v, 3, axis=0))


@pytest.mark.parametrize("n,splits", [(1, 1), (4, 2), (5, 3), (5, 5), (6, 4)])
def test_split_forward_matches_brute_force(n, splits):
    q, k, v = rnd((3, 4), 33), rnd((n, 4), 34), rnd((n, 4), 35)
    ref = brute_attention(q.tolist(), k.tolist(), v.tolist())
    o, _, _ = oracle.split_fwd(q, k, v, splits)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16, 64, 200])
def test_split_forward_equals_naive(splits):
    q, k, v = rnd((2, 3, 17, 16), 36), rnd((2, 3, 129, 16), 37), rnd((2, 3, 129, 16), 38)
    o, m, l = oracle.naive_fwd(q, k, v)
    o2, m2, l2 = oracle.split_fwd(q, k, v, splits)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(m2, m, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, l, rtol=1e-13, atol=0)


def test_merge_is_order_independent():
    q, k, v = rnd((9, 8), 39), rnd((40, 8), 40), rnd((40, 8), 41)
    parts = [oracle.block_summary(q, k[a:b], v[a:b]) for a, b in oracle.split_ranges(40, 5)]
    o1, m1, l1 = oracle.merge_summaries(parts)
    o2, m2, l2 = oracle.merge_summaries(parts[::-1])
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(m2, m1)


def test_split_forward_at_1e4_scores():
    # scaled scores in the thousands: block maxima differ by far more than exp's range
    q, k, v = rnd((2, 6, 64), 42, 30.0), rnd((2, 300, 64), 43, 30.0), rnd((2, 300, 64), 44)
    o, m, l = oracle.naive_fwd(q, k, v)
    assert np.abs(m).max() > 1e3
    for splits in (2, 9, 300):
        o2, m2, l2 = oracle.split_fwd(q, k, v, splits)
        assert np.isfinite(o2).all()
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)


@pytest.mark.parametrize("n_k,splits", [(1, 1), (1, 4), (10, 3), (128, 8), (129, 8), (7, 7)])
def test_split_ranges_tile_the_keys(n_k, splits):
    r = oracle.split_ranges(n_k, splits)
    assert 1 <= len(r) <= splits
    assert r[0][0] == 0 and r[-1][1] == n_k
    for (a, b), (c, _) in zip(r, r[1:]):
        assert b == c
    assert all(b > a for a, b in r)


# ---------------------------------------------------------- planted mistakes

def test_planted_wrong_head_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(A, "kv_head_of", lambda h, H, H_kv: h % H_kv)
    with pytest.raises(AssertionError):
        test_gqa_head_mapping_closed_form(6, 2)


def test_planted_unsummed_group_gradient_is_caught(monkeypatch):
    real = A.gqa_bwd

    def bad(q, k, v, do, rows=None, cols=None):
        # takes the gradient of the first query head of each group only
        q = np.asarray(q, dtype=np.float64)
        H, H_kv = q.shape[1], np.asarray(k).shape[1]
        G = H // H_kv
        dq, dk, dv = real(q, k, v, do, rows, cols)
        _, dk1, dv1 = A.naive_bwd(q[:, ::G], k, v, np.asarray(do)[:, ::G], rows=rows, cols=cols)
        return dq, dk1, dv1

    monkeypatch.setattr(oracle, "gqa_bwd", bad)
    with pytest.raises(AssertionError):
        test_gqa_backward_central_finite_differences()


def test_planted_merge_without_rebase_is_caught(monkeypatch):
    def bad_merge(parts):
        l = sum(p[1] for p in parts)
        u = sum(p[2] for p in parts)
        m = parts[0][0]
        for p in parts[1:]:
            m = np.maximum(m, p[0])
        return u / l[..., None], m, l

    monkeypatch.setattr(A, "merge_summaries", bad_merge)
    with pytest.raises(AssertionError):
        test_split_forward_equals_naive(3)


def test_planted_merge_on_smallest_maximum_is_caught(monkeypatch):
    # re-basing on the smallest block maximum is exact in real arithmetic but
    # overflows exp once block maxima differ by more than ~709
    def bad_merge(parts):
        m = parts[0][0]
        for p in parts[1:]:
            m = np.minimum(m, p[0])
        with np.errstate(over="ignore", invalid="ignore"):
            w = [np.exp(p[0] - m) for p in parts]
            l = sum(wi * p[1] for wi, p in zip(w, parts))
            u = sum(wi[..., None] * p[2] for wi, p in zip(w, parts))
            return u / l[..., None], m, l

    monkeypatch.setattr(A, "merge_summaries", bad_merge)
    with pytest.raises(AssertionError):
        test_split_forward_at_1e4_scores()
