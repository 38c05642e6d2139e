"""Pins for the CPU oracle: each check ties it to something other than itself.

Kinds of pin used here (no test retypes the oracle's own formula):
* brute force: pure-Python loops over math.exp on tiny inputs, using the
  plain softmax definition exp(x_j) / sum_k exp(x_k) with no max subtraction;
* closed forms: two keys reduce softmax to a logistic function of the score
  gap, which fixes the scale 1/sqrt(d); the argmax limit; identical keys;
* a library routine: torch's scaled_dot_product_attention and autograd in
  float64 on the CPU (the oracle never calls torch);
* invariants fixed by the mathematics: n = 1, permutation of (k, v) pairs,
  translation of all keys, V = 1, linearity in V, gradient sum identities;
* central finite differences for the backward.
Planted-mistake tests at the end mutate the oracle (on the CPU) and show the
pins catch each mistake.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def brute_attention(q, k, v):
    """Pure-Python definition on [n, d] lists: softmax without max subtraction."""
    n, d = len(q), len(q[0])
    nk = len(k)
    out = []
    for i in range(n):
        s = [sum(q[i][t] * k[j][t] for t in range(d)) / math.sqrt(d) for j in range(nk)]
        e = [math.exp(x) for x in s]
        z = sum(e)
        out.append([sum(e[j] * v[j][c] for j in range(nk)) / z for c in range(len(v[0]))])
    return np.array(out)


# ---------------------------------------------------------------- forward pins

@pytest.mark.parametrize("n,d", [(1, 1), (2, 1), (3, 2), (5, 4), (4, 3)])
def test_naive_and_chunked_match_brute_force(n, d):
    q, k, v = rnd((n, d), 1), rnd((n, d), 2), rnd((n, d), 3)
    ref = brute_attention(q.tolist(), k.tolist(), v.tolist())
    o, _, _ = oracle.naive_fwd(q, k, v)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-14)
    for c in (1, 2, n):
        oc, _, _ = oracle.chunked_fwd(q, k, v, chunk=c)
        np.testing.assert_allclose(oc, ref, rtol=0, atol=1e-14)


def test_single_query_matches_brute_force():
    q, k, v = rnd((1, 6), 4), rnd((9, 6), 5), rnd((9, 6), 6)
    ref = brute_attention(q.tolist(), k.tolist(), v.tolist())[0]
    o, m, s = oracle.single_query(q[0], k, v)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-14)
    scores = [float(q[0] @ k[j]) / math.sqrt(6) for j in range(9)]
    assert m == pytest.approx(max(scores), abs=1e-15)
    assert s == pytest.approx(sum(math.exp(x - max(scores)) for x in scores), rel=1e-14)


@pytest.mark.parametrize("t", [0.3, -1.1, 2.5])
def test_two_key_closed_form_fixes_scale(t):
    # d = 4, q = (1,1,1,1), k1 = 0, k2 = (t,t,t,t): raw gap 4t, scaled gap 4t / sqrt(4) = 2t.
    # Softmax over two scores is the logistic of the gap: w2 = 1 / (1 + exp(-2t)).
    q = np.ones((1, 4))
    k = np.array([[0.0] * 4, [t] * 4])
    v = np.array([[1.0, -2.0, 0.5, 3.0], [-1.0, 4.0, 2.5, 0.0]])
    w2 = 1.0 / (1.0 + math.exp(-2.0 * t))
    expect = v[0] + (v[1] - v[0]) * w2
    for fn in (oracle.naive_fwd, lambda a, b, c: oracle.chunked_fwd(a, b, c, chunk=1)):
        o, m, l = fn(q, k, v)
        np.testing.assert_allclose(o[0], expect, rtol=0, atol=1e-15)
        assert m[0] == pytest.approx(max(0.0, 2.0 * t), abs=1e-15)
        assert l[0] == pytest.approx(1.0 + math.exp(-abs(2.0 * t)), abs=1e-15)


def test_matches_torch_sdpa_fp64():
    q, k, v = rnd((2, 3, 37, 16), 7), rnd((2, 3, 37, 16), 8), rnd((2, 3, 37, 16), 9)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    o, _, _ = oracle.naive_fwd(q, k, v)
    oc, _, _ = oracle.chunked_fwd(q, k, v)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oc, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("chunk", [1, 7, None, 300])
def test_chunked_equals_naive(chunk):
    q, k, v = rnd((2, 300, 32), 10), rnd((2, 300, 32), 11), rnd((2, 300, 32), 12)
    o, m, l = oracle.naive_fwd(q, k, v)
    oc, mc, lc = oracle.chunked_fwd(q, k, v, chunk=chunk)
    np.testing.assert_allclose(oc, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(mc, m, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lc, l, rtol=1e-12, atol=0)


def test_n1_returns_v_bitwise():
    q, k, v = rnd((3, 1, 64), 13), rnd((3, 1, 64), 14), rnd((3, 1, 64), 15)
    for fn in (oracle.naive_fwd, oracle.chunked_fwd):
        o, m, l = fn(q, k, v)
        assert np.array_equal(o, v)
        assert np.all(l == 1.0)


@pytest.mark.parametrize("scale", [1.0, 30.0])
def test_identical_keys_give_mean_of_values(scale):
    q = rnd((64, 128), 16, scale)
    k = np.repeat(rnd((1, 128), 17, scale), 50, axis=0)
    v = rnd((50, 128), 18)
    for fn in (oracle.naive_fwd, oracle.chunked_fwd):
        o, m, l = fn(q, k, v)
        np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, 50.0, rtol=0, atol=1e-12)


def test_permuting_kv_pairs_leaves_output_unchanged():
    q, k, v = rnd((40, 16), 19), rnd((70, 16), 20), rnd((70, 16), 21)
    perm = np.random.default_rng(22).permutation(70)
    for fn in (oracle.naive_fwd, oracle.chunked_fwd):
        o, _, _ = fn(q, k, v)
        op, _, _ = fn(q, k[perm], v[perm])
        np.testing.assert_allclose(op, o, rtol=0, atol=1e-13)


def test_v_all_ones_gives_ones():
    q, k = rnd((33, 8), 23, 3.0), rnd((45, 8), 24, 3.0)
    v = np.ones((45, 8))
    for fn in (oracle.naive_fwd, oracle.chunked_fwd):
        o, _, _ = fn(q, k, v)
        np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


def test_translating_all_keys_leaves_output_unchanged():
    q, k, v = rnd((30, 16), 25), rnd((50, 16), 26), rnd((50, 16), 27)
    w = rnd((1, 16), 28, 2.0)
    for fn in (oracle.naive_fwd, oracle.chunked_fwd):
        o, _, _ = fn(q, k, v)
        o2, _, _ = fn(q, k + w, v)
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)


def test_linear_in_v():
    q, k = rnd((20, 8), 29), rnd((30, 8), 30)
    v1, v2 = rnd((30, 8), 31), rnd((30, 8), 32)
    o1, _, _ = oracle.naive_fwd(q, k, v1)
    o2, _, _ = oracle.naive_fwd(q, k, v2)
    o3, _, _ = oracle.naive_fwd(q, k, 2.5 * v1 - 0.75 * v2)
    np.testing.assert_allclose(o3, 2.5 * o1 - 0.75 * o2, rtol=0, atol=1e-13)


def test_argmax_limit_at_1e4_scores():
    # Q, K ~ 30 N(0,1) at d = 128: raw scores ~1e4. Where the top two scaled
    # scores differ by more than 40, exp(-40) < 5e-18 so o_i = v_argmax to fp64.
    q, k, v = rnd((200, 128), 33, 30.0), rnd((300, 128), 34, 30.0), rnd((300, 128), 35)
    raw = q @ k.T
    assert np.abs(raw).max() > 5e3
    s = raw / math.sqrt(128)
    srt = np.sort(s, axis=1)
    clear = (srt[:, -1] - srt[:, -2]) > 40.0
    assert clear.sum() > 100
    for fn in (oracle.naive_fwd, oracle.chunked_fwd):
        o, _, _ = fn(q, k, v)
        assert np.all(np.isfinite(o))
        np.testing.assert_allclose(o[clear], v[np.argmax(s, axis=1)][clear], rtol=0, atol=1e-15)


def test_row_stats_brute_force():
    q, k = rnd((6, 5), 36), rnd((9, 5), 37)
    m, l = oracle.row_stats(q, k)
    _, m2, l2 = oracle.naive_fwd(q, k, rnd((9, 5), 38))
    for i in range(6):
        s = [sum(q[i][t] * k[j][t] for t in range(5)) / math.sqrt(5) for j in range(9)]
        assert m[i] == pytest.approx(max(s), abs=1e-15)
        assert l[i] == pytest.approx(sum(math.exp(x - max(s)) for x in s), rel=1e-14)
        assert 1.0 <= l[i] <= 9.0
    np.testing.assert_allclose(m2, m, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, l, rtol=1e-14, atol=0)


def test_row_subset_equals_full():
    q, k, v = rnd((2, 3, 50, 8), 39), rnd((2, 3, 50, 8), 40), rnd((2, 3, 50, 8), 41)
    rows = np.array([0, 7, 49, 13])
    o, m, l = oracle.naive_fwd(q, k, v)
    os_, ms, ls = oracle.naive_fwd(q, k, v, rows=rows, row_block=3)
    np.testing.assert_allclose(os_, o[..., rows, :], rtol=0, atol=1e-14)
    np.testing.assert_allclose(ms, m[..., rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(ls, l[..., rows], rtol=1e-14, atol=0)


def test_empty_inputs():
    z = np.zeros((2, 0, 64))
    o, m, l = oracle.naive_fwd(z, z, z)
    assert o.shape == (2, 0, 64) and m.shape == (2, 0)
    o, m, l = oracle.chunked_fwd(z, z, z)
    assert o.shape == (2, 0, 64)
    dq, dk, dv = oracle.naive_bwd(z, z, z, z)
    assert dq.shape == (2, 0, 64)


# --------------------------------------------------------------- backward pins

def _loss(q, k, v, do):
    o, _, _ = oracle.naive_fwd(q, k, v)
    return float((o * do).sum())


@pytest.mark.parametrize("G,n,d", [(1, 1, 1), (1, 2, 2), (2, 3, 4), (1, 5, 8), (2, 8, 2), (1, 8, 8)])
def test_backward_central_finite_differences(G, n, d):
    rng = np.random.default_rng(100 + n * 10 + d)
    q, k, v, do = (rng.standard_normal((G, n, d)) for _ in range(4))
    dq, dk, dv = oracle.naive_bwd(q, k, v, do)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], do)) / (2 * h)
        err = np.abs(num - g).max()
        scale = max(1.0, np.abs(g).max())
        assert err / scale <= 1e-6, (name, err)


def test_backward_matches_torch_autograd_fp64():
    rng = np.random.default_rng(200)
    q, k, v, do = (rng.standard_normal((2, 2, 29, 16)) for _ in range(4))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    out.backward(torch.from_numpy(do))
    dq, dk, dv = oracle.naive_bwd(q, k, v, do, row_block=7)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_sum_identities():
    # sum_j dK_j = 0 (softmax rows are shift-invariant) and sum_j dV_j = sum_i dO_i (rows of P sum to 1).
    rng = np.random.default_rng(201)
    q, k, v, do = (rng.standard_normal((3, 64, 32)) for _ in range(4))
    dq, dk, dv = oracle.naive_bwd(q, k, v, do)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), rtol=0, atol=1e-12)


def test_backward_special_cases():
    rng = np.random.default_rng(202)
    q, k, v, do = (rng.standard_normal((2, 1, 16)) for _ in range(4))
    dq, dk, dv = oracle.naive_bwd(q, k, v, do)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv, do, rtol=0, atol=0)
    # identical keys: uniform P, so dQ = 0
    q, v, do = (rng.standard_normal((20, 16)) for _ in range(3))
    k = np.repeat(rng.standard_normal((1, 16)), 20, axis=0)
    dq, dk, dv = oracle.naive_bwd(q, k, v, do)
    np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-14)


def test_backward_subsets_equal_full():
    rng = np.random.default_rng(203)
    q, k, v, do = (rng.standard_normal((2, 40, 8)) for _ in range(4))
    dq, dk, dv = oracle.naive_bwd(q, k, v, do)
    rows, cols = np.array([3, 0, 39]), np.array([5, 38])
    dq2, dk2, dv2 = oracle.naive_bwd(q, k, v, do, rows=rows, cols=cols, row_block=6)
    np.testing.assert_allclose(dq2, dq[:, rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk2, dk[:, cols], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv2, dv[:, cols], rtol=0, atol=1e-13)


def test_backward_row_term_from_the_exact_output_is_the_default():
    # D_i = dO_i . O_i equals sum_j P_ij dP_ij when O is the exact output
    rng = np.random.default_rng(204)
    q, k, v, do = (rng.standard_normal((2, 37, 16)) for _ in range(4))
    o, _, _ = oracle.naive_fwd(q, k, v)
    ref = oracle.naive_bwd(q, k, v, do)
    got = oracle.naive_bwd(q, k, v, do, o=o, row_block=10)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_backward_row_term_from_a_perturbed_output_closed_form():
    # o' = o + delta changes D by dD_i = dO_i . delta_i, hence dS by -P_ij dD_i:
    # dQ_i moves by -dD_i (P K)_i / sqrt(d), dK_j by -sum_i dD_i P_ij q_i / sqrt(d),
    # and dV not at all
    rng = np.random.default_rng(205)
    G, n, d = 2, 23, 8
    q, k, v, do = (rng.standard_normal((G, n, d)) for _ in range(4))
    o, _, _ = oracle.naive_fwd(q, k, v)
    delta = 1e-3 * rng.standard_normal(o.shape)
    dq0, dk0, dv0 = oracle.naive_bwd(q, k, v, do)
    dq1, dk1, dv1 = oracle.naive_bwd(q, k, v, do, o=o + delta)
    scale = 1.0 / math.sqrt(d)
    s = np.einsum("gid,gjd->gij", q, k) * scale
    p = np.exp(s - s.max(axis=2, keepdims=True))
    p /= p.sum(axis=2, keepdims=True)
    dD = (do * delta).sum(axis=2)
    np.testing.assert_allclose(dq1 - dq0, -dD[:, :, None] * np.einsum("gij,gjd->gid", p, k) * scale,
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk1 - dk0, -np.einsum("gi,gij,gid->gjd", dD, p, q) * scale,
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv1, dv0, rtol=0, atol=0)


# --------------------------------------------------------- planted mistakes
# Each test plants a plausible bug in the oracle (CPU only) and checks that a
# pin above detects it.

def test_planted_wrong_scale_is_caught(monkeypatch):
    monkeypatch.setattr(A, "softmax_scale", lambda d: 1.0 / float(d))
    with pytest.raises(AssertionError):
        test_two_key_closed_form_fixes_scale(0.3)


def test_planted_transposed_scores_are_caught(monkeypatch):
    real = A.naive_fwd

    def transposed(q, k, v, rows=None, row_block=1024):
        # uses K Q^T instead of Q K^T
        return real(k, q, v, rows=rows, row_block=row_block)

    monkeypatch.setattr(oracle, "naive_fwd", transposed)
    with pytest.raises(AssertionError):
        test_matches_torch_sdpa_fp64()


def test_planted_missing_rescale_is_caught(monkeypatch):
    # a chunked loop that forgets to rescale acc by alpha when the max moves
    def bad_chunked(q, k, v, chunk=None):
        q3, k3, v3 = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        scale = A.softmax_scale(q3.shape[-1])
        chunk = chunk or 1
        n = q3.shape[-2]
        m = np.full(n, -np.inf)
        l = np.zeros(n)
        acc = np.zeros((n, v3.shape[-1]))
        for c0 in range(0, k3.shape[-2], chunk):
            s = (q3 @ k3[c0:c0 + chunk].T) * scale
            m_new = np.maximum(m, s.max(axis=1))
            p = np.exp(s - m_new[:, None])
            l = np.exp(m - m_new) * l + p.sum(axis=1)
            acc = acc + p @ v3[c0:c0 + chunk]
            m = m_new
        return acc / l[:, None], m, l

    monkeypatch.setattr(oracle, "chunked_fwd", bad_chunked)
    with pytest.raises(AssertionError):
        test_naive_and_chunked_match_brute_force(5, 4)


def test_planted_wrong_gradient_sign_is_caught(monkeypatch):
    real = A.naive_bwd

    def bad(q, k, v, do, rows=None, cols=None, row_block=1024):
        dq, dk, dv = real(q, k, v, do, rows, cols, row_block)
        return dq, -dk, dv

    monkeypatch.setattr(oracle, "naive_bwd", bad)
    with pytest.raises(AssertionError):
        test_backward_central_finite_differences(1, 5, 8)


# ---------------------------------------------------- fp32 error floor (design)

def test_fp32_scores_cannot_meet_1e5_on_stress_inputs_but_fp64_scores_can():
    """Why the fp32-input kernel forms scores in fp64.

    With Q, K ~ 30 N(0,1) at d = 128 (raw scores ~1e4), fp32 rounding of the
    scores (~1e-3 absolute) moves near-tied softmax weights, so an all-fp32
    pipeline misses the 1e-5 output tolerance. fp32 inputs multiply exactly in
    fp64, and with fp64 scores (fp32 exp and accumulation after the max is
    subtracted) the error falls well below it.
    """
    import inputgen
    t = inputgen.draw(1, 1, 8192, 128, "fp32", seed=1004, qk_scale=30.0)
    q = t["q"][0, 0, :384].numpy()
    k = t["k"][0, 0].numpy()
    v = t["v"][0, 0].numpy()
    ref, _, _ = oracle.naive_fwd(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    sc = np.float32(1.0 / math.sqrt(128))
    # all-fp32 pipeline
    s32 = (q @ k.T) * sc
    p32 = np.exp(s32 - s32.max(axis=1, keepdims=True))
    o32 = (p32 @ v) / p32.sum(axis=1, keepdims=True)
    err32 = np.abs(o32 - ref).max()
    # fp64 scores and max-subtraction, then fp32 exp / sum / PV
    s64 = (q.astype(np.float64) @ k.astype(np.float64).T) / math.sqrt(128)
    p = np.exp((s64 - s64.max(axis=1, keepdims=True)).astype(np.float32))
    o = (p @ v) / p.sum(axis=1, keepdims=True)
    err64 = np.abs(o - ref).max()
    assert err32 > 1e-5, err32
    assert err64 < 2e-6, err64


def test_backward_rows_only_equals_full():
    # an empty cols list visits only the blocks holding the requested rows
    rng = np.random.default_rng(204)
    q, k, v, do = (rng.standard_normal((2, 50, 8)) for _ in range(4))
    dq, _, _ = oracle.naive_bwd(q, k, v, do)
    rows = np.array([49, 3, 20])
    dq2, dk2, dv2 = oracle.naive_bwd(q, k, v, do, rows=rows, cols=np.array([], dtype=np.int64),
                                     row_block=7)
    np.testing.assert_allclose(dq2, dq[:, rows], rtol=0, atol=1e-13)
    assert dk2.shape == (2, 0, 8) and dv2.shape == (2, 0, 8)
