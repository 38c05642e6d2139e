"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances (max |gpu - oracle| per element, separately for O, dQ, dK, dV):
  * fp32 inputs: 1e-5;
  * bf16 inputs: 2e-2, and additionally relative L2 error <= 1e-2 (bf16
    outputs are small, |O| <~ 0.1 at n >= 4096, so 2e-2 alone would admit
    a badly wrong kernel).
Both bars are absolute for outputs of magnitude <= 1 (every workload) and
scale with max |reference| beyond that (see ``check``).
Small shapes are compared in full; the full-size workloads are compared on
sampled query rows (and sampled key rows for dK/dV), which the oracle
computes exactly from the complete key set.
"""

import math

import numpy as np
import pytest
import torch

import inputgen
import memory_efficient_exact_amd as mea
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"fp32": 1e-5, "bf16": 2e-2}
REL_L2_BF16 = 1e-2


def say(*a):
    print("[case]", *a, flush=True)


def gpu(t):
    return t.to(DEV)


def f64(t):
    return inputgen.to_f64(t)


def run_fwd(t):
    q, k, v = gpu(t["q"]), gpu(t["k"]), gpu(t["v"])
    o, m, l = mea.attn_fwd(q, k, v)
    torch.cuda.synchronize()
    return o, m, l


def check(name, got, ref, dtype):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = np.abs(got - ref).max() if got.size else 0.0
    # The bar is absolute for outputs of magnitude <= 1, which holds for every
    # workload (bf16: |O|, |dQ|, |dK|, |dV| <~ 0.2). Where a test shape has
    # larger outputs (one key shared by hundreds of query rows sums their dO
    # into dV), an output in the input type cannot be closer than half its
    # ulp, so the bar scales with the largest reference value.
    bar = TOL[dtype] * max(1.0, float(np.abs(ref).max()) if ref.size else 0.0)
    assert err <= bar, f"{name}: max abs err {err:.3e} > {bar:.3e}"
    if dtype == "bf16" and got.size:
        # relative L2, with a floor of 1e-3 rms on the denominator. An exactly
        # zero reference (dQ at n = 1; dK with a single key, where dP - D
        # vanishes) leaves only fp32 rounding noise of the order of 1e-6 (the
        # same dot product summed in two orders); the floor keeps that from
        # becoming an unbounded ratio. It lies below every output scale of
        # the workloads (rms |O| >= 0.014 at n = 16384, rms dQ/dK/dV ~ 0.018).
        den = max(np.linalg.norm(ref), 1e-3 * math.sqrt(ref.size))
        rel = np.linalg.norm(got - ref) / den
        assert rel <= REL_L2_BF16, f"{name}: rel L2 {rel:.3e}"
    return err


def check_stats(m, l, m_ref, l_ref, dtype):
    """Row statistics: m (natural units, fp32 rounding of a score of size |m|)
    and the log-sum-exp m + log(l). The pair is stored so that l sums
    exp(s - m) for the stored m; where m was rounded only l absorbs it, and
    m + log(l) does not depend on the rounding (at scores of ~1e4 fp32
    rounding of m alone moves l by 2e-4)."""
    m = np.asarray(m, np.float64)
    l = np.asarray(l, np.float64)
    np.testing.assert_allclose(m, m_ref, rtol=2e-6, atol=1e-6)
    lse = m + np.log(l)
    lse_ref = np.asarray(m_ref, np.float64) + np.log(np.asarray(l_ref, np.float64))
    # the same relative allowance as m (fp32 scores of size |m|) plus the absolute
    # accuracy of the sum
    np.testing.assert_allclose(lse, lse_ref, rtol=2e-6, atol=1e-4 if dtype == "bf16" else 1e-5)


# ------------------------------------------------------------ small, full compare

SMALL = [(1, 1, 1), (1, 1, 2), (1, 1, 3), (1, 3, 17), (1, 1, 63), (1, 1, 64), (1, 1, 65),
         (3, 1, 127), (1, 1, 129), (1, 3, 300), (2, 1, 1000), (1, 1, 257)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,n", SMALL)
def test_fwd_small_full(dtype, d, B, H, n):
    say("fwd small", dtype, d, B, H, n)
    t = inputgen.draw(B, H, n, d, dtype, seed=7 + n + d)
    o, m, l = run_fwd(t)
    o_ref, m_ref, l_ref = oracle.naive_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]))
    check("O", f64(o.cpu()), o_ref, dtype)
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,n", [(1, 1, 1), (1, 1, 17), (1, 3, 130), (2, 1, 300), (1, 1, 256)])
def test_bwd_small_full(dtype, d, B, H, n):
    say("bwd small", dtype, d, B, H, n)
    t = inputgen.draw(B, H, n, d, dtype, seed=11 + n + d, with_do=True)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o, m, l = mea.attn_fwd(q, k, v)
    dq, dk, dv = mea.attn_bwd(q, k, v, o, do, m, l)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.naive_bwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"]))
    check("dQ", f64(dq.cpu()), rq, dtype)
    check("dK", f64(dk.cpu()), rk, dtype)
    check("dV", f64(dv.cpu()), rv, dtype)


def test_bwd_fp32_single_head_workload_full():
    # the 1 x 1 x 1024 x 64 fp32 workload, forward then backward, every element
    w = inputgen.WORKLOADS["c1_single_head_fp32"]
    say("bwd fp32", w.name)
    t = inputgen.make_inputs(w, with_do=True)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o, m, l = mea.attn_fwd(q, k, v)
    dq, dk, dv = mea.attn_bwd(q, k, v, o, do, m, l)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.naive_bwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"]))
    check("dQ", f64(dq.cpu()), rq, "fp32")
    check("dK", f64(dk.cpu()), rk, "fp32")
    check("dV", f64(dv.cpu()), rv, "fp32")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_fp32_stress_scores(d):
    # Q and K scaled by 30 (scaled scores in the hundreds to thousands) and one head of
    # all-equal keys, as in the fp32 stress workload: the probabilities are rebuilt from
    # the stored statistics, so their fp32 rounding must not leak into the gradients
    say("bwd fp32 stress", d)
    t = inputgen.draw(1, 2, 1500, d, "fp32", seed=17 + d, qk_scale=30.0, equal_key_heads=(0,),
                      with_do=True)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o, m, l = mea.attn_fwd(q, k, v)
    dq, dk, dv = mea.attn_bwd(q, k, v, o, do, m, l)
    torch.cuda.synchronize()
    assert float(m.abs().max()) > 300.0
    rq, rk, rv = oracle.naive_bwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"]))
    check("dQ", f64(dq.cpu()), rq, "fp32")
    check("dK", f64(dk.cpu()), rk, "fp32")
    check("dV", f64(dv.cpu()), rv, "fp32")


# ------------------------------------------------------------ invariants on GPU output

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_n1_returns_v_bitwise(dtype, d):
    say("n=1", dtype, d)
    t = inputgen.draw(2, 3, 1, d, dtype, seed=3)
    o, m, l = run_fwd(t)
    assert torch.equal(o.cpu(), t["v"])
    if dtype == "bf16":
        assert torch.all(l.cpu() == 1.0)
    else:
        # fp32: m is the fp64 score rounded to fp32 and l = exp(s - m) absorbs that
        # rounding, so m + log(l) is the score itself
        s = (f64(t["q"]) * f64(t["k"])).sum(-1) / math.sqrt(d)
        lse = m.cpu().double().numpy() + np.log(l.cpu().double().numpy())
        np.testing.assert_allclose(lse, s, rtol=0, atol=1e-6)
        assert np.all(np.abs(l.cpu().numpy() - 1.0) <= 2.0 ** -20)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_identical_keys_give_mean_of_values(dtype):
    say("equal keys", dtype)
    t = inputgen.draw(1, 2, 333, 128, dtype, seed=4, qk_scale=30.0, equal_key_heads=(0, 1))
    o, m, l = run_fwd(t)
    mean = f64(t["v"]).mean(axis=2, keepdims=True)
    check("O", f64(o.cpu()), np.broadcast_to(mean, o.shape), dtype)
    if dtype == "bf16":
        np.testing.assert_allclose(l.cpu().numpy(), 333.0, rtol=1e-5)
    else:
        # fp32 at scores of ~1e4: l is re-based onto the fp32-rounded maximum, so the
        # log-sum-exp is what equals s + log(333)
        s = (f64(t["q"]) * f64(t["k"])[:, :, :1, :]).sum(-1) / math.sqrt(128)
        lse = m.cpu().double().numpy() + np.log(l.cpu().double().numpy())
        np.testing.assert_allclose(lse, s + math.log(333.0), rtol=0, atol=1e-5)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_permuting_kv_pairs(dtype):
    say("permutation", dtype)
    t = inputgen.draw(1, 2, 200, 64, dtype, seed=5)
    perm = torch.from_numpy(np.random.default_rng(6).permutation(200))
    o1, _, _ = run_fwd(t)
    t2 = dict(t, k=t["k"][:, :, perm].contiguous(), v=t["v"][:, :, perm].contiguous())
    o2, _, _ = run_fwd(t2)
    check("O perm", f64(o2.cpu()), f64(o1.cpu()), dtype)


def test_runs_are_bitwise_deterministic():
    say("determinism")
    t = inputgen.draw(2, 4, 1000, 64, "bf16", seed=8, with_do=True)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    outs = []
    for _ in range(2):
        o, m, l = mea.attn_fwd(q, k, v)
        dq, dk, dv = mea.attn_bwd(q, k, v, o, do, m, l)
        torch.cuda.synchronize()
        outs.append([x.cpu() for x in (o, m, l, dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_gradient_sum_identities_on_gpu():
    say("grad sums")
    t = inputgen.draw(1, 2, 512, 64, "bf16", seed=9, with_do=True)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o, m, l = mea.attn_fwd(q, k, v)
    dq, dk, dv = mea.attn_bwd(q, k, v, o, do, m, l)
    torch.cuda.synchronize()
    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i hold exactly; bf16 outputs allow
    # a rounding error of ~2^-9 per element
    assert f64(dk.cpu()).sum(axis=2).__abs__().max() < 0.05
    np.testing.assert_allclose(f64(dv.cpu()).sum(axis=2), f64(t["do"]).sum(axis=2), atol=0.3)


# ------------------------------------------------------------ full-size workloads

def sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    fixed = np.array([0, 1, n // 2, n - 2, n - 1])
    return np.unique(np.concatenate([fixed, rng.choice(n, size=count, replace=False)]))


@pytest.mark.parametrize("name", ["c1_single_head_fp32", "c2_multihead_bf16", "c3_long_bf16",
                                  "c4_stress_fp32"])
def test_workload_forward(name):
    w = inputgen.WORKLOADS[name]
    say("workload fwd", name)
    t = inputgen.make_inputs(w)
    o, m, l = run_fwd(t)
    o, m, l = f64(o.cpu()), m.cpu().numpy(), l.cpu().numpy()
    rows = np.arange(w.n) if w.n <= 1024 else sample_rows(w.n, 96, w.seed)
    q, k, v = f64(t["q"]), f64(t["k"]), f64(t["v"])
    o_ref, m_ref, l_ref = oracle.naive_fwd(q, k, v, rows=rows)
    err = check("O", o[:, :, rows], o_ref, w.dtype)
    check_stats(m[:, :, rows], l[:, :, rows], m_ref, l_ref, w.dtype)
    say(name, "max abs err", f"{err:.3e}")
    if w.equal_key_heads:
        # every query in an all-equal-key head gets the mean of the values
        for h in w.equal_key_heads:
            mean = v[:, h].mean(axis=1, keepdims=True)
            check("O equal-key head", o[:, h], np.broadcast_to(mean, o[:, h].shape), w.dtype)


def test_workload_training_step():
    w = inputgen.WORKLOADS["c5_train_bf16"]
    say("workload fwd+bwd", w.name)
    t = inputgen.make_inputs(w)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o, m, l = mea.attn_fwd(q, k, v)
    dq, dk, dv = mea.attn_bwd(q, k, v, o, do, m, l)
    torch.cuda.synchronize()
    o, dq, dk, dv = (f64(x.cpu()) for x in (o, dq, dk, dv))
    rows = sample_rows(w.n, 48, w.seed)
    cols = sample_rows(w.n, 48, w.seed + 1)
    for b, h in ((0, 0), (1, 7)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        qs, ks, vs, dos = (f64(t[x])[sl] for x in ("q", "k", "v", "do"))
        o_ref, _, _ = oracle.naive_fwd(qs, ks, vs, rows=rows)
        check("O", o[sl][:, :, rows], o_ref, "bf16")
        rq, rk, rv = oracle.naive_bwd(qs, ks, vs, dos, rows=rows, cols=cols)
        check("dQ", dq[sl][:, :, rows], rq, "bf16")
        check("dK", dk[sl][:, :, cols], rk, "bf16")
        check("dV", dv[sl][:, :, cols], rv, "bf16")


def test_forward_allocates_nothing_beyond_outputs():
    w = inputgen.WORKLOADS["c3_long_bf16"]
    say("memory", w.name)
    t = inputgen.make_inputs(w)
    q, k, v = gpu(t["q"]), gpu(t["k"]), gpu(t["v"])
    o = torch.empty_like(q)
    m = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    l = torch.empty_like(m)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    mea.attn_fwd(q, k, v, out=o, row_max=m, row_sum=l)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == before
    # the only state beyond Q, K, V, O is 8 bytes per row of statistics
    assert m.numel() * 4 + l.numel() * 4 == 8 * w.B * w.H * w.n


def test_bench_step_workload_backward():
    # the step bench.py times: 1 x 16 x 16384 x 64 bf16, inputs drawn exactly as the bench
    # draws them, forward with statistics then backward with a caller workspace
    w = inputgen.WORKLOADS["c3_long_bf16"]
    say("bench step fwd+bwd", w.name)
    t = inputgen.draw(w.B, w.H, w.n, w.d, w.dtype, seed=w.seed, with_do=True)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    m = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    l = torch.empty_like(m)
    ws = torch.empty(mea.attn_bwd_workspace_bytes(mea.DTYPE_BF16, w.B, w.H, w.n, w.d),
                     dtype=torch.uint8, device=DEV)
    mea.attn_fwd(q, k, v, out=o, row_max=m, row_sum=l)
    dq, dk, dv = mea.attn_bwd(q, k, v, o, do, m, l, workspace=ws)
    torch.cuda.synchronize()
    dq, dk, dv = (f64(x.cpu()) for x in (dq, dk, dv))
    rows = sample_rows(w.n, 24, w.seed + 2)
    cols = sample_rows(w.n, 24, w.seed + 3)
    q64, k64, v64, do64 = (f64(t[x]) for x in ("q", "k", "v", "do"))
    # dQ rows on every head (each row needs only its own softmax)
    rq, _, _ = oracle.naive_bwd(q64, k64, v64, do64, rows=rows, cols=np.array([], dtype=np.int64),
                                row_block=64)
    check("dQ", dq[:, :, rows], rq, "bf16")
    # dK, dV key rows on two heads (every query row contributes)
    for h in (0, 11):
        sl = (slice(0, 1), slice(h, h + 1))
        _, rk, rv = oracle.naive_bwd(q64[sl], k64[sl], v64[sl], do64[sl], rows=rows[:1], cols=cols)
        check("dK", dk[sl][:, :, cols], rk, "bf16")
        check("dV", dv[sl][:, :, cols], rv, "bf16")
    # identities on every head: sum_j dK_j = 0, sum_j dV_j = sum_i dO_i
    for h in range(w.H):
        sk = np.abs(dk[0, h]).sum(axis=0)
        sv = np.abs(dv[0, h]).sum(axis=0)
        assert np.all(np.abs(dk[0, h].sum(axis=0)) <= 1e-3 * sk), h
        assert np.all(np.abs(dv[0, h].sum(axis=0) - do64[0, h].sum(axis=0)) <= 1e-3 * sv), h
