"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances (max |gpu - oracle| per element, separately for O, dQ, dK, dV):
  * fp32 inputs: 1e-5, absolute, for every element;
  * bf16 inputs: 2e-2 absolute, or one bf16 ulp of the reference value where
    that is larger (only |ref| >= 4, which no workload reaches: an output in
    bf16 can be no closer than one of the two bf16 neighbours of the exact
    value), and additionally relative L2 error <= 1e-2 (bf16 outputs are
    small, |O| <~ 0.1 at n >= 4096, so 2e-2 alone would admit a badly wrong
    kernel).
Every element of every workload is compared, forward and backward; the
oracle runs per (batch, head) on a thread pool to keep the full sizes within
a minute or two of host time. With MEA_PARITY_RECORD=<path> set, every check
appends its error figures to that file as one JSON line.
"""

import json
import math
import os
from concurrent.futures import ThreadPoolExecutor

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


def ulp(x, dtype):
    """Spacing of the output type at |x|: 2^(e - 7) for bf16 (8 significant
    bits), 2^(e - 23) for fp32, with e = floor(log2 |x|); the smallest normal
    spacing below that."""
    a = np.abs(np.asarray(x, np.float64))
    bits = 8 if dtype == "bf16" else 24
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - (bits - 1))


def bar_of(ref, dtype):
    """Per-element bar: 1e-5 for fp32; for bf16 the larger of 2e-2 and one bf16
    ulp of the reference value (representability: the exact result lies
    between two bf16 neighbours, which are one ulp apart)."""
    if dtype == "fp32":
        return np.full(np.shape(ref), TOL["fp32"])
    return np.maximum(TOL["bf16"], ulp(ref, "bf16"))


def record(entry):
    path = os.environ.get("MEA_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(entry) + "\n")


def check(name, got, ref, dtype, tag=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    if not got.size:
        return 0.0
    diff = np.abs(got - ref)
    err = float(diff.max())
    bar = bar_of(ref, dtype)
    worst = int(np.argmax(diff - bar))
    rel = None
    if dtype == "bf16":
        # relative L2, with a floor of 1e-3 rms on the denominator. An exactly
        # zero reference (dQ at n = 1; dK with a single key, where dP - D
        # vanishes) leaves only fp32 rounding noise of the order of 1e-6 (the
        # same dot product summed in two orders); the floor keeps that from
        # becoming an unbounded ratio. It lies below every output scale of
        # the workloads (rms |O| >= 0.014 at n = 16384, rms dQ/dK/dV ~ 0.018).
        den = max(np.linalg.norm(ref), 1e-3 * math.sqrt(ref.size))
        rel = float(np.linalg.norm(got - ref) / den)
    if tag is not None:
        record({"case": tag, "output": name, "dtype": dtype, "elements": int(ref.size),
                "max_abs_err": err, "max_abs_ref": float(np.abs(ref).max()),
                "bar": float(bar.max()) if dtype == "bf16" else TOL["fp32"],
                "rel_l2": rel if rel is not None else float(
                    np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))})
    assert diff.flat[worst] <= bar.flat[worst], (
        f"{name}: abs err {diff.flat[worst]:.3e} > bar {bar.flat[worst]:.3e} at flat index "
        f"{worst} (ref {ref.flat[worst]:.6g}, got {got.flat[worst]:.6g}); max abs err {err:.3e}")
    if rel is not None:
        assert rel <= REL_L2_BF16, f"{name}: rel L2 {rel:.3e}"
    return err


def check_relative(name, got, ref, dtype):
    """The bf16 bar taken relative to the tensor's largest reference value,
    2e-2 * max(1, max |ref|), plus the relative L2 gate: only for shapes whose
    outputs lie far above the workloads' scale and where bf16 operands alone
    cannot meet the absolute bar (each use says why)."""
    assert dtype == "bf16"
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape and np.all(np.isfinite(got)), name
    if not got.size:
        return 0.0
    err = float(np.abs(got - ref).max())
    bar = TOL["bf16"] * max(1.0, float(np.abs(ref).max()))
    assert err <= bar, f"{name}: max abs err {err:.3e} > {bar:.3e}"
    den = max(np.linalg.norm(ref), 1e-3 * math.sqrt(ref.size))
    rel = float(np.linalg.norm(got - ref) / den)
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
    check("dQ", f64(dq.cpu()), rq, "fp32", tag=w.name + " backward")
    check("dK", f64(dk.cpu()), rk, "fp32", tag=w.name + " backward")
    check("dV", f64(dv.cpu()), rv, "fp32", tag=w.name + " backward")


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
    tag = f"fp32 stress backward 1x2x1500x{d}"
    check("dQ", f64(dq.cpu()), rq, "fp32", tag=tag)
    check("dK", f64(dk.cpu()), rk, "fp32", tag=tag)
    check("dV", f64(dv.cpu()), rv, "fp32", tag=tag)


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


# Scores that climb past the reference in every 32-key block: key j carries
# alpha * j in column 0 and q has 1 there, so each block's row maximum exceeds
# the previous block's by about 32 * alpha raw units (> 8 in log2 units), and
# every block takes the rebase path (new reference, rescaled acc and l, the
# block's weights formed again). One shape per forward layout.
CLIMB = [
    (1, 2, 1000, 64),    # decoding layout (small grid)
    (1, 40, 1000, 64),   # 4-wave row-tiled layout
    (1, 130, 1000, 64),  # 8-wave row-tiled layout
    (1, 20, 1000, 128),  # 4-wave row-tiled layout, d = 128
    (1, 64, 1000, 128),  # 8-wave row-tiled layout, d = 128
]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,H,n,d,splits", [c + (1,) for c in CLIMB] + [(1, 2, 1000, 64, 4),
                                                                         (1, 2, 1000, 128, 4)])
def test_scores_climbing_every_block(dtype, B, H, n, d, splits):
    say("climbing scores", dtype, B, H, n, d, "splits", splits)
    t = inputgen.draw(B, H, n, d, "fp32", seed=11)
    alpha = 2.5 if d == 64 else 3.5
    q = t["q"] * 0.5
    q[..., 0] = 1.0
    k = t["k"].clone()
    k[..., 0] = alpha * torch.arange(n, dtype=torch.float32)
    cast = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = {"q": q.to(cast), "k": k.to(cast), "v": t["v"].to(cast)}
    if splits == 1:
        o, m, l = run_fwd(t)
    else:  # key ranges whose maxima differ by far more than the threshold, then the merge
        o, m, l = mea.attn_fwd_splitkv(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]), num_splits=splits)
        torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle_heads(oracle.naive_fwd, f64(t["q"]), f64(t["k"]), f64(t["v"]))
    check("O", f64(o.cpu()), o_ref, dtype, tag=f"climb {dtype} {B}x{H}x{n}x{d} splits {splits}")
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, dtype)


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

def oracle_heads(fn, *arrays, **kw):
    """fn(*[a[b, h] for a in arrays], **kw) for every (b, h) of [B, H, n, d]
    arrays, on a pool of host threads (one BLAS thread each; numpy releases the
    interpreter lock in its matrix products and elementwise loops). Returns the
    per-head results stacked back to [B, H, ...], one array per output of fn."""
    from threadpoolctl import threadpool_limits
    B, H = arrays[0].shape[:2]
    jobs = [(b, h) for b in range(B) for h in range(H)]
    workers = max(1, min(len(jobs), 16, len(os.sched_getaffinity(0))))
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(lambda bh: fn(*(a[bh[0], bh[1]] for a in arrays), **kw), jobs))
    outs = []
    for i in range(len(res[0])):
        stacked = np.stack([r[i] for r in res])
        outs.append(stacked.reshape((B, H) + stacked.shape[1:]))
    return outs


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["c1_single_head_fp32", "c2_multihead_bf16", "c3_long_bf16",
                                  "c4_stress_fp32"])
def test_workload_forward(name):
    # every query row of every head against the oracle's definition
    w = inputgen.WORKLOADS[name]
    say("workload fwd", name)
    t = inputgen.make_inputs(w)
    o, m, l = run_fwd(t)
    o, m, l = f64(o.cpu()), m.cpu().numpy(), l.cpu().numpy()
    q, k, v = f64(t["q"]), f64(t["k"]), f64(t["v"])
    o_ref, m_ref, l_ref = oracle_heads(oracle.naive_fwd, q, k, v, row_block=512)
    err = check("O", o, o_ref, w.dtype, tag=name)
    check_stats(m, l, m_ref, l_ref, w.dtype)
    say(name, "max abs err", f"{err:.3e}")
    if w.equal_key_heads:
        # every query in an all-equal-key head gets the mean of the values
        for h in w.equal_key_heads:
            mean = v[:, h].mean(axis=1, keepdims=True)
            check("O equal-key head", o[:, h], np.broadcast_to(mean, o[:, h].shape), w.dtype)


@pytest.mark.timeout(900)
def test_workload_training_step():
    # 2 x 8 x 8192 x 64 bf16: O, dQ, dK and dV, every element
    w = inputgen.WORKLOADS["c5_train_bf16"]
    say("workload fwd+bwd", w.name)
    t = inputgen.make_inputs(w)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o, m, l = mea.attn_fwd(q, k, v)
    dq, dk, dv = mea.attn_bwd(q, k, v, o, do, m, l)
    torch.cuda.synchronize()
    o, dq, dk, dv = (f64(x.cpu()) for x in (o, dq, dk, dv))
    q64, k64, v64, do64 = (f64(t[x]) for x in ("q", "k", "v", "do"))
    o_ref, m_ref, l_ref = oracle_heads(oracle.naive_fwd, q64, k64, v64, row_block=512)
    check("O", o, o_ref, "bf16", tag=w.name)
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, "bf16")
    rq, rk, rv = oracle_heads(oracle.naive_bwd, q64, k64, v64, do64, row_block=512)
    for nm, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        err = check(nm, got, ref, "bf16", tag=w.name)
        say(w.name, nm, "max abs err", f"{err:.3e}")


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


@pytest.mark.timeout(900)
def test_bench_step_workload_backward():
    # the step bench.py times: 1 x 16 x 16384 x 64 bf16, inputs drawn exactly as the bench
    # draws them, forward with statistics then backward with a caller workspace; every
    # element of dQ, dK and dV against the oracle
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
    q64, k64, v64, do64 = (f64(t[x]) for x in ("q", "k", "v", "do"))
    rq, rk, rv = oracle_heads(oracle.naive_bwd, q64, k64, v64, do64, row_block=512)
    for nm, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        err = check(nm, got, ref, "bf16", tag="c3_long_bf16 backward")
        say("bench step", nm, "max abs err", f"{err:.3e}")
    # identities on every head: sum_j dK_j = 0, sum_j dV_j = sum_i dO_i
    for h in range(w.H):
        sk = np.abs(dk[0, h]).sum(axis=0)
        sv = np.abs(dv[0, h]).sum(axis=0)
        assert np.all(np.abs(dk[0, h].sum(axis=0)) <= 1e-3 * sk), h
        assert np.all(np.abs(dv[0, h].sum(axis=0) - do64[0, h].sum(axis=0)) <= 1e-3 * sv), h
