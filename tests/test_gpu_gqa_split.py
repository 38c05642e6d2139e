"""GPU parity for grouped-query heads, separate query/key lengths and the
split-key forward, through the C ABI, against the fp64 oracle.

Tolerances are those of test_gpu_parity.py (fp32: 1e-5; bf16: 2e-2 plus
relative L2 <= 1e-2), element by element on the same seeded inputs. The
oracle's ``gqa_fwd``/``gqa_bwd`` give query head h the key/value head
h // (H / H_kv) and ``split_fwd`` is pinned to ``naive_fwd``; here the GPU is
compared with the plain definitions directly.
"""

import numpy as np
import pytest
import torch

import inputgen
import memory_efficient_exact_amd as mea
import oracle

from test_gpu_parity import check, check_stats, f64, gpu, say

pytestmark = pytest.mark.gpu

# (B, H, H_kv, n_q, n_k): grouped, multi-query, cross lengths, ragged tiles, a single key
GQA_CASES = [(1, 4, 2, 17, 300), (2, 8, 1, 5, 129), (1, 6, 3, 257, 64), (1, 2, 2, 1, 1000),
             (1, 3, 3, 300, 1), (1, 4, 4, 100, 33), (2, 8, 2, 64, 513)]


def draw(B, H, H_kv, n_q, n_k, d, dtype, seed, with_do=False, qk_scale=1.0):
    return inputgen.draw_gqa(B, H, H_kv, n_q, n_k, d, dtype, seed=seed, with_do=with_do,
                             qk_scale=qk_scale)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,H_kv,n_q,n_k", GQA_CASES)
def test_fwd_ex_small_full(dtype, d, B, H, H_kv, n_q, n_k):
    say("fwd_ex", dtype, d, B, H, H_kv, n_q, n_k)
    t = draw(B, H, H_kv, n_q, n_k, d, dtype, seed=21 + n_q + n_k + d)
    o, m, l = mea.attn_fwd_ex(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]))
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle.gqa_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]))
    check("O", f64(o.cpu()), o_ref, dtype)
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,H_kv,n_q,n_k", [(1, 4, 2, 17, 300), (1, 8, 1, 33, 129),
                                              (2, 4, 4, 100, 37), (1, 2, 1, 1, 200),
                                              (1, 4, 2, 300, 1), (1, 6, 2, 130, 260)])
def test_bwd_ex_small_full(dtype, d, B, H, H_kv, n_q, n_k):
    say("bwd_ex", dtype, d, B, H, H_kv, n_q, n_k)
    t = draw(B, H, H_kv, n_q, n_k, d, dtype, seed=31 + n_q + n_k + d, with_do=True)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o, m, l = mea.attn_fwd_ex(q, k, v)
    dq, dk, dv = mea.attn_bwd_ex(q, k, v, o, do, m, l)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.gqa_bwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"]))
    check("dQ", f64(dq.cpu()), rq, dtype)
    check("dK", f64(dk.cpu()), rk, dtype)
    check("dV", f64(dv.cpu()), rv, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bwd_ex_without_queries_gives_zero_key_gradients(dtype):
    say("bwd_ex n_q=0", dtype)
    t = draw(1, 4, 2, 0, 200, 64, dtype, seed=41, with_do=True)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    m = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    l = torch.empty_like(m)
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    _, dk, dv = mea.attn_bwd_ex(q, k, v, o, do, m, l, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


# ------------------------------------------------------------------ split keys

SPLIT_CASES = [(1, 1, 1, 1, 2000), (1, 4, 2, 33, 1500), (2, 2, 2, 130, 777), (1, 8, 1, 3, 4100)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7, 1000])
@pytest.mark.parametrize("B,H,H_kv,n_q,n_k", SPLIT_CASES)
def test_splitkv_small_full(dtype, d, splits, B, H, H_kv, n_q, n_k):
    used = mea.attn_fwd_splitkv_num_splits(mea.DTYPE_BF16 if dtype == "bf16" else mea.DTYPE_F32,
                                           B, H, H_kv, n_q, n_k, d, splits)
    say("splitkv", dtype, d, splits, "->", used, B, H, H_kv, n_q, n_k)
    t = draw(B, H, H_kv, n_q, n_k, d, dtype, seed=51 + n_q + n_k + d)
    o, m, l = mea.attn_fwd_splitkv(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]), num_splits=splits)
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle.gqa_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]))
    check("O", f64(o.cpu()), o_ref, dtype)
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, dtype)


def test_splitkv_workspace_is_reused_across_calls():
    # the second, smaller call reads nothing the first one left behind
    say("splitkv workspace reuse")
    big = draw(1, 2, 1, 40, 3000, 64, "bf16", seed=61)
    small = draw(1, 2, 1, 9, 700, 64, "bf16", seed=62)
    need = mea.attn_fwd_splitkv_workspace_bytes(mea.DTYPE_BF16, 1, 2, 1, 40, 3000, 64, 16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for t, s in ((big, 16), (small, 5)):
        o, m, l = mea.attn_fwd_splitkv(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]), num_splits=s,
                                       workspace=ws)
        torch.cuda.synchronize()
        o_ref, m_ref, l_ref = oracle.gqa_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]))
        check("O", f64(o.cpu()), o_ref, "bf16")
        check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, "bf16")


def test_splitkv_single_head_fp32_workload_full():
    # the 1 x 1 x 1024 x 64 fp32 workload: 16 query tiles alone leave most of the GPU idle
    w = inputgen.WORKLOADS["c1_single_head_fp32"]
    t = inputgen.make_inputs(w)
    used = mea.attn_fwd_splitkv_num_splits(mea.DTYPE_F32, w.B, w.H, w.H, w.n, w.n, w.d, 0)
    say("splitkv", w.name, "splits", used)
    assert used > 1
    o, m, l = mea.attn_fwd_splitkv(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]))
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle.naive_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]))
    check("O", f64(o.cpu()), o_ref, "fp32")
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, "fp32")


def test_splitkv_stress_fp32_sampled_rows():
    # 2 x 8 x 8192 x 128 fp32, Q and K scaled by 30 (scores ~1e4), all-equal keys in head 0:
    # range maxima differ by thousands, so the merge must re-base every range exactly
    w = inputgen.WORKLOADS["c4_stress_fp32"]
    t = inputgen.make_inputs(w)
    say("splitkv", w.name, "splits 8")
    o, m, l = mea.attn_fwd_splitkv(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]), num_splits=8)
    torch.cuda.synchronize()
    rows = np.random.default_rng(71).choice(w.n, 48, replace=False)
    rows = np.concatenate([rows, [0, w.n - 1]])
    o_ref, m_ref, l_ref = oracle.naive_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), rows=rows)
    check("O", f64(o.cpu())[:, :, rows], o_ref, "fp32")
    check_stats(m.cpu().numpy()[:, :, rows], l.cpu().numpy()[:, :, rows], m_ref, l_ref, "fp32")
    mean = f64(t["v"])[:, 0].mean(axis=1)  # equal keys: uniform weights
    check("O equal-key head", f64(o.cpu())[:, 0], np.broadcast_to(mean[:, None, :], (2, w.n, 128)),
          "fp32")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 128)])
def test_splitkv_decode_step(dtype, d):
    # one new query per head against a 16384-entry key/value cache, 4 query heads per K/V head
    B, H, H_kv, n_q, n_k = 1, 8, 2, 1, 16384
    dt = mea.DTYPE_BF16 if dtype == "bf16" else mea.DTYPE_F32
    used = mea.attn_fwd_splitkv_num_splits(dt, B, H, H_kv, n_q, n_k, d, 0)
    say("decode", dtype, d, "splits", used)
    assert used >= 16
    t = draw(B, H, H_kv, n_q, n_k, d, dtype, seed=81)
    o, m, l = mea.attn_fwd_splitkv(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]))
    o1, m1, l1 = mea.attn_fwd_ex(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]))
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle.gqa_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]))
    check("O split", f64(o.cpu()), o_ref, dtype)
    check("O unsplit", f64(o1.cpu()), o_ref, dtype)
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, dtype)


# ------------------------------------------------------- larger grouped-query shapes

def test_gqa_prefill_sampled_rows_fwd_bwd():
    # 32 query heads over 8 key/value heads, 2048 tokens, d = 128, forward and backward;
    # sampled query rows for O and dQ, sampled key rows for dK and dV (the oracle forms
    # every row's full softmax for them)
    B, H, H_kv, n, d = 1, 32, 8, 2048, 128
    say("gqa prefill", B, H, H_kv, n, d)
    t = draw(B, H, H_kv, n, n, d, "bf16", seed=91, with_do=True)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o, m, l = mea.attn_fwd_ex(q, k, v)
    dq, dk, dv = mea.attn_bwd_ex(q, k, v, o, do, m, l)
    torch.cuda.synchronize()
    rng = np.random.default_rng(92)
    rows = np.concatenate([rng.choice(n, 30, replace=False), [0, n - 1]])
    cols = np.concatenate([rng.choice(n, 30, replace=False), [0, n - 1]])
    o_ref, m_ref, l_ref = oracle.gqa_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), rows=rows)
    check("O", f64(o.cpu())[:, :, rows], o_ref, "bf16")
    check_stats(m.cpu().numpy()[:, :, rows], l.cpu().numpy()[:, :, rows], m_ref, l_ref, "bf16")
    rq, rk, rv = oracle.gqa_bwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"]), rows=rows,
                                cols=cols)
    check("dQ", f64(dq.cpu())[:, :, rows], rq, "bf16")
    check("dK", f64(dk.cpu())[:, :, cols], rk, "bf16")
    check("dV", f64(dv.cpu())[:, :, cols], rv, "bf16")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_multi_token_decode_split(dtype, d):
    # 4 new queries per head (32 heads over 8 key/value heads) against a 32768-entry cache
    B, H, H_kv, n_q, n_k = 2, 32, 8, 4, 32768
    say("decode 4 tokens", dtype, d)
    t = draw(B, H, H_kv, n_q, n_k, d, dtype, seed=93)
    o, m, l = mea.attn_fwd_splitkv(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]))
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle.gqa_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]))
    check("O", f64(o.cpu()), o_ref, dtype)
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, dtype)


def test_splitkv_bf16_large_scores():
    # bf16 inputs with Q and K scaled by 30: range maxima far apart, every range re-based
    say("splitkv bf16 x30")
    t = draw(1, 4, 2, 200, 3000, 64, "bf16", seed=94, qk_scale=30.0)
    o, m, l = mea.attn_fwd_splitkv(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]), num_splits=12)
    o1, m1, l1 = mea.attn_fwd_ex(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]))
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle.gqa_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]))
    check("O split", f64(o.cpu()), o_ref, "bf16")
    check("O unsplit", f64(o1.cpu()), o_ref, "bf16")
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, "bf16")


# ------------------------------------------------------- 8-wave forward workgroups
# The bf16 forward takes 8-wave workgroups (512 query rows at d = 64, 256 at
# d = 128) when heads x tiles of that size reach 256; these shapes do, with a
# ragged last tile, grouped heads and key counts that are not tile multiples.
WIDE_CASES = [(1, 256, 256, 600, 300, 64), (2, 256, 64, 150, 200, 64),
              (1, 128, 128, 300, 333, 128), (4, 256, 32, 40, 97, 128)]


@pytest.mark.parametrize("B,H,H_kv,n_q,n_k,d", WIDE_CASES)
@pytest.mark.parametrize("splits", [None, 3])
def test_wide_workgroups_full(B, H, H_kv, n_q, n_k, d, splits):
    rows = (512 if d == 64 else 256)
    assert B * H_kv * -(-(H // H_kv) * n_q // rows) >= 256  # the 8-wave layout is taken
    say("wide", B, H, H_kv, n_q, n_k, d, splits)
    t = draw(B, H, H_kv, n_q, n_k, d, "bf16", seed=151 + n_q + d)
    q, k, v = (gpu(t[x]) for x in ("q", "k", "v"))
    if splits is None:
        o, m, l = mea.attn_fwd_ex(q, k, v)
    else:
        assert mea.attn_fwd_splitkv_num_splits(mea.DTYPE_BF16, B, H, H_kv, n_q, n_k, d, splits) > 1
        o, m, l = mea.attn_fwd_splitkv(q, k, v, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle.gqa_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]))
    check("O", f64(o.cpu()), o_ref, "bf16")
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, "bf16")


# Row-tiled 4-wave forward workgroups. Grids of at most 128 such workgroups
# take the decoding layout instead (keys split across the waves), so these
# shapes sit between 128 and 256 workgroups: bf16 at d = 64 (256 rows per
# workgroup) and d = 128 (128 rows), fp32 (64 rows), with ragged tiles and
# grouped heads.
ROW_TILED_CASES = [("bf16", 1, 33, 33, 1000, 300, 64), ("bf16", 2, 64, 16, 300, 257, 64),
                   ("bf16", 1, 17, 17, 1000, 333, 128), ("fp32", 1, 9, 9, 1000, 300, 64),
                   ("fp32", 1, 12, 3, 1000, 200, 128)]


@pytest.mark.parametrize("dtype,B,H,H_kv,n_q,n_k,d", ROW_TILED_CASES)
@pytest.mark.parametrize("splits", [None, 3])
def test_row_tiled_workgroups_full(dtype, B, H, H_kv, n_q, n_k, d, splits):
    rows = {("bf16", 64): 256, ("bf16", 128): 128}.get((dtype, d), 64)
    grid = B * H_kv * -(-(H // H_kv) * n_q // rows)
    assert 128 < grid < 256  # the row-tiled 4-wave layout is taken
    say("row-tiled", dtype, B, H, H_kv, n_q, n_k, d, splits)
    t = draw(B, H, H_kv, n_q, n_k, d, dtype, seed=171 + n_q + d)
    q, k, v = (gpu(t[x]) for x in ("q", "k", "v"))
    if splits is None:
        o, m, l = mea.attn_fwd_ex(q, k, v)
    else:
        dt = mea.DTYPE_BF16 if dtype == "bf16" else mea.DTYPE_F32
        assert mea.attn_fwd_splitkv_num_splits(dt, B, H, H_kv, n_q, n_k, d, splits) > 1
        o, m, l = mea.attn_fwd_splitkv(q, k, v, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle.gqa_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]))
    check("O", f64(o.cpu()), o_ref, dtype)
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, dtype)


# Grids of at most 128 row-tiled workgroups take the decoding layout whatever
# the number of query rows: thousands of rows per head here, grouped heads,
# ragged key counts, and one shape exactly at the 128-workgroup threshold.
DECODE_GRID_CASES = [("bf16", 1, 1, 1, 8192, 8192, 64), ("bf16", 1, 2, 1, 4096, 3000, 128),
                     ("fp32", 1, 2, 2, 2000, 2100, 64), ("fp32", 2, 4, 2, 1000, 777, 128)]


@pytest.mark.parametrize("dtype,B,H,H_kv,n_q,n_k,d", DECODE_GRID_CASES)
def test_small_grid_decoding_layout_full(dtype, B, H, H_kv, n_q, n_k, d):
    rows = {("bf16", 64): 256, ("bf16", 128): 128}.get((dtype, d), 64)
    grid = B * H_kv * -(-(H // H_kv) * n_q // rows)
    assert 2 * grid <= 256 and (H // H_kv) * n_q > 64  # decoding layout by grid size only
    say("small-grid decode", dtype, B, H, H_kv, n_q, n_k, d)
    t = draw(B, H, H_kv, n_q, n_k, d, dtype, seed=181 + n_q + d)
    o, m, l = mea.attn_fwd_ex(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]))
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle.gqa_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]))
    check("O", f64(o.cpu()), o_ref, dtype)
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, dtype)


@pytest.mark.parametrize("d", [64, 128])
def test_small_grid_decoding_layout_fp32_stress_full(d):
    # fp32 at the x30 score scale of the stress workload (scores of ~1e4), on a grid
    # small enough for the decoding layout: the waves' partial results, each formed
    # against its own fp64 maximum, merge through LDS within the 1e-5 bar
    B, H, H_kv, n_q, n_k = 1, 2, 2, 2048, 2048
    grid = B * H_kv * -(-n_q // 64)
    assert 2 * grid <= 256
    say("small-grid decode fp32 x30", d)
    t = draw(B, H, H_kv, n_q, n_k, d, "fp32", seed=191 + d, qk_scale=30.0)
    o, m, l = mea.attn_fwd_ex(gpu(t["q"]), gpu(t["k"]), gpu(t["v"]))
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle.gqa_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]))
    assert np.abs(m_ref).max() > 1e3  # the stress scale is reached
    check("O", f64(o.cpu()), o_ref, "fp32")
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, "fp32")


# Split backward: on grids of at most 256 unsplit workgroups each workgroup's sweep
# is cut into ranges whose fp32 partials a reduce pass sums, when the workspace
# holds them (the size the workspace query reports). With only the row terms the
# same call runs unsplit. Both are checked against the oracle and against each
# other, with ragged tiles, grouped heads, both head dimensions and both types.
SPLIT_BWD_CASES = [("bf16", 1, 1, 1, 1024, 1024, 64), ("bf16", 1, 3, 3, 700, 333, 64),
                   ("bf16", 2, 4, 2, 300, 1000, 128), ("bf16", 1, 16, 16, 1024, 1024, 64),
                   ("fp32", 1, 1, 1, 1024, 1024, 64), ("fp32", 1, 4, 1, 200, 777, 128),
                   ("fp32", 2, 2, 2, 129, 1500, 64)]


@pytest.mark.parametrize("dtype,B,H,H_kv,n_q,n_k,d", SPLIT_BWD_CASES)
def test_split_backward_full(dtype, B, H, H_kv, n_q, n_k, d):
    dt = mea.DTYPE_BF16 if dtype == "bf16" else mea.DTYPE_F32
    row = 8 if dtype == "bf16" else 16
    full = mea.attn_bwd_ex_workspace_bytes(dt, B, H, H_kv, n_q, n_k, d)
    assert full > row * B * H * n_q  # the shape is split
    say("split bwd", dtype, B, H, H_kv, n_q, n_k, d, full)
    t = draw(B, H, H_kv, n_q, n_k, d, dtype, seed=201 + n_q + n_k + d, with_do=True)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o, m, l = mea.attn_fwd_ex(q, k, v)
    ws_full = torch.empty(full, dtype=torch.uint8, device=q.device)
    ws_min = torch.empty(row * B * H * n_q, dtype=torch.uint8, device=q.device)
    s_dq, s_dk, s_dv = mea.attn_bwd_ex(q, k, v, o, do, m, l, workspace=ws_full)
    u_dq, u_dk, u_dv = mea.attn_bwd_ex(q, k, v, o, do, m, l, workspace=ws_min)
    # one byte short of the split layout: the unsplit backward, bit for bit
    c_dq, c_dk, c_dv = mea.attn_bwd_ex(q, k, v, o, do, m, l, workspace=ws_full[:full - 1])
    torch.cuda.synchronize()
    assert torch.equal(c_dq, u_dq) and torch.equal(c_dk, u_dk) and torch.equal(c_dv, u_dv)
    rq, rk, rv = oracle.gqa_bwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"]))
    for name, got, ref in (("dQ", s_dq, rq), ("dK", s_dk, rk), ("dV", s_dv, rv),
                           ("dQ unsplit", u_dq, rq), ("dK unsplit", u_dk, rk),
                           ("dV unsplit", u_dv, rv)):
        check(name, f64(got.cpu()), ref, dtype)
    # split and unsplit differ only by the order of fp32 additions
    for a, b in ((s_dq, u_dq), (s_dk, u_dk), (s_dv, u_dv)):
        check("split vs unsplit", f64(a.cpu()), f64(b.cpu()), dtype)


# The bf16 backward at d = 64 takes 8-wave workgroups (256 keys or queries each)
# when heads x (key tiles + query tiles) of that size reach 256: ragged tiles on both
# sides, grouped heads, and fewer keys than one workgroup covers.
WIDE_BWD_CASES = [(1, 128, 128, 300, 300), (4, 64, 16, 70, 300), (1, 64, 64, 1000, 77)]


@pytest.mark.parametrize("B,H,H_kv,n_q,n_k", WIDE_BWD_CASES)
def test_wide_workgroups_backward_full(B, H, H_kv, n_q, n_k):
    rows_q = (H // H_kv) * n_q
    assert B * H_kv * (-(-n_k // 256) - (-rows_q // 256)) >= 256  # the 8-wave layout is taken
    say("wide bwd", B, H, H_kv, n_q, n_k)
    t = draw(B, H, H_kv, n_q, n_k, 64, "bf16", seed=161 + n_q, with_do=True)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o, m, l = mea.attn_fwd_ex(q, k, v)
    dq, dk, dv = mea.attn_bwd_ex(q, k, v, o, do, m, l)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.gqa_bwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"]))
    check("dQ", f64(dq.cpu()), rq, "bf16")
    check("dK", f64(dk.cpu()), rk, "bf16")
    check("dV", f64(dv.cpu()), rv, "bf16")


@pytest.mark.parametrize("B,H,H_kv,n", [(1, 32, 8, 4096), (1, 4, 4, 3001)])
def test_backward_d128_long_sampled(B, H, H_kv, n):
    # the d = 128 backward at a prefill-sized grouped shape (8-wave layout) and a ragged
    # length (4-wave layout): sampled dQ rows of two query heads and sampled dK, dV rows
    # of their key/value heads against the oracle
    say("bwd d128 long", B, H, H_kv, n)
    t = draw(B, H, H_kv, n, n, 128, "bf16", seed=171 + n, with_do=True)
    q, k, v, do = (gpu(t[x]) for x in ("q", "k", "v", "do"))
    o, m, l = mea.attn_fwd_ex(q, k, v)
    dq, dk, dv = mea.attn_bwd_ex(q, k, v, o, do, m, l)
    torch.cuda.synchronize()
    dq, dk, dv = (f64(x.cpu()) for x in (dq, dk, dv))
    rng = np.random.default_rng(n)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 30, replace=False)]))
    G = H // H_kv
    for hk in (0, H_kv - 1):
        qh = slice(hk * G, hk * G + G)  # the query heads of key/value head hk
        qs, dos = f64(t["q"])[:, qh], f64(t["do"])[:, qh]
        ks, vs = f64(t["k"])[:, hk:hk + 1], f64(t["v"])[:, hk:hk + 1]
        rq, rk, rv = oracle.gqa_bwd(qs[:, :1], ks, vs, dos[:, :1], rows=rows,
                                    cols=np.array([], dtype=np.int64))
        check("dQ", dq[:, hk * G:hk * G + 1][:, :, rows], rq, "bf16")
        _, rk, rv = oracle.gqa_bwd(qs, ks, vs, dos, rows=np.array([], dtype=np.int64), cols=rows)
        check("dK", dk[:, hk:hk + 1][:, :, rows], rk, "bf16")
        check("dV", dv[:, hk:hk + 1][:, :, rows], rv, "bf16")
