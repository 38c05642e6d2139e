"""attn_bwd_noalloc (the backward for callers that cannot allocate) against
attn_bwd, through the C ABI, on two calls in a row with the second smaller,
and captured in a HIP graph (its first call in the process) and replayed.

attn_bwd_noalloc runs in the library's per-GPU scratch array instead of a
caller workspace. The split layout of a small grid (at most about 25 MiB)
always fits that array and is used exactly as attn_bwd uses it when given
attn_bwd_workspace_bytes, so the gradients must be equal bit for bit. Small
results are also held to the oracle's bar (fp32 1e-5, bf16 2e-2) so that two
equal wrong answers cannot pass. The second call reuses the array the first
one filled, with fewer rows, so stale contents would show.
"""

import numpy as np
import pytest
import torch

import inputgen
import memory_efficient_exact_amd as mea
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"fp32": 1e-5, "bf16": 2e-2}


def say(*a):
    print("[case]", *a, flush=True)


def run_pair(B, H, n, d, dtype, seed):
    t = inputgen.draw(B, H, n, d, dtype, seed=seed, with_do=True)
    q, k, v, do = (t[x].to(DEV) for x in ("q", "k", "v", "do"))
    o, m, l = mea.attn_fwd(q, k, v)
    dt = mea.DTYPE_BF16 if dtype == "bf16" else mea.DTYPE_F32
    ws = torch.empty(max(16, mea.attn_bwd_workspace_bytes(dt, B, H, n, d)), dtype=torch.uint8,
                     device=DEV)
    ref = mea.attn_bwd(q, k, v, o, do, m, l, workspace=ws)
    outs = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    before = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    got = mea.attn_bwd_noalloc(q, k, v, o, do, m, l, *outs)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == before  # nothing allocated by the call
    return t, ref, got


def check_oracle(t, got, dtype):
    f = inputgen.to_f64
    refs = oracle.naive_bwd(f(t["q"]), f(t["k"]), f(t["v"]), f(t["do"]))
    for name, g, r in zip(("dQ", "dK", "dV"), got, refs):
        err = np.abs(f(g.cpu()) - r).max()
        say(name, f"max abs err vs oracle {err:.3e}")
        assert err <= TOL[dtype], (name, err)


def test_noalloc_first_call_inside_graph_capture():
    # The callers this entry point is for capture it in HIP graphs. Defined first in
    # the last test file, this test makes the process's first attn_bwd_noalloc call
    # inside a capture (that call also looks up the scratch array's device address);
    # nothing runs it earlier. A small grid, so the split layout runs in the array.
    # Every replay, with new inputs copied in and eager work between replays, must
    # equal the eager attn_bwd given its workspace, bit for bit.
    say("noalloc captured in a graph")
    shape = (1, 2, 1000, 64)
    B, H, n, d = shape
    q, k, v, do, o = (torch.empty(shape, dtype=torch.bfloat16, device=DEV) for _ in range(5))
    m = torch.empty(shape[:3], device=DEV)
    l = torch.empty_like(m)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    ws = torch.empty(mea.attn_bwd_workspace_bytes(mea.DTYPE_BF16, B, H, n, d), dtype=torch.uint8,
                     device=DEV)

    def load(seed):
        t = inputgen.draw(*shape, "bf16", seed=seed, with_do=True)
        for buf, name in zip((q, k, v, do), ("q", "k", "v", "do")):
            buf.copy_(t[name])
        mea.attn_fwd(q, k, v, out=o, row_max=m, row_sum=l)
        torch.cuda.synchronize()
        return t

    load(150)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            mea.attn_bwd_noalloc(q, k, v, o, do, m, l, *grads)
    torch.cuda.synchronize()
    for replay, seed in enumerate((151, 152, 153)):
        t = load(seed)
        g.replay()
        torch.cuda.synchronize()
        ref = mea.attn_bwd(q, k, v, o, do, m, l, workspace=ws)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), grads, ref):
            assert torch.equal(a, b), (replay, name)
    check_oracle(t, grads, "bf16")


@pytest.mark.parametrize("dtype,d,first,second", [
    # 4-wave grids small enough for the split backward: the split layout fits the array
    ("bf16", 64, (1, 4, 2048), (1, 2, 300)),
    ("bf16", 128, (2, 2, 1024), (1, 1, 129)),
    ("fp32", 64, (1, 2, 1024), (1, 1, 257)),
    ("fp32", 128, (1, 2, 1000), (1, 1, 65)),
    # a grid that fills the chip (unsplit, row terms only), then a split one
    ("bf16", 64, (1, 16, 4096), (2, 4, 1000)),
])
def test_noalloc_matches_attn_bwd_twice(dtype, d, first, second):
    for i, (B, H, n) in enumerate((first, second)):
        say("noalloc vs attn_bwd", dtype, d, B, H, n)
        t, ref, got = run_pair(B, H, n, d, dtype, seed=500 + 7 * i + n + d)
        for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.equal(a, b), f"{name} differs from attn_bwd ({dtype}, {B}x{H}x{n}x{d})"
        if n <= 2048:
            check_oracle(t, got, dtype)


def test_noalloc_bench_step_then_small():
    # the 1 x 16 x 16384 x 64 bf16 step (unsplit; 2 MiB of row terms in the array),
    # then a small split grid that reuses the array
    for i, (B, H, n, d) in enumerate(((1, 16, 16384, 64), (1, 1, 700, 64))):
        say("noalloc vs attn_bwd", B, H, n, d)
        t, ref, got = run_pair(B, H, n, d, "bf16", seed=90 + i)
        for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.equal(a, b), name
    check_oracle(t, got, "bf16")


def test_noalloc_rejects_more_rows_than_the_array_holds():
    # bf16 row terms take 8 bytes per query row: 2^22 rows fill the 32 MiB array
    # exactly, one more row is rejected before anything runs
    say("noalloc size limit")
    x = torch.empty(16, dtype=torch.bfloat16, device=DEV)
    p = x.data_ptr()
    L = mea.lib()
    st = L.attn_bwd_noalloc(mea.DTYPE_BF16, 1, 1, (1 << 22) + 1, 64, *([p] * 10), None)
    assert mea.attn_status_str(st) == "MEA_ERR_WORKSPACE"
    # at exactly 2^22 rows the size passes and validation goes on to the next rule
    # (every pointer is the same buffer here, so the outputs overlap the inputs)
    st = L.attn_bwd_noalloc(mea.DTYPE_BF16, 1, 1, 1 << 22, 64, *([p] * 10), None)
    assert mea.attn_status_str(st) == "MEA_ERR_ALIAS"
