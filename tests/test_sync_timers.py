"""The timing library (libmea_synctimers.so): the same kernels built with
MEA_SYNC_TIMERS=1, which count per wave the core cycles of each tiled loop and
of its end-of-tile copy wait and barrier, and per SIMD pair of an 8-wave
workgroup the cycles both waves sit at the barrier (bench.py --mode sync).

CPU: what the library exports, and the reduction of its counters. GPU: its
outputs equal libmea.so's bit for bit, and its tile counts match the loops."""

import math
import os
import subprocess

import pytest

import memory_efficient_exact_amd as mea

from test_abi import header_functions

READERS = {"mea_sync_timers_fwd", "mea_sync_timers_bwd"}


def test_timing_library_exports_the_c_abi_and_its_two_readers():
    path = mea.timing_library_path()
    if not os.path.exists(path):
        pytest.fail("libmea_synctimers.so is not built; run __graft_entry__.build() first")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.split()[1:2] == ["T"]}
    assert exported == set(header_functions()) | READERS, exported ^ (set(header_functions()) | READERS)


def test_sync_counter_reduction():
    import bench
    # forward row-tiled layout: 16 waves (two 8-wave workgroups) x 8 tiles, 1000
    # loop cycles per tile of which 100 copy wait and 250 barrier; the 8 first
    # waves of the SIMD pairs saw both waves at the barrier 40 cycles per tile;
    # decoding layout unused
    fwd = [16 * 8 * 100, 16 * 8 * 250, 16 * 8 * 1000, 16 * 8, 16, 8 * 8 * 40, 8 * 8 * 1000] + [0] * 7
    # backward: only the d = 64 dQ role ran (one 4-wave workgroup x 3 tiles: no pairs)
    bwd = [0] * 7 + [12 * 30, 12 * 60, 12 * 600, 12, 4, 0, 0] + [0] * 14
    d = bench.derive_sync(fwd, bwd)
    assert set(d) == {"fwd row-tiled", "bwd d=64 dQ"}
    f = d["fwd row-tiled"]
    assert f["tiles_per_wave"] == 8 and f["loop_cycles_per_tile"] == 1000
    assert f["copy_wait_cycles_per_tile"] == 100 and f["barrier_cycles_per_tile"] == 250
    assert f["copy_wait_share"] == pytest.approx(0.1) and f["barrier_share"] == pytest.approx(0.25)
    assert f["pair_idle_share"] == pytest.approx(0.04)
    q = d["bwd d=64 dQ"]
    assert q["tiles_per_wave"] == 3 and q["barrier_share"] == pytest.approx(0.1)
    assert q["pair_idle_share"] is None


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,n,d", [(1, 16, 2048, 64), (1, 8, 1000, 128)])
def test_timing_library_matches_libmea_and_counts_every_tile(B, H, n, d):
    import torch

    import bench
    import inputgen
    from test_gpu_parity import say
    say(f"timing library {B}x{H}x{n}x{d}")
    dev = torch.device("cuda:0")
    t = inputgen.draw(B, H, n, d, "bf16", seed=1003, with_do=True)
    q, k, v, do = (t[x].to(dev) for x in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    m = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    ws = torch.empty(mea.attn_bwd_workspace_bytes(mea.DTYPE_BF16, B, H, n, d), dtype=torch.uint8,
                     device=dev)

    def step():
        mea.attn_fwd(q, k, v, out=o, row_max=m, row_sum=l)
        mea.attn_bwd(q, k, v, o, do, m, l, dq=dq, dk=dk, dv=dv, workspace=ws)

    r = bench.run_sync(step, (o, m, l, dq, dk, dv), 3, dev)
    assert r["bitwise_equal_to_libmea"]
    loops = r["loops"]
    assert any(name.startswith("fwd") for name in loops)
    assert any(name.startswith(f"bwd d={d} ") for name in loops)
    for name, x in loops.items():
        assert x["waves"] > 0 and x["tiles_per_wave"] >= 1
        assert 0 <= x["copy_wait_share"] <= 1 and 0 <= x["barrier_share"] <= 1
        assert x["copy_wait_cycles_per_tile"] + x["barrier_cycles_per_tile"] <= x["loop_cycles_per_tile"]
        if x["pair_idle_share"] is not None:  # both waves idle only while each waits
            assert 0 <= x["pair_idle_share"] <= x["barrier_share"] * 1.05
    if d == 64:
        # a grid that fills the chip runs the backward unsplit: every wave of both
        # roles sweeps all 64-row tiles of its head
        for role in ("bwd d=64 dK/dV", "bwd d=64 dQ"):
            assert loops[role]["tiles_per_wave"] == math.ceil(n / 64), (role, loops[role])
