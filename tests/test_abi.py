"""The C ABI on the CPU: symbols, status strings and host-side validation.

Validation runs before any HIP call, so every error code is reachable here
without a GPU. No test in this file launches a kernel.
"""

import ctypes
import os
import re
import subprocess

import pytest
import torch

import memory_efficient_exact_amd as mea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mea.h")

F32, BF16 = mea.DTYPE_F32, mea.DTYPE_BF16
OK, NULL, SHAPE, UNSUP, ALIGN, WS, LAUNCH, ALIAS = range(8)
A = 0x10000  # aligned fake device addresses: validation never dereferences them


def header_functions():
    """Names of the functions include/mea.h declares (every one is marked MEA_API)."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^MEA_API\b[^;(]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    # every prototype in the header carries the export marker
    protos = re.findall(r"^[A-Za-z_][^;{}#]*?\b([a-z_][a-z0-9_]*)\s*\([^;{}]*\)\s*;", text, flags=re.M)
    assert sorted(set(protos)) == sorted(set(names)), (protos, names)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mea.library_path()):
        pytest.fail("libmea.so is not built; run __graft_entry__.build() first")
    return mea.lib()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert set(names) >= {"attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_status_str",
                          "mea_version", "attn_fwd_ex", "attn_bwd_ex", "attn_bwd_ex_workspace_bytes",
                          "attn_fwd_splitkv", "attn_fwd_splitkv_num_splits",
                          "attn_fwd_splitkv_workspace_bytes", "attn_bwd_noalloc"}
    for nm in names:
        assert hasattr(L, nm), f"libmea.so does not export {nm}"


def test_exports_nothing_but_the_c_abi():
    out = subprocess.run(["nm", "-D", "--defined-only", mea.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.split()[1:2] == ["T"]}
    assert exported == set(header_functions()), exported ^ set(header_functions())


def test_status_strings(L):
    for code, name in enumerate(["MEA_OK", "MEA_ERR_NULL", "MEA_ERR_SHAPE", "MEA_ERR_UNSUPPORTED",
                                 "MEA_ERR_ALIGN", "MEA_ERR_WORKSPACE", "MEA_ERR_LAUNCH",
                                 "MEA_ERR_ALIAS"]):
        assert mea.attn_status_str(code) == name
    assert mea.attn_status_str(99) == "MEA_UNKNOWN_STATUS"
    assert mea.mea_version() == 400


def fwd(L, dt=BF16, B=1, H=1, n=128, d=64, q=A, k=A, v=A, o=A, m=0, l=0):
    return L.attn_fwd(dt, B, H, n, d, q, k, v, o, m, l, None)


def bwd(L, dt=BF16, B=1, H=1, n=128, d=64, ptrs=None, ws=A, wsb=1 << 20):
    p = dict(q=A, k=A, v=A, o=A, do=A, m=A, l=A, dq=A, dk=A, dv=A)
    p.update(ptrs or {})
    return L.attn_bwd(dt, B, H, n, d, p["q"], p["k"], p["v"], p["o"], p["do"], p["m"], p["l"],
                      p["dq"], p["dk"], p["dv"], ws, wsb, None)


def test_fwd_validation(L):
    assert fwd(L, dt=2) == UNSUP
    assert fwd(L, dt=-1) == UNSUP
    assert fwd(L, B=-1) == SHAPE
    assert fwd(L, H=-3) == SHAPE
    assert fwd(L, n=-1) == SHAPE
    assert fwd(L, n=(1 << 24) + 1) == SHAPE
    assert fwd(L, B=1 << 20, H=1 << 20) == SHAPE
    # grid bound: B*H * ceil(n / 64) <= 2^22 keeps every launch within 2^31 work-items
    assert fwd(L, B=1, H=(1 << 22) + 1, n=64) == SHAPE
    assert fwd(L, B=1 << 10, H=1 << 10, n=(1 << 12) + 1) == SHAPE
    assert fwd(L, d=96) == UNSUP
    assert fwd(L, d=32) == UNSUP
    assert fwd(L, q=0) == NULL
    assert fwd(L, o=0) == NULL
    assert fwd(L, m=A, l=0) == NULL
    assert fwd(L, m=0, l=A) == NULL
    assert fwd(L, v=A + 8) == ALIGN
    assert fwd(L, m=A + 4, l=A) == ALIGN


def test_fwd_empty_is_noop(L):
    # B, H or n = 0: nothing to do, no HIP call, pointers may be NULL
    assert fwd(L, B=0, q=0, k=0, v=0, o=0) == OK
    assert fwd(L, H=0, q=0, k=0, v=0, o=0) == OK
    assert fwd(L, n=0, q=0, k=0, v=0, o=0, dt=F32, d=128) == OK


def test_bwd_validation(L):
    assert bwd(L, dt=2) == UNSUP
    # fp32 keeps 16 bytes per query row (fp64 log-sum-exp); every call below stops
    # in validation (a passing fp32 call would launch on the fake pointers)
    assert bwd(L, dt=F32, wsb=16 * 128 - 1) == WS
    assert bwd(L, dt=F32, ws=0) == WS
    assert bwd(L, dt=F32, ptrs={"dq": 0}) == NULL
    assert bwd(L, dt=F32, d=96) == UNSUP
    assert bwd(L, d=256) == UNSUP
    assert bwd(L, n=-5) == SHAPE
    for name in ("q", "k", "v", "o", "do", "m", "l", "dq", "dk", "dv"):
        assert bwd(L, ptrs={name: 0}) == NULL, name
        assert bwd(L, ptrs={name: A + 2}) == ALIGN, name
    assert bwd(L, ws=0) == WS
    assert bwd(L, wsb=8 * 128 - 1) == WS
    assert bwd(L, wsb=8 * 128, ws=A + 8) == ALIGN
    assert bwd(L, B=0, ws=0, wsb=0, ptrs={k: 0 for k in ("q", "k", "v")}) == OK


def test_bwd_noalloc_validation(L):
    # the backward without a workspace: same rules as attn_bwd, and the row terms
    # (8 bytes per query row for bf16, 16 for fp32) must fit the 32 MiB scratch
    # array. Every call below stops in validation (the pointers are fake).
    assert mea.NOALLOC_SCRATCH_BYTES == 32 << 20
    f = L.attn_bwd_noalloc

    def call(dt=BF16, B=1, H=1, n=128, d=64, ptrs=None):
        p = dict(zip(("q", "k", "v", "o", "do", "m", "l", "dq", "dk", "dv"), [A] * 10))
        p.update(ptrs or {})
        return f(dt, B, H, n, d, *p.values(), None)

    assert call(dt=2) == UNSUP
    assert call(d=96) == UNSUP
    assert call(n=-1) == SHAPE
    for name in ("q", "k", "v", "o", "do", "m", "l", "dq", "dk", "dv"):
        assert call(ptrs={name: 0}) == NULL, name
        assert call(ptrs={name: A + 4}) == ALIGN, name
    rows = mea.NOALLOC_SCRATCH_BYTES // 8
    assert call(n=rows + 1) == WS
    assert call(H=2, n=rows // 2 + 1) == WS
    assert call(dt=F32, n=rows // 2 + 1) == WS
    # at the limit the size passes; these outputs overlap the inputs
    assert call(n=rows) == ALIAS
    assert call(dt=F32, n=rows // 2) == ALIAS
    assert call(B=0, ptrs={"q": 0}) == OK


# distinct fake buffers 1 MiB apart (every tensor below is far smaller)
Q, K, V, O, M, LS, DO, DQ, DK, DV, W = (A + (i << 20) for i in range(11))


def test_outputs_must_not_overlap(L):
    # n = 128, d = 64, bf16: q-side tensors 16 KiB, statistics 512 B, workspace 1 KiB.
    # Every call below stops at the overlap check (a passing call would launch).
    qb = 128 * 64 * 2
    f = lambda **kw: fwd(L, **dict(dict(q=Q, k=K, v=V, o=O, m=M, l=LS), **kw))
    assert f(o=Q) == ALIAS                      # in place
    assert f(o=Q + qb - 16) == ALIAS            # last 16 bytes shared
    assert f(o=V - qb + 16) == ALIAS
    assert f(m=O + qb - 16) == ALIAS            # statistics inside the output
    assert f(l=M) == ALIAS
    assert f(l=M + 512 - 16) == ALIAS
    b = lambda ws=W, **kw: bwd(L, ws=ws, wsb=1 << 20, ptrs=dict(
        dict(q=Q, k=K, v=V, o=O, do=DO, m=M, l=LS, dq=DQ, dk=DK, dv=DV), **kw))
    assert b(dq=Q) == ALIAS
    assert b(dq=DO) == ALIAS
    assert b(dk=DV) == ALIAS
    assert b(dv=K + qb - 16) == ALIAS
    assert b(ws=DQ + qb - 16) == ALIAS          # the workspace is written too
    assert b(ws=LS) == ALIAS
    assert b(dk=M) == ALIAS
    # without query rows only dk, dv and the key side remain
    assert bwd_ex(L, n_q=0, ws=0, wsb=0, ptrs=dict(q=0, o=0, do=0, m=0, l=0, dq=0,
                                                   k=K, v=V, dk=K, dv=DV)) == ALIAS
    # the split backward of a small grid writes its whole layout, but only when the
    # workspace holds it: one head of 1024 rows, buffers 16 MiB apart
    bq, bk, bv, bo, bd, bm, bl, bdq, bdk, bdv, bw = (A + (i << 24) for i in range(11))
    full = mea.attn_bwd_workspace_bytes(BF16, 1, 1, 1024, 64)
    assert full > 8 * 1024
    sb = lambda wsb, **kw: bwd(L, n=1024, ws=bw, wsb=wsb, ptrs=dict(
        dict(q=bq, k=bk, v=bv, o=bo, do=bd, m=bm, l=bl, dq=bdq, dk=bdk, dv=bdv), **kw))
    assert sb(full, dq=bw + full - 16) == ALIAS      # the partials are written too
    assert sb(full, dk=bw + 8 * 1024) == ALIAS
    assert sb(8 * 1024, dq=bw + 8 * 1024 - 16) == ALIAS
    # split-key: 16384 keys make K and V 2 MiB each, so these buffers sit 16 MiB apart
    sq, sk, sv, so, sm, sl, sw = (A + (i << 24) for i in range(7))
    need = mea.attn_fwd_splitkv_workspace_bytes(BF16, 1, 1, 1, 1, 16384, 64, 0)
    sp = lambda **kw: split(L, **dict(dict(q=sq, k=sk, v=sv, o=so, m=sm, l=sl, ws=sw, wsb=need), **kw))
    assert sp(ws=so) == ALIAS
    assert sp(ws=sl - need + 16) == ALIAS
    assert sp(ws=sk + (2 << 20) - 16) == ALIAS
    assert sp(o=sv + (2 << 20) - 16) == ALIAS


def test_workspace_bytes(L):
    assert mea.attn_bwd_workspace_bytes(BF16, 2, 8, 8192, 64) == 8 * 2 * 8 * 8192
    assert mea.attn_bwd_workspace_bytes(F32, 2, 8, 8192, 128) == 16 * 2 * 8 * 8192
    assert mea.attn_bwd_workspace_bytes(BF16, 0, 8, 8192, 64) == 0
    assert mea.attn_bwd_workspace_bytes(BF16, 1, 1, 5, 96) == 0
    assert mea.attn_bwd_workspace_bytes(BF16, -1, 1, 5, 64) == 0


def test_split_backward_workspace_bytes(L):
    # Grids of at most 256 unsplit workgroups: the row terms, then from a 256-byte
    # boundary the split's fp32 partials of dK and of dV ([ranges][B*H_kv*n_k][d]
    # each) and of dQ ([ranges][B*H*n_q][d]); ranges = min(16, 512 // workgroups),
    # each of at least two staged tiles.
    ws = mea.attn_bwd_workspace_bytes
    # bf16 d = 64: 128 rows per workgroup, 64-row tiles; one head of 1024 is 8 + 8
    # workgroups and 16 tiles a side: 8 ranges of 2 tiles
    assert ws(BF16, 1, 1, 1024, 64) == 8 * 1024 + 3 * 8 * 1024 * 64 * 4
    # fp32 d = 64: 64 rows per workgroup, 32-row tiles: 16 + 16 workgroups, 16 ranges
    assert ws(F32, 1, 1, 1024, 64) == 16 * 1024 + 3 * 16 * 1024 * 64 * 4
    # 16 heads: 256 workgroups, two ranges of 8 tiles; 32 heads (512) are not split
    assert ws(BF16, 1, 16, 1024, 64) == 8 * 16 * 1024 + 3 * 2 * 16 * 1024 * 64 * 4
    assert ws(BF16, 1, 32, 1024, 64) == 8 * 32 * 1024
    # bf16 d = 128: 64 rows per workgroup and per tile. The dK/dV workgroups sweep the
    # stacked query rows of a group (4 x 300 = 1200), so their ranges cut the query
    # tiles; the dQ workgroups sweep the keys, so theirs cut the key tiles.
    exb = mea.attn_bwd_ex_workspace_bytes
    k_tiles, q_tiles = 1000 // 64 + 1, 1200 // 64 + 1       # 16 and 19
    wgs = 1 * (k_tiles + q_tiles)                            # 35 workgroups of 64 rows
    r = min(16, 512 // wgs)                                  # 14
    len_q, len_k = max(2, -(-q_tiles // r)), max(2, -(-k_tiles // r))
    kv, q = -(-q_tiles // len_q), -(-k_tiles // len_k)       # 10 and 8
    rows = 8 * 1200
    off = -(-rows // 256) * 256
    assert exb(BF16, 1, 4, 1, 300, 1000, 128) == off + 2 * kv * 1000 * 128 * 4 + q * 1200 * 128 * 4
    # at most 32 MiB of partials whatever the small shape
    for dt, d in ((BF16, 64), (BF16, 128), (F32, 64), (F32, 128)):
        for n in (64, 300, 1024, 4096, 8192, 20000):
            for H in (1, 2, 3, 8):
                assert ws(dt, 1, H, n, d) - (8 if dt == BF16 else 16) * H * n <= 32 << 20 + 256


def test_binding_rejects_cpu_and_mismatched_tensors():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mea.attn_fwd(q, q, q)
    with pytest.raises(ValueError):
        mea.attn_fwd(q.float(), q.float(), q.float()[..., :32])
    with pytest.raises(ValueError):
        mea.attn_fwd(q.half(), q.half(), q.half())


def test_product_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "memory_efficient_exact_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"\boracle\b", text), f"{f} mentions the oracle"
    assert not re.search(r"\boracle\b", open(HEADER).read())


# ------------------------------------------------------------- _ex entry points

def fwd_ex(L, dt=BF16, B=1, H=4, H_kv=2, n_q=16, n_k=128, d=64, q=A, k=A, v=A, o=A, m=0, l=0):
    return L.attn_fwd_ex(dt, B, H, H_kv, n_q, n_k, d, q, k, v, o, m, l, None)


def bwd_ex(L, dt=BF16, B=1, H=4, H_kv=2, n_q=16, n_k=128, d=64, ptrs=None, ws=A, wsb=1 << 20):
    p = dict(q=A, k=A, v=A, o=A, do=A, m=A, l=A, dq=A, dk=A, dv=A)
    p.update(ptrs or {})
    return L.attn_bwd_ex(dt, B, H, H_kv, n_q, n_k, d, p["q"], p["k"], p["v"], p["o"], p["do"],
                         p["m"], p["l"], p["dq"], p["dk"], p["dv"], ws, wsb, None)


def test_fwd_ex_validation(L):
    assert fwd_ex(L, dt=3) == UNSUP
    assert fwd_ex(L, H_kv=3) == SHAPE          # 4 query heads cannot form 3 groups
    assert fwd_ex(L, H_kv=0) == SHAPE
    assert fwd_ex(L, H_kv=-2) == SHAPE
    assert fwd_ex(L, n_q=-1) == SHAPE
    assert fwd_ex(L, n_k=-1) == SHAPE
    assert fwd_ex(L, n_k=(1 << 24) + 1) == SHAPE
    assert fwd_ex(L, H=8, H_kv=1, n_q=(1 << 22)) == SHAPE   # G * n_q rows > 2^24
    # B*H_kv * ceil(max(G*n_q, n_k) / 64) > 2^22
    assert fwd_ex(L, B=1 << 19, H=8, H_kv=8, n_q=65, n_k=64) == SHAPE
    assert fwd_ex(L, B=1 << 19, H=8, H_kv=8, n_q=64, n_k=65) == SHAPE
    assert fwd_ex(L, n_k=0) == SHAPE           # queries but no keys
    assert fwd_ex(L, d=80) == UNSUP
    assert fwd_ex(L, k=0) == NULL
    assert fwd_ex(L, m=A) == NULL
    assert fwd_ex(L, o=A + 4) == ALIGN
    # no query rows: nothing to do, pointers may be NULL
    assert fwd_ex(L, n_q=0, n_k=0, q=0, k=0, v=0, o=0) == OK
    assert fwd_ex(L, n_q=0, q=0, k=0, v=0, o=0) == OK
    assert fwd_ex(L, B=0, q=0, k=0, v=0, o=0) == OK
    assert fwd_ex(L, H=0, H_kv=0, q=0, k=0, v=0, o=0) == OK


def test_bwd_ex_validation(L):
    assert bwd_ex(L, dt=5) == UNSUP
    assert bwd_ex(L, dt=F32, wsb=16 * 4 * 16 - 1) == WS
    assert bwd_ex(L, H_kv=3) == SHAPE
    assert bwd_ex(L, n_k=0) == SHAPE
    for name in ("q", "k", "v", "o", "do", "m", "l", "dq", "dk", "dv"):
        assert bwd_ex(L, ptrs={name: 0}) == NULL, name
        assert bwd_ex(L, ptrs={name: A + 2}) == ALIGN, name
    need = 8 * 1 * 4 * 16  # 8 bytes per query row of every query head
    assert mea.attn_bwd_ex_workspace_bytes(BF16, 1, 4, 2, 16, 128, 64) == need
    assert bwd_ex(L, wsb=need - 1) == WS
    assert bwd_ex(L, ws=0) == WS
    assert bwd_ex(L, wsb=need, ws=A + 8) == ALIGN
    assert bwd_ex(L, B=0, ws=0, wsb=0) == OK
    assert bwd_ex(L, n_q=0, n_k=0, ws=0, wsb=0) == OK
    # no query rows: only the key side is checked; no workspace needed
    q_side = {nm: 0 for nm in ("q", "o", "do", "m", "l", "dq")}
    assert bwd_ex(L, n_q=0, ptrs=dict(q_side, dk=0), ws=0, wsb=0) == NULL


def test_ex_workspace_bytes(L):
    assert mea.attn_bwd_ex_workspace_bytes(BF16, 2, 32, 8, 100, 7000, 128) == 8 * 2 * 32 * 100
    assert mea.attn_bwd_ex_workspace_bytes(BF16, 2, 32, 5, 100, 7000, 128) == 0
    assert mea.attn_bwd_ex_workspace_bytes(BF16, 2, 32, 8, 0, 0, 128) == 0


# ---------------------------------------------------------- split-key entry point

def split(L, dt=BF16, B=1, H=1, H_kv=1, n_q=1, n_k=16384, d=64, q=A, k=A, v=A, o=A, m=0, l=0,
          s=0, ws=A, wsb=1 << 30):
    return L.attn_fwd_splitkv(dt, B, H, H_kv, n_q, n_k, d, q, k, v, o, m, l, s, ws, wsb, None)


# key tile of the split ranges at one query row per head: both forwards then use their
# decoding layouts (bf16: 128-key tiles, fp32: 64-key tiles)
@pytest.mark.parametrize("dt,d,tile", [(BF16, 64, 128), (BF16, 128, 128), (F32, 64, 64), (F32, 128, 64)])
def test_split_planning(L, dt, d, tile):
    ns = mea.attn_fwd_splitkv_num_splits
    wsb = mea.attn_fwd_splitkv_workspace_bytes
    # explicit requests: honoured up to one range per key tile and 256 ranges
    assert ns(dt, 1, 1, 1, 1, 4096, d, 1) == 1
    assert ns(dt, 1, 1, 1, 1, 4096, d, 4) == 4
    assert ns(dt, 1, 1, 1, 1, 4096, d, 10 ** 6) == min(256, 4096 // tile)
    assert ns(dt, 1, 1, 1, 1, tile, d, 8) == 1          # one key tile: one range
    assert ns(dt, 1, 1, 1, 1, 3 * tile + 1, d, 3) == 2  # ranges of whole tiles, none empty
    # automatic choice: a single query against many keys is split; a full grid is not
    assert ns(dt, 1, 1, 1, 1, 1 << 16, d, 0) > 1
    assert ns(dt, 64, 64, 64, 4096, 4096, d, 0) == 1
    # workspace: splits * rows * (d + 4) * 4 bytes, 0 when unsplit
    s = ns(dt, 2, 8, 2, 5, 4096, d, 4)
    assert s == 4 and wsb(dt, 2, 8, 2, 5, 4096, d, 4) == 4 * 2 * 8 * 5 * (d + 4) * 4
    assert wsb(dt, 2, 8, 2, 5, 4096, d, 1) == 0
    assert ns(dt, 1, 1, 1, 1, 4096, d, -1) == 0
    assert wsb(dt, 1, 1, 1, 1, 4096, d, -1) == 0
    assert ns(dt, 1, 3, 2, 1, 4096, d, 0) == 0           # invalid grouping


def test_split_planning_full_tiles(L):
    # more than 64 (bf16) or 32 (fp32) query rows per head on grids of more than 128
    # row-tiled 4-wave workgroups: the regular layouts (bf16 d = 128 uses 64-key tiles,
    # fp32 32-key tiles)
    ns = mea.attn_fwd_splitkv_num_splits
    big = 10 ** 6
    assert ns(BF16, 1, 64, 64, 4096, 4096, 128, big) == 4096 // 64
    assert ns(BF16, 1, 64, 64, 4096, 4096, 64, big) == 4096 // 128
    assert ns(BF16, 1, 256, 256, 65, 4096, 128, big) == 4096 // 64
    assert ns(BF16, 1, 256, 256, 64, 4096, 128, big) == 4096 // 128  # still decoding
    assert ns(F32, 1, 64, 64, 4096, 4096, 128, big) == 4096 // 32
    assert ns(F32, 1, 256, 256, 33, 4096, 64, big) == 4096 // 32
    assert ns(F32, 1, 256, 256, 32, 4096, 64, big) == 4096 // 64     # fp32 decoding
    # grids of at most 128 row-tiled workgroups take the decoding layouts at any row count
    assert ns(BF16, 1, 1, 1, 4096, 4096, 128, big) == 4096 // 128
    assert ns(BF16, 1, 64, 64, 256, 4096, 128, big) == 4096 // 128   # 128 workgroups
    assert ns(BF16, 1, 65, 65, 256, 4096, 128, big) == 4096 // 64    # 130
    assert ns(F32, 1, 1, 1, 4096, 4096, 64, big) == 4096 // 64
    assert ns(F32, 1, 64, 64, 128, 4096, 64, big) == 4096 // 64      # 128 workgroups
    assert ns(F32, 1, 65, 65, 128, 4096, 64, big) == 4096 // 32      # 130


def test_split_validation(L):
    need = mea.attn_fwd_splitkv_workspace_bytes(BF16, 1, 1, 1, 1, 16384, 64, 0)
    assert need > 0
    assert split(L, wsb=need - 1) == WS
    assert split(L, ws=0) == WS
    assert split(L, ws=A + 4, wsb=need) == ALIGN
    assert split(L, s=-1) == SHAPE
    assert split(L, H=3, H_kv=2) == SHAPE
    assert split(L, n_k=0) == SHAPE
    assert split(L, dt=7) == UNSUP
    assert split(L, q=0) == NULL
    assert split(L, m=A) == NULL
    # empty problems: OK without touching anything
    assert split(L, n_q=0, q=0, k=0, v=0, o=0, ws=0, wsb=0) == OK
    # one range needs no workspace
    assert split(L, n_k=100, s=1, ws=0, wsb=0, q=0) == NULL  # pointer checks still run


def test_binding_rejects_bad_group_shapes():
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 9, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mea.attn_fwd_ex(q, k, k)  # CPU tensors
    with pytest.raises(ValueError):
        mea.attn_fwd_splitkv(q, k, k[..., :32])


C_PROGRAM = r"""
#include <stdio.h>
#include "mea.h"
int main(void) {
  char buf[16] __attribute__((aligned(16)));
  void* p = buf;
  /* validation paths only: no call below reaches a kernel launch */
  if (mea_version() != 400) return 1;
  if (attn_fwd(MEA_DTYPE_BF16, 1, 1, 8, 96, p, p, p, p, NULL, NULL, NULL) != MEA_ERR_UNSUPPORTED) return 2;
  if (attn_fwd_ex(MEA_DTYPE_F32, 1, 4, 3, 8, 8, 64, p, p, p, p, NULL, NULL, NULL) != MEA_ERR_SHAPE) return 3;
  if (attn_bwd(MEA_DTYPE_BF16, 0, 1, 8, 64, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
               NULL, NULL, 0, NULL) != MEA_OK) return 4;
  if (attn_bwd_workspace_bytes(MEA_DTYPE_F32, 2, 8, 8192, 128) != (size_t)16 * 2 * 8 * 8192) return 5;
  if (attn_bwd_workspace_bytes(MEA_DTYPE_F32, 2, 8, 100, 128) <= (size_t)16 * 2 * 8 * 100) return 7;
  if (attn_fwd_splitkv_num_splits(MEA_DTYPE_BF16, 1, 32, 8, 1, 16384, 128, 0) < 2) return 6;
  printf("%s\n", attn_status_str(MEA_ERR_WORKSPACE));
  return 0;
}
"""


def test_header_compiles_as_c99_and_links(tmp_path):
    src = tmp_path / "abi.c"
    exe = tmp_path / "abi"
    src.write_text(C_PROGRAM)
    libdir = os.path.dirname(mea.library_path())
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), "-L", libdir, "-lmea", f"-Wl,-rpath,{libdir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert r.stdout.strip() == "MEA_ERR_WORKSPACE"
