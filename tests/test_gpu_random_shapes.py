"""Seeded random sweep of shapes against the fp64 oracle, through the C ABI.

The hand-picked parity cases pin each feature on its own. This sweep mixes
them: dtype, head dimension, batch, grouped heads, ragged query and key
lengths on both sides of every tile size, explicit and automatic split
counts, and head counts large enough to take the 8-wave layouts. The list is
drawn once from a fixed seed, so every run checks the same cases, and each
case names its parameters. The tolerances are those of test_gpu_parity.py.
"""

import random

import pytest
import torch

import inputgen
import memory_efficient_exact_amd as mea
import oracle

from test_gpu_parity import check, check_relative, check_stats, f64, gpu, say

pytestmark = pytest.mark.gpu


def _cases(count=96, seed=20261203):
    rng = random.Random(seed)
    lengths = [1, 2, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 255, 256, 257, 300, 511,
               513, 700]
    out = []
    i = 0
    while len(out) < count:
        i += 1
        dtype = rng.choice(["bf16", "bf16", "fp32"])
        d = rng.choice([64, 128])
        B = rng.choice([1, 2, 3])
        H_kv = rng.choice([1, 2, 3, 4])
        G = rng.choice([1, 1, 2, 4])
        n_q, n_k = rng.choice(lengths), rng.choice(lengths)
        mode = rng.choice(["fwd", "bwd", "split"])
        if i % 6 == 5 and dtype == "bf16":
            # enough heads that the grid takes the 8-wave layouts
            H_kv, G, B = rng.choice([64, 128]), 1, 2
            n_q = rng.choice([257, 300, 513])
            n_k = rng.choice([65, 257, 300])
        splits = rng.choice([0, 2, 3, 5]) if mode == "split" else None
        case = (dtype, d, B, H_kv * G, H_kv, n_q, n_k, mode, splits)
        if case not in out:
            out.append(case)
    return out


CASES = _cases()


@pytest.mark.parametrize("dtype,d,B,H,H_kv,n_q,n_k,mode,splits", CASES)
def test_random_shape(dtype, d, B, H, H_kv, n_q, n_k, mode, splits):
    say("random", dtype, d, B, H, H_kv, n_q, n_k, mode, splits)
    t = inputgen.draw_gqa(B, H, H_kv, n_q, n_k, d, dtype, seed=n_q * 1000 + n_k + d + H,
                          with_do=mode == "bwd")
    q, k, v = (gpu(t[x]) for x in ("q", "k", "v"))
    if mode == "split":
        o, m, l = mea.attn_fwd_splitkv(q, k, v, num_splits=splits)
    else:
        o, m, l = mea.attn_fwd_ex(q, k, v)
    if mode == "bwd":
        do = gpu(t["do"])
        dq, dk, dv = mea.attn_bwd_ex(q, k, v, o, do, m, l)
    torch.cuda.synchronize()
    q64, k64, v64 = f64(t["q"]), f64(t["k"]), f64(t["v"])
    o_ref, m_ref, l_ref = oracle.gqa_fwd(q64, k64, v64)
    check("O", f64(o.cpu()), o_ref, dtype)
    check_stats(m.cpu().numpy(), l.cpu().numpy(), m_ref, l_ref, dtype)
    if mode == "bwd":
        rq, rk, rv = oracle.gqa_bwd(q64, k64, v64, f64(t["do"]))
        chk = check
        if dtype == "bf16" and d == 128 and n_k <= 2:
            # Two keys per head at d = 128: dS = P (dP - D) reaches ~4 and dQ, dK reach
            # 2-4, ten times the workloads' output scale. There the rounding of P and dS
            # to bf16 operands alone costs more than 2e-2: a CPU model of a bf16-operand
            # backward with the exact D misses by the same amount (dQ 0.020-0.027, dK
            # 0.041-0.091 on these three shapes). These cases are held to 2e-2 relative
            # to the tensor's largest reference value, and to the relative L2 gate.
            chk = check_relative
        chk("dQ", f64(dq.cpu()), rq, dtype)
        chk("dK", f64(dk.cpu()), rk, dtype)
        chk("dV", f64(dv.cpu()), rv, dtype)


def _large_cases(count=16, seed=4242):
    # thousands of rows per head: the row-tiled, 8-wave and decoding layouts, split keys
    # and the split backward all appear, with ragged lengths on both sides
    rng = random.Random(seed)
    out = []
    while len(out) < count:
        dtype = rng.choice(["bf16", "bf16", "fp32"])
        d = rng.choice([64, 128])
        B = rng.choice([1, 2])
        H_kv = rng.choice([1, 2, 4, 8])
        G = rng.choice([1, 2, 4])
        n_q = rng.choice([511, 1000, 1537, 2048, 3001])
        n_k = rng.choice([129, 1000, 2048, 3999])
        mode = rng.choice(["fwd", "bwd", "split"])
        case = (dtype, d, B, H_kv * G, H_kv, n_q, n_k, mode, 0 if mode == "split" else None)
        if case not in out:
            out.append(case)
    return out


LARGE_CASES = _large_cases()


@pytest.mark.parametrize("dtype,d,B,H,H_kv,n_q,n_k,mode,splits", LARGE_CASES)
def test_random_large_shape(dtype, d, B, H, H_kv, n_q, n_k, mode, splits):
    test_random_shape(dtype, d, B, H, H_kv, n_q, n_k, mode, splits)

