"""Why three bf16 backward shapes of the random sweep take a relative bar.

A bf16 backward multiplies on bf16 MFMA, so the probabilities P (for dV = P^T dO)
and dS = P * (dP - D) (for dQ = dS K / sqrt(d) and dK = dS^T Q / sqrt(d)) are
rounded to bf16 before the products, and the outputs are rounded to bf16. This
file models exactly that on the CPU, with everything else exact (fp64 scores,
the exact row term D from the oracle's own output, fp64 sums), and shows that
on heads with two keys at d = 128 (dS ~ 4, outputs of 2-4) the model alone
misses the 2e-2 absolute bar; the same model stays far inside it on a
workload-like shape. The model is test infrastructure: it shares nothing
with the library and uses the oracle only for the reference gradients.
"""

import math

import numpy as np
import torch

import inputgen
import oracle


def bf16(x):
    """Round to bfloat16 (round-to-nearest-even, torch CPU) and back to fp64."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def bf16_operand_backward(q, k, v, do, G):
    """dQ, dK, dV of grouped-query attention with P and dS rounded to bf16
    operands and bf16 outputs; scores, D and all sums exact (fp64)."""
    B, H, n_q, d = q.shape
    scale = 1.0 / math.sqrt(d)
    o, _, _ = oracle.gqa_fwd(q, k, v)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            hk = h // G
            s = q[b, h] @ k[b, hk].T * scale
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = do[b, h] @ v[b, hk].T
            D = (o[b, h] * do[b, h]).sum(axis=1)  # exact: the oracle's fp64 output
            ds = bf16(p * (dp - D[:, None]))
            dq[b, h] = ds @ k[b, hk] * scale
            dk[b, hk] += ds.T @ q[b, h] * scale
            dv[b, hk] += bf16(p).T @ do[b, h]
    return bf16(dq), bf16(dk), bf16(dv)


def model_errors(B, H, H_kv, n_q, n_k, d, seed):
    t = inputgen.draw_gqa(B, H, H_kv, n_q, n_k, d, "bf16", seed=seed, with_do=True)
    q, k, v, do = (inputgen.to_f64(t[x]) for x in ("q", "k", "v", "do"))
    ref = oracle.gqa_bwd(q, k, v, do)
    got = bf16_operand_backward(q, k, v, do, H // H_kv)
    return [float(np.abs(g - r).max()) for g, r in zip(got, ref)], [float(np.abs(r).max()) for r in ref]


def test_two_key_heads_exceed_the_absolute_bar_in_bf16_operands():
    # the three random-sweep shapes (B, H, H_kv, n_q, n_k, d) with their sweep seeds
    for B, H, H_kv, n_q, n_k, d in ((3, 4, 4, 200, 2, 128), (3, 8, 4, 513, 2, 128),
                                    (2, 16, 4, 64, 2, 128)):
        errs, mags = model_errors(B, H, H_kv, n_q, n_k, d, seed=n_q * 1000 + n_k + d + H)
        # dQ or dK of the model misses 2e-2 although D and every sum are exact ...
        assert max(errs[0], errs[1]) > 2e-2, errs
        # ... while staying within 2e-2 of the tensor's largest value
        for e, m in zip(errs, mags):
            assert m > 1.0 and e <= 2e-2 * m, (errs, mags)


def test_workload_like_heads_stay_far_inside_the_bar():
    # many keys per head (diffuse rows, outputs ~0.1): the same model is ~50x inside 2e-2
    errs, mags = model_errors(1, 2, 2, 256, 2048, 64, seed=11)
    assert max(errs) < 1e-3 and max(mags) < 1.0, (errs, mags)
