"""Seeded synthetic inputs for attention workloads.

This module only draws and rounds random numbers; it holds none of the
attention arithmetic. Both the CPU oracle (through the tests) and the HIP
library consume exactly the tensors it returns, so parity compares like with
like.

Recipe (identical for every workload):

1. ``rng = numpy.random.default_rng(seed)`` (PCG64).
2. Draw ``standard_normal`` float64 arrays of shape [B, H, n, d] in the fixed
   order Q, K, V, dO (dO last, so Q, K, V do not depend on whether dO is used).
3. Optional workload structure, applied in float64:
   * ``qk_scale``: Q and K multiplied by this factor (the stress workload uses
     30, so that raw scores q.k reach about 1e4 at d=128);
   * ``equal_key_heads``: for each listed head h and every batch b, every key
     row K[b, h, j, :] is replaced by K[b, h, 0, :] (all keys identical).
4. Round to float32 (numpy, round-to-nearest-even), then, for bf16 workloads,
   to bfloat16 (torch CPU, round-to-nearest-even).

The pages measure self-attention at sequence lengths up to 16384 and name no
input distribution; i.i.d. N(0, 1) entries are the plain reading.
"""

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n: int
    d: int
    dtype: str  # "fp32" or "bf16"
    backward: bool = False
    qk_scale: float = 1.0
    equal_key_heads: Tuple[int, ...] = field(default_factory=tuple)
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def fwd_flops(self):
        """4 B H n^2 d: two n x n x d contractions (QK^T and PV)."""
        return 4.0 * self.B * self.H * self.n * self.n * self.d

    def bwd_flops(self):
        """10 B H n^2 d: five n x n x d contractions (S recompute, dV, dP, dQ, dK)."""
        return 10.0 * self.B * self.H * self.n * self.n * self.d


# The five workloads. Seeds are ours: workload c uses 1000 + c.
WORKLOADS = {
    "c1_single_head_fp32": Workload("c1_single_head_fp32", 1, 1, 1024, 64, "fp32", seed=1001),
    "c2_multihead_bf16": Workload("c2_multihead_bf16", 4, 8, 4096, 64, "bf16", seed=1002),
    "c3_long_bf16": Workload("c3_long_bf16", 1, 16, 16384, 64, "bf16", seed=1003),
    "c4_stress_fp32": Workload("c4_stress_fp32", 2, 8, 8192, 128, "fp32", qk_scale=30.0,
                               equal_key_heads=(0,), seed=1004),
    "c5_train_bf16": Workload("c5_train_bf16", 2, 8, 8192, 64, "bf16", backward=True, seed=1005),
}


def draw(B, H, n, d, dtype="bf16", seed=0, qk_scale=1.0, equal_key_heads=(), with_do=False):
    """Draw Q, K, V (and dO) per the recipe above.

    Returns a dict of contiguous CPU torch tensors in ``dtype`` ("fp32" or
    "bf16"), keys "q", "k", "v" and, if ``with_do``, "do".
    """
    if dtype not in ("fp32", "bf16"):
        raise ValueError(f"dtype must be 'fp32' or 'bf16', got {dtype!r}")
    rng = np.random.default_rng(seed)
    shape = (B, H, n, d)
    names = ["q", "k", "v", "do"]
    raw = {}
    for nm in names:
        if nm == "do" and not with_do:
            break
        raw[nm] = rng.standard_normal(shape, dtype=np.float64)
    if qk_scale != 1.0:
        raw["q"] = raw["q"] * qk_scale
        raw["k"] = raw["k"] * qk_scale
    for h in equal_key_heads:
        if 0 <= h < H and n > 0:
            raw["k"][:, h, :, :] = raw["k"][:, h, 0:1, :]
    out = {}
    for nm, a in raw.items():
        t = torch.from_numpy(np.ascontiguousarray(a.astype(np.float32)))
        if dtype == "bf16":
            t = t.to(torch.bfloat16)
        out[nm] = t.contiguous()
    return out


def draw_gqa(B, H, H_kv, n_q, n_k, d, dtype="bf16", seed=0, qk_scale=1.0, with_do=False):
    """Like ``draw`` for separate shapes: q (and do) [B, H, n_q, d], k and v
    [B, H_kv, n_k, d]; same generator, same draw order (q, k, v, do), same
    rounding. With H_kv = H and n_q = n_k it returns exactly ``draw``'s tensors.
    """
    if dtype not in ("fp32", "bf16"):
        raise ValueError(f"dtype must be 'fp32' or 'bf16', got {dtype!r}")
    rng = np.random.default_rng(seed)
    shapes = {"q": (B, H, n_q, d), "k": (B, H_kv, n_k, d), "v": (B, H_kv, n_k, d),
              "do": (B, H, n_q, d)}
    raw = {}
    for nm in ("q", "k", "v", "do"):
        if nm == "do" and not with_do:
            break
        raw[nm] = rng.standard_normal(shapes[nm], dtype=np.float64)
    if qk_scale != 1.0:
        raw["q"] = raw["q"] * qk_scale
        raw["k"] = raw["k"] * qk_scale
    out = {}
    for nm, a in raw.items():
        t = torch.from_numpy(np.ascontiguousarray(a.astype(np.float32)))
        if dtype == "bf16":
            t = t.to(torch.bfloat16)
        out[nm] = t.contiguous()
    return out


def make_inputs(w: Workload, seed=None, with_do=None):
    """Inputs for workload ``w`` (seed defaults to the workload's own)."""
    return draw(w.B, w.H, w.n, w.d, w.dtype, w.seed if seed is None else seed,
                w.qk_scale, w.equal_key_heads, w.backward if with_do is None else with_do)


def to_f64(t):
    """Exact upcast of a CPU tensor (bf16 or fp32) to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
