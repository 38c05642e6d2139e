"""The seeded generator: determinism, rounding recipe and workload structure."""

import numpy as np
import torch

import inputgen


def test_same_seed_same_bytes():
    a = inputgen.draw(2, 3, 17, 64, "bf16", seed=5, with_do=True)
    b = inputgen.draw(2, 3, 17, 64, "bf16", seed=5, with_do=True)
    for k in ("q", "k", "v", "do"):
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16))


def test_different_seed_differs_and_do_is_drawn_last():
    a = inputgen.draw(1, 2, 33, 64, "fp32", seed=1)
    b = inputgen.draw(1, 2, 33, 64, "fp32", seed=2)
    assert not torch.equal(a["q"], b["q"])
    c = inputgen.draw(1, 2, 33, 64, "fp32", seed=1, with_do=True)
    for k in ("q", "k", "v"):
        assert torch.equal(a[k], c[k])


def test_rounding_recipe():
    rng = np.random.default_rng(9)
    ref = rng.standard_normal(4 * 512)[:512].reshape(1, 1, 8, 64).astype(np.float32)
    t = inputgen.draw(1, 1, 8, 64, "fp32", seed=9)
    assert np.array_equal(t["q"].numpy(), ref)
    tb = inputgen.draw(1, 1, 8, 64, "bf16", seed=9)
    assert torch.equal(tb["q"], torch.from_numpy(ref).to(torch.bfloat16))
    assert tb["q"].dtype == torch.bfloat16 and tb["q"].is_contiguous()


def test_stress_structure():
    w = inputgen.WORKLOADS["c4_stress_fp32"]
    t = inputgen.draw(2, 3, 40, 128, "fp32", seed=w.seed, qk_scale=w.qk_scale,
                      equal_key_heads=w.equal_key_heads)
    k = t["k"]
    assert torch.equal(k[:, 0], k[:, 0, :1].expand_as(k[:, 0]))
    assert not torch.equal(k[:, 1], k[:, 1, :1].expand_as(k[:, 1]))
    raw = (t["q"][0, 1].double() @ t["k"][0, 1].double().T).abs().max().item()
    assert raw > 3e3


def test_workload_table():
    w = inputgen.WORKLOADS
    assert (w["c3_long_bf16"].B, w["c3_long_bf16"].H, w["c3_long_bf16"].n, w["c3_long_bf16"].d) == (1, 16, 16384, 64)
    assert w["c3_long_bf16"].fwd_flops() == 4.0 * 16 * 16384 ** 2 * 64
    assert w["c5_train_bf16"].backward and w["c5_train_bf16"].bwd_flops() == 10.0 * 16 * 8192 ** 2 * 64
    assert w["c1_single_head_fp32"].dtype == "fp32" and w["c4_stress_fp32"].d == 128


def test_draw_gqa_matches_draw_on_equal_shapes():
    a = inputgen.draw(2, 3, 17, 64, "bf16", seed=9, qk_scale=2.0, with_do=True)
    b = inputgen.draw_gqa(2, 3, 3, 17, 17, 64, "bf16", seed=9, qk_scale=2.0, with_do=True)
    for nm in ("q", "k", "v", "do"):
        assert torch.equal(a[nm], b[nm]), nm
    c = inputgen.draw_gqa(1, 4, 2, 5, 9, 64, "fp32", seed=1)
    assert c["q"].shape == (1, 4, 5, 64) and c["k"].shape == (1, 2, 9, 64) and "do" not in c
