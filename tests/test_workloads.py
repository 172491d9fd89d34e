"""Input-generator checks (no GPU, no method arithmetic)."""

import math

import torch

from transformer_attention_diffattn_amd import workloads as W


def test_seeded_and_reproducible():
    a = W.prefill_inputs(1, 2, 33, 16, "bf16", seed=5)
    b = W.prefill_inputs(1, 2, 33, 16, "bf16", seed=5)
    for k in ("q1", "k1", "q2", "k2", "v", "lq1"):
        assert torch.equal(a[k], b[k])
    assert a["v"].shape == (1, 2, 33, 32) and a["q1"].dtype == torch.bfloat16


def test_lambda_init_drawn_in_range():
    w = W.WORKLOADS["layer3b_bf16_b2h12n4096d128"]
    x = W.prefill_inputs(1, 1, 4, w.d, w.dtype, w.seed, lambda_init=None)
    assert 0.2 <= x["lambda_init"] <= 0.8


def test_needle_adds_exact_logit_boost():
    g = torch.Generator().manual_seed(0)
    q = torch.randn(1, 1, 64, 32, generator=g, dtype=torch.float64)
    k = torch.randn(1, 1, 64, 32, generator=g, dtype=torch.float64)
    k0 = k.clone()
    W.plant_needles(q, k, offsets=(7,), boost=3.0)
    i = 40
    delta = (q[0, 0, i] @ (k[0, 0, i - 7] - k0[0, 0, i - 7])) / math.sqrt(32)
    assert abs(delta.item() - 3.0) < 1e-12


def test_workload_table_shapes():
    # the headline prefill is the largest one that fits a GPU: the 64K context
    w = W.WORKLOADS[W.HEADLINE_PREFILL]
    assert (w.B, w.H, w.N, w.d, w.dtype) == (1, 12, 65536, 128, "bf16")
    assert w.pairs() == 65536 * 65537 // 2
    big = max((v for v in W.WORKLOADS.values() if v.kind == "prefill"), key=lambda v: v.pairs() * v.B * v.H * v.d)
    assert big.name == W.HEADLINE_PREFILL
    w = W.WORKLOADS[W.PREFILL_SUBLEGS[0]]
    assert (w.B, w.H, w.N, w.d, w.dtype) == (4, 16, 2048, 64, "bf16")
    assert w.pairs() == 2048 * 2049 // 2
    assert set(W.PREFILL_TRAFFIC) == {W.HEADLINE_PREFILL, *W.PREFILL_SUBLEGS}
    x = W.workload_inputs("tiny_fp32_b1h1n128d16")
    assert x["q1"].dtype == torch.float32 and x["v"].shape == (1, 1, 128, 32)
