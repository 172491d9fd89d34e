"""Seeded synthetic inputs for the differential-attention forward.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  It is the one piece that both the HIP path's callers and
the oracle's tests share: the same seeded tensors go to both sides.

The workloads stand in for the pages' evaluations (language modelling at
1.4B/3B scale, 64K-token long context with needle retrieval, KV-cache
decoding) with synthetic data of the same shapes: every value is a seeded
normal draw, so no dataset is needed.  Draw order for every workload is
lambda_q1, lambda_k1, lambda_q2, lambda_k2, (lambda_init if drawn), Q1, K1,
Q2, K2, V.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """One named workload: shapes, dtype and the recipe of its values."""

    name: str
    kind: str  # "prefill" or "decode"
    dtype: str  # "fp32" or "bf16"
    B: int
    H: int
    N: int  # prefill: sequence length; decode: cached keys per sequence (L)
    d: int  # per-map query/key width; the value width is 2d
    seed: int
    causal: bool = True
    lambda_init: float | None = 0.8  # None: drawn once, uniform in lambda_init_range
    lambda_init_range: tuple = (0.2, 0.8)
    lam_std: float = 0.1
    needle_offsets: tuple = field(default_factory=tuple)
    needle_boost: float = 0.0
    eps: float = 1e-5

    def pairs(self) -> int:
        """(query, key) pairs that take part, per head."""
        if self.kind == "decode":
            return self.N
        return self.N * (self.N + 1) // 2 if self.causal else self.N * self.N


WORKLOADS = {
    w.name: w
    for w in (
        # oracle-scale case: fp32, one head of 128 tokens, d = 16
        Workload("tiny_fp32_b1h1n128d16", "prefill", "fp32", 1, 1, 128, 16, seed=20261),
        # one attention layer of a 1.4B-scale model: d_model 2048 = 16 heads x 2d
        Workload("layer1p4b_bf16_b4h16n2048d64", "prefill", "bf16", 4, 16, 2048, 64, seed=20262),
        # one layer of a 3B-scale model: d_model 3072 = 12 heads x 2d
        Workload("layer3b_bf16_b2h12n4096d128", "prefill", "bf16", 2, 12, 4096, 128, seed=20263,
                 lambda_init=None),
        # 64K-token prefill with a sparse signal: each query row gets up to four keys
        # whose map-1 logit is raised by +3 over an N(0,1) noise floor
        Workload("longctx_bf16_b1h12n65536d128", "prefill", "bf16", 1, 12, 65536, 128, seed=20264,
                 needle_offsets=(7, 311, 5003, 40009), needle_boost=3.0),
        # one decode step: 64 sequences, one new token each, 32768 cached keys
        Workload("decode_bf16_b64h16l32768d128", "decode", "bf16", 64, 16, 32768, 128, seed=20265),
    )
}

# the headline prefill workload: the largest prefill that fits one GPU (the
# 64K-token context); the two model-layer prefills are reported beside it
HEADLINE_PREFILL = "longctx_bf16_b1h12n65536d128"
PREFILL_SUBLEGS = ("layer1p4b_bf16_b4h16n2048d64", "layer3b_bf16_b2h12n4096d128")
HEADLINE_DECODE = "decode_bf16_b64h16l32768d128"
# traffic summaries under profiles/ per prefill workload (prefill.hip counters)
PREFILL_TRAFFIC = {"longctx_bf16_b1h12n65536d128": "prefill_longctx", "layer1p4b_bf16_b4h16n2048d64":
                   "prefill_layer1p4b", "layer3b_bf16_b2h12n4096d128": "prefill_layer3b"}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _lambda_params(g, d, lam_std, lambda_init, lo_hi, device):
    vecs = [torch.randn(d, generator=g, device=device, dtype=torch.float32) * lam_std for _ in range(4)]
    if lambda_init is None:
        u = torch.rand(1, generator=g, device=device, dtype=torch.float32).item()
        lambda_init = lo_hi[0] + (lo_hi[1] - lo_hi[0]) * u
    return vecs, float(lambda_init)


def plant_needles(q1: torch.Tensor, k1: torch.Tensor, offsets, boost: float) -> None:
    """Raise selected map-1 logits by exactly ``boost`` (in place, fp32).

    For each offset o and query i >= o, key i - o gets boost*sqrt(d)/|q_i|^2
    times q_i added, so q_i . k_{i-o} / sqrt(d) grows by exactly ``boost``.
    Cross terms on other rows are ~N(0, boost^2/d).  Input construction only.
    """
    d = q1.shape[-1]
    n = q1.shape[-2]
    coef = (boost * math.sqrt(d)) / (q1 * q1).sum(-1, keepdim=True)
    for o in offsets:
        if o < n:
            k1[..., : n - o, :] += coef[..., o:, :] * q1[..., o:, :]


def prefill_inputs(B, H, N, d, dtype="bf16", seed=0, *, lambda_init=0.8, lam_std=0.1,
                   lambda_init_range=(0.2, 0.8), needle_offsets=(), needle_boost=0.0,
                   qk_scale=1.0, device="cpu", eps=1e-5):
    """Seeded prefill inputs.  Values are drawn in fp32 on ``device`` and
    rounded (RNE) to ``dtype``.  Returns a dict of tensors and scalars."""
    g = _gen(seed, device)
    (lq1, lk1, lq2, lk2), lambda_init = _lambda_params(g, d, lam_std, lambda_init, lambda_init_range, device)
    shp = (B, H, N, d)
    q1 = torch.randn(shp, generator=g, device=device) * qk_scale
    k1 = torch.randn(shp, generator=g, device=device) * qk_scale
    q2 = torch.randn(shp, generator=g, device=device) * qk_scale
    k2 = torch.randn(shp, generator=g, device=device) * qk_scale
    v = torch.randn((B, H, N, 2 * d), generator=g, device=device)
    if needle_offsets:
        plant_needles(q1, k1, needle_offsets, needle_boost)
    dt = DTYPES[dtype]
    return dict(
        lq1=lq1, lk1=lk1, lq2=lq2, lk2=lk2, lambda_init=lambda_init,
        q1=q1.to(dt).contiguous(), k1=k1.to(dt).contiguous(), q2=q2.to(dt).contiguous(),
        k2=k2.to(dt).contiguous(), v=v.to(dt).contiguous(),
        weight=torch.ones(2 * d, device=device, dtype=torch.float32), eps=eps,
    )


def projection_inputs(B, N, d_model, H, d, seed=0, *, d_out=None, device="cpu"):
    """Seeded inputs of the projections either side of the attention (bf16):
    x [B, N, d_model] ~ N(0, 1); w_qkv [3*H*2d, d_model] and
    w_o [d_out, H*2d] ~ N(0, 1/fan_in) (fan-in scaled, as a linear layer's
    initialisation); o [B, H, N, 2d] ~ N(0, 1) stands in for the attention
    output."""
    g = _gen(seed, device)
    width = H * 2 * d
    d_out = d_model if d_out is None else d_out
    x = torch.randn((B, N, d_model), generator=g, device=device)
    w_qkv = torch.randn((3 * width, d_model), generator=g, device=device) / math.sqrt(d_model)
    w_o = torch.randn((d_out, width), generator=g, device=device) / math.sqrt(width)
    o = torch.randn((B, H, N, 2 * d), generator=g, device=device)
    bf = torch.bfloat16
    return dict(x=x.to(bf).contiguous(), w_qkv=w_qkv.to(bf).contiguous(), w_o=w_o.to(bf).contiguous(),
                o=o.to(bf).contiguous())


def decode_inputs(B, H, L, d, dtype="bf16", seed=0, *, lambda_init=0.8, lam_std=0.1,
                  cache_len=None, device="cpu", eps=1e-5):
    """Seeded decode inputs: one query token per sequence and a KV cache of
    L_max = L keys.  ``cache_len``: None (all L), or a list of B ints.
    Large caches are drawn directly in ``dtype`` on ``device``."""
    g = _gen(seed, device)
    (lq1, lk1, lq2, lk2), lambda_init = _lambda_params(g, d, lam_std, lambda_init, (0.2, 0.8), device)
    dt = DTYPES[dtype]
    q1 = torch.randn((B, H, 1, d), generator=g, device=device).to(dt)
    k1c = torch.randn((B, H, L, d), generator=g, device=device, dtype=dt)
    q2 = torch.randn((B, H, 1, d), generator=g, device=device).to(dt)
    k2c = torch.randn((B, H, L, d), generator=g, device=device, dtype=dt)
    vc = torch.randn((B, H, L, 2 * d), generator=g, device=device, dtype=dt)
    lens = [L] * B if cache_len is None else list(cache_len)
    return dict(
        lq1=lq1, lk1=lk1, lq2=lq2, lk2=lk2, lambda_init=lambda_init,
        q1=q1.contiguous(), q2=q2.contiguous(), k1c=k1c, k2c=k2c, vc=vc,
        cache_len=torch.tensor(lens, dtype=torch.int32, device=device),
        weight=torch.ones(2 * d, device=device, dtype=torch.float32), eps=eps,
    )


def workload_inputs(name: str, device="cpu"):
    """Inputs of a named workload (see ``WORKLOADS``)."""
    w = WORKLOADS[name]
    if w.kind == "decode":
        return decode_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, lambda_init=w.lambda_init,
                             lam_std=w.lam_std, device=device, eps=w.eps)
    return prefill_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, lambda_init=w.lambda_init,
                          lam_std=w.lam_std, lambda_init_range=w.lambda_init_range,
                          needle_offsets=w.needle_offsets, needle_boost=w.needle_boost,
                          device=device, eps=w.eps)
