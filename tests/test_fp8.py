"""GPU parity of the fp8 (e4m3) query/key path against the oracles.

* diffattn_quantize_fp8 against oracle/fp8_oracle.quantize: codes and scale
  bit-exact (byte work; the scale is one float32 division of an exact max).
* diffattn_fwd_fp8qk against oracle/diffattn_oracle.forward on the
  dequantised inputs (code value * scale, exact in float64): the matrix cores
  sum exact e4m3 products in fp32, so what remains is the bf16 rounding of
  the weights, bounded per element as for the bf16 prefill (2e-2, or the
  propagated rounding where the two maps nearly cancel).
* the whole fp8 path (quantise, then attend) against the unquantised oracle
  at a looser, derived bound: quantising q and k perturbs every logit; the
  perturbation's standard deviation (measured per head from the oracle's own
  quantised and exact logits) joins the bf16 rounding as a relative error of
  each weight, and six standard deviations of its propagation through
  (A1 - lambda A2) V and the norm bound each element.
"""

import numpy as np
import pytest
import torch

from oracle import diffattn_oracle as O
from oracle import fp8_oracle as F
from transformer_attention_diffattn_amd import binding as da
from transformer_attention_diffattn_amd import workloads as W

pytestmark = pytest.mark.gpu

D = 128
U_BF16 = 2.0 ** -9


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _lam_host(x):
    return O.lambda_scalar(x["lq1"], x["lk1"], x["lq2"], x["lk2"], x["lambda_init"])


def _oracle_quant(x):
    """oracle codes and scales of q1, k1, q2, k2 and their dequantised values"""
    codes, scales, deq = {}, [], {}
    for k in ("q1", "k1", "q2", "k2"):
        c, s = F.quantize(x[k].float().numpy())
        codes[k], deq[k] = c, F.dequantize(c, s)
        scales.append(float(s))
    return codes, np.array(scales, np.float32), deq


def _gpu_fp8(codes, scales, x, dev, causal, lam_t=None):
    g = {k: torch.from_numpy(codes[k]).to(dev) for k in codes}
    sc = torch.from_numpy(scales).to(dev)
    if lam_t is None:
        lam_t = da.lam(*(x[k].to(dev) for k in ("lq1", "lk1", "lq2", "lk2")), x["lambda_init"])
    out = da.fwd_fp8qk(g["q1"], g["k1"], g["q2"], g["k2"], sc, x["v"].to(dev), lam_t, x["lambda_init"],
                       eps=x["eps"], causal=causal)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _bound(q1, k1, q2, k2, v, lam, lambda_init, eps, causal, rel_std):
    """6 standard deviations of a relative error rel_std[b, h] of every
    weight, propagated through (A1 - lambda A2) V and the norm, plus the
    output's own bf16 rounding; never below 2e-2."""
    s = 1.0 - lambda_init
    B, H, N, _ = q1.shape
    tol = np.empty((B, H, N, 2 * D))
    for b in range(B):
        for h in range(H):
            a1 = O.attention_map(O._f64(q1[b, h]), O._f64(k1[b, h]), causal)
            a2 = O.attention_map(O._f64(q2[b, h]), O._f64(k2[b, h]), causal)
            vv = O._f64(v[b, h])
            y = (a1 - lam * a2) @ vv
            r = np.sqrt(np.mean(y * y, axis=1, keepdims=True) + eps)
            sig = rel_std[b, h] * np.sqrt((a1 * a1 + lam * lam * a2 * a2) @ (vv * vv))
            tol[b, h] = np.maximum(2e-2, (6.0 * s * sig + U_BF16 * s * np.abs(y)) / r)
    return tol


# ---------------------------------------------------------------------------
# quantiser


@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 4099, 2 * 2 * 77 * D, 65536 * 8 + 5])
def test_quantize_bit_exact(dev, n):
    print(f"case quantize n={n}", flush=True)
    g = torch.Generator().manual_seed(4000 + n)
    x = (torch.randn(n, generator=g) * 1.7).to(torch.bfloat16)
    codes, scale = da.quantize_fp8(x.to(dev))
    ref_c, ref_s = F.quantize(x.float().numpy())
    assert np.array_equal(codes.cpu().numpy(), ref_c)
    assert scale.item() == float(ref_s)


@pytest.mark.parametrize("kind", ["tiny", "huge", "zeros", "mixed", "signed_zero"])
def test_quantize_special_values(dev, kind):
    print(f"case quantize {kind}", flush=True)
    g = torch.Generator().manual_seed(77)
    n = 3000
    if kind == "tiny":  # most values land in e4m3's subnormal range after scaling
        x = torch.randn(n, generator=g) * 1e-3
        x[0] = 1.0
    elif kind == "huge":
        x = torch.randn(n, generator=g) * 3e4
    elif kind == "zeros":
        x = torch.zeros(n)
    elif kind == "mixed":
        x = torch.randn(n, generator=g) * torch.exp2(torch.randint(-20, 10, (n,), generator=g).float())
    else:
        x = torch.zeros(n)
        x[::2] = -0.0
        x[5] = 2.0
    x = x.to(torch.bfloat16)
    codes, scale = da.quantize_fp8(x.to(dev))
    ref_c, ref_s = F.quantize(x.float().numpy())
    assert np.array_equal(codes.cpu().numpy(), ref_c)
    assert scale.item() == float(ref_s)


@pytest.mark.parametrize("count,n", [(1, 1000), (2, 7), (4, 4099), (4, 2 * 12 * 4096 * D)])
def test_quantize_batch_equals_oracle(dev, count, n):
    print(f"case quantize batch count={count} n={n}", flush=True)
    g = torch.Generator().manual_seed(7000 + n + count)
    xs = [(torch.randn(n, generator=g) * (0.5 + t)).to(torch.bfloat16) for t in range(count)]
    codes, scales = da.quantize_fp8_batch([x.to(dev) for x in xs])
    for t in range(count):
        ref_c, ref_s = F.quantize(xs[t].float().numpy())
        assert np.array_equal(codes[t].cpu().numpy(), ref_c), t
        assert scales[t].item() == float(ref_s), t


def test_quantize_full_size_3b_layer(dev):
    # every query/key tensor of the 3B-layer prefill (2 x 12 x 4096 x 128)
    x = W.workload_inputs("layer3b_bf16_b2h12n4096d128", device=dev)
    for k in ("q1", "k1", "q2", "k2"):
        print(f"case quantize layer3b {k}", flush=True)
        codes, scale = da.quantize_fp8(x[k])
        ref_c, ref_s = F.quantize(x[k].float().cpu().numpy())
        assert np.array_equal(codes.cpu().numpy(), ref_c), k
        assert scale.item() == float(ref_s), k


# ---------------------------------------------------------------------------
# attention on e4m3 queries and keys


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N", [1, 15, 33, 64, 65, 200, 257])
def test_fp8qk_matches_oracle_on_dequantised_inputs(dev, causal, N):
    print(f"case fp8qk N={N} causal={causal}", flush=True)
    x = W.prefill_inputs(2, 2, N, D, "bf16", seed=5000 + N)
    codes, scales, deq = _oracle_quant(x)
    lam = _lam_host(x)
    got = _gpu_fp8(codes, scales, x, dev, causal)
    ref = O.forward(deq["q1"], deq["k1"], deq["q2"], deq["k2"], x["v"], lam, x["lambda_init"], eps=x["eps"],
                    causal=causal)
    err = np.abs(got - ref)
    tol = _bound(deq["q1"], deq["k1"], deq["q2"], deq["k2"], x["v"], lam, x["lambda_init"], x["eps"], causal,
                 np.full((2, 2), U_BF16 / np.sqrt(3.0)))
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    print(f"max err {err.max():.3e}; worst vs bound {err[worst]:.3e} / {tol[worst]:.3e}", flush=True)
    assert np.all(err <= tol)


def test_fp8qk_with_norm_weight(dev):
    """A non-unit per-channel norm weight (review page, "Summary", Eq. 3):
    the weight scales each output channel after the norm, so the bound of
    the unweighted output scales by it channel by channel."""
    N, causal = 130, True
    x = W.prefill_inputs(2, 2, N, D, "bf16", seed=5400)
    codes, scales, deq = _oracle_quant(x)
    wt = (0.5 + torch.rand(2 * D, generator=torch.Generator().manual_seed(5401))).float()
    g = {k: torch.from_numpy(codes[k]).to(dev) for k in codes}
    lam_t = da.lam(*(x[k].to(dev) for k in ("lq1", "lk1", "lq2", "lk2")), x["lambda_init"])
    got = da.fwd_fp8qk(g["q1"], g["k1"], g["q2"], g["k2"], torch.from_numpy(scales).to(dev), x["v"].to(dev), lam_t,
                       x["lambda_init"], weight=wt.to(dev), eps=x["eps"], causal=causal).float().cpu().numpy()
    lam = _lam_host(x)
    ref = O.forward(deq["q1"], deq["k1"], deq["q2"], deq["k2"], x["v"], lam, x["lambda_init"], weight=wt.numpy(),
                    eps=x["eps"], causal=causal)
    tol = _bound(deq["q1"], deq["k1"], deq["q2"], deq["k2"], x["v"], lam, x["lambda_init"], x["eps"], causal,
                 np.full((2, 2), U_BF16 / np.sqrt(3.0))) * wt.numpy().astype(np.float64)
    err = np.abs(got - ref)
    print(f"max err {err.max():.3e}", flush=True)
    assert np.all(err <= tol)


def _gpu_fp8_nonorm(codes, scales, v, lam_value, dev, causal):
    g = {k: torch.from_numpy(codes[k]).to(dev) for k in codes}
    lam_t = torch.tensor([lam_value], dtype=torch.float32, device=dev)
    out = da.fwd_fp8qk(g["q1"], g["k1"], g["q2"], g["k2"], torch.from_numpy(scales).to(dev), v.to(dev), lam_t, 0.8,
                       causal=causal, norm=False)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("causal", [True, False])
def test_fp8qk_without_norm(dev, causal):
    # Eq. 1's Y = (A1 - lambda A2) V (the testing hook without the norm), to
    # the bf16 path's 2e-2 on the dequantised inputs
    x = W.prefill_inputs(1, 2, 190, D, "bf16", seed=81)
    codes, scales, deq = _oracle_quant(x)
    got = _gpu_fp8_nonorm(codes, scales, x["v"], 0.6, dev, causal)
    ref = O.forward(deq["q1"], deq["k1"], deq["q2"], deq["k2"], x["v"], 0.6, 0.8, causal=causal, norm=False)
    assert np.max(np.abs(got - ref)) <= 2e-2


@pytest.mark.parametrize("lam_value", [-0.3, 0.5, 1.7])
def test_fp8qk_rows_sum_to_one_minus_lambda(dev, lam_value):
    # V = ones and no norm: every row of Y is 1 - lambda (each map's rows sum to 1)
    x = W.prefill_inputs(1, 2, 130, D, "bf16", seed=82)
    codes, scales, _ = _oracle_quant(x)
    out = _gpu_fp8_nonorm(codes, scales, torch.ones_like(x["v"]), lam_value, dev, True)
    assert np.max(np.abs(out - (1.0 - lam_value))) <= 4e-3


def test_fp8qk_every_row_3b_shape(dev):
    """Every row of the fp8 prefill at the 3B layer's shape is written (768
    items of 128 rows: exactly three rounds of a 256-CU part, whose last three
    take the three-permutation order): the codes come from the library's own
    quantiser (any codes do: with V = ones and no norm every row of Y is
    1 - lambda), and the output starts as NaN."""
    print("case fp8 every-row B=2 H=12 N=4096 d=128", flush=True)
    x = W.prefill_inputs(2, 12, 4096, D, "bf16", seed=84, device=dev)
    xs = [x[k] for k in ("q1", "k1", "q2", "k2")]
    ws = torch.empty(max(4, 4 * da.quantize_fp8_workspace_bytes(xs[0].numel())), dtype=torch.uint8, device=dev)
    codes, scales = da.quantize_fp8_batch(xs, workspace=ws)
    lam = 0.37
    lam_t = torch.tensor([lam], dtype=torch.float32, device=dev)
    v = torch.ones_like(x["v"])
    out = torch.full_like(v, float("nan"))
    da.fwd_fp8qk(codes[0], codes[1], codes[2], codes[3], scales, v, lam_t, 0.8, causal=True, norm=False, out=out)
    torch.cuda.synchronize()
    err = (out.float() - (1.0 - lam)).abs().max().item()
    assert err <= 4e-3, err


@pytest.mark.parametrize("lam_value", [-0.3, 0.0, 1.0])
def test_fp8qk_lambda_values(dev, lam_value):
    x = W.prefill_inputs(1, 3, 150, D, "bf16", seed=51)
    codes, scales, deq = _oracle_quant(x)
    lam_t = torch.tensor([lam_value], dtype=torch.float32, device=dev)
    got = _gpu_fp8(codes, scales, x, dev, True, lam_t=lam_t)
    ref = O.forward(deq["q1"], deq["k1"], deq["q2"], deq["k2"], x["v"], lam_value, x["lambda_init"],
                    eps=x["eps"])
    tol = _bound(deq["q1"], deq["k1"], deq["q2"], deq["k2"], x["v"], lam_value, x["lambda_init"], x["eps"], True,
                 np.full((1, 3), U_BF16 / np.sqrt(3.0)))
    assert np.all(np.abs(got - ref) <= tol)


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_path_end_to_end_against_unquantised_oracle(dev, causal):
    # GPU quantiser + fp8 attention against the oracle on the bf16 inputs
    x = W.prefill_inputs(2, 2, 300, D, "bf16", seed=61)
    g = {k: x[k].to(dev) for k in ("q1", "k1", "q2", "k2")}
    codes, scales = {}, torch.empty(4, dtype=torch.float32, device=dev)
    for i, k in enumerate(("q1", "k1", "q2", "k2")):
        codes[k], _ = da.quantize_fp8(g[k], scale=scales[i:i + 1])
    lam_t = da.lam(*(x[k].to(dev) for k in ("lq1", "lk1", "lq2", "lk2")), x["lambda_init"])
    got = da.fwd_fp8qk(codes["q1"], codes["k1"], codes["q2"], codes["k2"], scales, x["v"].to(dev), lam_t,
                       x["lambda_init"], eps=x["eps"], causal=causal).float().cpu().numpy()
    lam = _lam_host(x)
    ref = O.forward(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, x["lambda_init"], eps=x["eps"],
                    causal=causal)
    _, _, deq = _oracle_quant(x)
    rel = np.empty((2, 2))
    for b in range(2):
        for h in range(2):
            ds = []
            for qk in (("q1", "k1"), ("q2", "k2")):
                exact = O._f64(x[qk[0]][b, h]) @ O._f64(x[qk[1]][b, h]).T
                quant = deq[qk[0]][b, h] @ deq[qk[1]][b, h].T
                ds.append(((quant - exact) / np.sqrt(D)).ravel())
            rel[b, h] = np.sqrt(np.std(np.concatenate(ds)) ** 2 + U_BF16 ** 2 / 3.0)
    tol = _bound(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, x["lambda_init"], x["eps"], causal, rel)
    err = np.abs(got - ref)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    print(f"logit perturbation std {rel.ravel()}; max err {err.max():.3e}; worst vs bound "
          f"{err[worst]:.3e} / {tol[worst]:.3e}", flush=True)
    assert np.all(err <= tol)


def test_fp8qk_full_size_3b_layer_sampled(dev):
    # the benchmarked launch: 2 x 12 heads, N = 4096, causal; sampled rows of
    # sampled heads (each with its full causal prefix) against the oracle on
    # the dequantised inputs
    name = "layer3b_bf16_b2h12n4096d128"
    x = W.workload_inputs(name, device=dev)
    codes, scales = {}, torch.empty(4, dtype=torch.float32, device=dev)
    for i, k in enumerate(("q1", "k1", "q2", "k2")):
        codes[k], _ = da.quantize_fp8(x[k], scale=scales[i:i + 1])
    lam_t = da.lam(x["lq1"], x["lk1"], x["lq2"], x["lk2"], x["lambda_init"])
    out = da.fwd_fp8qk(codes["q1"], codes["k1"], codes["q2"], codes["k2"], scales, x["v"], lam_t,
                       x["lambda_init"], eps=x["eps"], causal=True)
    torch.cuda.synchronize()
    lam = float(lam_t.item())
    sc = scales.cpu().numpy()
    rng = np.random.default_rng(7)
    N = x["q1"].shape[2]
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, N - 2, N - 1], rng.integers(0, N, 24)]))
    worst = 0.0
    for b, h in ((0, 0), (1, 11), (0, 5)):
        deq = [F.dequantize(codes[k][b, h].cpu().numpy(), sc[i]) for i, k in enumerate(("q1", "k1", "q2", "k2"))]
        ref = O.forward_rows(deq[0], deq[1], deq[2], deq[3], x["v"][b, h].cpu(), rows, lam, x["lambda_init"],
                             eps=x["eps"], causal=True)
        got = out[b, h][torch.from_numpy(rows).to(dev)].float().cpu().numpy()
        assert np.all(np.isfinite(got))
        worst = max(worst, float(np.max(np.abs(got - ref))))
    print(f"{name} fp8qk: sampled max|err| = {worst:.3e}", flush=True)
    assert worst <= 2e-2


def test_fp8qk_longctx_64k_sampled(dev):
    # 64K tokens, 12 heads, d = 128, with the planted needles: sampled rows
    # (needle offsets, first and last rows) of two heads against the oracle
    # on the dequantised inputs, each row with its full causal prefix
    name = "longctx_bf16_b1h12n65536d128"
    x = W.workload_inputs(name, device=dev)
    codes, scales = {}, torch.empty(4, dtype=torch.float32, device=dev)
    for i, k in enumerate(("q1", "k1", "q2", "k2")):
        codes[k], _ = da.quantize_fp8(x[k], scale=scales[i:i + 1])
    lam_t = da.lam(x["lq1"], x["lk1"], x["lq2"], x["lk2"], x["lambda_init"])
    out = da.fwd_fp8qk(codes["q1"], codes["k1"], codes["q2"], codes["k2"], scales, x["v"], lam_t,
                       x["lambda_init"], eps=x["eps"], causal=True)
    torch.cuda.synchronize()
    lam = float(lam_t.item())
    sc = scales.cpu().numpy()
    N = x["q1"].shape[2]
    rows = np.array([0, 6, 7, 8, 311, 312, 5003, 40009, 40010, N - 1])
    worst = 0.0
    for h in (0, 11):
        deq = [F.dequantize(codes[k][0, h].cpu().numpy(), sc[i]) for i, k in enumerate(("q1", "k1", "q2", "k2"))]
        ref = O.forward_rows(deq[0], deq[1], deq[2], deq[3], x["v"][0, h].cpu(), rows, lam, x["lambda_init"],
                             eps=x["eps"], causal=True)
        got = out[0, h][torch.from_numpy(rows).to(dev)].float().cpu().numpy()
        assert np.all(np.isfinite(got))
        worst = max(worst, float(np.max(np.abs(got - ref))))
    print(f"{name} fp8qk: sampled max|err| = {worst:.3e}", flush=True)
    assert worst <= 2e-2


def test_fp8qk_deterministic(dev):
    x = W.prefill_inputs(1, 2, 700, D, "bf16", seed=71)
    codes, scales, _ = _oracle_quant(x)
    a = _gpu_fp8(codes, scales, x, dev, True)
    b = _gpu_fp8(codes, scales, x, dev, True)
    assert np.array_equal(a, b)


def test_fp8_bindings_refuse_wrong_inputs(dev):
    c = torch.zeros(1, 1, 8, D, dtype=torch.uint8, device=dev)
    v = torch.zeros(1, 1, 8, 2 * D, dtype=torch.bfloat16, device=dev)
    s = torch.ones(4, device=dev)
    lam_t = torch.zeros(1, device=dev)
    with pytest.raises(ValueError):
        da.fwd_fp8qk(c.to(torch.bfloat16), c, c, c, s, v, lam_t, 0.8)
    with pytest.raises(ValueError):
        da.fwd_fp8qk(c, c, c, c, s[:3], v, lam_t, 0.8)
    with pytest.raises(RuntimeError):  # d = 64 is refused by the library
        c64 = torch.zeros(1, 1, 8, 64, dtype=torch.uint8, device=dev)
        da.fwd_fp8qk(c64, c64, c64, c64, s, v[..., :128].contiguous(), lam_t, 0.8)
    with pytest.raises(ValueError):
        da.quantize_fp8(torch.zeros(8, device=dev))  # fp32 input
