"""GPU parity of the in- and out-projections (diffattn_in_proj,
diffattn_out_proj) against oracle/projection_oracle.py.

Bound per element, from the arithmetic: the inputs are bf16 (exact in the
oracle's float64), the kernel sums exact products in fp32 and rounds the
result to bf16, so |gpu - oracle| <= 2^-8 |oracle| (round to nearest) +
K 2^-24 sum_k |x_k w_k| (fp32 summation of K terms), with the magnitudes
summed by the oracle on |x| and |w|.
"""

import numpy as np
import pytest
import torch

from oracle import diffattn_oracle as O
from oracle import projection_oracle as P
from transformer_attention_diffattn_amd import binding as da
from transformer_attention_diffattn_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _check(got, ref, mag, K):
    got = got.float().cpu().numpy()
    tol = 2.0 ** -8 * np.abs(ref) + K * 2.0 ** -24 * (1 + 2.0 ** -8) * mag + 1e-30
    err = np.abs(got - ref)
    worst = np.unravel_index(np.argmax(err / tol), err.shape)
    print(f"max err {err.max():.3e}; worst vs bound {err[worst]:.3e} / {tol[worst]:.3e}", flush=True)
    assert np.all(err <= tol)


def _abs(t):
    return t.float().abs().numpy()


IN_CASES = [(2, 77, 256, 2, 64), (1, 130, 200, 3, 32), (2, 33, 128, 1, 128), (1, 1, 64, 2, 16),
            (3, 129, 72, 4, 16)]


@pytest.mark.parametrize("B,N,dm,H,d", IN_CASES)
def test_in_proj(dev, B, N, dm, H, d):
    print(f"case in_proj B={B} N={N} d_model={dm} H={H} d={d}", flush=True)
    x = W.projection_inputs(B, N, dm, H, d, seed=900 + N)
    outs = da.in_proj(x["x"].to(dev), x["w_qkv"].to(dev), H, d)
    torch.cuda.synchronize()
    ref = P.in_projection(x["x"], x["w_qkv"], H, d)
    mag = P.in_projection(_abs(x["x"]), _abs(x["w_qkv"]), H, d)
    for g, r, m in zip(outs, ref, mag):
        _check(g, r, m, dm)


# reduction lengths H*2d of 32 and 96 leave the last 64-wide step half empty
OUT_CASES = [(2, 2, 77, 64, 256), (1, 3, 130, 32, 100), (2, 1, 33, 128, 4), (1, 4, 129, 16, 36),
             (1, 1, 50, 16, 8), (2, 3, 20, 16, 12)]


@pytest.mark.parametrize("B,H,N,d,dout", OUT_CASES)
def test_out_proj(dev, B, H, N, d, dout):
    print(f"case out_proj B={B} H={H} N={N} d={d} d_out={dout}", flush=True)
    x = W.projection_inputs(B, N, 64, H, d, seed=950 + N, d_out=dout)
    y = da.out_proj(x["o"].to(dev), x["w_o"].to(dev))
    torch.cuda.synchronize()
    _check(y, P.out_projection(x["o"], x["w_o"]), P.out_projection(_abs(x["o"]), _abs(x["w_o"])), H * 2 * d)


# shapes large enough for the 256 x 256 large-tile form (reduction a multiple
# of 64), with ragged token and feature edges and workgroups past the tile
# grid: every element against the oracle
# (1, 2048, 256, 25, 64): 9600 features, whose large-tile blocks make one and
# a quarter rounds, so the last 1408 features go to the 128 x 128 form
@pytest.mark.parametrize("B,N,dm,H,d", [(1, 3000, 512, 8, 64), (2, 2100, 256, 6, 128), (1, 2048, 256, 25, 64)])
def test_in_proj_large_tiles_ragged(dev, B, N, dm, H, d):
    print(f"case in_proj large B={B} N={N} d_model={dm} H={H} d={d}", flush=True)
    x = W.projection_inputs(B, N, dm, H, d, seed=970 + N)
    outs = da.in_proj(x["x"].to(dev), x["w_qkv"].to(dev), H, d)
    torch.cuda.synchronize()
    ref = P.in_projection(x["x"], x["w_qkv"], H, d)
    mag = P.in_projection(_abs(x["x"]), _abs(x["w_qkv"]), H, d)
    for g, r, m in zip(outs, ref, mag):
        _check(g, r, m, dm)


# (1, 4, 8192, 64, 2600): blocks making one and a half rounds; features
# 2048..2599 (a ragged 128-tile at the end) go to the 128 x 128 form
@pytest.mark.parametrize("B,H,N,d,dout", [(1, 8, 8300, 32, 1000), (2, 4, 4150, 64, 1028), (1, 4, 8192, 64, 2600)])
def test_out_proj_large_tiles_ragged(dev, B, H, N, d, dout):
    print(f"case out_proj large B={B} H={H} N={N} d={d} d_out={dout}", flush=True)
    x = W.projection_inputs(B, N, 64, H, d, seed=990 + N, d_out=dout)
    y = da.out_proj(x["o"].to(dev), x["w_o"].to(dev))
    torch.cuda.synchronize()
    _check(y, P.out_projection(x["o"], x["w_o"]), P.out_projection(_abs(x["o"]), _abs(x["w_o"])), H * 2 * d)


def test_projections_full_size_1p4b_layer_sampled(dev):
    # the benchmarked shapes: 4 x 2048 tokens, d_model 2048, 16 heads of 2d = 128;
    # every output feature of sampled tokens against the oracle
    B, N, dm, H, d = 4, 2048, 2048, 16, 64
    x = W.projection_inputs(B, N, dm, H, d, seed=20266, device=dev)
    outs = da.in_proj(x["x"], x["w_qkv"], H, d)
    y = da.out_proj(x["o"], x["w_o"])
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 1000, N - 2, N - 1])
    xs = x["x"][:, rows].cpu()
    ref = P.in_projection(xs, x["w_qkv"].cpu(), H, d)
    mag = P.in_projection(_abs(xs), _abs(x["w_qkv"].cpu()), H, d)
    for g, r, m in zip(outs, ref, mag):
        _check(g[:, :, rows], r, m, dm)
    os_ = x["o"][:, :, rows].cpu()
    _check(y[:, rows], P.out_projection(os_, x["w_o"].cpu()),
           P.out_projection(_abs(os_), _abs(x["w_o"].cpu())), H * 2 * d)


def test_projections_full_size_3b_layer_sampled(dev):
    # 2 x 4096 tokens, d_model 3072, 12 heads of 2d = 256 (d = 128)
    B, N, dm, H, d = 2, 4096, 3072, 12, 128
    x = W.projection_inputs(B, N, dm, H, d, seed=20267, device=dev)
    outs = da.in_proj(x["x"], x["w_qkv"], H, d)
    y = da.out_proj(x["o"], x["w_o"])
    torch.cuda.synchronize()
    rows = np.array([0, 127, 128, 2049, N - 1])
    xs = x["x"][:, rows].cpu()
    ref = P.in_projection(xs, x["w_qkv"].cpu(), H, d)
    mag = P.in_projection(_abs(xs), _abs(x["w_qkv"].cpu()), H, d)
    for g, r, m in zip(outs, ref, mag):
        _check(g[:, :, rows], r, m, dm)
    os_ = x["o"][:, :, rows].cpu()
    _check(y[:, rows], P.out_projection(os_, x["w_o"].cpu()),
           P.out_projection(_abs(os_), _abs(x["w_o"].cpu())), H * 2 * d)


def test_layer_chain_parity_1p4b_slice(dev):
    """in_proj -> lambda -> diffattn_fwd -> out_proj on the device layouts (no
    copies between the calls) against projection_oracle then diffattn_oracle
    then projection_oracle, all computed from x and the weights alone: a
    slice of the 1.4B-scale layer (256 tokens, d_model 2048, 16 heads of
    2d = 128).  Tutorial page "Differential attention", section "How it's
    wired": the layer drops into the block in place of ordinary attention.

    Composed bound, stage by stage against the fp64 chain:
    * q1, k1, q2, k2, v: the projection bound above;
    * attention output: the bf16 tolerance 2e-2 per element (it covers the
      kernel's own rounding and the bf16 storage of its inputs, which moves
      this output by under 8e-3 here);
    * y: the attention errors e_c enter y_f = sum_c o_c W_O[f, c] as
      independent per-channel errors of size at most 2e-2, so six standard
      deviations give 6 * 2e-2 * ||W_O[f]||_2, plus the out-projection's own
      rounding (the projection bound)."""
    B, N, dm, H, d = 1, 256, 2048, 16, 64
    lam_init = 0.8
    x = W.projection_inputs(B, N, dm, H, d, seed=31)
    g = torch.Generator().manual_seed(32)
    lv = [0.1 * torch.randn(d, generator=g) for _ in range(4)]
    # device chain
    q1, k1, q2, k2, v = da.in_proj(x["x"].to(dev), x["w_qkv"].to(dev), H, d)
    lam_t = da.lam(*(t.to(dev) for t in lv), lam_init)
    o = da.fwd(q1, k1, q2, k2, v, lam_t, lam_init)
    y = da.out_proj(o, x["w_o"].to(dev))
    torch.cuda.synchronize()
    # oracle chain
    ref_in = P.in_projection(x["x"], x["w_qkv"], H, d)
    mag_in = P.in_projection(_abs(x["x"]), _abs(x["w_qkv"]), H, d)
    for gt, r, m in zip((q1, k1, q2, k2, v), ref_in, mag_in):
        _check(gt, r, m, dm)
    lam = O.lambda_scalar(*lv, lam_init)
    ref_o = O.forward(*ref_in, lam, lam_init)
    err_o = float(np.max(np.abs(o.float().cpu().numpy() - ref_o)))
    print(f"attention stage: max err {err_o:.3e} (bound 2e-2)", flush=True)
    assert err_o <= 2e-2
    ref_y = P.out_projection(ref_o, x["w_o"])
    mag_y = P.out_projection(np.abs(ref_o), _abs(x["w_o"]))
    wn = np.linalg.norm(x["w_o"].double().numpy(), axis=1)
    K = H * 2 * d
    tol = 6.0 * 2e-2 * wn + 2.0 ** -8 * np.abs(ref_y) + K * 2.0 ** -24 * (1 + 2.0 ** -8) * mag_y
    err_y = np.abs(y.float().cpu().numpy() - ref_y)
    worst = np.unravel_index(np.argmax(err_y / tol), err_y.shape)
    print(f"output stage: max err {err_y.max():.3e}; worst vs bound {err_y[worst]:.3e} / {tol[worst]:.3e} "
          f"(rms of y {np.sqrt(np.mean(ref_y ** 2)):.3e})", flush=True)
    assert np.all(err_y <= tol)


def test_projection_deterministic(dev):
    x = W.projection_inputs(2, 300, 512, 4, 64, seed=41, device=dev)
    a = da.in_proj(x["x"], x["w_qkv"], 4, 64)
    b = da.in_proj(x["x"], x["w_qkv"], 4, 64)
    for s, t in zip(a, b):
        assert torch.equal(s, t)
