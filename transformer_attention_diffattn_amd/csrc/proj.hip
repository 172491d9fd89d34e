// Projections on either side of differential attention ("Differential
// attention" page, section "How it's wired": each head's query and key
// projections split into the halves Q1/K1 and Q2/K2; "Differential
// Transformer" sample peer review, "Strengths": heads halved, h = d_model/2d,
// a drop-in for the attention of a standard block).
//
// Both are one bf16 matrix product with fp32 accumulation, C^T = W X^T, in
// which both operands are contiguous along the reduction (W[out, in] rows,
// token rows of X), so 16-byte loads feed the 16x16x32 bf16 MFMA directly:
// W rows are the A operand (output features), token rows the B operand.
// What differs is where the operands come from and where results go:
//
//   in-projection  : X = x [B*N, d_model] row-major; the epilogue writes each
//                    output feature to Q1/K1/Q2/K2 [B, H, N, d] or V
//                    [B, H, N, 2d] (the attention kernels' layouts), so no
//                    split or transpose pass follows;
//   out-projection : X = the attention output [B, H, N, 2d] read as the
//                    head concatenation [B*N, H*2d] (reduction index
//                    h*2d + c), y = X W_O^T written row-major [B*N, d_out].
//
// Workgroup: 4 waves as 2 x 2, a 128-feature x 128-token tile; each wave
// owns 64 x 64 (4 x 4 MFMA blocks) and streams its fragments straight from
// global memory (the four waves' overlapping rows meet in the L1/L2), the
// next reduction step's loads issued before the current step's products.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace diffattn {

namespace {

constexpr int kProjTile = 128;

template <int MODE>  // 0: in-projection, 1: out-projection
__global__ __launch_bounds__(256, 2) void proj_kernel(ProjArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * kProjTile + (wave & 1) * 64;  // output features
  const int m0 = blockIdx.y * kProjTile + (wave >> 1) * 64;  // tokens (M < 2^23)
  const int K = a.K, F = a.F, M = a.M, N = a.N, H = a.H;
  const int l2dv = a.log2_dv;  // 2d = 1 << l2dv (out-projection reads; in-projection writes)

  const uint16_t* wrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wrow[i] = (const uint16_t*)a.w + (size_t)min(n0 + 16 * i + lr, F - 1) * K;
  // token rows (b, t) of this lane's four tokens; the x rows (in-projection)
  // or head 0 of the token (out-projection; head h lies h*N*2d further)
  int tb[4], tt[4];
  const uint16_t* xrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = min(m0 + 16 * j + lr, M - 1);
    tb[j] = m / N;
    tt[j] = m - tb[j] * N;
    if (MODE == 0)
      xrow[j] = (const uint16_t*)a.x + (size_t)m * K;
    else
      xrow[j] = (const uint16_t*)a.x + (((size_t)tb[j] * H * N + (size_t)tt[j]) << l2dv);
  }
  const size_t head_stride = (size_t)N << l2dv;  // out-projection: elements between heads

  // fragments of reduction step k0; past K they are zero (the address is
  // clamped to the last chunk, so every load stays inside its row)
  auto load = [&](int k0, bf16x8 (&af)[4], bf16x8 (&bfr)[4]) {
    const int kk0 = k0 + 8 * lg;
    const bool ok = kk0 < K;
    const int kk = min(kk0, K - 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 t = ld16(wrow[i] + kk);
      af[i] = as_bf16x8(ok ? t : zero_u32x4());
    }
    size_t off = (size_t)kk;
    if (MODE == 1) off = (size_t)(kk >> l2dv) * head_stride + (size_t)(kk & ((1 << l2dv) - 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 t = ld16(xrow[j] + off);
      bfr[j] = as_bf16x8(ok ? t : zero_u32x4());
    }
  };
  auto mma = [&](const bf16x8 (&af)[4], const bf16x8 (&bfr)[4], f32x4 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32_bf16(af[i], bfr[j], acc[i][j]);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero_f32x4();

  // two register buffers, the loop unrolled by two so that both are named
  // at compile time; each step's loads are issued before the previous
  // step's products
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  load(0, a0, b0);
  for (int k0 = 0; k0 < K; k0 += 64) {
    load(k0 + 32, a1, b1);
    mma(a0, b0, acc);
    if (k0 + 32 >= K) break;
    load(k0 + 64, a0, b0);
    mma(a1, b1, acc);
  }

  // lane: token m0 + 16j + lr, features n0 + 16i + 4lg .. +3 (8 bytes of bf16)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + 16 * i + 4 * lg;
    if (n >= F) continue;
    // in-projection: feature n of [W_Q; W_K; W_V] -> destination tensor,
    // its row width, the head and the channel within a row
    uint16_t* base = (uint16_t*)a.y;
    int l2w = 0, h = 0, ch = n;
    if (MODE == 0) {
      const int width = H << l2dv;
      const int part = n / width, r = n - part * width;
      h = r >> l2dv;
      const int c = r & ((1 << l2dv) - 1);
      if (part == 2) {
        base = (uint16_t*)a.v;
        l2w = l2dv;
        ch = c;
      } else {
        const int half = c >> (l2dv - 1);
        base = (uint16_t*)(part == 0 ? (half ? a.q2 : a.q1) : (half ? a.k2 : a.k1));
        l2w = l2dv - 1;
        ch = c & ((1 << l2w) - 1);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + 16 * j + lr;
      if (m >= M) continue;
      const u32x2 pk = {pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
      size_t off;
      if (MODE == 0)
        off = ((((size_t)tb[j] * H + h) * N + (size_t)tt[j]) << l2w) + ch;
      else
        off = (size_t)m * F + n;
      *reinterpret_cast<u32x2*>(base + off) = pk;
    }
  }
}

}  // namespace

hipError_t launch_proj(int mode, const ProjArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.F + kProjTile - 1) / kProjTile), (unsigned)((a.M + kProjTile - 1) / kProjTile));
  if (mode == 0)
    hipLaunchKernelGGL(proj_kernel<0>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(proj_kernel<1>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace diffattn
