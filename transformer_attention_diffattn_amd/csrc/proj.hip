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
// owns 64 x 64 (4 x 4 MFMA blocks).  Operand tiles are staged in LDS, 64
// reduction elements per step, the next step's global loads in flight while
// the current step's products run.

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
  // Tile order.  Workgroups are dealt to the 8 XCDs round-robin by launch
  // index, each XCD with its own L2: XCD x takes the x-th eighth of a
  // sequence in which GM token tiles run with all feature tiles before the
  // next GM, so each XCD keeps a few token slabs resident while it streams
  // the weight rows (a bijection of the tile grid; plain order if the tile
  // count is not a multiple of 8).
  constexpr int GM = 8;
  const int nF = gridDim.x, nMt = gridDim.y, total = nF * nMt;
  const int L = blockIdx.x + nF * blockIdx.y;
  const int seq = (total % 8 == 0) ? (L % 8) * (total / 8) + L / 8 : L;
  const int grp = seq / (GM * nF), first_m = grp * GM;
  const int gm = min(nMt - first_m, GM);
  const int rem = seq - grp * GM * nF;
  const int tile_m = first_m + rem % gm, tile_f = rem / gm;
  const int n0 = tile_f * kProjTile + (wave & 1) * 64;  // output features
  const int m0 = tile_m * kProjTile + (wave >> 1) * 64;  // tokens (M < 2^23)
  const int K = a.K, F = a.F, M = a.M, N = a.N, H = a.H;
  const int l2dv = a.log2_dv;  // 2d = 1 << l2dv (out-projection reads; in-projection writes)

  // The workgroup's operand tiles pass through LDS, 64 reduction elements
  // (128 bytes per row) at a time, double-buffered: 128 feature rows of W
  // and 128 token rows of X, each row's eight 16-byte chunks XOR-swizzled by
  // (row mod 8) so that each eight consecutive rows of a fragment read fall
  // on distinct 16-byte bank groups.  Thread t loads chunks t + 256u (u < 4) of each tile: eight
  // consecutive threads cover one row's 128 bytes.
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kProjTile * 64];  // [buffer][W, X][row*64 + k]
  const int tid = threadIdx.x;
  const int wf0 = tile_f * kProjTile, wm0 = tile_m * kProjTile;  // workgroup's first feature / token
  const uint16_t* wsrc[4];
  const uint16_t* xsrc[4];
  int lrow[4], lchk[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = tid + 256 * u;
    const int r = q >> 3, c = q & 7;
    lrow[u] = r;
    lchk[u] = c;
    wsrc[u] = (const uint16_t*)a.w + (size_t)min(wf0 + r, F - 1) * K;
    const int m = min(wm0 + r, M - 1);
    if (MODE == 0) {
      xsrc[u] = (const uint16_t*)a.x + (size_t)m * K;
    } else {
      const int b = m / N, t = m - b * N;
      xsrc[u] = (const uint16_t*)a.x + (((size_t)b * H * N + (size_t)t) << l2dv);
    }
  }
  const size_t head_stride = (size_t)N << l2dv;  // out-projection: elements between heads
  u32x4 stw[4], stx[4];
  // global -> registers: chunk (row, c) of step k0; zero past K (address clamped)
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk0 = k0 + 8 * lchk[u];
      const bool ok = kk0 < K;
      const int kk = min(kk0, K - 8);
      const u32x4 tw = ld16(wsrc[u] + kk);
      size_t off = (size_t)kk;
      if (MODE == 1) off = (size_t)(kk >> l2dv) * head_stride + (size_t)(kk & ((1 << l2dv) - 1));
      const u32x4 tx = ld16(xsrc[u] + off);
      stw[u] = ok ? tw : zero_u32x4();
      stx[u] = ok ? tx : zero_u32x4();
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = lrow[u] * 64 + 8 * (lchk[u] ^ (lrow[u] & 7));
      *reinterpret_cast<u32x4*>(&lds[buf][0][e]) = stw[u];
      *reinterpret_cast<u32x4*>(&lds[buf][1][e]) = stx[u];
    }
  };
  // fragments of half s (k 32s..32s+31) of the staged step: row 16i + lr of
  // the wave's 64 rows, chunk 4s + lg
  const int wrow0 = (wave & 1) * 64, xrow0 = (wave >> 1) * 64;
  auto frag = [&](const uint16_t* t, int row, int s) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(t + row * 64 + 8 * ((4 * s + lg) ^ (row & 7))));
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero_f32x4();

  const int nk = (K + 63) / 64;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) fetch(64 * (ks + 1));
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = frag(lds[buf][0], wrow0 + 16 * i + lr, s);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = frag(lds[buf][1], xrow0 + 16 * j + lr, s);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32_bf16(af[i], bfr[j], acc[i][j]);
    }
    // the other buffer was last read in the previous step, before its barrier
    if (ks + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }

  // token rows (b, t) of this lane's four tokens, for the epilogue
  int tb[4], tt[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = min(m0 + 16 * j + lr, M - 1);
    tb[j] = m / N;
    tt[j] = m - tb[j] * N;
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
