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
  const int n0 = a.f_lo + tile_f * kProjTile + (wave & 1) * 64;  // output features
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
  const int wf0 = a.f_lo + tile_f * kProjTile, wm0 = tile_m * kProjTile;  // workgroup's first feature / token
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

// ---------------------------------------------------------------------------
// The large-tile form (reduction length a multiple of 64; for the
// out-projection a head width 2d of at least 64, so that a 64-wide step of
// the reduction lies inside one head): a workgroup of 8 waves owns 256
// features x 256 tokens, each wave 128 features x 64 tokens (8 x 4 MFMA
// blocks), one workgroup per compute unit.  Operand tiles go from global
// memory straight into LDS (global_load_lds_dwordx4, 1 KB = 8 rows of 64
// reduction elements per instruction), double-buffered, 64 reduction
// elements per step; each 128-byte row's eight 16-byte chunks are
// XOR-swizzled by (row mod 8) on the global side, so that the eight rows of
// each fragment read fall on distinct bank groups.  Per wave and step, 12
// fragment reads (12 KB) feed 64 products: a quarter fewer LDS bytes per
// product than the 128 x 128 form.
//   Tile order: workgroups are dealt to the 8 XCDs round robin by launch
// index; the tile grid is cut into blocks of 4 feature tiles x 8 token tiles,
// block b going to XCD b % 8 as its (b / 8)-th round, so the 32 workgroups
// that an XCD runs together share 1024 weight rows and 2048 token rows,
// streamed through its L2 in step.

constexpr int kBigTile = 256;
constexpr int kBigFB = 4, kBigMB = 8;  // tiles per XCD block: features x tokens

template <int MODE>
__global__ __launch_bounds__(512, 1) void proj256_kernel(ProjArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int K = a.K, F = a.F, M = a.M, N = a.N, H = a.H;
  const int l2dv = a.log2_dv;
  // tile order (see above); the grid covers whole rounds of 8 XCD blocks,
  // and a workgroup whose block or tile lies past the tile grid has nothing
  // to do (it leaves before any barrier)
  // (this form always starts at feature 0: f_lo = 0, f_hi = F or a multiple of 256)
  const int nFt = (a.f_hi + kBigTile - 1) / kBigTile, nMt = (M + kBigTile - 1) / kBigTile;
  const int nFb = (nFt + kBigFB - 1) / kBigFB, nMb = (nMt + kBigMB - 1) / kBigMB;
  const int L = blockIdx.x;
  const int bi = (L % 8) + 8 * ((L / 8) / (kBigFB * kBigMB));  // XCD block
  const int slot = (L / 8) % (kBigFB * kBigMB);
  const int tile_f = (bi % nFb) * kBigFB + slot % kBigFB;
  const int tile_m = (bi / nFb) * kBigMB + slot / kBigFB;
  if (bi >= nFb * nMb || tile_f >= nFt || tile_m >= nMt) return;
  const int wf0 = tile_f * kBigTile, wm0 = tile_m * kBigTile;
  const int n0 = wf0 + (wave & 1) * 128;   // this wave's features
  const int m0 = wm0 + (wave >> 1) * 64;   // this wave's tokens

  // LDS: [buffer][W, X][256 rows][64] bf16 = 2 x 2 x 32 KB
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kBigTile * 64];
  const uint32_t lds0 = lds_offset(lds);
  // Loads of one step: 32 instructions for the W tile and 32 for the X tile,
  // 8 rows each; wave w issues W instructions w, w + 8, w + 16, w + 24 and
  // the same X instructions.  Lane l fills LDS row 8 i + l / 8, physical
  // chunk l % 8, which holds logical chunk (l % 8) ^ (row % 8).
  const int prow = lane >> 3;
  const int lchunk = (lane & 7) ^ (prow & 7);  // rows 8i + prow: row % 8 == prow
  uint32_t woff[4];                    // byte offsets from the W tile's first row
  const uint16_t* xrow[4];             // X rows (token m) at reduction index 0
  size_t xh_stride = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 8 * (wave + 8 * u) + prow;  // row within the tile
    woff[u] = (uint32_t)(min(wf0 + r, F - 1) - wf0) * (uint32_t)K * 2u + 16u * (uint32_t)lchunk;
    const int m = min(wm0 + r, M - 1);
    if (MODE == 0) {
      xrow[u] = (const uint16_t*)a.x + (size_t)m * K + 8 * lchunk;
    } else {
      const int b = m / N, t = m - b * N;
      xrow[u] = (const uint16_t*)a.x + (((size_t)b * H * N + (size_t)t) << l2dv) + 8 * lchunk;
    }
  }
  if (MODE == 1) xh_stride = (size_t)N << l2dv;
  const uint16_t* wbase = (const uint16_t*)a.w + (size_t)wf0 * K;
  auto issue = [&](int ks, int buf) {
    const int k0 = 64 * ks;
    const uint32_t lw = lds0 + (uint32_t)(buf * 2 * kBigTile * 64 * 2);
    const uint32_t lx = lw + (uint32_t)(kBigTile * 64 * 2);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      lds_dma16_s(wbase, woff[u] + 2u * (uint32_t)k0, lw + 1024u * (uint32_t)(wave + 8 * u));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint16_t* src;
      if (MODE == 0)
        src = xrow[u] + k0;
      else
        src = xrow[u] + (size_t)(k0 >> l2dv) * xh_stride + (k0 & ((1 << l2dv) - 1));
      lds_dma16(src, lx + 1024u * (uint32_t)(wave + 8 * u));
    }
  };
  // fragment of half s (k 32s .. 32s + 31): row `row` of a tile, chunk 4s + lg
  auto frag = [&](const uint16_t* t, int row, int s) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(t + row * 64 + 8 * ((4 * s + lg) ^ (row & 7))));
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero_f32x4();

  const int nk = K / 64;
  const int wr0 = (wave & 1) * 128, xr0 = (wave >> 1) * 64;
  issue(0, 0);
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    // this wave's loads of step ks have landed; the barrier extends that to
    // everybody's, and everybody is done reading the other buffer (step ks-1)
    wait_vmem();
    __syncthreads();
    if (ks + 1 < nk) issue(ks + 1, buf ^ 1);
    const uint16_t* tw = lds[buf][0];
    const uint16_t* tx = lds[buf][1];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 bfr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = frag(tx, xr0 + 16 * j + lr, s);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 af = frag(tw, wr0 + 16 * i + lr, s);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32_bf16(af, bfr[j], acc[i][j]);
      }
    }
  }

  // epilogue as in proj_kernel: lane holds features n0 + 16i + 4lg .. +3 of
  // token m0 + 16j + lr
  int tb[4], tt[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = min(m0 + 16 * j + lr, M - 1);
    tb[j] = m / N;
    tt[j] = m - tb[j] * N;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = n0 + 16 * i + 4 * lg;
    if (n >= F) continue;
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

// The large-tile form needs a reduction length that is a multiple of 64 and
// a head width of at least 64 when it reads the per-head attention output;
// it pays for large products only (at least half a round of XCD blocks).
// Its grid: whole rounds of 8 XCD blocks of 4 x 8 tiles of 256, over the
// features [0, f_hi).
static bool proj256_fits(int mode, const ProjArgs& a) {
  if (a.K % 64 != 0 || (mode == 1 && a.log2_dv < 6)) return false;
  const long long nFt = (a.F + kBigTile - 1) / kBigTile, nMt = (a.M + kBigTile - 1) / kBigTile;
  return nFt * nMt >= 8LL * kBigFB * kBigMB / 2;
}
static long long proj256_grid(const ProjArgs& a) {
  const long long nFt = (a.f_hi + kBigTile - 1) / kBigTile, nMt = (a.M + kBigTile - 1) / kBigTile;
  const long long blocks = ((nFt + kBigFB - 1) / kBigFB) * ((nMt + kBigMB - 1) / kBigMB);
  return (blocks + 7) / 8 * 8 * kBigFB * kBigMB;
}

// Features of the large-tile launch.  When its XCD blocks make a last round
// that is only partly filled, the features of the blocks past the last
// whole round (whole feature blocks of 1024) go to the 128 x 128 form
// instead, in a second launch, if that takes less time than the partial
// round: the 128 x 128 form runs at about 0.7 of the large one's rate and
// fills all compute units with two workgroups each.
static int proj256_features(const ProjArgs& a) {
  const long long nFt = (a.F + kBigTile - 1) / kBigTile, nMt = (a.M + kBigTile - 1) / kBigTile;
  const long long nFb = (nFt + kBigFB - 1) / kBigFB, nMb = (nMt + kBigMB - 1) / kBigMB;
  const long long per_round = 8LL * kBigFB * kBigMB;  // tiles of 256 per round
  if ((nFb * nMb) % 8 == 0) return a.F;
  long long nf = nFb - 1;
  while (nf >= 1 && (nf * nMb) % 8 != 0) --nf;
  if (nf < 1) return a.F;
  const long long rounds_full = (nFb * nMb + 7) / 8, rounds_big = nf * nMb / 8;
  const double rest_rounds = (double)(nFt - nf * kBigFB) * (double)nMt / (double)per_round;
  if (rest_rounds / 0.7 >= (double)(rounds_full - rounds_big) - 0.05) return a.F;
  return (int)(nf * kBigFB * kBigTile);
}

static void launch_proj128(int mode, const ProjArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.F - a.f_lo + kProjTile - 1) / kProjTile), (unsigned)((a.M + kProjTile - 1) / kProjTile));
  if (mode == 0)
    hipLaunchKernelGGL(proj_kernel<0>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(proj_kernel<1>, grid, dim3(256), 0, stream, a);
}

hipError_t launch_proj(int mode, const ProjArgs& args, hipStream_t stream) {
  ProjArgs a = args;
  a.f_lo = 0;
  a.f_hi = a.F;
  if (proj256_fits(mode, a)) {
    a.f_hi = proj256_features(a);
    const unsigned grid = (unsigned)proj256_grid(a);
    if (mode == 0)
      hipLaunchKernelGGL(proj256_kernel<0>, dim3(grid), dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL(proj256_kernel<1>, dim3(grid), dim3(512), 0, stream, a);
    if (a.f_hi < a.F) {
      a.f_lo = a.f_hi;
      a.f_hi = a.F;
      launch_proj128(mode, a, stream);
    }
    return hipGetLastError();
  }
  launch_proj128(mode, a, stream);
  return hipGetLastError();
}

}  // namespace diffattn
