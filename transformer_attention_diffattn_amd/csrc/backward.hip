// Backward of the fused differential-attention forward for gfx950 (MI355X).
//
// The gradients follow from the forward's definitions (Eq. 1 of "Differential
// Transformer: Canceling Context Noise with Differential Attention", section
// "Cancelling Context Noise Through Attention Map Subtraction"; Eq. 2 and
// Eq. 3 of the "Differential Transformer" sample review, "Summary", with the
// head-wise RMSNorm of its "Weaknesses"), which the review's "Summary"
// describes as trained end to end.  Per row i (sigma = 1 - lambda_init,
// n = 2d, r = sqrt(mean(Y^2) + eps), g = sigma w dout):
//
//   dY    = g / r - Y (g . Y) / (n r^3)            dw = sum_i sigma dout Y / r
//   dV    = (A1 - lambda A2)^T dY                  dP = dY V^T
//   dS1   = A1 * (dP - delta1),  delta1 = dY . O1  (O_k = A_k V)
//   dS2   = A2 * (-lambda dP - delta2),  delta2 = -lambda dY . O2
//   dQk   = dSk Kk / sqrt d,  dKk = dSk^T Qk / sqrt d
//   dlambda = -sum_i dY . O2
//
// The forward run in training mode keeps, per map and row, the log2-sum-exp
// of the scaled scores and O_k; A_k is recomputed here as
// 2^(s log2(e)/sqrt(d) - lse_k).  The launches:
//   bwd_prep_kernel    row-wise: Y, r, dY (bf16), delta1, delta2, and per-
//                      workgroup partial sums of dw and dlambda (d = 128;
//                      at d <= 64 the dQ kernel does this for its own rows);
//   bwd_reduce_kernel  the partial sums in a fixed order (deterministic);
//   bwd_dq_kernel      query-parallel: S^T, dP^T and dQ^T += K^T dS^T;
//   bwd_dkv_kernel     key-parallel: S, dP and dV^T += dY^T D,
//                      dK^T += Q^T dS (D = A1 - lambda A2); at d = 128 as
//                      two launches, dV and dK apart (registers).
// Splitting dQ from dK/dV costs a second evaluation of S and dP but needs no
// atomics, so every gradient is deterministic.
//
// All products use the 16x16x32 bf16 MFMA with fp32 accumulation.  Staged
// tiles live in LDS as [16-column block][row][16 columns]: a 16-byte read
// gives an A operand whose k runs over columns, and the transposing read
// (lds_read_tr16) one whose k runs over rows.  A 16x16 result C holds, in
// lane L, column L % 16 and rows 4 (L / 16) + j; two such blocks over 32 rows,
// rounded to bf16 in-lane, are the B operand of a product whose k runs over
// those rows, in the same row order as the transposing read delivers them.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace diffattn {

namespace {

// element offset of (row r, column c) in an R-row tile stored as
// [16-column block][row][16 columns]
template <int R>
__device__ __forceinline__ int boff(int r, int c) {
  return ((c >> 4) * R + r) * 16 + (c & 15);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Tiles of 32 rows stream through a ring of LDS stage buffers by direct
// global->LDS loads.  One load instruction moves 32 rows x 16 columns (one
// column block, 1 KB) of a row-major [*, C] bf16 matrix: lane L fetches row
// r0 + L / 2 (rows past n_rows - 1 read row n_rows - 1), columns
// 16 cb + 8 (L % 2) .. + 7, which the blocked layout puts at byte 16 L of
// the block -- the position the instruction writes lane L's 16 bytes to.
constexpr int kTileRows = 32;
// Stage buffers: three (two tiles loading ahead) where two workgroups still
// fit a compute unit's LDS.  At d = 128 three would take 96 KB and leave one
// workgroup per CU, whose accumulators the compiler then shuttles through
// AGPRs, so two.
template <int D, bool DQ>
struct BwdStages {
  static constexpr int N = D >= 128 ? 2 : 3;
};

__device__ __forceinline__ void dma_block(const uint16_t* src, int C, int cb, int r0, int n_rows, int lane,
                                          uint32_t lds_block) {
  const int r = min(r0 + (lane >> 1), n_rows - 1);
  lds_dma16_s(src, (uint32_t)(r * C + 16 * cb + 8 * (lane & 1)) * 2u, lds_block);
}

// Make the compiler wait for a register's pending load here, where nothing
// else is in flight: inside a loop it cannot see the asynchronous tile
// loads and would wait for them too.
template <typename T>
__device__ __forceinline__ void settle(T& x) {
  asm volatile("" : "+v"(x));
}

// A operand with k over 32 rows starting at r0 of column block cb (R-row tile)
template <int R>
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tile, int cb, int r0, int lane) {
  const u32x2 lo = lds_read_tr16(tile + 16 * (R * cb + r0) + 4 * lane);
  const u32x2 hi = lds_read_tr16(tile + 16 * (R * cb + r0 + 16) + 4 * lane);
  const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return as_bf16x8(v);
}

// B operand from two C-layout blocks (rows 4 lg + j of block 0, then of block 1)
__device__ __forceinline__ bf16x8 pack_frag(const float (&x)[2][4]) {
  const u32x4 v = {pack_bf16x2(x[0][0], x[0][1]), pack_bf16x2(x[0][2], x[0][3]), pack_bf16x2(x[1][0], x[1][1]),
                   pack_bf16x2(x[1][2], x[1][3])};
  return as_bf16x8(v);
}

__device__ __forceinline__ void store_bf16x4(void* p, f32x4 v, float s) {
  const u32x2 w = {pack_bf16x2(v[0] * s, v[1] * s), pack_bf16x2(v[2] * s, v[3] * s)};
  *reinterpret_cast<u32x2*>(p) = w;
}

}  // namespace

// ---------------------------------------------------------------------------
// row-wise preparation: G = 2d/8 lanes per row, 8 consecutive channels per
// lane (two 16-byte loads of each fp32 per-map output, one of dout), 64/G
// rows per wave; row sums by shuffles within the G-lane group

constexpr int kPrepThreads = 256;

template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

template <int D>
__global__ __launch_bounds__(kPrepThreads) void bwd_prep_kernel(BwdArgs a) {
  constexpr int DV = 2 * D;
  constexpr int G = DV / 8;      // lanes per row
  constexpr int RPW = 64 / G;    // rows per wave
  constexpr int WAVES = kPrepThreads / 64;
  static_assert(G >= 8 && G <= 64 && 64 % G == 0, "row group");
  __shared__ float sdw[WAVES][DV];
  __shared__ float sdl[WAVES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / G, gl = lane % G;  // row within the wave, channel group
  const float lam = *a.lambda;
  const float sigma = a.out_scale;
  const long long rows = (long long)a.BH * a.N;
  float w[8], dw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    w[i] = a.norm_w ? a.norm_w[8 * gl + i] : 1.0f;
    dw[i] = 0.f;
  }
  float dl = 0.f;
  const uint16_t* dout = (const uint16_t*)a.dout;
  const long long stride = (long long)gridDim.x * WAVES * RPW;
  // the loop bound is wave-uniform: every lane takes part in the shuffles
  for (long long base = ((long long)blockIdx.x * WAVES + wave) * RPW; base < rows; base += stride) {
    const long long row = base + sub;
    const bool valid = row < rows;
    float x1[8], x2[8], gd[8], y[8];
    if (valid) {
      const f32x4* o1 = reinterpret_cast<const f32x4*>(a.osave + row * DV + 8 * gl);
      const f32x4* o2 = reinterpret_cast<const f32x4*>(a.osave + (rows + row) * DV + 8 * gl);
      const f32x4 p0 = o1[0], p1 = o1[1], r0 = o2[0], r1 = o2[1];
      const u32x4 g = ld16(dout + row * DV + 8 * gl);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x1[i] = p0[i];
        x1[4 + i] = p1[i];
        x2[i] = r0[i];
        x2[4 + i] = r1[i];
        gd[2 * i] = bf16_lo(g[i]);
        gd[2 * i + 1] = bf16_hi(g[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x1[i] = x2[i] = gd[i] = 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      y[i] = x1[i] - lam * x2[i];
      ss += y[i] * y[i];
    }
    ss = group_sum<G>(ss);
    const float ir = 1.0f / sqrtf(ss * (1.0f / DV) + a.eps);
    float gy = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) gy += sigma * w[i] * gd[i] * y[i];
    gy = group_sum<G>(gy);
    const float k3 = gy * ir * ir * ir * (1.0f / DV);
    // delta_k is formed from dY as rounded to bf16, the dY the products
    // dP = dY V^T see, so that dP - delta cancels where it should (a row
    // with one visible key has dS = 0 exactly); dlambda uses the fp32 dY
    float t1 = 0.f, t2 = 0.f, u2 = 0.f;
    uint32_t packed[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d0 = sigma * w[2 * i] * gd[2 * i] * ir - y[2 * i] * k3;
      const float d1 = sigma * w[2 * i + 1] * gd[2 * i + 1] * ir - y[2 * i + 1] * k3;
      packed[i] = pack_bf16x2(d0, d1);
      const float r0 = bf16_lo(packed[i]), r1 = bf16_hi(packed[i]);
      t1 += r0 * x1[2 * i] + r1 * x1[2 * i + 1];
      t2 += r0 * x2[2 * i] + r1 * x2[2 * i + 1];
      u2 += d0 * x2[2 * i] + d1 * x2[2 * i + 1];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) dw[i] += sigma * gd[i] * y[i] * ir;
    t1 = group_sum<G>(t1);
    t2 = group_sum<G>(t2);
    u2 = group_sum<G>(u2);
    if (valid) {
      const u32x4 pk = {packed[0], packed[1], packed[2], packed[3]};
      st16(a.dy + row * DV + 8 * gl, pk);
      if (gl == 0) {
        a.delta[row] = t1;
        a.delta[rows + row] = -lam * t2;
        dl -= u2;
      }
    }
  }
  // this wave's sums over its rows: lanes of equal gl, then dlambda over the wave
#pragma unroll
  for (int off = G; off < 64; off <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) dw[i] += __shfl_xor(dw[i], off);
  dl = wave_sum(dl);
  if (sub == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sdw[wave][8 * gl + i] = dw[i];
  }
  if (lane == 0) sdl[wave] = dl;
  __syncthreads();
  // partials stored column-major ([2d + 1][blocks]) so that the reduction
  // reads each column contiguously
  float* part = a.partial + blockIdx.x;
  const size_t np = gridDim.x;
  for (int c = threadIdx.x; c < DV; c += kPrepThreads) {
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) s += sdw[v][c];
    part[(size_t)c * np] = s;
  }
  if (threadIdx.x == 0) {
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) s += sdl[v];
    part[(size_t)DV * np] = s;
  }
}

// fixed-order sums of the per-workgroup partials, one wave per column:
// dw [2d] (columns 0..2d-1) and dlambda (column 2d); a column's nparts
// values are contiguous, read 256 at a time (four independent sums per lane)
__global__ __launch_bounds__(64) void bwd_reduce_kernel(const float* __restrict__ partial, int nparts, int width,
                                                        float* __restrict__ dweight, float* __restrict__ dlambda) {
  const int c = blockIdx.x;
  const float* col = partial + (size_t)c * nparts;
  float s4[4] = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < nparts; p0 += 256)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = p0 + 64 * k + threadIdx.x;
      if (p < nparts) s4[k] += col[p];
    }
  float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  s = wave_sum(s);
  if (threadIdx.x == 0) {
    if (c == width - 1)
      dlambda[0] = s;
    else
      dweight[c] = s;
  }
}

// ---------------------------------------------------------------------------
// dQ: a workgroup owns 4 x 16 x SUB query rows of one head (4 waves) and streams
// 32-key tiles of K1, K2, V through LDS.  Per wave and tile:
//   S_k^T (32 keys x 16 queries) = K_k Q_k^T, dP^T = V dY^T,
//   dS_k^T from A_k^T = 2^(S_k^T c - lse_k), then dQ_k^T += K_k^T dS_k^T.

constexpr int kDqKeys = 32;
// 16-row sub-tiles per wave: two where registers allow (d <= 64), so that
// every K and V fragment read from LDS feeds two matrix products
template <int D>
struct DqCfg {
  static constexpr int SUB = D <= 64 ? 2 : 1;
  static constexpr int ROWS = 4 * 16 * SUB;  // query rows per workgroup
  // d <= 64: the dQ kernel also does the row-wise preparation of its rows
  // (no bwd_prep_kernel launch); d = 128 keeps the separate kernel, whose
  // per-row values would not fit beside the dQ kernel's registers
  static constexpr bool FUSE_PREP = D <= 64;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int DV = 2 * D, KS = D / 32, KV = DV / 32, DB = D / 16, BN = kDqKeys;
  constexpr int SUB = DqCfg<D>::SUB, ROWS = DqCfg<D>::ROWS;
  constexpr bool FUSE = DqCfg<D>::FUSE_PREP;
  static_assert(BN == kTileRows, "one load instruction per 32-row column block");
  constexpr int STAGE = 2 * BN * D + BN * DV;  // K1, K2, V tiles
  constexpr int NI = D / 16;                   // load instructions per wave and tile
  constexpr int kStages = BwdStages<D, true>::N;
  __shared__ __attribute__((aligned(16))) uint16_t stg[kStages * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: branches on it stay uniform
  const int lr = lane & 15, lg = lane >> 4;
  const int N = a.N, BH = a.BH;
  const int nqt = (N + ROWS - 1) / ROWS;
  const int bh = blockIdx.x % BH;
  const int qt = CAUSAL ? nqt - 1 - (int)(blockIdx.x / BH) : (int)(blockIdx.x / BH);
  const int q0 = qt * ROWS, qw = q0 + 16 * SUB * wave;
  const size_t hb = (size_t)bh * (size_t)N;
  const size_t nrows = (size_t)BH * (size_t)N;
  const float c = a.c, lam = *a.lambda;

  const uint16_t* Q1 = (const uint16_t*)a.q1 + hb * D;
  const uint16_t* Q2 = (const uint16_t*)a.q2 + hb * D;
  const uint16_t* K1 = (const uint16_t*)a.k1 + hb * D;
  const uint16_t* K2 = (const uint16_t*)a.k2 + hb * D;
  const uint16_t* V = (const uint16_t*)a.v + hb * DV;
  const uint16_t* DY = a.dy + hb * DV;

  // per sub-tile u: this lane's query, its Q / dY rows (B operands) and
  // its row statistics
  int q[SUB];
  bf16x8 qf1[SUB][KS], qf2[SUB][KS], dyf[SUB][KV];
  float lse1[SUB], lse2[SUB], dl1[SUB], dl2[SUB];
  // the first key tiles load while the rows are prepared
  const int kend = CAUSAL ? min(N, q0 + ROWS) : N;
  const int nkt = (kend + BN - 1) / BN;
  // segments of a stage: the D/16 column blocks of K1, then of K2, then
  // the D/8 of V; wave w issues segments w, w + 4, ...
  const uint32_t lds0 = lds_offset(stg);
  auto issue = [&](int kt) {
    const uint32_t base = lds0 + 2u * (uint32_t)((kt % kStages) * STAGE);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int sg = wave + 4 * i;
      if (sg < D / 16)
        dma_block(K1, D, sg, kt * BN, N, lane, base + 1024u * sg);
      else if (sg < D / 8)
        dma_block(K2, D, sg - D / 16, kt * BN, N, lane, base + 2u * BN * D + 1024u * (sg - D / 16));
      else
        dma_block(V, DV, sg - D / 8, kt * BN, N, lane, base + 4u * BN * D + 1024u * (sg - D / 8));
    }
  };
  issue(0);
  if (kStages == 3 && nkt > 1) issue(1);
#pragma unroll
  for (int u = 0; u < SUB; ++u) q[u] = qw + 16 * u + lr;
  if constexpr (FUSE) {
    // The row-wise preparation of this workgroup's query rows (what
    // bwd_prep_kernel does for the other head widths), on the channels this
    // lane holds as dY B operands: 32 kv + 8 lg .. + 7 for kv < 2d/32, the
    // four lanes of equal lr covering the row.  dY and the deltas also go
    // to the workspace for the dK/dV kernel; the norm-weight and dlambda
    // sums of the workgroup's rows go to its column of the partials.
    const float sigma = a.out_scale;
    float dwp[KV][8];
#pragma unroll
    for (int kv = 0; kv < KV; ++kv)
#pragma unroll
      for (int e = 0; e < 8; ++e) dwp[kv][e] = 0.f;
    float dlp = 0.f;
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const bool valid = q[u] < N;
      const size_t row = hb + (size_t)min(q[u], N - 1);
      float x1[KV][8], x2[KV][8], gd[KV][8];
#pragma unroll
      for (int kv = 0; kv < KV; ++kv) {
        const int ch = 32 * kv + 8 * lg;
        const f32x4* o1 = reinterpret_cast<const f32x4*>(a.osave + row * DV + ch);
        const f32x4* o2 = reinterpret_cast<const f32x4*>(a.osave + (nrows + row) * DV + ch);
        const f32x4 p0 = o1[0], p1 = o1[1], r0 = o2[0], r1 = o2[1];
        const u32x4 g = ld16((const uint16_t*)a.dout + row * DV + ch);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x1[kv][i] = p0[i];
          x1[kv][4 + i] = p1[i];
          x2[kv][i] = r0[i];
          x2[kv][4 + i] = r1[i];
          gd[kv][2 * i] = bf16_lo(g[i]);
          gd[kv][2 * i + 1] = bf16_hi(g[i]);
        }
      }
      // the norm weight of channel c (read where used, not kept)
      auto wch = [&](int c) { return a.norm_w ? a.norm_w[c] : 1.0f; };
      float y[KV][8], ss = 0.f, gy = 0.f;
#pragma unroll
      for (int kv = 0; kv < KV; ++kv)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          y[kv][e] = x1[kv][e] - lam * x2[kv][e];
          ss += y[kv][e] * y[kv][e];
          gy += sigma * wch(32 * kv + 8 * lg + e) * gd[kv][e] * y[kv][e];
        }
      // the row's four lanes: lg = lane / 16
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      gy += __shfl_xor(gy, 16);
      gy += __shfl_xor(gy, 32);
      const float ir = 1.0f / sqrtf(ss * (1.0f / DV) + a.eps);
      const float k3 = gy * ir * ir * ir * (1.0f / DV);
      // delta_k from dY as rounded to bf16 (the dY the products see), so that
      // dP - delta cancels where it should; dlambda from the fp32 dY
      float t1 = 0.f, t2 = 0.f, u2 = 0.f;
#pragma unroll
      for (int kv = 0; kv < KV; ++kv) {
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = 32 * kv + 8 * lg + 2 * i;
          const float d0 = sigma * wch(ch) * gd[kv][2 * i] * ir - y[kv][2 * i] * k3;
          const float d1 = sigma * wch(ch + 1) * gd[kv][2 * i + 1] * ir - y[kv][2 * i + 1] * k3;
          pk[i] = pack_bf16x2(d0, d1);
          const float q0r = bf16_lo(pk[i]), q1r = bf16_hi(pk[i]);
          t1 += q0r * x1[kv][2 * i] + q1r * x1[kv][2 * i + 1];
          t2 += q0r * x2[kv][2 * i] + q1r * x2[kv][2 * i + 1];
          u2 += d0 * x2[kv][2 * i] + d1 * x2[kv][2 * i + 1];
        }
        const u32x4 pv = {pk[0], pk[1], pk[2], pk[3]};
        dyf[u][kv] = as_bf16x8(pv);
        if (valid) st16(a.dy + row * DV + 32 * kv + 8 * lg, pv);
        if (valid) {
#pragma unroll
          for (int e = 0; e < 8; ++e) dwp[kv][e] += sigma * gd[kv][e] * y[kv][e] * ir;
        }
      }
      t1 += __shfl_xor(t1, 16);
      t1 += __shfl_xor(t1, 32);
      t2 += __shfl_xor(t2, 16);
      t2 += __shfl_xor(t2, 32);
      u2 += __shfl_xor(u2, 16);
      u2 += __shfl_xor(u2, 32);
      dl1[u] = t1;
      dl2[u] = -lam * t2;
      if (valid && lg == 0) {
        a.delta[row] = dl1[u];
        a.delta[nrows + row] = dl2[u];
        dlp -= u2;
      }
    }
    // this workgroup's sums: over the 16 rows of a lane group (lr), then over
    // the waves through LDS, in a fixed order
    __shared__ float sdw[4][DV];
    __shared__ float sdl[4];
#pragma unroll
    for (int kv = 0; kv < KV; ++kv)
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) dwp[kv][e] += __shfl_xor(dwp[kv][e], off);
    dlp = wave_sum(dlp);
    if (lr == 0) {
#pragma unroll
      for (int kv = 0; kv < KV; ++kv)
#pragma unroll
        for (int e = 0; e < 8; ++e) sdw[wave][32 * kv + 8 * lg + e] = dwp[kv][e];
    }
    if (lane == 0) sdl[wave] = dlp;
    __syncthreads();
    float* part = a.partial + blockIdx.x;
    const size_t np = gridDim.x;
    for (int cix = tid; cix < DV; cix += 256) part[(size_t)cix * np] = ((sdw[0][cix] + sdw[1][cix]) + sdw[2][cix]) + sdw[3][cix];
    if (tid == 0) part[(size_t)DV * np] = ((sdl[0] + sdl[1]) + sdl[2]) + sdl[3];
  }
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    const int qc = min(q[u], N - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf1[u][ks] = as_bf16x8(ld16(Q1 + (size_t)qc * D + 32 * ks + 8 * lg));
      qf2[u][ks] = as_bf16x8(ld16(Q2 + (size_t)qc * D + 32 * ks + 8 * lg));
    }
    if constexpr (!FUSE) {
#pragma unroll
      for (int kv = 0; kv < KV; ++kv) dyf[u][kv] = as_bf16x8(ld16(DY + (size_t)qc * DV + 32 * kv + 8 * lg));
      dl1[u] = a.delta[hb + qc];
      dl2[u] = a.delta[nrows + hb + qc];
    }
    lse1[u] = a.lse[hb + qc];
    lse2[u] = a.lse[nrows + hb + qc];
  }

#pragma unroll
  for (int u = 0; u < SUB; ++u) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      settle(qf1[u][ks]);
      settle(qf2[u][ks]);
    }
#pragma unroll
    for (int kv = 0; kv < KV; ++kv) settle(dyf[u][kv]);
    settle(lse1[u]);
    settle(lse2[u]);
    settle(dl1[u]);
    settle(dl2[u]);
  }

  // the dP products start from -delta1 and so deliver dP - delta1; then
  // -lambda dP - delta2 = -lambda (dP - delta1) - (lambda delta1 + delta2)
  float nd1[SUB], c2[SUB];
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    nd1[u] = -dl1[u];
    c2[u] = lam * dl1[u] + dl2[u];
  }
  f32x4 dq1[SUB][DB], dq2[SUB][DB];
#pragma unroll
  for (int u = 0; u < SUB; ++u)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dq1[u][db] = zero_f32x4();
      dq2[u][db] = zero_f32x4();
    }
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BN;
    // tile kt has landed (with three stages tile kt+1 may still load) for
    // every wave, and everybody is done with the buffer the next issue reuses
    if (kStages == 3 && kt + 1 < nkt)
      wait_vmem_keep<NI>();
    else
      wait_vmem();
    __syncthreads();
    if (kt + kStages - 1 < nkt) issue(kt + kStages - 1);
    const uint16_t* sk1 = stg + (kt % kStages) * STAGE;
    const uint16_t* sk2 = sk1 + BN * D;
    const uint16_t* sv = sk1 + 2 * BN * D;
    // nothing visible to this wave: its dQ products still run, on zero dS,
    // so that every path through the loop updates the accumulators in place
    // (a path around them makes the compiler copy all of them every tile)
    const bool skip = qw >= N || (CAUSAL && k0 > qw + 16 * SUB - 1);

    float g1[SUB][2][4], g2[SUB][2][4];
    // the tile holds keys past a row of this wave's diagonal, or keys or
    // rows past N: only such tiles pay for the per-element mask
    const bool masked = (CAUSAL && k0 + BN - 1 > qw) || k0 + BN > N || qw + 16 * SUB > N;
    auto scores = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x4 s1[SUB], s2[SUB], dp[SUB];
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
          s1[u] = s2[u] = zero_f32x4();
          dp[u] = f32x4{nd1[u], nd1[u], nd1[u], nd1[u]};
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a1 = as_bf16x8(ld16(sk1 + boff<BN>(16 * kb + lr, 32 * ks + 8 * lg)));
          const bf16x8 a2 = as_bf16x8(ld16(sk2 + boff<BN>(16 * kb + lr, 32 * ks + 8 * lg)));
#pragma unroll
          for (int u = 0; u < SUB; ++u) {
            s1[u] = mfma16x16x32_bf16(a1, qf1[u][ks], s1[u]);
            s2[u] = mfma16x16x32_bf16(a2, qf2[u][ks], s2[u]);
          }
        }
#pragma unroll
        for (int kv = 0; kv < KV; ++kv) {
          const bf16x8 av = as_bf16x8(ld16(sv + boff<BN>(16 * kb + lr, 32 * kv + 8 * lg)));
#pragma unroll
          for (int u = 0; u < SUB; ++u) dp[u] = mfma16x16x32_bf16(av, dyf[u][kv], dp[u]);
        }
#pragma unroll
        for (int u = 0; u < SUB; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = k0 + 16 * kb + 4 * lg + j;
            const bool ok = !MASK || (key < N && q[u] < N && (!CAUSAL || key <= q[u]));
            const float e1 = ok ? exp2_fast(s1[u][j] * c - lse1[u]) : 0.f;
            const float e2 = ok ? exp2_fast(s2[u][j] * c - lse2[u]) : 0.f;
            g1[u][kb][j] = e1 * dp[u][j];
            g2[u][kb][j] = e2 * (-lam * dp[u][j] - c2[u]);
          }
        // at d = 128, keep the next block's fragment reads from being hoisted
        // here: all of a tile's fragments live at once would not fit
        if (D >= 128) __builtin_amdgcn_sched_barrier(0);
      }
    };
    // (at d = 128 a second copy of the tile body would not fit the registers)
    if (skip) {
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) g1[u][kb][j] = g2[u][kb][j] = 0.f;
    } else if (D >= 128 || masked) {
      scores(std::true_type{});
    } else {
      scores(std::false_type{});
    }
    bf16x8 b1[SUB], b2[SUB];
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      b1[u] = pack_frag(g1[u]);
      b2[u] = pack_frag(g2[u]);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 t1 = tr_frag<BN>(sk1, db, 0, lane), t2 = tr_frag<BN>(sk2, db, 0, lane);
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        dq1[u][db] = mfma16x16x32_bf16(t1, b1[u], dq1[u][db]);
        dq2[u][db] = mfma16x16x32_bf16(t2, b2[u], dq2[u][db]);
      }
    }
  }
  const float s = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    if (q[u] < N) {
      uint16_t* o1 = (uint16_t*)a.dq1 + (hb + q[u]) * D;
      uint16_t* o2 = (uint16_t*)a.dq2 + (hb + q[u]) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        store_bf16x4(o1 + 16 * db + 4 * lg, dq1[u][db], s);
        store_bf16x4(o2 + 16 * db + 4 * lg, dq2[u][db], s);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: a workgroup owns 64 keys of one head (4 waves x 16) and streams
// 32-query tiles of Q1, Q2, dY (and the rows' lse, delta) through LDS.  Per
// wave and tile: S_k (32 queries x 16 keys) = Q_k K_k^T, dP = dY V^T, then
//   dV^T += dY^T (A1 - lambda A2),  dK_k^T += Q_k^T dS_k.

// One 16-key sub-tile per wave: with two (each Q / dY fragment read feeding
// two products, as in the dQ kernel) the dK1, dK2 and dV accumulators alone
// take 128 registers at d = 64 and the kernel needs 416 (one wave per SIMD);
// that measured 19% slower than this form (66% slower squeezed into 256
// registers with spills).
// At d = 128 one kernel holding dK1, dK2 and dV (128 accumulator registers)
// plus the K and V operands needs more than 256 registers (one wave per SIMD,
// accumulators shuttled through AGPRs), so there the work is split over two
// launches of this kernel: MODE 1 accumulates dV only, MODE 2 dK1 and dK2
// only; each evaluates S again (20 d instead of 16 d flops per pair) but
// runs two waves per SIMD.  MODE 0 does both (d <= 64).
constexpr int kDkvKeys = 64;
constexpr int kDkvRows = 32;

template <int D, bool CAUSAL, int MODE>
__global__ __launch_bounds__(256, 2) void bwd_dkv_kernel(BwdArgs a) {
  constexpr bool DO_DV = MODE != 2, DO_DK = MODE != 1;
  constexpr int DV = 2 * D, KS = D / 32, KV = DV / 32, DB = D / 16, CB = DV / 16, BQ = kDkvRows;
  static_assert(BQ == kTileRows, "one load instruction per 32-row column block");
  constexpr int STAGE = 2 * BQ * D + BQ * DV;  // Q1, Q2, dY tiles
  constexpr int NI = D / 16;                   // tile load instructions per wave and tile
  constexpr int kStages = BwdStages<D, false>::N;
  __shared__ __attribute__((aligned(16))) uint16_t stg[kStages * STAGE];
  __shared__ __attribute__((aligned(16))) float sstat[kStages][4][BQ];  // lse1, lse2, delta1, delta2
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: branches on it stay uniform
  const int lr = lane & 15, lg = lane >> 4;
  const int N = a.N, BH = a.BH;
  const int bh = blockIdx.x % BH;
  const int kt = blockIdx.x / BH;  // causal: the first key tiles see the most queries
  const int k0 = kt * kDkvKeys, kw = k0 + 16 * wave, kk = kw + lr, kc = min(kk, N - 1);
  const size_t hb = (size_t)bh * (size_t)N;
  const size_t nrows = (size_t)BH * (size_t)N;
  const float c = a.c, lam = *a.lambda;

  const uint16_t* Q1 = (const uint16_t*)a.q1 + hb * D;
  const uint16_t* Q2 = (const uint16_t*)a.q2 + hb * D;
  const uint16_t* K1 = (const uint16_t*)a.k1 + hb * D;
  const uint16_t* K2 = (const uint16_t*)a.k2 + hb * D;
  const uint16_t* V = (const uint16_t*)a.v + hb * DV;
  const uint16_t* DY = a.dy + hb * DV;

  bf16x8 kf1[KS], kf2[KS], vf[KV];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf1[ks] = as_bf16x8(ld16(K1 + (size_t)kc * D + 32 * ks + 8 * lg));
    kf2[ks] = as_bf16x8(ld16(K2 + (size_t)kc * D + 32 * ks + 8 * lg));
  }
  if constexpr (DO_DK) {
#pragma unroll
    for (int kv = 0; kv < KV; ++kv) vf[kv] = as_bf16x8(ld16(V + (size_t)kc * DV + 32 * kv + 8 * lg));
  }

#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    settle(kf1[ks]);
    settle(kf2[ks]);
  }
  if constexpr (DO_DK) {
#pragma unroll
    for (int kv = 0; kv < KV; ++kv) settle(vf[kv]);
  }

  f32x4 dk1[DB], dk2[DB], dv[CB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk1[db] = zero_f32x4();
    dk2[db] = zero_f32x4();
  }
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) dv[cb] = zero_f32x4();

  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? k0 / BQ : 0;
  // segments of a stage: the D/16 column blocks of Q1, then of Q2, then the
  // D/8 of dY; wave w issues segments w, w + 4, ...; waves 0 and 1 also
  // load the rows' (lse1, lse2) and (delta1, delta2) pairs, one 4-byte
  // value per lane (lanes 0-31 the first of the pair, 32-63 the second)
  const uint32_t lds0 = lds_offset(stg);
  const uint32_t lds_st = lds_offset(sstat);
  auto issue = [&](int qt) {
    const int q0 = qt * BQ, buf = qt % kStages;
    const uint32_t base = lds0 + 2u * (uint32_t)(buf * STAGE);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int sg = wave + 4 * i;
      if (sg < D / 16)
        dma_block(Q1, D, sg, q0, N, lane, base + 1024u * sg);
      else if (sg < D / 8)
        dma_block(Q2, D, sg - D / 16, q0, N, lane, base + 2u * BQ * D + 1024u * (sg - D / 16));
      else
        dma_block(DY, DV, sg - D / 8, q0, N, lane, base + 4u * BQ * D + 1024u * (sg - D / 8));
    }
    if (wave < 2) {
      // two rows of nrows apart: the byte offset stays below 2^32 because
      // the host limits B * H * N to 2^28
      const float* src = (wave == 0 ? a.lse : a.delta) + hb;
      const uint32_t off = 4u * (uint32_t)((size_t)(lane >> 5) * nrows + (size_t)min(q0 + (lane & 31), N - 1));
      lds_dma4_s(src, off, lds_st + 4u * (uint32_t)((buf * 4 + 2 * wave) * BQ));
    }
  };
  issue(qt0);
  if (kStages == 3 && qt0 + 1 < nqt) issue(qt0 + 1);
  for (int qt = qt0; qt < nqt; ++qt) {
    const int q0 = qt * BQ;
    // tile qt has landed (with three stages tile qt+1 may still load) for
    // every wave, and everybody is done with the buffer the next issue reuses
    if (kStages == 3 && qt + 1 < nqt) {
      if (wave < 2)
        wait_vmem_keep<NI + 1>();
      else
        wait_vmem_keep<NI>();
    } else {
      wait_vmem();
    }
    __syncthreads();
    if (qt + kStages - 1 < nqt) issue(qt + kStages - 1);
    const uint16_t* sq1 = stg + (qt % kStages) * STAGE;
    const uint16_t* sq2 = sq1 + BQ * D;
    const uint16_t* sdy = sq1 + 2 * BQ * D;
    const float(*sst)[BQ] = sstat[qt % kStages];
    if (kw >= N || (CAUSAL && q0 + BQ - 1 < kw)) continue;  // nothing visible to this wave

    float d1[2][4], gs1[2][4], gs2[2][4];
    // the tile holds rows before one of this wave's keys, or rows or keys
    // past N: only such tiles pay for the per-element mask
    const bool masked = (CAUSAL && q0 < kw + 15) || q0 + BQ > N || kw + 16 > N;
    auto scores = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x4 s1 = zero_f32x4(), s2 = zero_f32x4(), dp = zero_f32x4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s1 = mfma16x16x32_bf16(as_bf16x8(ld16(sq1 + boff<BQ>(16 * qb + lr, 32 * ks + 8 * lg))), kf1[ks], s1);
          s2 = mfma16x16x32_bf16(as_bf16x8(ld16(sq2 + boff<BQ>(16 * qb + lr, 32 * ks + 8 * lg))), kf2[ks], s2);
        }
        if constexpr (DO_DK) {
#pragma unroll
          for (int kv = 0; kv < KV; ++kv)
            dp = mfma16x16x32_bf16(as_bf16x8(ld16(sdy + boff<BQ>(16 * qb + lr, 32 * kv + 8 * lg))), vf[kv], dp);
        }
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(&sst[0][16 * qb + 4 * lg]);
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(&sst[1][16 * qb + 4 * lg]);
        const f32x4 t1 = *reinterpret_cast<const f32x4*>(&sst[2][16 * qb + 4 * lg]);
        const f32x4 t2 = *reinterpret_cast<const f32x4*>(&sst[3][16 * qb + 4 * lg]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int qi = q0 + 16 * qb + 4 * lg + j;
          const bool ok = !MASK || (qi < N && kk < N && (!CAUSAL || kk <= qi));
          const float e1 = ok ? exp2_fast(s1[j] * c - l1[j]) : 0.f;
          const float e2 = ok ? exp2_fast(s2[j] * c - l2[j]) : 0.f;
          d1[qb][j] = e1 - lam * e2;
          gs1[qb][j] = e1 * (dp[j] - t1[j]);
          gs2[qb][j] = e2 * (-lam * dp[j] - t2[j]);
        }
        if (D >= 128) __builtin_amdgcn_sched_barrier(0);  // as in the dQ kernel
      }
    };
    // (at d = 128 without the causal mask the compiler's schedule of a second,
    // unmasked copy of the tile body spills, so there every tile takes the
    // masked one)
    if ((D >= 128 && !CAUSAL) || masked)
      scores(std::true_type{});
    else
      scores(std::false_type{});
    if constexpr (DO_DV) {
      const bf16x8 bd = pack_frag(d1);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) dv[cb] = mfma16x16x32_bf16(tr_frag<BQ>(sdy, cb, 0, lane), bd, dv[cb]);
    }
    if constexpr (DO_DK) {
      const bf16x8 b1 = pack_frag(gs1), b2 = pack_frag(gs2);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dk1[db] = mfma16x16x32_bf16(tr_frag<BQ>(sq1, db, 0, lane), b1, dk1[db]);
        dk2[db] = mfma16x16x32_bf16(tr_frag<BQ>(sq2, db, 0, lane), b2, dk2[db]);
      }
    }
  }
  if (kk < N) {
    const float s = 1.0f / sqrtf((float)D);
    if constexpr (DO_DK) {
      uint16_t* o1 = (uint16_t*)a.dk1 + (hb + kk) * D;
      uint16_t* o2 = (uint16_t*)a.dk2 + (hb + kk) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        store_bf16x4(o1 + 16 * db + 4 * lg, dk1[db], s);
        store_bf16x4(o2 + 16 * db + 4 * lg, dk2[db], s);
      }
    }
    if constexpr (DO_DV) {
      uint16_t* ov = (uint16_t*)a.dv + (hb + kk) * DV;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) store_bf16x4(ov + 16 * cb + 4 * lg, dv[cb], 1.0f);
    }
  }
}

// Eq. 2 backward: dlq1 = dl e1 lk1, dlk1 = dl e1 lq1, dlq2 = -dl e2 lk2,
// dlk2 = -dl e2 lq2 with e_k = exp(lqk . lkk).  One wave.
__global__ __launch_bounds__(64) void lambda_bwd_kernel(const float* __restrict__ lq1, const float* __restrict__ lk1,
                                                        const float* __restrict__ lq2, const float* __restrict__ lk2,
                                                        int d, const float* __restrict__ dlambda,
                                                        float* __restrict__ dlq1, float* __restrict__ dlk1,
                                                        float* __restrict__ dlq2, float* __restrict__ dlk2) {
  float x = 0.f, y = 0.f;
  for (int i = threadIdx.x; i < d; i += 64) {
    x += lq1[i] * lk1[i];
    y += lq2[i] * lk2[i];
  }
  x = wave_sum(x);
  y = wave_sum(y);
  const float g = dlambda[0];
  const float g1 = g * expf(x), g2 = -g * expf(y);
  for (int i = threadIdx.x; i < d; i += 64) {
    dlq1[i] = g1 * lk1[i];
    dlk1[i] = g1 * lq1[i];
    dlq2[i] = g2 * lk2[i];
    dlk2[i] = g2 * lq2[i];
  }
}

// ---------------------------------------------------------------------------
// dispatch

// columns of per-workgroup partial sums the backward writes (one per dQ
// workgroup where the dQ kernel does the row-wise preparation)
int bwd_partial_count(int BH, int N, int d) {
  const long long rows = (long long)BH * N;
  switch (d) {
    case 32: return (int)(((N + DqCfg<32>::ROWS - 1) / DqCfg<32>::ROWS) * (long long)BH);
    case 64: return (int)(((N + DqCfg<64>::ROWS - 1) / DqCfg<64>::ROWS) * (long long)BH);
    default: return bwd_prep_blocks(rows);
  }
}

int bwd_prep_blocks(long long rows) {
  const long long per = kPrepThreads / 64;
  const long long need = (rows + per - 1) / per;
  return (int)(need < 1024 ? (need > 0 ? need : 1) : 1024);
}

template <int D, bool C>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
  const long long rows = (long long)a.BH * a.N;
  const unsigned gq = (unsigned)(((a.N + DqCfg<D>::ROWS - 1) / DqCfg<D>::ROWS) * (long long)a.BH);
  if constexpr (DqCfg<D>::FUSE_PREP) {
    // dQ first: it writes dY, the deltas and the partial sums
    hipLaunchKernelGGL((bwd_dq_kernel<D, C>), dim3(gq), dim3(256), 0, s, a);
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3(2 * D + 1), dim3(64), 0, s, a.partial, (int)gq, 2 * D + 1, a.dweight,
                       a.dlambda);
  } else {
    const int np = bwd_prep_blocks(rows);
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3(np), dim3(kPrepThreads), 0, s, a);
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3(2 * D + 1), dim3(64), 0, s, a.partial, np, 2 * D + 1, a.dweight,
                       a.dlambda);
    hipLaunchKernelGGL((bwd_dq_kernel<D, C>), dim3(gq), dim3(256), 0, s, a);
  }
  const unsigned gk = (unsigned)(((a.N + kDkvKeys - 1) / kDkvKeys) * (long long)a.BH);
  if constexpr (D >= 128) {
    hipLaunchKernelGGL((bwd_dkv_kernel<D, C, 1>), dim3(gk), dim3(256), 0, s, a);
    hipLaunchKernelGGL((bwd_dkv_kernel<D, C, 2>), dim3(gk), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((bwd_dkv_kernel<D, C, 0>), dim3(gk), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(int d, bool causal, const BwdArgs& a, hipStream_t stream) {
  switch (d) {
    case 32: return causal ? launch_bwd_d<32, true>(a, stream) : launch_bwd_d<32, false>(a, stream);
    case 64: return causal ? launch_bwd_d<64, true>(a, stream) : launch_bwd_d<64, false>(a, stream);
    case 128: return causal ? launch_bwd_d<128, true>(a, stream) : launch_bwd_d<128, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lambda_bwd(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int d,
                             const float* dlambda, float* dlq1, float* dlk1, float* dlq2, float* dlk2,
                             hipStream_t stream) {
  hipLaunchKernelGGL(lambda_bwd_kernel, dim3(1), dim3(64), 0, stream, lq1, lk1, lq2, lk2, d, dlambda, dlq1, dlk1,
                     dlq2, dlk2);
  return hipGetLastError();
}

}  // namespace diffattn
