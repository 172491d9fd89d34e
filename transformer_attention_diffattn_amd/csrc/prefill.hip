// Fused differential-attention prefill for gfx950 (MI355X).
//
// Computes, for every query row i of every (batch, head):
//   Y_i   = sum_j [softmax_j(Q1_i.K1_j/sqrt d) - lambda softmax_j(Q2_i.K2_j/sqrt d)] V_j
//   out_i = (1 - lambda_init) w * Y_i / sqrt(mean(Y_i^2) + eps)
// (Eq. 1 of "Differential Transformer: Canceling Context Noise with
// Differential Attention", section "Cancelling Context Noise Through Attention
// Map Subtraction"; Eq. 3 of the "Differential Transformer" sample review,
// "Summary", with the head-wise RMSNorm of its "Weaknesses" section.)
//
// One pass over the keys.  Because the two maps' normalisers are only known
// at the end, each query row carries two online-softmax states (running
// reference maximum m, denominator l, numerator O[2d]); the V tile staged in
// LDS feeds both maps' PV products (A1 V - lambda A2 V = (A1 - lambda A2) V).
//
// Layout of the work (bf16 kernel): a workgroup takes (128 query rows, head)
// items in turn (8 waves, 32 rows and one map each) and streams BN-key tiles
// of K1, K2, V through a ring of LDS stage buffers.  Products are computed
// transposed so that every per-row quantity lives in the lane of its query:
//   S^T = K Q^T   (16x16x32 bf16 MFMA, A = K rows from LDS, B = Q^T in VGPRs)
//   O^T += V^T P^T (A = V^T from LDS, B = P^T built in-lane from S^T)
//   l   += 1^T P^T (the same MFMA with A = ones: row sums of the rounded P)
// In a 16x16 MFMA result lane L holds column L%16 (the query) and rows
// 4*(L/16)+j, so a lane owns one query's scores for 4 keys per 16-key block
// and one query's outputs for 4 channels per 16-channel block.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace diffattn {

// ---------------------------------------------------------------------------
// online softmax step for one map (shared by both element types)
//
// t[]: this lane's scaled scores (log2 units) for the tile, -inf if masked.
// m:   the row's reference maximum; l/O: accumulators to rescale.
template <int NT, int CB>
__device__ __forceinline__ void softmax_step(float (&t)[NT], float& m, f32x4& l, f32x4 (&O)[CB]) {
  float mt = t[0];
#pragma unroll
  for (int i = 1; i < NT; ++i) mt = fmaxf(mt, t[i]);
  mt = max_over_lane_groups(mt);
  if (wave_any(mt > m + kRescaleThreshold)) {
    const float mn = fmaxf(m, mt);
    const float alpha = (mn == -INFINITY) ? 1.0f : exp2_fast(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) O[cb] *= alpha;
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) t[i] = exp2_fast(t[i] - m);
}

// Y = O1/l1 - lambda O2/l2, then (optionally) the head-wise RMSNorm and the
// (1 - lambda_init) scale.  Returns the 4*CB values this lane owns.
template <int CB, bool NORM>
__device__ __forceinline__ void epilogue_values(const f32x4 (&O1)[CB], const f32x4 (&O2)[CB], float l1,
                                                float l2, float lam, float out_scale, float eps,
                                                const float* __restrict__ w, int lg, f32x4 (&y)[CB]) {
  constexpr int DV = CB * 16;
  const float i1 = 1.0f / l1;
  const float i2 = lam / l2;
  float ss = 0.f;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float yv = O1[cb][j] * i1 - O2[cb][j] * i2;
      y[cb][j] = yv;
      ss += yv * yv;
    }
  }
  if (NORM) {
    ss = sum_over_lane_groups(ss);
    const float r = out_scale / sqrtf(ss * (1.0f / DV) + eps);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = 16 * cb + 4 * lg + j;
        y[cb][j] *= r * (w ? w[col] : 1.0f);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel
//
// A work item is BM = 128 query rows of one head; a workgroup runs 8 waves:
// wave w computes map (w & 1) for the 32 rows of row group (w >> 1), as two
// 16-row sub-tiles so that each K or V fragment read from LDS feeds two
// MFMAs.  The two maps of a row group only meet in the epilogue, where the
// map-2 wave hands O2/l2 to the map-1 wave through LDS.  K1, K2 and V tiles
// of BN keys arrive by direct global->LDS loads into a ring of stage buffers
// (later tiles load while earlier ones are consumed).  Rows are XOR-swizzled in 16-byte
// chunks so that K fragment reads are free of bank conflicts.  A V tile is
// stored as [16-channel block][key][16 channels]: the transposing LDS read
// (ds_read_b64_tr_b16) of a V^T fragment then covers 512 contiguous bytes,
// and every such read of a wave uses one address register plus an immediate.

// Shape per head width: waves per workgroup (two per row group), 16-row
// sub-tiles per wave, keys per tile.
template <int D>
struct Bf16Cfg {
  static constexpr int WAVES = 8;
  static constexpr int SUB = 2;
  static constexpr int BN = D >= 128 ? 32 : 64;  // d = 128: keeps a wave within 256 registers
  // Software-pipelined tile loop (QK^T of the next tile overlaps the
  // softmax of the current one): tiles t and t+1 are read while t+2 loads,
  // so three LDS stage buffers.
  static constexpr int STAGES = 3;
  static constexpr int PV_FENCE = D >= 128 ? 4 : 0;  // channel blocks between scheduling fences
  // LDS fragment reads issued ahead of their MFMAs in the pipelined loop
  static constexpr int K_AHEAD = 1;  // 16-key blocks of K
  static constexpr int V_AHEAD = 2;  // V^T fragments
};

// F8: queries and keys are e4m3 bytes (QK^T on the 16x16x128 fp8 product,
// d = 128 only); a K tile then fills the first half of its slot.
template <int D, bool F8 = false>
struct Bf16Tile {
  static_assert(!F8 || D == 128, "the fp8 QK^T product is 128 deep");
  static constexpr int DV = 2 * D;
  static constexpr int KB = F8 ? 1 : 2;  // bytes per query/key element
  static constexpr int WAVES = Bf16Cfg<D>::WAVES;  // row groups x 2 maps
  static constexpr int SUB = Bf16Cfg<D>::SUB;      // 16-row sub-tiles per wave
  static constexpr int BM = 16 * SUB * (WAVES / 2);
  static constexpr int BN = Bf16Cfg<D>::BN;
  static constexpr int STAGES = Bf16Cfg<D>::STAGES;
  static constexpr int K_AHEAD = Bf16Cfg<D>::K_AHEAD;
  static constexpr int V_AHEAD = Bf16Cfg<D>::V_AHEAD;
  static_assert(STAGES >= 3, "stage ring of the pipelined tile loop");
  static constexpr int PV_FENCE = Bf16Cfg<D>::PV_FENCE;
  static constexpr int KS = F8 ? 1 : (D + 31) / 32;  // k-steps of the QK^T MFMA
  static constexpr int NB = BN / 16;        // 16-key score blocks per tile
  static constexpr int NC = BN / 32;        // 32-key PV k-steps per tile
  static constexpr int CB = DV / 16;        // 16-channel output blocks
  static constexpr int NCH = D * KB / 16;   // 16-byte chunks per K row
  static constexpr int RPK = NCH >= 16 ? 1 : 16 / NCH;  // K rows per 256 bytes
  static constexpr int KSEG = BN * NCH / 64;            // 1 KB segments per K tile
  static constexpr int VSEG = CB * BN / 32;             // 1 KB = 32 keys of one channel block
  static constexpr int NSEG = 2 * KSEG + VSEG;
  static constexpr int KTILE = BN * D;  // 16-bit elements (slot of one K tile)
  static constexpr int VTILE = BN * DV;
  static constexpr int STAGE = 2 * KTILE + VTILE;
  static_assert(NSEG % (WAVES / 2) == 0, "segments split evenly over the loading waves");

  // physical 16-byte chunk of logical chunk c in K row r
  static __device__ __forceinline__ int kchunk(int r, int c) { return c ^ ((r / RPK) % NCH); }
};


// v_max_f32 as such: the operands here are never NaN (scores, or -inf
// where masked), so the quieting copies fmaxf would add are not needed
__device__ __forceinline__ float max_f32(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// max over lanes l, l^16, l^32, l^48 without LDS traffic (v_permlane*_swap)
__device__ __forceinline__ float max4_groups(float x) {
  const uint32_t xb = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
  x = max_f32(u32_as_f32(r[0]), u32_as_f32(r[1]));
  const uint32_t yb = __builtin_bit_cast(uint32_t, x);
  auto q = __builtin_amdgcn_permlane16_swap(yb, yb, false, false);
  return max_f32(u32_as_f32(q[0]), u32_as_f32(q[1]));
}

// QK^T operand fragments: 8 bf16, or 32 e4m3 bytes
__device__ __forceinline__ f32x4 mma_qk(bf16x8 a, bf16x8 b, f32x4 c) { return mfma16x16x32_bf16(a, b, c); }
__device__ __forceinline__ f32x4 mma_qk(i32x8 a, i32x8 b, f32x4 c) { return mfma16x16x128_fp8(a, b, c); }
__device__ __forceinline__ i32x8 cat_i32x8(u32x4 lo, u32x4 hi) {
  i32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (int)lo[i];
    r[4 + i] = (int)hi[i];
  }
  return r;
}

// SAVE: the training forward (also writes the per-map statistics).
// F8: e4m3 queries and keys with per-tensor scales (a.qk_scale).
// XCD: the per-XCD schedule of long sequences (see the schedule below; the
// host picks it when its conditions hold).
template <int D, bool CAUSAL, bool NORM, bool SAVE, bool F8, bool XCD = false>
__global__ __launch_bounds__(64 * Bf16Cfg<D>::WAVES) void prefill_bf16_kernel(PrefillArgs a) {
  using T = Bf16Tile<D, F8>;
  using QFrag = std::conditional_t<F8, i32x8, bf16x8>;
  constexpr int DV = T::DV, BN = T::BN, KS = T::KS, NB = T::NB, NC = T::NC, CB = T::CB, SUB = T::SUB;
  constexpr int NCH = T::NCH, KSEG = T::KSEG, KTILE = T::KTILE;
  constexpr int RG = T::WAVES / 2;  // row groups

  constexpr int STAGES = T::STAGES;
  __shared__ __attribute__((aligned(16))) uint16_t stages[STAGES * T::STAGE];
  __shared__ float wsh[DV];  // norm weight
  __shared__ float ssx[T::WAVES][T::SUB * 16];  // epilogue: half-row sums of squares
  __shared__ float dnx[T::WAVES][T::SUB * 16];  // epilogue: per-row scales

  const int lane = threadIdx.x & 63;
  // wave-uniform values live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mp = wave & 1;   // which map this wave computes
  const int rg = wave >> 1;  // row group
  const int lr = lane & 15;  // query column of the 16x16 blocks owned by this lane
  const int lg = lane >> 4;  // lane group: rows 4*lg..4*lg+3 of each block
  const int N = a.N;
  // fp8: the dequantisation scales of this wave's map fold into the logit scale
  const float c = F8 ? a.c * (mp ? a.qk_scale[2] * a.qk_scale[3] : a.qk_scale[0] * a.qk_scale[1]) : a.c;
  const float lam = *a.lambda;
  for (int i = threadIdx.x; i < DV; i += blockDim.x) wsh[i] = a.norm_w ? a.norm_w[i] : 1.0f;

  // Persistent schedule: work items (query tile, head) are ordered longest
  // first under the causal mask, heads fastest; workgroup g takes one item
  // per round of G items, walking the rounds in alternating directions so
  // that every workgroup's total is about the same.  When G is a multiple of
  // B*H only the tile order is reversed, keeping each head on one workgroup
  // position (and so on one XCD's L2).
  //   Long sequences (XCD: a multiple of, and at least four, chunks of W =
  // G/8 query tiles per head) are grouped per XCD instead: workgroups are dealt
  // to the 8 XCDs round robin (g % 8), and in each round the W workgroups of
  // one XCD take the W query tiles of one chunk of ONE head, so they stream
  // the same key tiles through that XCD's L2 at about the same time (rather
  // than each L2 serving the key streams of several heads).  Chunks go
  // longest first, heads fastest, chunk c of the order to XCD c % 8 in round
  // c / 8 (to XCD 7 - c % 8 in odd rounds, so that the XCDs' totals even
  // out); within a chunk workgroup j takes tile j, or W-1-j in odd rounds,
  // so that the totals of an XCD's workgroups even out.
  const int G = gridDim.x, g = blockIdx.x, BH = a.BH;
  const int n_items = a.n_qtiles * BH;  // below 2^31 (checked by the host)
  // An odd number R >= 3 of whole rounds: alternating directions leave the
  // last round's spread (item lengths fall about linearly with the item
  // index), so the last three rounds take the three permutations P_k of
  // 0..n-1 (n even, h = n/2): P_0(v) = v, P_1(v) = (v + h - 1) mod n,
  // P_2(v) = n - 1 - 2v (v < h), 0 (v = h), 2n - 2v (v > h), whose sum is
  // n + h - 2 or n + h - 1 for every v.  With G a multiple of 16 they act on
  // g / 8 and g % 8 apart (position 8 P_k(g / 8) + P_k(g % 8)), which keeps
  // every XCD's items of a round on a few heads (a head's items differ by
  // multiples of B*H, and XCD = g % 8).  Positions 1 and 2 of this
  // workgroup, computed once.
  // (scalar registers: the grid size arrives through a vector load, and the
  // values live through the whole kernel)
  const int R_all = __builtin_amdgcn_readfirstlane(n_items / G);
  const bool tail3 = __builtin_amdgcn_readfirstlane(n_items == R_all * G && (R_all & 1) && R_all >= 3 && !(G & 1));
  const int R3 = R_all - 3;
  auto tail_perm = [](int k, int v, int n) {  // (no division: v + h - 1 < 2n)
    const int h = n / 2, w = v + h - 1;
    return k == 1 ? (w >= n ? w - n : w) : v < h ? n - 1 - 2 * v : v == h ? 0 : 2 * n - 2 * v;
  };
  const int tail_pos1 = __builtin_amdgcn_readfirstlane(
      (G % 16 == 0) ? 8 * tail_perm(1, g / 8, G / 8) + tail_perm(1, g % 8, 8) : tail_perm(1, g, G));
  const int tail_pos2 = __builtin_amdgcn_readfirstlane(
      (G % 16 == 0) ? 8 * tail_perm(2, g / 8, G / 8) + tail_perm(2, g % 8, 8) : tail_perm(2, g, G));
  auto item_at = [&](int r) -> int {
    if constexpr (XCD) {
      constexpr int NXCD = 8;
      const int W = G / NXCD;
      // c / BH without the vector code of an integer division: a multiply
      // by ceil(2^32 / BH) in scalar registers, corrected by one either way
      const uint32_t inv_bh = __builtin_amdgcn_readfirstlane((uint32_t)(0xffffffffu / (uint32_t)BH) + 1u);
      // chunk: XCD x takes chunk 8 r + x in even rounds, 8 r + 7 - x in odd
      // ones, so every XCD's chunks add up to the same number of key tiles
      const int c = r * NXCD + ((r & 1) ? NXCD - 1 - g % NXCD : g % NXCD);
      if (c >= n_items / W) return -1;
      int kk = (int)__umulhi((uint32_t)c, inv_bh);
      kk -= kk * BH > c ? 1 : 0;
      kk += (kk + 1) * BH <= c ? 1 : 0;
      kk = __builtin_amdgcn_readfirstlane(kk);
      const int j = g / NXCD;
      const int qi = kk * W + ((r & 1) ? W - 1 - j : j);
      return __builtin_amdgcn_readfirstlane(qi * BH + (c - kk * BH));
    } else {
      // integer division expands to vector code: keep the result scalar
      const int alt = __builtin_amdgcn_readfirstlane((G % BH == 0) ? ((G / BH - 1 - g / BH) * BH + g % BH) : (G - 1 - g));
      int x = (r & 1) ? alt : g;
      if (tail3 && r >= R3) {
        // (arithmetic, not a chain of selects: the compiler turns such a
        // chain into a small indexed table in memory)
        const int k = r - R3;
        x = g + (k == 1 ? 1 : 0) * (tail_pos1 - g) + (k == 2 ? 1 : 0) * (tail_pos2 - g);
      }
      const int i = r * G + x;
      return __builtin_amdgcn_readfirstlane(i < n_items ? i : -1);
    }
  };

  // One item; every field is wave-uniform and kept in scalar registers.
  struct Item {
    int bh, q0, qw0, nkt;
  };
  auto decode_item = [&](int i) {
    Item it;
    const int qi = __builtin_amdgcn_readfirstlane(i / BH);
    it.bh = __builtin_amdgcn_readfirstlane(i - qi * BH);
    const int qt = CAUSAL ? a.n_qtiles - 1 - qi : qi;
    it.q0 = qt * T::BM;
    it.qw0 = it.q0 + 16 * SUB * rg;
    const int kend = CAUSAL ? min(N, it.q0 + T::BM) : N;
    it.nkt = (kend + BN - 1) / BN;
    return it;
  };
  auto head_row = [&](const Item& it) { return (size_t)it.bh * (size_t)N; };

  // Q^T fragments (B operand of S^T = K Q^T): dims 32ks+8lg..+7 of the row
  // (fp8: bytes 32lg..+31 of the row)
  QFrag qf[SUB][KS];
  auto load_q = [&](const Item& it) {
    if constexpr (F8) {
      const uint8_t* Qm = (const uint8_t*)(mp ? a.q2 : a.q1) + head_row(it) * D;
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const uint8_t* qp = Qm + (size_t)min(it.qw0 + 16 * u + lr, N - 1) * D + 32 * lg;
        qf[u][0] = cat_i32x8(ld16(qp), ld16(qp + 16));
      }
      return;
    } else {
    const uint16_t* Qm = (const uint16_t*)(mp ? a.q2 : a.q1) + head_row(it) * D;
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int qrow = min(it.qw0 + 16 * u + lr, N - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int dc = 32 * ks + 8 * lg;
        qf[u][ks] = as_bf16x8(dc < D ? ld16(Qm + (size_t)qrow * D + dc) : zero_u32x4());
      }
    }
    }
  };

  // Direct global->LDS loads of one key tile: each instruction moves 1 KB
  // (64 lanes x 16 B) to consecutive LDS; a lane fetches the global chunk
  // that the swizzle assigns to its LDS position.  Segment i of this wave is
  // one 1 KB piece of the K1 (sel 0), K2 (1) or V (2) tile; which piece, its
  // LDS offset in a stage (wave-uniform), and the lane's byte offset inside
  // the tile and key row (per lane) are the same for every tile.
  // Only the first wave on each SIMD (waves 0..3, which the SIMD's
  // arbitration favours and which therefore run ahead within a tile step)
  // issues loads: the texture unit takes a tile's instructions one after the
  // other, so an issuing wave stalls until its last one is accepted, and that
  // stall then falls on the wave that would otherwise wait at the next barrier.
  constexpr int LOADERS = T::WAVES / 2;
  constexpr int SPW = T::NSEG / LOADERS;  // segments per loading wave
  int seg_sel[SPW];
  uint32_t seg_lds[SPW], seg_off[SPW];
  int seg_row[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int seg = (wave % LOADERS) + i * LOADERS;
    if (seg < 2 * KSEG) {
      const int sg = seg % KSEG;
      const int r = sg * (64 / NCH) + lane / NCH;
      seg_sel[i] = seg / KSEG;
      seg_lds[i] = 2u * (uint32_t)((seg / KSEG) * KTILE + sg * 512);
      seg_row[i] = r;
      seg_off[i] = (uint32_t)(r * D * T::KB + 16 * T::kchunk(r, lane % NCH));
    } else {
      // segment sg: keys 32*(sg % (BN/32)).. of channel block sg / (BN/32);
      // lane: key +lane/2, channels +8*(lane&1)
      const int sg = seg - 2 * KSEG;
      const int r = 32 * (sg % (BN / 32)) + (lane >> 1);
      seg_sel[i] = 2;
      seg_lds[i] = 2u * (uint32_t)(2 * KTILE + sg * 512);
      seg_row[i] = r;
      seg_off[i] = 2u * (uint32_t)(r * DV + 16 * (sg / (BN / 32)) + 8 * (lane & 1));
    }
  }
  const uint32_t lds_stages = lds_offset(stages);  // LDS byte address of the ring
  auto issue_tile = [&](int buf, const Item& it, int kt) {
    const int kb = kt * BN;
    const size_t row0 = head_row(it) + (size_t)kb;
    const char* bk1 = (const char*)a.k1 + row0 * (T::KB * D);
    const char* bk2 = (const char*)a.k2 + row0 * (T::KB * D);
    const char* bv = (const char*)a.v + row0 * (2 * DV);
    const uint32_t lds0 = lds_stages + (uint32_t)(buf * T::STAGE * 2);
    if (wave >= LOADERS) return;
    if (kb + BN <= N) {
#pragma unroll
      for (int i = 0; i < SPW; ++i)
        lds_dma16_s(seg_sel[i] == 0 ? bk1 : (seg_sel[i] == 1 ? bk2 : bv), seg_off[i], lds0 + seg_lds[i]);
    } else {
      // ragged last tile: rows past N - 1 read row N - 1 instead
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const uint32_t row_bytes = seg_sel[i] == 2 ? 2 * DV : T::KB * D;
        const uint32_t off = seg_off[i] - (uint32_t)max(0, kb + seg_row[i] - (N - 1)) * row_bytes;
        lds_dma16_s(seg_sel[i] == 0 ? bk1 : (seg_sel[i] == 1 ? bk2 : bv), off, lds0 + seg_lds[i]);
      }
    }
  };

  f32x4 O[SUB][CB], L[SUB];
  float m[SUB];
  const u32x4 ones_u = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  const bf16x8 ones = as_bf16x8(ones_u);

  using Scores = float[SUB][4 * NB];  // this lane's raw scores of one tile
  using PFrags = bf16x8[NC][SUB];      // P^T fragments of one tile

  // K fragment (A operand) of key row kr of the K tile at ks_, k-step ks
  auto kfrag = [&](const uint16_t* ks_, int kr, int ks) -> QFrag {
    if constexpr (F8) {
      const uint8_t* row = (const uint8_t*)ks_ + kr * D;
      return cat_i32x8(ld16(row + 16 * T::kchunk(kr, 2 * lg)), ld16(row + 16 * T::kchunk(kr, 2 * lg + 1)));
    } else {
      const int ch = 4 * ks + lg;
      return as_bf16x8(ch < NCH ? ld16(ks_ + kr * D + 8 * T::kchunk(kr, ch)) : zero_u32x4());
    }
  };

  // S^T = K Q^T for both sub-tiles; block b of sc holds keys 16b+4lg+j.
  // MASK: the tile holds keys past some row's diagonal or past N; those
  // tiles take a separate instantiation so that the common unmasked tiles
  // carry no per-element compare/select work.
  auto qk = [&](Scores& sc, const uint16_t* stg, int kb, int qw0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const uint16_t* ks_ = stg + mp * KTILE;
    // key 16b+4lg+j of the tile is visible to sub-tile u's query iff
    // 16b+j <= lim[u] (a compile-time constant against one register)
    int lim[SUB];
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int last_key = CAUSAL ? min(qw0 + 16 * u + lr, N - 1) : N - 1;
      lim[u] = last_key - kb - 4 * lg;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int kr = 16 * b + lr;
      f32x4 acc[SUB];
#pragma unroll
      for (int u = 0; u < SUB; ++u) acc[u] = zero_f32x4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const QFrag ka = kfrag(ks_, kr, ks);
#pragma unroll
        for (int u = 0; u < SUB; ++u) acc[u] = mma_qk(ka, qf[u][ks], acc[u]);
      }
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x = acc[u][j];
          if (MASK) x = (16 * b + j <= lim[u]) ? x : -INFINITY;
          sc[u][4 * b + j] = x;
        }
    }
  };

  // running maxima: the tile's row maxima (log2 units) and whether any row
  // of the wave needs a new reference; then one rescale branch per tile for
  // both sub-tiles
  auto tile_max = [&](const Scores& sc, float (&mt)[SUB]) {
    bool need = false;
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      float x = sc[u][0];
#pragma unroll
      for (int i = 1; i < 4 * NB; ++i) x = fmaxf(x, sc[u][i]);
      mt[u] = max4_groups(x) * c;
      need |= mt[u] > m[u] + kRescaleThreshold;
    }
    return need;
  };
  auto rescale = [&](const float (&mt)[SUB], bool need) {
    if (wave_any(need)) {
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const float mn = fmaxf(m[u], mt[u]);
        const float alpha = (mn == -INFINITY) ? 1.0f : exp2_fast(m[u] - mn);
        m[u] = mn;
        L[u] *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) O[u][cb] *= alpha;
      }
    }
  };
  auto update_max = [&](const Scores& sc) {
    float mt[SUB];
    const bool need = tile_max(sc, mt);
    rescale(mt, need);
  };

  // O^T += V^T P^T.  With a second set of fragments (lo), each V fragment
  // read also feeds O^T += V^T lo^T: P enters as the sum of two bf16 terms.
  auto pv = [&](const uint16_t* stg, const PFrags& pf, const PFrags& lo, bool split) {
    const uint16_t* vs = stg + 2 * KTILE;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        u32x4 vu;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // lane lr of group lg points at key 32cc+16h+4lg+lr/4, channels
          // 16cb+4(lr%4)..+3: in the [block][key][16] layout that is
          // element 16*(BN*cb + 32cc + 16h) + 4*lane
          const u32x2 t2 = lds_read_tr16(vs + 16 * (BN * cb + 32 * cc + 16 * h) + 4 * lane);
          vu[2 * h] = t2[0];
          vu[2 * h + 1] = t2[1];
        }
        const bf16x8 va = as_bf16x8(vu);
#pragma unroll
        for (int u = 0; u < SUB; ++u) O[u][cb] = mfma16x16x32_bf16(va, pf[cc][u], O[u][cb]);
        if (split) {
#pragma unroll
          for (int u = 0; u < SUB; ++u) O[u][cb] = mfma16x16x32_bf16(va, lo[cc][u], O[u][cb]);
        }
        // keep the scheduler from hoisting every V fragment read at once
        if (T::PV_FENCE > 0 && cb % T::PV_FENCE == T::PV_FENCE - 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- pieces of the software-pipelined iteration ----
  // There a tile's scores are kept as t = s c - m (log2 units, -inf where
  // masked): the row maxima are then taken over FMA results, which need no
  // canonicalisation, and a rescale only shifts t.  Each group of
  // instructions below ends in a scheduling fence, so that the matrix-core
  // work of one tile and the VALU work of the other stay interleaved.

  // K fragments (A operand) of 16-key block b
  auto load_kf = [&](const uint16_t* ks_, int b, QFrag (&kf)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = kfrag(ks_, 16 * b + lr, ks);
  };
  // V^T fragment j = (32-key chunk j / CB, channel block j % CB)
  auto load_vf = [&](const uint16_t* vs, int j) {
    const int cc = j / CB, cb = j % CB;
    u32x4 vu;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x2 t2 = lds_read_tr16(vs + 16 * (BN * cb + 32 * cc + 16 * h) + 4 * lane);
      vu[2 * h] = t2[0];
      vu[2 * h + 1] = t2[1];
    }
    return as_bf16x8(vu);
  };
  // P^T chunk q = (32-key chunk q / SUB, sub-tile q % SUB) of the
  // exponentiated tile e, rounded to bf16
  auto pack_chunk = [&](const Scores& e, int q) {
    const int cc = q / SUB, u = q % SUB;
    u32x4 pu;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* ep = &e[u][4 * (2 * cc + h)];
      pu[2 * h] = pack_bf16x2(ep[0], ep[1]);
      pu[2 * h + 1] = pack_bf16x2(ep[2], ep[3]);
    }
    return as_bf16x8(pu);
  };
  // P^T chunk q straight from t
  auto p_chunk = [&](const Scores& t, int q) {
    const int cc = q / SUB, u = q % SUB;
    u32x4 pu;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* tp = &t[u][4 * (2 * cc + h)];
      pu[2 * h] = pack_bf16x2(exp2_fast(tp[0]), exp2_fast(tp[1]));
      pu[2 * h + 1] = pack_bf16x2(exp2_fast(tp[2]), exp2_fast(tp[3]));
    }
    return as_bf16x8(pu);
  };

  // The bf16 remainder P - bf16(P) of chunk q of the exponentiated tile e.
  // P - bf16(P) is exact in fp32 (at most 16 significant bits), so
  // bf16(P) + bf16(P - bf16(P)) carries P to a relative 2^-17 instead of the
  // 2^-9 of bf16(P) alone.
  auto pack_lo_chunk = [&](const Scores& e, int q) {
    const int cc = q / SUB, u = q % SUB;
    u32x4 pu;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* ep = &e[u][4 * (2 * cc + h)];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t hi = pack_bf16x2(ep[2 * k], ep[2 * k + 1]);
        pu[2 * h + k] = pack_bf16x2(ep[2 * k] - bf16_lo(hi), ep[2 * k + 1] - bf16_hi(hi));
      }
    }
    return as_bf16x8(pu);
  };

  // Phase A: S^T of the next tile (raw, into sn) from the K tile at ks_,
  // block by block, each block with the exponentials of one block of the
  // current tile (t -> 2^t in place).
  auto phase_a = [&](const uint16_t* ks_, Scores& sn, Scores& t) {
    constexpr int KA = T::K_AHEAD;  // K blocks read ahead
    QFrag kf[KA + 1][KS];
#pragma unroll
    for (int b = 0; b < KA && b < NB; ++b) load_kf(ks_, b, kf[b]);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b + KA < NB) load_kf(ks_, b + KA, kf[(b + KA) % (KA + 1)]);
      f32x4 acc[SUB];
#pragma unroll
      for (int u = 0; u < SUB; ++u) acc[u] = zero_f32x4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int u = 0; u < SUB; ++u) acc[u] = mma_qk(kf[b % (KA + 1)][ks], qf[u][ks], acc[u]);
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) sn[u][4 * b + j] = acc[u][j];
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) t[u][4 * b + j] = exp2_fast(t[u][4 * b + j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Phase B: P^T of the current tile (bf16, from the exponentials e) with
  // its row sums, and O^T += V^T P^T (V tile at vs) fragment by fragment,
  // each fragment with a slice of the next tile's t = s c - m (masked) and
  // its maxima.  Returns whether some row needs a new reference; mt gets
  // this lane's maxima of t (a row's maximum is that over its four lane
  // groups, which only the rare rescale needs: the lane maxima already tell
  // whether any row's exceeds the threshold).
  auto phase_b = [&](const uint16_t* vs, const Scores& e, Scores& sn, int kb, int qw0, float (&mt)[SUB],
                     auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    int lim[SUB];
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int last_key = CAUSAL ? min(qw0 + 16 * u + lr, N - 1) : N - 1;
      lim[u] = last_key - kb - 4 * lg;
    }
    constexpr int J = NC * CB;
    constexpr int NQ = NC * SUB;             // P chunks
    constexpr int NV = SUB * 4 * NB;         // score values per lane
    constexpr int PER = (NV + J - 1) / J;    // of them per group
    static_assert(NQ - SUB <= CB, "later P chunks are packed before their PV products");
    PFrags pf;
    // chunks of the first 32 keys now; the others in the first groups
#pragma unroll
    for (int q = 0; q < SUB; ++q) pf[0][q] = pack_chunk(e, q);
    float mx[SUB];
#pragma unroll
    for (int u = 0; u < SUB; ++u) mx[u] = -INFINITY;
    constexpr int VA = T::V_AHEAD;  // V fragments read ahead
    bf16x8 vf[VA + 1];
#pragma unroll
    for (int j = 0; j < VA && j < J; ++j) vf[j] = load_vf(vs, j);
#pragma unroll
    for (int q = 0; q < SUB; ++q) L[q] = mfma16x16x32_bf16(ones, pf[0][q], L[q]);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (j + VA < J) vf[(j + VA) % (VA + 1)] = load_vf(vs, j + VA);
#pragma unroll
      for (int u = 0; u < SUB; ++u) O[u][j % CB] = mfma16x16x32_bf16(vf[j % (VA + 1)], pf[j / CB][u], O[u][j % CB]);
      if (j >= 1 && j - 1 < NQ - SUB) {
        const int q = SUB + j - 1;  // packed in the group before
        L[q % SUB] = mfma16x16x32_bf16(ones, pf[q / SUB][q % SUB], L[q % SUB]);
      }
      if (j < NQ - SUB) {
        const int q = SUB + j;
        pf[q / SUB][q % SUB] = pack_chunk(e, q);
      }
#pragma unroll
      for (int q = j * PER; q < (j + 1) * PER && q < NV; ++q) {
        const int u = q / (4 * NB), i = q % (4 * NB);
        float x = __builtin_fmaf(sn[u][i], c, -m[u]);
        if (MASK) x = (16 * (i / 4) + (i % 4) <= lim[u]) ? x : -INFINITY;
        sn[u][i] = x;
        mx[u] = fmaxf(mx[u], x);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    bool need = false;
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      mt[u] = mx[u];
      need |= mx[u] > kRescaleThreshold;
    }
    return need;
  };
  // raise the references of all rows whose t exceeds 0 (t, O, l follow);
  // mt: the lanes' maxima of t
  auto rescale_t = [&](Scores& t, const float (&mt)[SUB], bool need) {
    if (wave_any(need)) {
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const float dm = max_f32(max4_groups(mt[u]), 0.0f);
        const float alpha = exp2_fast(-dm);
        m[u] += dm;
        L[u] *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) O[u][cb] *= alpha;
#pragma unroll
        for (int i = 0; i < 4 * NB; ++i) t[u][i] -= dm;
      }
    }
  };

  // tile kt of the current item holds keys past a row's diagonal or past N
  auto tile_masked = [&](const Item& it, int kb) {
    return (CAUSAL && kb + BN - 1 > it.qw0) || (kb + BN > N);
  };
  // key tiles of the item that hold keys visible to this wave's rows
  auto visible_tiles = [&](const Item& it) {
    if (it.qw0 >= N) return 0;
    return CAUSAL ? min(it.nkt, (it.qw0 + 16 * SUB - 1) / BN + 1) : it.nkt;
  };

  // Epilogue of one item.  The two waves of a row group (one per map) each
  // finish half of the channels: a wave sends the other half of its
  // accumulators and its per-row scale (1/l1, or lambda/l2 for map 2)
  // through LDS, receives its partner's part of its own half, forms
  // Y = O1/l1 - lambda O2/l2 there, and the two halves' sums of squares meet
  // through a small LDS array for the RMSNorm.  The exchange uses the stage
  // buffers that no load targets during the epilogue (all but the one
  // receiving the next item's first tile), for all row groups at once and
  // UR sub-tiles per round.  The next item's Q rows are loaded once the
  // first round's sent halves have left the registers.
  constexpr int HC = CB / 2;                  // channel blocks per half
  constexpr int LPR = DV / 16;                // output store lanes per row (16 bytes each)
  constexpr int RPI = 64 / LPR;               // rows per store instruction
  constexpr int XS = HC * 4 * 64;             // floats one wave sends per sub-tile
  constexpr int XU = 2 * XS;                  // floats per row group and sub-tile
  constexpr int CAP = (STAGES - 1) * T::STAGE / 2;  // floats in the free buffers
  constexpr int UR_FIT = CAP / (RG * XU);
  constexpr int UR = UR_FIT >= SUB ? SUB : UR_FIT;  // sub-tiles per round
  constexpr int RPB = (T::STAGE / 2) / (UR * XU);   // row groups per stage buffer
  static_assert(CB % 2 == 0 && UR >= 1 && SUB % UR == 0 && RPB >= 1 && RG <= RPB * (STAGES - 1),
                "epilogue exchange");
  constexpr int EPI_STORES = (SUB / UR) * (16 * UR / RPI);  // vector-memory stores per wave
  // row pitch (elements) of the row-major staging of Y: 16 bytes more than a
  // half row, so the 16 rows one write instruction touches fall on distinct
  // banks, and every row stays 16-byte aligned for the 16-byte reads
  constexpr int SP = DV / 2 + 8;
  static_assert(16 * UR * SP * 2 <= UR * XS * 4, "staging fits the wave's send region");
  // The next item's Q rows load during the epilogue where registers allow
  // (d <= 64); otherwise after it, their latency exposed once per item.
  constexpr bool EARLY_Q = D <= 64;
  auto epilogue_map = [&](const Item& it, int nb, int ni, const Item& nxt, auto map_tag) {
    constexpr int MP = decltype(map_tag)::value;          // this wave's map
    constexpr int own0 = MP * HC, send0 = (1 - MP) * HC;  // first channel block of each half
    // lane indices re-derived from an opaque copy of the lane id, so that the
    // epilogue's lane-dependent addresses are formed here rather than kept
    // in registers through the tile loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lr = ln & 15, lg = ln >> 4;
    // Training forward: this map's per-row log-sum-exp (log2 units: m plus
    // log2 of the row sum) and its normalised output O/l, kept for the
    // backward.  Issued before the output stores, so the wait for the next
    // tile (which leaves only those outstanding) also covers them.
    if constexpr (SAVE) {
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const int row = it.qw0 + 16 * u + lr;
        if (row < N) {
          const size_t srow = (size_t)(MP * BH + it.bh) * (size_t)N + (size_t)row;
          const float il = 1.0f / L[u][0];
          if (lg == 0) a.lse[srow] = m[u] + log2f(L[u][0]);
          float* op = a.osave + srow * DV + 4 * lg;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) *reinterpret_cast<f32x4*>(op + 16 * cb) = O[u][cb] * il;
        }
      }
    }
    // nb: the buffer of the next tile to consume (the next item's first)
    const int fb0 = nb == 0 ? STAGES - 1 : nb - 1;  // the buffer the last tile used
    const int fb1 = fb0 == 0 ? STAGES - 1 : fb0 - 1;
    float* region = (float*)(stages + (rg / RPB == 0 ? fb0 : fb1) * T::STAGE) + (rg % RPB) * UR * XU;
    float* sent = region + MP * UR * XS;
    const float* recv = region + (1 - MP) * UR * XS;
    // waves whose rows all lie past N run the exchange too (no store
    // follows), so the accumulators are updated on one path only
    float dn[SUB];
#pragma unroll
    for (int u = 0; u < SUB; ++u) dn[u] = (MP ? lam : 1.0f) / L[u][0];
#pragma unroll
    for (int u0 = 0; u0 < SUB; u0 += UR) {
#pragma unroll
      for (int v = 0; v < UR; ++v) {
#pragma unroll
        for (int h = 0; h < HC; ++h)
          *reinterpret_cast<f32x4*>(sent + ((v * HC + h) * 64 + ln) * 4) = O[u0 + v][send0 + h];
        if (lg == 0) dnx[wave][16 * (u0 + v) + lr] = dn[u0 + v];
      }
      __syncthreads();
      if (EARLY_Q && u0 == 0 && ni >= 0) load_q(nxt);  // qf is free since the last tile's QK^T
      float ssp[UR];
#pragma unroll
      for (int v = 0; v < UR; ++v) {
        const int u = u0 + v;
        float ss = 0.f;
        const float dp = dnx[wave ^ 1][16 * u + lr];  // the partner's scale
#pragma unroll
        for (int h = 0; h < HC; ++h) {
          const f32x4 o = *reinterpret_cast<const f32x4*>(recv + ((v * HC + h) * 64 + ln) * 4);
          const f32x4 y = MP ? o * dp - O[u][own0 + h] * dn[u] : O[u][own0 + h] * dn[u] - o * dp;
          O[u][own0 + h] = y;
#pragma unroll
          for (int j = 0; j < 4; ++j) ss += y[j] * y[j];
        }
        ssp[v] = sum_over_lane_groups(ss);
        if (NORM && lg == 0) ssx[wave][16 * u + lr] = ssp[v];
      }
      // the partner's sum of squares; also the last read of this round's region
      __syncthreads();
      // Y of this wave's half, bf16, staged row-major in its half of the
      // region (everybody's reads of it are done) and stored as whole row
      // segments: DV bytes per row, 16 bytes per lane.
      uint16_t* stg = (uint16_t*)(region + MP * UR * XS);
#pragma unroll
      for (int v = 0; v < UR; ++v) {
        const int u = u0 + v;
        float r = 1.0f;
        if (NORM) r = a.out_scale / sqrtf((ssp[v] + ssx[wave ^ 1][16 * u + lr]) * (1.0f / DV) + a.eps);
#pragma unroll
        for (int h = 0; h < HC; ++h) {
          const int cb = own0 + h;
          float y[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = O[u][cb][j] * (NORM ? r * wsh[16 * cb + 4 * lg + j] : 1.0f);
          u32x2 pk = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
          *reinterpret_cast<u32x2*>(stg + (16 * v + lr) * SP + 16 * h + 4 * lg) = pk;
        }
      }
      // Buffer stores against the head's N output rows: rows past N are
      // dropped by the hardware's range check, so every wave issues the
      // same EPI_STORES stores and no branch hides them from the counters.
      const __amdgpu_buffer_rsrc_t ob = __builtin_amdgcn_make_buffer_rsrc(
          (uint16_t*)a.out + head_row(it) * DV, 0, N * DV * 2, kBufferRsrcWord3);
#pragma unroll
      for (int q = 0; q < 16 * UR / RPI; ++q) {
        const int rr = q * RPI + ln / LPR;  // row within the round: 16 v + lr
        const int row = it.qw0 + 16 * (u0 + rr / 16) + rr % 16;
        const u32x4 val = *reinterpret_cast<const u32x4*>(stg + rr * SP + 8 * (ln % LPR));
        __builtin_amdgcn_raw_buffer_store_b128(val, ob, (row * DV + 16 * own0 + 8 * (ln % LPR)) * 2, 0, kStoreStreaming);
      }
      // the region is reused by the next round's sends
      if (u0 + UR < SUB) __syncthreads();
    }
  };
  auto epilogue = [&](const Item& it, int nb, int ni, const Item& nxt) {
    if (mp)
      epilogue_map(it, nb, ni, nxt, std::integral_constant<int, 1>{});
    else
      epilogue_map(it, nb, ni, nxt, std::integral_constant<int, 0>{});
  };

  // The key tiles of all this workgroup's items form one stream through the
  // ring of stage buffers, across item boundaries; the load cursor runs one
  // tile ahead of the tile last made available.
  struct Cursor {
    int r, kt;
    bool ok;
    Item it;
  };
  // Tiles loading ahead of the one made available next: the pipelined loop
  // reads two tiles at a time, so one buffer fewer is free for loads.
  constexpr int LOOK = STAGES - 2;
  int ib = 0;       // stage buffer of the next tile to load
  int pending = 0;  // tiles loading and not yet made available
  auto load_next = [&](Cursor& q) {
    if (!q.ok) return;
    issue_tile(ib, q.it, q.kt);
    ib = ib + 1 == STAGES ? 0 : ib + 1;
    ++pending;
    if (++q.kt < q.it.nkt) return;
    q.kt = 0;
    const int i = __builtin_amdgcn_readfirstlane(item_at(++q.r));
    q.ok = i >= 0;
    if (q.ok) q.it = decode_item(i);
  };

  // The Q rows of an item come in through ordinary loads that the compiler
  // waits for itself; the empty asm makes that wait happen here, once per
  // item, where waiting for everything outstanding costs nothing, instead
  // of inside the tile loop.
  auto settle_q = [&]() {
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[u][ks]));
  };

  // Make the oldest loading tile available: this wave's loads of it have
  // landed (those of a newer tile, the wave's newest vector-memory work, may
  // still be in flight), the barrier extends that to everybody's and
  // guarantees that nobody still reads the buffer the next load reuses.
  // after an epilogue its output stores are the wave's newest vector-memory
  // work: the tile (and Q rows) issued before them may be waited for alone
  bool after_epilogue = false;
  auto avail = [&](Cursor& q) {
    if (after_epilogue) {
      static_assert(LOOK == 1, "after an epilogue only the tile being made available is loading");
      wait_vmem_keep<EPI_STORES>();
      after_epilogue = false;
    } else if (LOOK > 1 && __builtin_amdgcn_readfirstlane(pending) > 1) {
      wait_vmem_keep<SPW>();
    } else {
      wait_vmem();
    }
    --pending;
    __syncthreads();
    load_next(q);
  };

  int r = 0;
  const int i0 = item_at(0);
  if (i0 < 0) return;
  Item cur = decode_item(i0);
  Cursor ld{0, 0, true, cur};
  load_next(ld);
  load_q(cur);
  settle_q();
#pragma unroll
  for (int p = 1; p < LOOK; ++p) load_next(ld);
  int tb = 0;  // stage buffer of the current item's next tile to consume
  auto next_buf = [&](int i) { return i + 1 == STAGES ? 0 : i + 1; };
  Scores sA, sB;
  while (true) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) O[u][cb] = zero_f32x4();
      L[u] = zero_f32x4();
      m[u] = -INFINITY;
    }
    {
      // Iteration kt forms P of tile kt (VALU) while the QK^T products of
      // tile kt+1 run on the matrix cores, then runs PV of tile kt while the
      // row maxima of tile kt+1 are taken.  Tiles kt and kt+1 are read
      // together, so when tile t+1 becomes available tile t+2 loads into the
      // third buffer (that of tile t-1, finished by everybody).
      const int nvis = visible_tiles(cur);
      // Every wave makes the same nkt calls of avail() per item (each holds
      // a barrier): one for tile 0 here, then one at the start of step kt
      // for tile kt+1, visible to this wave or not.
      avail(ld);
      // full step: P and PV of tile kt (t in sc) with S^T of tile kt+1 into
      // sn, which leaves as t
      auto full = [&](int kt, Scores& sc, Scores& sn, auto mask_tag) {
        const uint16_t* bc = stages + tb * T::STAGE;
        tb = next_buf(tb);
        const uint16_t* bn = stages + tb * T::STAGE;
        avail(ld);
        float mt[SUB];
        phase_a(bn + mp * KTILE, sn, sc);
        const bool need = phase_b(bc + 2 * KTILE, sc, sn, (kt + 1) * BN, cur.qw0, mt, mask_tag);
        rescale_t(sn, mt, need);
      };
      // last visible tile of this wave: P and PV only.  When it is also the
      // wave's only one (every row sees at most BN keys: the first rows of a
      // causal head, or a sequence no longer than a tile), P enters the
      // products as bf16(P) + bf16(P - bf16(P)).  Those rows have few keys,
      // and where the two maps nearly cancel (lambda near 1) the norm divides
      // by an rms(Y) far below the size of A1 V and lambda A2 V, which would
      // amplify the bf16 rounding of P beyond the output tolerance.  Rows
      // with more keys average that rounding out.
      auto last = [&](int kt, Scores& t) {
        const uint16_t* bc = stages + tb * T::STAGE;
        tb = next_buf(tb);
        if (kt + 1 < cur.nkt) avail(ld);
        const bool split = kt == 0;
#pragma unroll
        for (int u = 0; u < SUB; ++u)
#pragma unroll
          for (int i = 0; i < 4 * NB; ++i) t[u][i] = exp2_fast(t[u][i]);
        PFrags pf, lo;
#pragma unroll
        for (int q = 0; q < NC * SUB; ++q) {
          pf[q / SUB][q % SUB] = pack_chunk(t, q);
          L[q % SUB] = mfma16x16x32_bf16(ones, pf[q / SUB][q % SUB], L[q % SUB]);
          if (split) {
            lo[q / SUB][q % SUB] = pack_lo_chunk(t, q);
            L[q % SUB] = mfma16x16x32_bf16(ones, lo[q / SUB][q % SUB], L[q % SUB]);
          }
        }
        pv(bc, pf, lo, split);
      };
      // this wave's visible tiles: the first nfree carry no mask, the rest
      // (the diagonal and the ragged end) do
      const int nfree = min(nvis, min(CAUSAL ? (cur.qw0 + 1) / BN : N / BN, N / BN));
      int kt = 0;
      if (nvis > 0) {
        // tile 0: scores, the first reference, then t
        if (nfree == 0)
          qk(sA, stages + tb * T::STAGE, 0, cur.qw0, std::true_type{});
        else
          qk(sA, stages + tb * T::STAGE, 0, cur.qw0, std::false_type{});
        update_max(sA);
#pragma unroll
        for (int u = 0; u < SUB; ++u)
#pragma unroll
          for (int i = 0; i < 4 * NB; ++i) sA[u][i] = __builtin_fmaf(sA[u][i], c, -m[u]);
        for (; kt + 1 < nfree; ++kt) {
          full(kt, sA, sB, std::false_type{});
#pragma unroll
          for (int u = 0; u < SUB; ++u)
#pragma unroll
            for (int i = 0; i < 4 * NB; ++i) sA[u][i] = sB[u][i];
        }
        for (; kt + 1 < nvis; ++kt) {
          full(kt, sA, sB, std::true_type{});
#pragma unroll
          for (int u = 0; u < SUB; ++u)
#pragma unroll
            for (int i = 0; i < 4 * NB; ++i) sA[u][i] = sB[u][i];
        }
        last(kt, sA);
        ++kt;
      }
      for (; kt < cur.nkt; ++kt) {  // tiles no row of this wave sees
        tb = next_buf(tb);
        if (kt + 1 < cur.nkt) avail(ld);
      }
    }
    const int ni = item_at(r + 1);
    const Item nxt = decode_item(ni < 0 ? i0 : ni);
    __syncthreads();  // everybody is done with the last tiles' buffers
    epilogue(cur, tb, ni, nxt);
    if (!EARLY_Q && ni >= 0) load_q(nxt);
    after_epilogue = EARLY_Q;
    settle_q();
    if (ni < 0) break;
    cur = nxt;
    ++r;
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: same schedule with the 16x16x4 f32 MFMA (products exact in
// fp32).  A workgroup owns 64 query rows (4 waves); tiles of 16 keys.

template <int D, bool CAUSAL, bool NORM>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int DV = 2 * D;
  constexpr int WAVES = 4;
  constexpr int BM = 16 * WAVES;
  constexpr int BN = 16;
  constexpr int KD = D / 4;   // k-steps of the QK^T MFMA
  constexpr int CB = DV / 16;
  constexpr int KP = D + 4;   // K row pitch (floats)
  constexpr int VP = DV + 16; // V row pitch (floats)
  constexpr int KTILE = BN * KP;
  constexpr int VTILE = BN * VP;
  constexpr int STAGE = 2 * KTILE + VTILE;
  constexpr int NTH = 64 * WAVES;
  constexpr int KCH = BN * D / 4;   // 16-byte chunks per K tile
  constexpr int VCH = BN * DV / 4;  // 16-byte chunks per V tile
  constexpr int KPT = (KCH + NTH - 1) / NTH;
  constexpr int VPT = (VCH + NTH - 1) / NTH;

  __shared__ __attribute__((aligned(16))) float lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int N = a.N;

  const int bid = blockIdx.x;
  const int bh = bid % a.BH;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - bid / a.BH) : (bid / a.BH);
  const int q0 = qt * BM;
  const int qw0 = q0 + 16 * wave;

  const size_t hrow = (size_t)bh * (size_t)N;
  const float* __restrict__ Q1 = (const float*)a.q1 + hrow * D;
  const float* __restrict__ Q2 = (const float*)a.q2 + hrow * D;
  const float* __restrict__ K1 = (const float*)a.k1 + hrow * D;
  const float* __restrict__ K2 = (const float*)a.k2 + hrow * D;
  const float* __restrict__ V = (const float*)a.v + hrow * DV;

  // Q^T fragments: lane holds dim 4ks+lg of its query row
  float qf1[KD], qf2[KD];
  {
    const int qrow = min(qw0 + lr, N - 1);
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) {
      qf1[ks] = Q1[(size_t)qrow * D + 4 * ks + lg];
      qf2[ks] = Q2[(size_t)qrow * D + 4 * ks + lg];
    }
  }

  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int nkt = (kend + BN - 1) / BN;

  u32x4 rk1[KPT], rk2[KPT], rv[VPT];
  auto load_tile = [&](int kt) {
    const int kb = kt * BN;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * NTH;
      if (idx < KCH) {
        const int r = min(kb + idx / (D / 4), N - 1);
        rk1[i] = ld16(K1 + (size_t)r * D + 4 * (idx % (D / 4)));
        rk2[i] = ld16(K2 + (size_t)r * D + 4 * (idx % (D / 4)));
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * NTH;
      if (idx < VCH) {
        const int r = min(kb + idx / (DV / 4), N - 1);
        rv[i] = ld16(V + (size_t)r * DV + 4 * (idx % (DV / 4)));
      }
    }
  };
  auto store_tile = [&](int buf) {
    float* Ks1 = lds + buf * STAGE;
    float* Ks2 = Ks1 + KTILE;
    float* Vs = Ks1 + 2 * KTILE;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * NTH;
      if (idx < KCH) {
        st16(Ks1 + (idx / (D / 4)) * KP + 4 * (idx % (D / 4)), rk1[i]);
        st16(Ks2 + (idx / (D / 4)) * KP + 4 * (idx % (D / 4)), rk2[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * NTH;
      if (idx < VCH) st16(Vs + (idx / (DV / 4)) * VP + 4 * (idx % (DV / 4)), rv[i]);
    }
  };

  f32x4 O1[CB], O2[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    O1[cb] = zero_f32x4();
    O2[cb] = zero_f32x4();
  }
  f32x4 L1 = zero_f32x4(), L2 = zero_f32x4();
  float m1 = -INFINITY, m2 = -INFINITY;
  const float c = a.c;
  const int qabs = qw0 + lr;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool has_next = kt + 1 < nkt;
    if (has_next) load_tile(kt + 1);
    const int kb = kt * BN;
    const bool active = (qw0 < N) && (!CAUSAL || kb <= qw0 + 15);
    if (active) {
      const float* Ks1 = lds + buf * STAGE;
      const float* Ks2 = Ks1 + KTILE;
      const float* Vs = Ks1 + 2 * KTILE;
      const bool need_mask = (CAUSAL && kb + BN - 1 > qw0) || (kb + BN > N);

      // S^T block: lane holds keys 4lg+j of its query
      f32x4 s1 = zero_f32x4(), s2 = zero_f32x4();
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) {
        s1 = mfma16x16x4_f32(Ks1[lr * KP + 4 * ks + lg], qf1[ks], s1);
        s2 = mfma16x16x4_f32(Ks2[lr * KP + 4 * ks + lg], qf2[ks], s2);
      }
      float t1[4], t2[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x1 = s1[j] * c, x2 = s2[j] * c;
        if (need_mask) {
          const int kabs = kb + 4 * lg + j;
          const bool ok = (kabs < N) && (!CAUSAL || kabs <= qabs);
          x1 = ok ? x1 : -INFINITY;
          x2 = ok ? x2 : -INFINITY;
        }
        t1[j] = x1;
        t2[j] = x2;
      }
      softmax_step<4, CB>(t1, m1, L1, O1);
      softmax_step<4, CB>(t2, m2, L2, O2);

      // PV: MFMA j consumes key 4*lg + j from every lane group
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        L1 = mfma16x16x4_f32(1.0f, t1[j], L1);
        L2 = mfma16x16x4_f32(1.0f, t2[j], L2);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const float va = Vs[(4 * lg + j) * VP + 16 * cb + lr];
          O1[cb] = mfma16x16x4_f32(va, t1[j], O1[cb]);
          O2[cb] = mfma16x16x4_f32(va, t2[j], O2[cb]);
        }
      }
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (qw0 < N) {
    f32x4 y[CB];
    epilogue_values<CB, NORM>(O1, O2, L1[0], L2[0], *a.lambda, a.out_scale, a.eps, a.norm_w, lg, y);
    const int row = qw0 + lr;
    if (row < N) {
      float* __restrict__ Out = (float*)a.out + (hrow + row) * DV;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) *reinterpret_cast<f32x4*>(Out + 16 * cb + 4 * lg) = y[cb];
    }
  }
}

// ---------------------------------------------------------------------------
// dispatch

int prefill_block_rows(bool bf16, int d) {
  if (!bf16) return 64;
  switch (d) {
    case 16: return Bf16Tile<16>::BM;
    case 32: return Bf16Tile<32>::BM;
    case 64: return Bf16Tile<64>::BM;
    default: return Bf16Tile<128>::BM;
  }
}
int prefill_block_threads(bool bf16, int d) {
  if (!bf16) return 256;
  switch (d) {
    case 16: return 64 * Bf16Tile<16>::WAVES;
    case 32: return 64 * Bf16Tile<32>::WAVES;
    case 64: return 64 * Bf16Tile<64>::WAVES;
    default: return 64 * Bf16Tile<128>::WAVES;
  }
}

// Compute units of the current device, queried once per device.
static hipError_t compute_units(int* ncu) {
  static int cache[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *ncu = cache[dev];
    return hipSuccess;
  }
  e = hipDeviceGetAttribute(ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && dev >= 0 && dev < 64) cache[dev] = *ncu;
  return e;
}

// schedule.hip: whether a causal launch of G workgroups takes the per-XCD
// schedule (the XCD instantiation) rather than the item-wise one
bool prefill_xcd_schedule(long long grid, int BH, int n_qtiles);

template <int D, bool C, bool NM, bool SV, bool F8 = false>
static hipError_t launch_one(bool bf16, const PrefillArgs& a, hipStream_t s) {
  const long long items = (long long)a.n_qtiles * (long long)a.BH;
  const dim3 block(prefill_block_threads(bf16, D));
  if (bf16) {
    // persistent: one workgroup per compute unit walks the item list
    int ncu = 0;
    const hipError_t e = compute_units(&ncu);
    if (e != hipSuccess) return e;
    const long long grid = items < ncu ? items : (ncu > 0 ? ncu : 1);
    bool xcd = false;
    if constexpr (C) xcd = prefill_xcd_schedule(grid, a.BH, a.n_qtiles);  // causal only
    if (xcd)
      hipLaunchKernelGGL((prefill_bf16_kernel<D, C, NM, SV, F8, C>), dim3((unsigned)grid), block, 0, s, a);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<D, C, NM, SV, F8, false>), dim3((unsigned)grid), block, 0, s, a);
  } else if constexpr (!SV && !F8) {
    hipLaunchKernelGGL((prefill_f32_kernel<D, C, NM>), dim3((unsigned)items), block, 0, s, a);
  } else {
    return hipErrorInvalidValue;  // no fp32 training forward
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(bool bf16, bool causal, bool norm, bool save, const PrefillArgs& a, hipStream_t s) {
  if constexpr (D >= 32) {
    // the training forward: bf16, normalised output
    if (save) {
      if (!bf16 || !norm) return hipErrorInvalidValue;
      return causal ? launch_one<D, true, true, true>(bf16, a, s) : launch_one<D, false, true, true>(bf16, a, s);
    }
  } else {
    if (save) return hipErrorInvalidValue;
  }
  if (causal)
    return norm ? launch_one<D, true, true, false>(bf16, a, s) : launch_one<D, true, false, false>(bf16, a, s);
  return norm ? launch_one<D, false, true, false>(bf16, a, s) : launch_one<D, false, false, false>(bf16, a, s);
}

hipError_t launch_prefill(bool bf16, int d, bool causal, bool norm, const PrefillArgs& a,
                          hipStream_t stream) {
  const bool save = a.osave != nullptr;
  switch (d) {
    case 16: return launch_d<16>(bf16, causal, norm, save, a, stream);
    case 32: return launch_d<32>(bf16, causal, norm, save, a, stream);
    case 64: return launch_d<64>(bf16, causal, norm, save, a, stream);
    case 128: return launch_d<128>(bf16, causal, norm, save, a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_fp8qk(bool causal, bool norm, const PrefillArgs& a, hipStream_t stream) {
  if (causal)
    return norm ? launch_one<128, true, true, false, true>(true, a, stream)
                : launch_one<128, true, false, false, true>(true, a, stream);
  return norm ? launch_one<128, false, true, false, true>(true, a, stream)
              : launch_one<128, false, false, false, true>(true, a, stream);
}

}  // namespace diffattn
