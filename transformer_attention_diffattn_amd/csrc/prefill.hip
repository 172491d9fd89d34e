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
// Layout of the work (bf16 kernel): a workgroup owns BM = 128 query rows of
// one head (8 waves x 16 rows) and streams BN-key tiles of K1, K2, V through
// double-buffered LDS.  Products are computed transposed so that every
// per-row quantity lives in the lane of its query:
//   S^T = K Q^T   (16x16x32 bf16 MFMA, A = K rows from LDS, B = Q^T in VGPRs)
//   O^T += V^T P^T (A = V^T from LDS, B = P^T built in-lane from S^T)
//   l   += 1^T P^T (the same MFMA with A = ones: row sums of the rounded P)
// In a 16x16 MFMA result lane L holds column L%16 (the query) and rows
// 4*(L/16)+j, so a lane owns one query's scores for 4 keys per 16-key block
// and one query's outputs for 4 channels per 16-channel block.

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

template <int D, bool CAUSAL, bool NORM>
__global__ __launch_bounds__(512) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int DV = 2 * D;
  constexpr int WAVES = 8;
  constexpr int BM = 16 * WAVES;
  constexpr int BN = (D >= 128) ? 32 : 64;
  constexpr int KS = (D + 31) / 32;  // 32-wide k-steps of the QK^T MFMA
  constexpr int NB = BN / 16;        // 16-key score blocks per tile
  constexpr int NC = BN / 32;        // 32-key chunks per tile (PV k-steps)
  constexpr int CB = DV / 16;        // 16-channel output blocks
  constexpr int KP = D + 8;          // K tile row pitch (elements); rows stay 16-byte aligned
  constexpr int VP = BN + 8;         // V^T tile row pitch (elements)
  constexpr int KTILE = BN * KP;
  constexpr int VTILE = DV * VP;
  constexpr int STAGE = 2 * KTILE + VTILE;
  constexpr int KCH = BN * D / 8;              // 16-byte chunks per K tile
  constexpr int VITEMS = (BN / 2) * (DV / 8);  // (key pair, 8-channel chunk) items per V tile
  static_assert(KCH <= 64 * WAVES && VITEMS <= 64 * WAVES, "one staging item per thread");

  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;  // query (MFMA column) owned by this lane
  const int lg = lane >> 4;  // lane group: selects rows 4*lg..4*lg+3 of each block
  const int N = a.N;

  // Longest tiles first under the causal mask; heads vary fastest.
  const int bid = blockIdx.x;
  const int bh = bid % a.BH;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - bid / a.BH) : (bid / a.BH);
  const int q0 = qt * BM;
  const int qw0 = q0 + 16 * wave;

  const size_t hrow = (size_t)bh * (size_t)N;
  const uint16_t* __restrict__ Q1 = (const uint16_t*)a.q1 + hrow * D;
  const uint16_t* __restrict__ Q2 = (const uint16_t*)a.q2 + hrow * D;
  const uint16_t* __restrict__ K1 = (const uint16_t*)a.k1 + hrow * D;
  const uint16_t* __restrict__ K2 = (const uint16_t*)a.k2 + hrow * D;
  const uint16_t* __restrict__ V = (const uint16_t*)a.v + hrow * DV;

  // Q^T fragments: lane holds dims 32ks+8lg..+7 of its query row (zeros past d).
  bf16x8 qf1[KS], qf2[KS];
  {
    const int qrow = min(qw0 + lr, N - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int dc = 32 * ks + 8 * lg;
      qf1[ks] = as_bf16x8(dc < D ? ld16(Q1 + (size_t)qrow * D + dc) : zero_u32x4());
      qf2[ks] = as_bf16x8(dc < D ? ld16(Q2 + (size_t)qrow * D + dc) : zero_u32x4());
    }
  }

  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int nkt = (kend + BN - 1) / BN;

  // staging registers: one K1 chunk, one K2 chunk, one V key pair per thread
  u32x4 rk1 = zero_u32x4(), rk2 = zero_u32x4(), rva = zero_u32x4(), rvb = zero_u32x4();
  const int k_row = tid / (D / 8), k_ch = tid % (D / 8);
  const int v_kp = tid % (BN / 2), v_ch = tid / (BN / 2);

  auto load_tile = [&](int kt) {
    const int kb = kt * BN;
    if (tid < KCH) {
      const int r = min(kb + k_row, N - 1);
      rk1 = ld16(K1 + (size_t)r * D + 8 * k_ch);
      rk2 = ld16(K2 + (size_t)r * D + 8 * k_ch);
    }
    if (tid < VITEMS) {
      const int r0 = min(kb + 2 * v_kp, N - 1);
      const int r1 = min(kb + 2 * v_kp + 1, N - 1);
      rva = ld16(V + (size_t)r0 * DV + 8 * v_ch);
      rvb = ld16(V + (size_t)r1 * DV + 8 * v_ch);
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* Ks1 = lds + buf * STAGE;
    uint16_t* Ks2 = Ks1 + KTILE;
    uint16_t* Vt = Ks1 + 2 * KTILE;
    if (tid < KCH) {
      st16(Ks1 + k_row * KP + 8 * k_ch, rk1);
      st16(Ks2 + k_row * KP + 8 * k_ch, rk2);
    }
    if (tid < VITEMS) {
      // transpose a 2-key x 8-channel block: channel e of keys (2kp, 2kp+1)
      // becomes one dword of V^T row (8ch+e)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t x = rva[e >> 1], y = rvb[e >> 1];
        const uint32_t wd = (e & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
        *reinterpret_cast<uint32_t*>(Vt + (8 * v_ch + e) * VP + 2 * v_kp) = wd;
      }
    }
  };

  // accumulators
  f32x4 O1[CB], O2[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    O1[cb] = zero_f32x4();
    O2[cb] = zero_f32x4();
  }
  f32x4 L1 = zero_f32x4(), L2 = zero_f32x4();
  float m1 = -INFINITY, m2 = -INFINITY;
  const float c = a.c;
  u32x4 ones_u = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  const bf16x8 ones = as_bf16x8(ones_u);
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
      const uint16_t* Ks1 = lds + buf * STAGE;
      const uint16_t* Ks2 = Ks1 + KTILE;
      const uint16_t* Vt = Ks1 + 2 * KTILE;
      const bool need_mask = (CAUSAL && kb + BN - 1 > qw0) || (kb + BN > N);

      // scores S^T for both maps; block b covers keys 32(b/2) + {8q + 4(b%2) + j}
      float t1[4 * NB], t2[4 * NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int krow = 32 * (b >> 1) + 8 * (lr >> 2) + 4 * (b & 1) + (lr & 3);
        f32x4 s1 = zero_f32x4(), s2 = zero_f32x4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int dc = 32 * ks + 8 * lg;
          const bf16x8 ka1 = as_bf16x8(dc < D ? ld16(Ks1 + krow * KP + dc) : zero_u32x4());
          const bf16x8 ka2 = as_bf16x8(dc < D ? ld16(Ks2 + krow * KP + dc) : zero_u32x4());
          s1 = mfma16x16x32_bf16(ka1, qf1[ks], s1);
          s2 = mfma16x16x32_bf16(ka2, qf2[ks], s2);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x1 = s1[j] * c, x2 = s2[j] * c;
          if (need_mask) {
            const int kabs = kb + 32 * (b >> 1) + 8 * lg + 4 * (b & 1) + j;
            const bool ok = (kabs < N) && (!CAUSAL || kabs <= qabs);
            x1 = ok ? x1 : -INFINITY;
            x2 = ok ? x2 : -INFINITY;
          }
          t1[4 * b + j] = x1;
          t2[4 * b + j] = x2;
        }
      }

      softmax_step<4 * NB, CB>(t1, m1, L1, O1);
      softmax_step<4 * NB, CB>(t2, m2, L2, O2);

      // P^T fragments: chunk cc takes blocks 2cc (keys 8q+0..3) and 2cc+1 (keys 8q+4..7)
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        u32x4 p1u, p2u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int b = 2 * cc + h;
          p1u[2 * h] = pack_bf16x2(t1[4 * b + 0], t1[4 * b + 1]);
          p1u[2 * h + 1] = pack_bf16x2(t1[4 * b + 2], t1[4 * b + 3]);
          p2u[2 * h] = pack_bf16x2(t2[4 * b + 0], t2[4 * b + 1]);
          p2u[2 * h + 1] = pack_bf16x2(t2[4 * b + 2], t2[4 * b + 3]);
        }
        const bf16x8 p1 = as_bf16x8(p1u), p2 = as_bf16x8(p2u);
        L1 = mfma16x16x32_bf16(ones, p1, L1);
        L2 = mfma16x16x32_bf16(ones, p2, L2);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const bf16x8 va = as_bf16x8(ld16(Vt + (16 * cb + lr) * VP + 32 * cc + 8 * lg));
          O1[cb] = mfma16x16x32_bf16(va, p1, O1[cb]);
          O2[cb] = mfma16x16x32_bf16(va, p2, O2[cb]);
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
      uint16_t* __restrict__ Out = (uint16_t*)a.out + (hrow + row) * DV;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        u32x2 pk = {pack_bf16x2(y[cb][0], y[cb][1]), pack_bf16x2(y[cb][2], y[cb][3])};
        *reinterpret_cast<u32x2*>(Out + 16 * cb + 4 * lg) = pk;
      }
    }
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

int prefill_block_rows(bool bf16) { return bf16 ? 128 : 64; }
int prefill_block_threads(bool bf16) { return bf16 ? 512 : 256; }

template <int D, bool C, bool NM>
static hipError_t launch_one(bool bf16, const PrefillArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.n_qtiles * (unsigned)a.BH);
  const dim3 block(prefill_block_threads(bf16));
  if (bf16)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, C, NM>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((prefill_f32_kernel<D, C, NM>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(bool bf16, bool causal, bool norm, const PrefillArgs& a, hipStream_t s) {
  if (causal) return norm ? launch_one<D, true, true>(bf16, a, s) : launch_one<D, true, false>(bf16, a, s);
  return norm ? launch_one<D, false, true>(bf16, a, s) : launch_one<D, false, false>(bf16, a, s);
}

hipError_t launch_prefill(bool bf16, int d, bool causal, bool norm, const PrefillArgs& a,
                          hipStream_t stream) {
  switch (d) {
    case 16: return launch_d<16>(bf16, causal, norm, a, stream);
    case 32: return launch_d<32>(bf16, causal, norm, a, stream);
    case 64: return launch_d<64>(bf16, causal, norm, a, stream);
    case 128: return launch_d<128>(bf16, causal, norm, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace diffattn
