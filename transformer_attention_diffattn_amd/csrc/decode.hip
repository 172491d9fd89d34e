// Differential-attention decode against a KV cache, for gfx950 (MI355X).
//
// One new query token per sequence attends its cache_len cached keys
// (Eq. 1 of "Differential Transformer: Canceling Context Noise with
// Differential Attention", section "Cancelling Context Noise Through Attention
// Map Subtraction", with one query row), then the head-wise RMSNorm and the
// (1 - lambda_init) scale (Eq. 3 of the "Differential Transformer" sample
// review, "Summary").
//
// The work is a stream over K1, K2 and V (8d bytes per cached key in bf16)
// with 12d flops per key: bound by HBM bandwidth.  Split-K: each (b, h) cache
// is cut into S contiguous splits, one 256-thread workgroup per split.
//   decode_split_kernel: per split, two online-softmax states (reference
//     maximum, denominator, numerator over 2d channels); 16-byte
//     non-temporal loads, 16 lanes per key row for the dots, all loads of an
//     unrolled group issued before use; lanes that hold different keys of the same channels merge
//     with cross-lane shuffles at the end, the 4 waves through LDS.
//   decode_merge_kernel: per (b, h), merges the S partial states (wavefront
//     shuffle reductions of the maxima and denominators, a fixed split order
//     for the numerators), then forms Y and applies the epilogue.

#include <mutex>

#include "../../include/diffattn.h"
#include "device_common.h"
#include "kernels.h"

namespace diffattn {

namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 4;

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int per16 = 4;
  // dot of 4 fp32 pairs
  static __device__ __forceinline__ float dot(u32x4 q, u32x4 k) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += u32_as_f32(q[i]) * u32_as_f32(k[i]);
    return s;
  }
  static __device__ __forceinline__ float get(u32x4 v, int i) { return u32_as_f32(v[i]); }
  static __device__ __forceinline__ void store(void* p, float x) { *(float*)p = x; }
};
template <>
struct Elem<__bf16> {
  static constexpr int per16 = 8;
  // dot of 8 bf16 pairs with fp32 accumulation (v_dot2c_f32_bf16)
  static __device__ __forceinline__ float dot(u32x4 q, u32x4 k) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s = __builtin_amdgcn_fdot2_f32_bf16(u32_as_bf16x2(q[i]), u32_as_bf16x2(k[i]), s, false);
    return s;
  }
  static __device__ __forceinline__ float get(u32x4 v, int i) {
    return (i & 1) ? bf16_hi(v[i >> 1]) : bf16_lo(v[i >> 1]);
  }
  static __device__ __forceinline__ void store(void* p, float x) {
    f32x2 t = {x, 0.f};
    *(uint16_t*)p = (uint16_t)(pack_bf16x2(t[0], t[1]) & 0xffffu);
  }
};

__device__ __forceinline__ float xor_max(float x, int off) { return fmaxf(x, __shfl_xor(x, off)); }
__device__ __forceinline__ float xor_sum(float x, int off) { return x + __shfl_xor(x, off); }

// Online-softmax update of one map for one group of keys whose scaled scores
// t (log2 units) are spread over the wave; tmax is the wave-wide maximum.
template <int EPC>
__device__ __forceinline__ void rescale_if_needed(float tmax, float& m, float& l, float (&o)[EPC]) {
  if (wave_any(tmax > m + kRescaleThreshold)) {
    const float mn = fmaxf(m, tmax);
    const float alpha = (mn == -INFINITY) ? 1.0f : exp2_fast(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < EPC; ++e) o[e] *= alpha;
  }
}

}  // namespace

size_t decode_record_floats(int d) { return 4 + 4 * (size_t)d; }

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  using E = Elem<T>;
  constexpr int DV = 2 * D;
  constexpr int EPC = E::per16;  // elements per 16-byte chunk
  constexpr int KL = D / EPC;    // lanes per K row
  constexpr int KPS = 64 / KL;   // keys per wave step
  constexpr int VL = DV / EPC;   // lanes per V row
  constexpr int VKPL = 64 / VL;  // keys per V load instruction (KPS / 2)
  static_assert(KL >= 1 && KL <= 64 && VL <= 64 && 2 * VKPL == KPS, "tiling");
  constexpr size_t REC = 4 + 2 * DV;

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = a.L;
  const int len = a.cache_len ? min(max(a.cache_len[b], 0), L) : L;
  const int k0 = s * a.chunk;
  const int k1 = min(k0 + a.chunk, len);
  const size_t bh = (size_t)b * a.H + h;

  const T* __restrict__ K1 = (const T*)a.k1c + bh * (size_t)L * D;
  const T* __restrict__ K2 = (const T*)a.k2c + bh * (size_t)L * D;
  const T* __restrict__ V = (const T*)a.vc + bh * (size_t)L * DV;

  const int kl = lane % KL, kg = lane / KL;  // K chunk, key within step
  const int vl = lane % VL, vg = lane / VL;  // V chunk, key within a V load
  const u32x4 q1v = ld16((const T*)a.q1 + bh * D + kl * EPC);
  const u32x4 q2v = ld16((const T*)a.q2 + bh * D + kl * EPC);
  const float c = a.c;

  float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
  float o1[EPC], o2[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) o1[e] = o2[e] = 0.f;

  const int nsteps = (k1 > k0) ? (k1 - k0 + KPS - 1) / KPS : 0;
  for (int st0 = wave; st0 < nsteps; st0 += kWaves * kUnroll) {
    u32x4 kk1[kUnroll], kk2[kUnroll], vv[kUnroll][2];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int kbase = k0 + (st0 + u * kWaves) * KPS;
      const int kr = min(kbase + kg, k1 - 1);
      // the cache is read once: non-temporal loads keep it from churning the caches
      kk1[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(K1 + (size_t)kr * D + kl * EPC));
      kk2[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(K2 + (size_t)kr * D + kl * EPC));
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int vr = min(kbase + x * VKPL + vg, k1 - 1);
        vv[u][x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(V + (size_t)vr * DV + vl * EPC));
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int kbase = k0 + (st0 + u * kWaves) * KPS;
      float s1 = E::dot(q1v, kk1[u]);
      float s2 = E::dot(q2v, kk2[u]);
#pragma unroll
      for (int off = 1; off < KL; off <<= 1) {
        s1 = xor_sum(s1, off);
        s2 = xor_sum(s2, off);
      }
      const bool valid = kbase + kg < k1;  // also false for steps past the end
      const float t1 = valid ? s1 * c : -INFINITY;
      const float t2 = valid ? s2 * c : -INFINITY;
      float mx1 = t1, mx2 = t2;
#pragma unroll
      for (int off = KL; off < 64; off <<= 1) {
        mx1 = xor_max(mx1, off);
        mx2 = xor_max(mx2, off);
      }
      rescale_if_needed<EPC>(mx1, m1, l1, o1);
      rescale_if_needed<EPC>(mx2, m2, l2, o2);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int src = (x * VKPL + vg) * KL;  // a lane holding this V row's key score
        const float p1 = exp2_fast(__shfl(t1, src) - m1);
        const float p2 = exp2_fast(__shfl(t2, src) - m2);
        l1 += p1;
        l2 += p2;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const float vx = E::get(vv[u][x], e);
          o1[e] += p1 * vx;
          o2[e] += p2 * vx;
        }
      }
    }
  }

  // lanes with the same channels but different keys: sum (same reference m)
#pragma unroll
  for (int off = VL; off < 64; off <<= 1) {
    l1 = xor_sum(l1, off);
    l2 = xor_sum(l2, off);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      o1[e] = xor_sum(o1[e], off);
      o2[e] = xor_sum(o2[e], off);
    }
  }

  __shared__ float sm[kWaves][4];
  __shared__ float so[kWaves][2][DV];
  if (lane < VL) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      so[wave][0][vl * EPC + e] = o1[e];
      so[wave][1][vl * EPC + e] = o2[e];
    }
  }
  if (lane == 0) {
    sm[wave][0] = m1;
    sm[wave][1] = l1;
    sm[wave][2] = m2;
    sm[wave][3] = l2;
  }
  __syncthreads();

  float M1 = -INFINITY, M2 = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    M1 = fmaxf(M1, sm[w][0]);
    M2 = fmaxf(M2, sm[w][2]);
  }
  float w1[kWaves], w2[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    w1[w] = (M1 == -INFINITY) ? 0.f : exp2_fast(sm[w][0] - M1);
    w2[w] = (M2 == -INFINITY) ? 0.f : exp2_fast(sm[w][2] - M2);
  }
  float* __restrict__ rec = a.ws + (bh * a.S + s) * REC;
  for (int t = threadIdx.x; t < DV; t += blockDim.x) {
    float x1 = 0.f, x2 = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      x1 += so[w][0][t] * w1[w];
      x2 += so[w][1][t] * w2[w];
    }
    rec[4 + t] = x1;
    rec[4 + DV + t] = x2;
  }
  if (threadIdx.x == 0) {
    float L1 = 0.f, L2 = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      L1 += sm[w][1] * w1[w];
      L2 += sm[w][3] * w2[w];
    }
    rec[0] = M1;
    rec[1] = L1;
    rec[2] = M2;
    rec[3] = L2;
  }
}

template <typename T, int D, bool NORM>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  using E = Elem<T>;
  constexpr int DV = 2 * D;
  constexpr size_t REC = 4 + 2 * DV;
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t bh = (size_t)b * a.H + h;
  const int S = a.S;
  const float* __restrict__ rec = a.ws + bh * S * REC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // wavefront-shuffle merge of the split maxima and denominators
  float M1 = -INFINITY, M2 = -INFINITY;
  for (int s = lane; s < S; s += 64) {
    M1 = fmaxf(M1, rec[s * REC + 0]);
    M2 = fmaxf(M2, rec[s * REC + 2]);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    M1 = xor_max(M1, off);
    M2 = xor_max(M2, off);
  }
  float L1 = 0.f, L2 = 0.f;
  if (M1 != -INFINITY) {
    for (int s = lane; s < S; s += 64) {
      L1 += rec[s * REC + 1] * exp2_fast(rec[s * REC + 0] - M1);
      L2 += rec[s * REC + 3] * exp2_fast(rec[s * REC + 2] - M2);
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    L1 = xor_sum(L1, off);
    L2 = xor_sum(L2, off);
  }

  // numerators: each thread owns one channel, splits in a fixed order
  const int t = threadIdx.x;
  float y = 0.f;
  if (t < DV && M1 != -INFINITY && L1 > 0.f && L2 > 0.f) {
    float x1 = 0.f, x2 = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* r = rec + s * REC;
      x1 += r[4 + t] * exp2_fast(r[0] - M1);
      x2 += r[4 + DV + t] * exp2_fast(r[2] - M2);
    }
    y = x1 / L1 - (*a.lambda) * (x2 / L2);
  }

  float outv = y;
  if (NORM) {
    __shared__ float red[4];
    float ss = y * y;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) ss = xor_sum(ss, off);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    ss = red[0] + red[1] + red[2] + red[3];
    const float r = a.out_scale / sqrtf(ss * (1.0f / DV) + a.eps);
    outv = y * r * ((a.norm_w && t < DV) ? a.norm_w[t] : 1.0f);
  }
  if (t < DV) E::store((T*)a.out + bh * DV + t, outv);
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: the split records of one call
// (B*H*S records of 4 + 4d floats).  Every split writes its whole record
// before the merge reads it, so the array never needs clearing; calls that
// overlap on one GPU share it and race.

static __device__ __align__(256) unsigned char scratch[DIFFATTN_NOALLOC_SCRATCH_BYTES];

// The array's address on the device that runs `stream`, looked up once per
// device with that device current (the host-side name is only a stand-in
// and never reaches a kernel).  No allocation happens.
hipError_t decode_scratch(hipStream_t stream, float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = (float*)addr[dev];
  return hipSuccess;
}

void decode_plan(int B, int H, int L, int d, int* S, int* chunk) {
  (void)d;
  const long long BH = (long long)B * H;
  if (L <= 0 || BH <= 0) {
    *S = 1;
    *chunk = 0;
    return;
  }
  // aim for ~8192 workgroups in flight, splits of at least 256 keys
  const long long target = 8192;
  long long s = (target + BH - 1) / BH;
  const long long smax = (L + 255) / 256;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  long long ch = (L + s - 1) / s;
  ch = (ch + 63) / 64 * 64;
  s = (L + ch - 1) / ch;
  *S = (int)s;
  *chunk = (int)ch;
}

template <typename T, int D>
static hipError_t launch_t(bool norm, const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(a.S, a.H, a.B), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (norm)
    hipLaunchKernelGGL((decode_merge_kernel<T, D, true>), dim3(a.H, a.B), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_merge_kernel<T, D, false>), dim3(a.H, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dd(bool bf16, bool norm, const DecodeArgs& a, hipStream_t st) {
  return bf16 ? launch_t<__bf16, D>(norm, a, st) : launch_t<float, D>(norm, a, st);
}

hipError_t launch_decode(bool bf16, int d, bool norm, const DecodeArgs& a, hipStream_t stream) {
  switch (d) {
    case 16: return launch_dd<16>(bf16, norm, a, stream);
    case 32: return launch_dd<32>(bf16, norm, a, stream);
    case 64: return launch_dd<64>(bf16, norm, a, stream);
    case 128: return launch_dd<128>(bf16, norm, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace diffattn
