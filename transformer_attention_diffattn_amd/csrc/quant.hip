// Per-tensor absmax quantisation of bf16 queries/keys to OCP e4m3 bytes, the
// input of the fp8 QK^T forward (low-bit attention logits: "Differential
// Transformer" sample peer review, "Strengths", and the figure on low-bit
// attention logits, Fig. 8, that it discusses).
//
//   scale = amax / 448,   code = e4m3(x * (448 / amax))   (amax = max |x|)
//
// with float32 division and product, round to nearest even, saturation at
// 448, and scale 1 for an all-zero tensor.  Two passes over HBM: partial
// maxima per workgroup, then every workgroup reduces the (few) partials
// itself and encodes its share.  Both passes are bandwidth-bound streams of
// 16-byte loads.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace diffattn {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kMaxPartials = 256;   // pass 1 workgroups: few partials for every pass-2 workgroup to reduce
constexpr int kMaxEncodeGroups = 2048;

// fp32 -> e4m3 code: round to nearest even, saturating at 448.
//   |y| >= 448          -> 0x7E
//   |y| <  2^-6         -> subnormal: the nearest multiple of 2^-9 (8 of them
//                          is 2^-6, whose code 0x08 is the smallest normal)
//   otherwise           -> the fp32 exponent/mantissa field rounded to 3
//                          mantissa bits, exponent rebased from 127 to 7
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t mag = u & 0x7fffffffu;
  uint32_t c;
  if (mag >= 0x43E00000u)
    c = 0x7Eu;
  else if (mag < 0x3C800000u)
    c = (uint32_t)__builtin_rintf(__builtin_bit_cast(float, mag) * 512.0f);
  else
    c = ((mag + 0x7FFFFu + ((mag >> 20) & 1u)) >> 20) - 960u;
  return ((u >> 24) & 0x80u) | c;
}

// max over the workgroup of a non-negative value held as bits (finite
// non-negative floats order like their bit patterns)
__device__ __forceinline__ uint32_t block_max_u32(uint32_t x, uint32_t* sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, off));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = x;
  __syncthreads();
  uint32_t r = sh[0];
#pragma unroll
  for (int i = 1; i < kQuantThreads / 64; ++i) r = max(r, sh[i]);
  __syncthreads();
  return r;
}

// Both passes take up to kQuantBatch tensors of n values at once, one per
// blockIdx.y: the same two launches then serve all of them.
// Pass 1: partial[t][blockIdx.x] = max |x_t| over this workgroup's 8-value
// chunks (and, for workgroup 0, the n % 8 values after the last whole chunk).
__global__ __launch_bounds__(kQuantThreads) void amax_partial_kernel(QuantBatch q) {
  __shared__ uint32_t sh[kQuantThreads / 64];
  const uint16_t* __restrict__ x = q.x[blockIdx.y];
  float* __restrict__ partial = q.partial + (size_t)blockIdx.y * q.P;
  const long long n = q.n;
  const long long chunks = n / 8;
  uint32_t m = 0;  // bf16 magnitude bits
#pragma unroll 4
  for (long long i = (long long)blockIdx.x * kQuantThreads + threadIdx.x; i < chunks;
       i += (long long)gridDim.x * kQuantThreads) {
    const u32x4 w = ld16(x + 8 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = w[j];
      m = max(m, max(v & 0x7fffu, (v >> 16) & 0x7fffu));
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < (unsigned)(n - 8 * chunks)) m = max(m, x[8 * chunks + threadIdx.x] & 0x7fffu);
  m = block_max_u32(m, sh);
  if (threadIdx.x == 0) partial[blockIdx.x] = __builtin_bit_cast(float, m << 16);
}

// Pass 2: amax from the P partials, then codes of this workgroup's chunks;
// workgroup 0 writes the scale and the codes of the tail.
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(QuantBatch q) {
  __shared__ uint32_t sh[kQuantThreads / 64];
  const uint16_t* __restrict__ x = q.x[blockIdx.y];
  const float* __restrict__ partial = q.partial + (size_t)blockIdx.y * q.P;
  uint8_t* __restrict__ codes = q.codes[blockIdx.y];
  float* __restrict__ scale = q.scale + blockIdx.y;
  const long long n = q.n;
  const int P = q.P;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < P; i += kQuantThreads) m = max(m, __builtin_bit_cast(uint32_t, partial[i]));
  m = block_max_u32(m, sh);
  const float amax = __builtin_bit_cast(float, m);
  const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = amax > 0.f ? amax / 448.0f : 1.0f;
  const long long chunks = n / 8;
#pragma unroll 2
  for (long long i = (long long)blockIdx.x * kQuantThreads + threadIdx.x; i < chunks;
       i += (long long)gridDim.x * kQuantThreads) {
    const u32x4 w = ld16(x + 8 * i);
    u32x2 out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t v = w[2 * h + j];
        word |= e4m3_code(bf16_lo(v) * inv) << (16 * j);
        word |= e4m3_code(bf16_hi(v) * inv) << (16 * j + 8);
      }
      out[h] = word;
    }
    *reinterpret_cast<u32x2*>(codes + 8 * i) = out;
  }
  if (blockIdx.x == 0 && threadIdx.x < (unsigned)(n - 8 * chunks)) {
    const long long k = 8 * chunks + threadIdx.x;
    codes[k] = (uint8_t)e4m3_code(__builtin_bit_cast(float, (uint32_t)x[k] << 16) * inv);
  }
}

}  // namespace

int quant_partial_blocks(long long n) {
  const long long chunks = (n + 7) / 8;
  const long long b = (chunks + 8 * kQuantThreads - 1) / (8 * kQuantThreads);
  return (int)(b < 1 ? 1 : (b > kMaxPartials ? kMaxPartials : b));
}

hipError_t launch_quantize_fp8(int count, const void* const* x, long long n, float* partial, void* const* codes,
                               float* scales, hipStream_t stream) {
  if (count < 1 || count > kQuantBatch) return hipErrorInvalidValue;
  QuantBatch q = {};
  for (int t = 0; t < count; ++t) {
    q.x[t] = (const uint16_t*)x[t];
    q.codes[t] = (uint8_t*)codes[t];
  }
  q.scale = scales;
  q.partial = partial;
  q.n = n;
  q.P = quant_partial_blocks(n);
  const long long chunks = n / 8;
  long long g = (chunks + kQuantThreads - 1) / kQuantThreads;
  g = g < 1 ? 1 : (g > kMaxEncodeGroups ? kMaxEncodeGroups : g);
  hipLaunchKernelGGL(amax_partial_kernel, dim3(q.P, count), dim3(kQuantThreads), 0, stream, q);
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)g, count), dim3(kQuantThreads), 0, stream, q);
  return hipGetLastError();
}

}  // namespace diffattn
