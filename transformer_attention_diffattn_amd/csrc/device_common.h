// Device helpers shared by the differential-attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;  // 32 fp8 values

// log2(e): softmax weights are formed as 2^(s * log2(e)/sqrt(d) - m) so that
// one FMA and one v_exp_f32 give exp((s - m')/sqrt(d)).
constexpr float kLog2e = 1.44269504088896340736f;

// Rescale threshold (log2 units): the running reference maximum of a row is
// raised only when a new score exceeds it by more than this, so weights stay
// below 2^8 = 256 -- harmless in fp32 accumulators and in bf16 -- and the
// accumulators are rescaled only when a row's maximum jumps.  Exact: the
// numerator and denominator always share the same reference.
constexpr float kRescaleThreshold = 8.0f;

// Fourth word of a buffer resource for raw (byte-offset) access: 32-bit data
// format, no swizzle; with stride 0 the hardware drops every access whose
// offset + size exceeds the resource's byte count.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Cache-policy operand of a store written once and not read again by the
// kernel (the non-temporal bit): the lines should not displace K/V tiles
// that other workgroups still read from the L2.
constexpr int kStoreStreaming = 2;

__device__ __forceinline__ f32x4 mfma16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x128 product of e4m3 operands (both format fields 0 = fp8 e4m3) with
// unit block scales (exponent byte 127 = 2^0).  Lane L holds row L % 16 of
// A (and of B) with 32 of its 128 reduction elements; any assignment of
// reduction elements to lane groups and bytes gives the same product as long
// as A and B use the same one.  C has the 16x16x32 bf16 product's layout.
__device__ __forceinline__ f32x4 mfma16x16x128_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ f32x4 mfma16x16x4_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Two floats -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), lo first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Reinterpret one 32-bit word.  Always pass a scalar copy: bit-casting a
// vector element expression (v[i]) directly reads element 0 with this
// compiler, so vector elements go through these by-value helpers.
__device__ __forceinline__ float u32_as_f32(uint32_t w) { return __builtin_bit_cast(float, w); }
__device__ __forceinline__ bf16x2 u32_as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 zero_u32x4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

__device__ __forceinline__ f32x4 zero_f32x4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// Transposing LDS read (ds_read_b64_tr_b16).  Each lane of a 16-lane group
// supplies the address of 4 consecutive bf16 of one row; the group's 16 x 4
// block comes back transposed.  With a tile stored as [16-column block][row]
// [16 columns] and lane L pointing at element 16 (r0 + L / 4) + 4 (L % 4) of
// a column block, lane L receives that block's column L % 16 for rows
// r0 + 4 (L / 16) .. + 3 -- half of the A operand of a 16x16x32 MFMA whose
// k runs over rows.
typedef __attribute__((ext_vector_type(4))) short s16x4;
#define DIFFATTN_LDS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Byte offset of an LDS location (wave-uniform callers only).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)DIFFATTN_LDS(p));
}

// 16 bytes per lane from global memory straight into LDS at lds + 16*lane
// (global_load_lds_dwordx4).  Issued through asm so that the compiler does
// not track it: it would otherwise wait for every outstanding tile before
// any LDS read.  Completion is awaited explicitly with s_waitcnt vmcnt plus
// a workgroup barrier before the data is read.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds) : "memory", "m0");
}
// The same with a wave-uniform 64-bit base (scalar registers) and a 32-bit
// per-lane byte offset.
__device__ __forceinline__ void lds_dma16_s(const void* base, uint32_t off, uint32_t lds) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t ul = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(ub), "s"(ul) : "memory", "m0");
}
// wait until at most K vector-memory operations of this wave are outstanding
template <int K>
__device__ __forceinline__ void wait_vmem_keep() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K) : "memory");
}
// 4 bytes per lane straight into LDS at lds + 4*lane (global_load_lds_dword),
// with a wave-uniform base and a per-lane byte offset; tracked like the
// 16-byte form.
__device__ __forceinline__ void lds_dma4_s(const void* base, uint32_t off, uint32_t lds) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t ul = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(ub), "s"(ul) : "memory", "m0");
}

// 16-byte global load / store through plain pointers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Reductions across the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max_over_lane_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float sum_over_lane_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

}  // namespace diffattn
