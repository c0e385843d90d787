// Shared device helpers for the gfx950 (CDNA4) kernels: vector types, MFMA
// wrappers, LDS transpose reads, bf16 conversion and wave-level reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define DSA_LDS __attribute__((address_space(3)))

// 16x16x32 bf16 MFMA. Lane l: A row l%16 with k = 8*(l/16)+e; B column l%16 with
// k = 8*(l/16)+e; C column l%16 with rows 4*(l/16)+j.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 32x32x16 bf16 MFMA. Lane l: A row l%32 with k = 8*(l/32)+e; B column l%32;
// C column l%32 with rows 8*(j/4) + 4*(l/32) + j%4.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x4 fp32 MFMA. Lane l: A row l%16 with k = l/16; B column l%16 with k = l/16.
__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS transpose read of 4 x 16-bit elements. Within each group of 16 lanes,
// lane j receives element j%4 of the 8 bytes addressed by lane 4*e + j/4, for
// e = 0..3. If lane j of the group points at row (base + j/4), column
// (col0 + 4*(j%4)) of a row-major 16-bit matrix, it receives column col0 + j of
// rows base .. base+3.
__device__ __forceinline__ short4v lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSA_LDS short4v*)(p));
}
// Same read from a pointer already in the LDS address space: a base plus a constant
// then folds into the instruction's offset field, one address register per base.
__device__ __forceinline__ short4v lds_read_tr16(DSA_LDS const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSA_LDS short4v*)(p));
}

__device__ __forceinline__ bf16x8 join_bf16x8(short4v lo, short4v hi) {
  typedef short short8v __attribute__((ext_vector_type(8)));
  short8v v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f2bf_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf_bits2f(uint16_t b) {
  return __builtin_bit_cast(float, ((uint32_t)b) << 16);
}

// Eight floats to bf16 with the hardware convert (round to nearest even, the same
// as f2bf_bits for finite values), two per instruction.
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, bf16x8);
}

// Workgroup barrier that orders LDS accesses only. __syncthreads() also waits for
// every outstanding global load (vmcnt(0)), which would drain the direct-to-LDS
// prefetch ring; tile data is instead waited for explicitly with s_waitcnt
// vmcnt(n) before the barrier that publishes a tile.
// 16-byte direct global->LDS load: lane l writes LDS bytes [m0 + 16 l, m0 + 16 l + 16).
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_base) : "memory");
}
// Same with a wave-uniform base address (SGPRs) plus a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_base) : "memory");
}

// A wave-uniform pointer, moved to scalar registers (direct loads take their base
// address from there). Both halves are read as unsigned 32-bit values, so the low
// word is zero-extended when the halves are joined.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 2^x with the hardware instruction alone (about 1 ulp; results below 2^-126
// flush to zero, which softmax weights never need). exp2f adds a range check and
// rescale for denormal results that costs several instructions per call.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum of the eight bf16 values of v, in fp32 (exact conversions), pairwise.
__device__ __forceinline__ float sum_bf16x8(bf16x8 v) {
  const u32x4 w = __builtin_bit_cast(u32x4, v);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    s += __uint_as_float(w[e] << 16) + __uint_as_float(w[e] & 0xFFFF0000u);
  return s;
}

// Combine lanes l, l^16, l^32, l^48 (the four 16-lane groups that hold the same
// 16x16 MFMA column) with the lane-swap instructions: each swap hands both lanes of
// a pair the two values in the same order, so all four lanes end bit-identical.
__device__ __forceinline__ float group4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace dsa
