// Device helpers shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// bf16 <-> fp32

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two floats to two bf16 values (round to nearest even) by the hardware
// pack conversion (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---------------------------------------------------------------------------
// order-preserving uint32 key of a float (larger float -> larger key);
// callers canonicalise -0.0 to +0.0 first.

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------------------
// 16-byte global loads reinterpreted as MFMA operands

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ bf16x8_t zero_bf16x8() {
  u32x4_t v = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ s16x4_t as_s16x4(u32x2_t v) { return __builtin_bit_cast(s16x4_t, v); }

// ---------------------------------------------------------------------------
// MFMA wrappers.
//
// v_mfma_f32_16x16x32_bf16 (gfx950): A 16x32, B 32x16, D 16x16.
//   lane l holds A[l%16][8*(l/16) + j], B[8*(l/16) + j][l%16], j = 0..7,
//   and D[4*(l/16) + r][l%16], r = 0..3.
// v_mfma_f32_16x16x16_bf16: the same with 4 k-values per lane,
//   A[l%16][4*(l/16) + j], B[4*(l/16) + j][l%16], j = 0..3.

__device__ __forceinline__ f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma16(s16x4_t a, s16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i%4 of the 8-byte chunks addressed by lanes
// i/4 + 4j, j = 0..3.  So if lane s of the group addresses row R0 + s/4 and
// columns C0 + 4(s%4) .. +3 of a row-major bf16 tile, lane i receives column
// C0 + i of rows R0 .. R0+3: a 4-value MFMA operand read across rows.

typedef short s16x4_lds_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4_t read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_lds_t*)p);
}

// Offset (in elements) of the chunk lane c16 addresses for read_tr from a
// tile with row stride `stride`: row c16/4, columns 4*(c16%4).
__device__ __forceinline__ int tr_offset(int c16, int stride) { return (c16 >> 2) * stride + 4 * (c16 & 3); }

// ---------------------------------------------------------------------------
// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// orders global memory, which on this ISA (loads and stores share one
// counter) waits for every global load in flight, prefetches included.

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// wave helpers

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of m in lanes below this one
__device__ __forceinline__ int mbcnt(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  for (int o = 32; o >= 1; o >>= 1) v |= (uint32_t)__shfl_xor((int)v, o, kWave);
  return v;
}

__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  for (int o = 32; o >= 1; o >>= 1) v &= (uint32_t)__shfl_xor((int)v, o, kWave);
  return v;
}

}  // namespace dsa
