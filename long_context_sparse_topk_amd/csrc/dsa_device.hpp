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

// ---------------------------------------------------------------------------
// Cross-lane steps on DPP (data-parallel primitives: a VALU operand read from
// another lane of the same row of 16), which need no LDS round trip as
// ds_bpermute (what __shfl lowers to) does.  dpp_ctrl values of this ISA:
// quad_perm [1,0,3,2] and [2,3,0,1] exchange lanes 1 and 2 apart within each
// quad, row_half_mirror reverses each half row of 8 lanes, row_mirror each
// row; after the first k of these four steps a lane holds the combination of
// 2^k lanes of its row.  row_shr:n reads the lane n before (0 before the row
// start, with bound_ctrl); row_bcast:15 / :31 read lane 15 of the row before /
// lane 31, in the rows that row_mask enables.  The helpers below read other
// lanes' values, so they are called with all 64 lanes of the wave active.
constexpr int kDppQuadSwap1 = 0xB1;
constexpr int kDppQuadSwap2 = 0x4E;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr3 = 0x113;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int kCtrl, int kRowMask = 0xF, int kBankMask = 0xF, bool kBoundZero = false>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, kBankMask, kBoundZero);
}

// every lane of a row of 16 gets op over the row's 16 values
template <class Op>
__device__ __forceinline__ int row_reduce16(int v, Op op) {
  v = op(v, dpp<kDppQuadSwap1>(v));
  v = op(v, dpp<kDppQuadSwap2>(v));
  v = op(v, dpp<kDppRowHalfMirror>(v));
  return op(v, dpp<kDppRowMirror>(v));
}

__device__ __forceinline__ int row_sum16(int v) {
  return row_reduce16(v, [](int x, int y) { return x + y; });
}

// op over the wave: the rows' results combined from lanes 0, 16, 32, 48
template <class Op>
__device__ __forceinline__ int wave_reduce(int v, Op op) {
  const int r = row_reduce16(v, op);
  return op(op(__builtin_amdgcn_readlane(r, 0), __builtin_amdgcn_readlane(r, 16)),
            op(__builtin_amdgcn_readlane(r, 32), __builtin_amdgcn_readlane(r, 48)));
}

__device__ __forceinline__ int wave_max(int v) {
  return wave_reduce(v, [](int x, int y) { return x > y ? x : y; });
}

__device__ __forceinline__ int wave_min(int v) {
  return wave_reduce(v, [](int x, int y) { return x < y ? x : y; });
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  return (uint32_t)wave_reduce((int)v, [](int x, int y) { return x | y; });
}

__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  return (uint32_t)wave_reduce((int)v, [](int x, int y) { return x & y; });
}

// inclusive prefix sum over the 64 lanes: sums of 4 within a row, then of 8
// and 16 (lanes 4.. and 8.. of each row), then the earlier rows' totals
__device__ __forceinline__ int wave_prefix_sum(int v) {
  int s = v + dpp<kDppRowShr1, 0xF, 0xF, true>(v);
  s += dpp<kDppRowShr2, 0xF, 0xF, true>(v);
  s += dpp<kDppRowShr3, 0xF, 0xF, true>(v);
  s += dpp<kDppRowShr4, 0xF, 0xE>(s);
  s += dpp<kDppRowShr8, 0xF, 0xC>(s);
  s += dpp<kDppRowBcast15, 0xA>(s);
  return s + dpp<kDppRowBcast31, 0xC>(s);
}

}  // namespace dsa
