// Pieces shared by the indexer kernels (internal): launch constants, the
// arguments, the threshold sampling constants and the exact top-k selection of
// one candidate list.
#pragma once

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {
namespace {

constexpr int kDI = 64;              // indexer head dim
constexpr int kQT = kIndexQueryTile; // queries per sub-tile of the wider variant
constexpr int kPT = kIndexPoolTile;  // 64 pools per staged tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kBufferWord3 = 0x00020000;  // raw buffer: 32-bit data format, no swizzle
constexpr int kWaitVmcnt0 = 0x0F70;        // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15)
constexpr int kWaitVmcnt2 = 0x0F72;        // s_waitcnt vmcnt(2) expcnt(7) lgkmcnt(15)
constexpr int kRing = 3;                   // LDS key-tile buffers
constexpr int kExactSharedSlots = 64;      // exact-pass grid when the CUs are shared

// exact top-k of one candidate list, wave-wide (all arguments wave-uniform).
// Keeps the k largest keys, equal keys in list order, stably compacted to the
// front of the list (or, with `out` set, written to `out` as pool ids).
// Returns the k-th largest key's float value.  The caller has made the
// wave's candidate stores visible (__threadfence_block) beforehand.
//
// The list is read in chunks of 64 x kR entries, keys and pool ids together,
// with all loads of a lane in flight; a list of up to 64 x kR entries is read
// once and stays in registers through every pass.  The k-th largest key is
// found by a radix select over the bits where the keys differ (their OR xor
// AND), 8 bits per pass, with a per-wave LDS histogram.  kR is the caller's
// register budget: with 24 a list of up to 1536 entries is read once, with 8
// a longer list is read again in every pass.

template <int kR>
__device__ __forceinline__ void load_chunk(const u32x2_t* __restrict__ list, int base, int n,
                                           u32x2_t (&e)[kR]) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    const int j = base + i * kWave + lane;
    e[i] = j < n ? list[j] : u32x2_t{0u, 0u};
  }
}

// Steps of a chunk are skipped (wave-uniformly) past the list end, so short
// lists cost in proportion to their length.
template <int kR>
__device__ __forceinline__ float select_and_compact(u32x2_t* __restrict__ list, int n, int k, uint32_t* hist,
                                    int32_t* __restrict__ out) {
  constexpr int kChunk = kWave * kR;
  const int lane = lane_id();
  const int nch = (n + kChunk - 1) / kChunk;
  u32x2_t e[kR];
  if (nch == 1) load_chunk(list, 0, n, e);

  uint32_t o = 0u, an = 0xFFFFFFFFu;
  for (int c = 0; c < nch; ++c) {
    if (nch > 1) load_chunk(list, c * kChunk, n, e);
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      if (c * kChunk + i * kWave >= n) break;
      if (c * kChunk + i * kWave + lane < n) {
        o |= e[i][0];
        an &= e[i][0];
      }
    }
  }
  o = wave_or(o);
  an = wave_and(an);
  const uint32_t X = o ^ an;        // bits where the keys differ
  uint32_t prefix = an & ~X;        // bits common to every key
  int rem = k;                      // keys still to take among those in play

  if (X != 0u) {
    const int hi = 31 - __clz((int)X);
    const int lo = __ffs((int)X) - 1;
    int top = hi + 1;               // bits >= top of the answer are fixed in prefix
    while (top > lo) {
      const int width = min(8, top - lo);
      const int shift = top - width;
      const uint32_t dmask = (1u << width) - 1u;
      const uint32_t hmask = top >= 32 ? 0u : (0xFFFFFFFFu << top);
      const uint32_t want = prefix & hmask;
#pragma unroll
      for (int b = 0; b < 4; ++b) hist[lane * 4 + b] = 0u;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      for (int c = 0; c < nch; ++c) {
        if (nch > 1) load_chunk(list, c * kChunk, n, e);
#pragma unroll
        for (int i = 0; i < kR; ++i) {
          if (c * kChunk + i * kWave >= n) break;
          const bool in = c * kChunk + i * kWave + lane < n;
          if (in && (e[i][0] & hmask) == want) atomicAdd(&hist[(e[i][0] >> shift) & dmask], 1u);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      const int h0 = (int)hist[lane * 4 + 0], h1 = (int)hist[lane * 4 + 1];
      const int h2 = (int)hist[lane * 4 + 2], h3 = (int)hist[lane * 4 + 3];
      const int tot = h0 + h1 + h2 + h3;
      // inclusive suffix sum over lanes (bins ascending with lane)
      const int pre = wave_prefix_sum(tot);
      const int suf = __builtin_amdgcn_readlane(pre, kWave - 1) - pre + tot;
      const uint64_t ge = ballot(suf >= rem);
      const int L = 63 - __clzll((long long)ge);
      const int s3 = suf - tot + h3, s2 = s3 + h2, s1 = s2 + h1;
      int d, above;
      if (s3 >= rem) { d = 3; above = s3 - h3; }
      else if (s2 >= rem) { d = 2; above = s2 - h2; }
      else if (s1 >= rem) { d = 1; above = s1 - h1; }
      else { d = 0; above = suf - h0; }
      const int digit = __builtin_amdgcn_readlane(lane * 4 + d, L);
      above = __builtin_amdgcn_readlane(above, L);
      rem -= above;
      prefix |= (uint32_t)digit << shift;
      top = shift;
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  }

  // keep every key > T and the first `rem` keys == T, in list order
  const uint32_t T = prefix;
  int kept = 0, eqseen = 0;
  for (int c = 0; c < nch; ++c) {
    if (nch > 1) load_chunk(list, c * kChunk, n, e);
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      if (c * kChunk + i * kWave >= n) break;
      const bool in = c * kChunk + i * kWave + lane < n;
      const bool gtf = in && e[i][0] > T;
      const bool eqf = in && e[i][0] == T;
      const uint64_t EQ = ballot(eqf);
      const bool keep = gtf || (eqf && (eqseen + mbcnt(EQ)) < rem);
      const uint64_t K = ballot(keep);
      if (keep) {
        const int dst = kept + mbcnt(K);
        if (out) out[dst] = (int32_t)e[i][1];
        else list[dst] = e[i];
      }
      kept += __popcll(K);
      eqseen += __popcll(EQ);
    }
  }
  // Chunk loads past the list end are never consumed; wait for them here so
  // that the callers' loops do not inherit outstanding loads (which would
  // make every later wait on the key prefetch a full vmcnt(0)).
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  return key_to_float(T);
}


struct KernelArgs {
  const uint16_t* q_idx;
  const uint16_t* w_idx;
  const uint16_t* kpool;
  const uint8_t* kpool8;   // the 32x32-layout kernel's pooled keys (fp8 or bf16 rows)
  const int32_t* q_pos;
  int64_t q_base;          // position of row 0 when q_pos is NULL
  int64_t Sq, Sk;
  int n_pools;
  int heads, topk, cap;
  const int32_t* rows;     // exact pass: rows to score (the fallback list)
  const uint32_t* nrows;   // exact pass: device count of rows
  uint32_t* fb_count;      // two-phase pass: fallback list length
  int32_t* fb_rows;        // two-phase pass: fallback list
  uint32_t* tile_next;     // this pass's tile queue (next tile rank)
  u32x2_t* cand;           // [slots][kQT][cap] (order key, pool id)
  int32_t* idx_out;
};

// Phase-1 sample: every kSampleStride-th pool tile.  With a fraction f of a
// query's causal pools sampled, about r/f pools score at or above the r-th
// best sampled score, with a spread of about sqrt(r)/f; r is the smallest
// value with r - z sqrt(r) >= k f, z spreads of margin.  A small margin
// keeps fewer survivors (a cheaper phase 2) and fails more often: phase 2
// runs with kSampleZ1 and, in a workgroup where some query failed, once more
// for those queries with kSampleZ2; a query failing twice goes to the exact
// pass.
constexpr int kSampleStride = 16;
// Query tiles whose causal range spans at most kSampleShortTiles pool tiles
// sample every kSampleStrideShort-th tile instead when k is small: their rows
// are short, so survivors weigh more against the sample (S = 4096, k = 128:
// 0.124 against 0.147 ms with fp8 operands, 0.079 against 0.082 with bf16;
// from S = 2^17 on the two strides are within run-to-run noise).  With a large
// k the denser sample pushes the rank r towards what the lanes keep (r near 96
// at k = 512), the kept-score threshold falls short of the true r-th best and
// survivors overflow, so k above kSampleShortMaxTopk keeps the wide stride
// (S = 2^15, k = 512: 0.87 against 0.46 ms without that bound).
constexpr int kSampleStrideShort = 8;
constexpr int kSampleShortTiles = 128;
constexpr int kSampleShortMaxTopk = 256;
__device__ inline int sample_stride(int ntp, int topk) {
  return (ntp <= kSampleShortTiles && topk <= kSampleShortMaxTopk) ? kSampleStrideShort
                                                                   : kSampleStride;
}
constexpr float kSampleZ1 = 3.f;
constexpr float kSampleZ2 = 5.f;
// Workgroups the device keeps resident at once, and its CU count.
struct Residency {
  int cus, per_cu;
};

constexpr int kFlushPeriod = 32;                 // tiles between periodic stage flushes

// largest float below x (x finite or -inf); +0 and -0 are one score
__device__ __forceinline__ float float_below(float x) {
  if (x == 0.f) return -__builtin_bit_cast(float, 1u);
  if (x == -__builtin_huge_valf()) return x;
  return key_to_float(order_key(x) - 1u);
}

}  // namespace
}  // namespace dsa
