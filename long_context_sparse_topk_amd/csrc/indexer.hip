// Lightning indexer with a fused per-query top-k (gfx950).
//
// What is computed (pages: "SkyRL 将 GLM-5.3-Flash 训练上下文扩至 100 万 token",
// sections "模型与瓶颈" and "四块优化 1. DSA 真稀疏"): every query is scored
// against every complete 4-token pool of indexer keys and keeps the top-k pools
// as an int32 id list.  The pages chunk the queries so the score matrix never
// exists in full; here no score row leaves the chip at all.
//
// Kernels:
//   pool_keys_kernel    kpool[p] = bf16(mean of k_idx[4p..4p+3])   (HBM-bound)
//   indexer_topk_kernel per workgroup sub-tile of 64 queries (256 rows of
//                       query x indexer-head), stream the causal pool range in
//                       tiles of 64 pools staged in LDS; bf16 MFMA 16x16x32 gives
//                       the 4 head dot products of a (query, pool) pair in one
//                       lane, so ReLU, the head weights and the head sum are an
//                       in-register epilogue.  Each score is compared with the
//                       query's running threshold (the k-th best key so far);
//                       survivors are appended, in pool order, to the query's
//                       candidate list in the workspace.  When a list could
//                       overflow, the owning wave selects its exact top-k with a
//                       radix select over the order-preserving float keys and
//                       compacts it stably, raising the threshold.  The final
//                       list is already ascending in pool id.
//
// Exactness: pools are streamed in ascending id order and a candidate joins the
// list only if its score is strictly greater than the threshold score, so an
// equal score with a higher id loses exactly as the rule "ties go to the lower
// pool id" demands; compaction breaks score ties by list position, which is
// pool order.

#include <cmath>
#include <mutex>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {
namespace {

constexpr int kDI = 64;              // indexer head dim
constexpr int kQT = kIndexQueryTile; // 64 queries per sub-tile
constexpr int kPT = kIndexPoolTile;  // 64 pools per staged tile
constexpr int kWaves = 4;            // 16 queries per wave
constexpr int kThreads = kWaves * kWave;
constexpr int kBufferWord3 = 0x00020000;  // raw buffer: 32-bit data format, no swizzle

// ---------------------------------------------------------------------------

// Pools [n_pools, n_padded) are zero-filled so that key tiles can be loaded
// whole, without bounds predicates.
// Thread 0 also clears the indexer's fallback-list length.
__global__ __launch_bounds__(256) void pool_keys_kernel(const uint16_t* __restrict__ k_idx,
                                                        uint16_t* __restrict__ kpool,
                                                        int64_t n_pools, int64_t n_padded,
                                                        uint32_t* __restrict__ fb_count) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t == 0) *fb_count = 0u;
  if (t >= n_padded * 8) return;
  const int64_t p = t >> 3;
  const int c = (int)(t & 7);
  if (p >= n_pools) {
    *reinterpret_cast<u32x4_t*>(kpool + p * kDI + c * 8) = u32x4_t{0u, 0u, 0u, 0u};
    return;
  }
  const uint16_t* src = k_idx + (4 * p) * kDI + c * 8;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll
  for (int tok = 0; tok < 4; ++tok) {
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + tok * kDI);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16_to_f32(v[j] & 0xFFFFu);
      acc[2 * j + 1] += bf16_to_f32(v[j] >> 16);
    }
  }
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[2 * j] * 0.25f, acc[2 * j + 1] * 0.25f);
  *reinterpret_cast<u32x4_t*>(kpool + p * kDI + c * 8) = o;
}

// ---------------------------------------------------------------------------
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
// AND), 8 bits per pass, with a per-wave LDS histogram.

constexpr int kR = 24;
constexpr int kChunk = kWave * kR;

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
__device__ __forceinline__ float select_and_compact(u32x2_t* __restrict__ list, int n, int k, uint32_t* hist,
                                    int32_t* __restrict__ out) {
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
      int suf = tot;  // inclusive suffix sum over lanes (bins ascending with lane)
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int t = __shfl_down(suf, off, kWave);
        if (lane + off < kWave) suf += t;
      }
      const uint64_t ge = ballot(suf >= rem);
      const int L = 63 - __clzll((long long)ge);
      const int s3 = suf - tot + h3, s2 = s3 + h2, s1 = s2 + h1;
      int d, above;
      if (s3 >= rem) { d = 3; above = s3 - h3; }
      else if (s2 >= rem) { d = 2; above = s2 - h2; }
      else if (s1 >= rem) { d = 1; above = s1 - h1; }
      else { d = 0; above = suf - h0; }
      const int digit = __shfl(lane * 4 + d, L, kWave);
      above = __shfl(above, L, kWave);
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
  return key_to_float(T);
}

// Tile order: each workgroup takes every gridDim-th tile, snaking, over tiles
// ranked from the longest causal range down (the last query tiles when q_pos
// is the identity).
__device__ __forceinline__ int64_t snake_rank(int64_t it, int slot, int nslots) {
  return (it & 1) ? it * nslots + (nslots - 1 - slot) : it * nslots + slot;
}

struct KernelArgs {
  const uint16_t* q_idx;
  const uint16_t* w_idx;
  const uint16_t* kpool;
  const int32_t* q_pos;
  int64_t Sq, Sk;
  int n_pools;
  int heads, topk, cap;
  const int32_t* rows;     // exact pass: rows to score (the fallback list)
  const uint32_t* nrows;   // exact pass: device count of rows
  uint32_t* fb_count;      // two-phase pass: fallback list length
  int32_t* fb_rows;        // two-phase pass: fallback list
  u32x2_t* cand;           // [slots][kQT][cap] (order key, pool id)
  int32_t* idx_out;
};

// Phase-1 sample: every kSampleStride-th pool tile.  With a fraction f of a
// query's causal pools sampled, about r/f pools score at or above the r-th
// best sampled score, with a spread of about sqrt(r)/f; r is the smallest
// value with r - kSampleZ sqrt(r) >= k f, kSampleZ spreads of margin before
// the query needs the exact pass.
constexpr int kSampleStride = 16;
constexpr float kSampleZ = 5.f;
constexpr int kSampleKeep = 8;   // sampled scores kept per lane and query

// largest float below x (x finite or -inf); +0 and -0 are one score
__device__ __forceinline__ float float_below(float x) {
  if (x == 0.f) return -__builtin_bit_cast(float, 1u);
  if (x == -__builtin_huge_valf()) return x;
  return key_to_float(order_key(x) - 1u);
}

// Two-phase pass (kTwoPhase): per query, phase 1 streams a strided sample of
// the pool tiles and takes the exact r-th best sampled score t; phase 2
// streams every tile keeping pools with score >= t, then the running top-k.
// If at least min(k, n_c) pools score >= t, every true top-k pool does (its
// score is >= the k-th best score >= t), so the result is exact; otherwise
// the query goes to the fallback list, which the exact pass (!kTwoPhase:
// one phase, threshold from -inf) then scores.
template <bool kTwoPhase>
__global__ __launch_bounds__(kThreads, 2) void indexer_topk_kernel(KernelArgs a) {
  __shared__ __align__(16) u32x4_t lds_k[2][kPT * 8];       // 2 x (64 pools x 128 B), swizzled
  __shared__ uint32_t lds_hist[kWaves][256];
  __shared__ int lds_np[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = uniform(tid >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int cap = a.cap;
  const int topk = a.topk;
  uint32_t* hist = lds_hist[wave];
  const float NEG_INF = -__builtin_huge_valf();
  const int64_t nrow = kTwoPhase ? a.Sq : (int64_t)__builtin_amdgcn_readfirstlane(*a.nrows);
  const int64_t ntiles = (nrow + kQT - 1) / kQT;

  for (int64_t it = 0;; ++it) {
    const int64_t rank = snake_rank(it, blockIdx.x, gridDim.x);
    if (rank >= ntiles) break;
    const int64_t q0 = (kTwoPhase ? ntiles - 1 - rank : rank) * kQT;
    auto row_of = [&](int64_t i) -> int64_t {
      if (i >= nrow) return -1;
      return kTwoPhase ? i : (int64_t)a.rows[i];
    };

    // A operands: row (4*qq + h) of row block rb -> query 16*wave + 4*rb + qq, head h
    bf16x8_t A[4][2];
    float w[4][4];
    int nc[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      {
        const int64_t qr = row_of(q0 + 16 * wave + 4 * rb + (c16 >> 2));
        const int h = c16 & 3;
        const bool ok = qr >= 0 && h < a.heads;
        const uint16_t* src = a.q_idx + (qr * a.heads + h) * kDI + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) A[rb][ks] = ok ? load_bf16x8(src + 32 * ks) : zero_bf16x8();
      }
      {
        const int64_t qr = row_of(q0 + 16 * wave + 4 * rb + g);
        const bool ok = qr >= 0;
        int64_t pos = qr;
        if (ok && a.q_pos) {
          pos = a.q_pos[qr];
          pos = pos < 0 ? 0 : (pos >= a.Sk ? a.Sk - 1 : pos);
        }
        nc[rb] = ok ? (int)((pos + 1) >> 2) : 0;
#pragma unroll
        for (int h = 0; h < 4; ++h)
          w[rb][h] = (ok && h < a.heads) ? bf16_to_f32(a.w_idx[qr * a.heads + h]) : 0.f;
      }
    }
    int ncm = max(max(nc[0], nc[1]), max(nc[2], nc[3]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ncm = max(ncm, __shfl_xor(ncm, o, kWave));
    int ncmin = min(min(nc[0], nc[1]), min(nc[2], nc[3]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ncmin = min(ncmin, __shfl_xor(ncmin, o, kWave));
    ncmin = uniform(ncmin);
    if (lane == 0) lds_np[wave] = ncm;
    lds_barrier();
    const int tp = max(max(lds_np[0], lds_np[1]), max(lds_np[2], lds_np[3]));
    const int ntp = (tp + kPT - 1) / kPT;   // pool tiles in the tile's causal range

    int cnt[4] = {0, 0, 0, 0};
    float tau[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
    const int64_t wbase = ((int64_t)blockIdx.x * kQT + 16 * wave) * cap;
    // this lane's query list of each row block: (order key, pool id) pairs
    u32x2_t* clist[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) clist[rb] = a.cand + wbase + (int64_t)(4 * rb + g) * cap;
    const uint32_t lane_below = (1u << c16) - 1u;

    // pool-key tiles: global -> registers two tiles ahead, registers -> LDS
    // one tile ahead (double buffer), one LDS-only barrier per tile.  The
    // loads are unconditional raw buffer loads (the keys are padded to whole
    // tiles) from a per-tile resource and a loop-invariant per-thread offset.
    u32x4_t pre[2];
    auto gload = [&](int tile) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.kpool + (int64_t)tile * kPT * kDI), (short)0, kPT * kDI * 2, kBufferWord3);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        pre[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (tid + kThreads * j) * 16, 0, 0);
    };
    auto lstore = [&](u32x4_t* buf) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = tid + kThreads * j;
        const int pr = c >> 3, ch = c & 7;
        buf[pr * 8 + (ch ^ (pr & 7))] = pre[j];
      }
    };

    // Stream pool tiles first, first+step, ... < ntp; `consume(sc, pt0, more)`
    // receives each tile's scores (-inf where a pool is not causal for the
    // query).  Tile 0 of a stream is always loaded (in bounds: the keys are
    // padded to >= 1 tile) so every path into the loop has waited for the A
    // operands.
    auto stream = [&](int first, int step, auto&& consume) {
      const int nt = first < ntp ? (ntp - first + step - 1) / step : 0;
      gload(first < ntp ? first : 0);
      lstore(lds_k[0]);
      if (nt > 1) gload(first + step);
      lds_barrier();
      for (int i = 0; i < nt; ++i) {
        const int pt0 = (first + i * step) * kPT;
        const u32x4_t* kb = lds_k[i & 1];
        if (i + 1 < nt) {
          lstore(lds_k[(i + 1) & 1]);
          if (i + 2 < nt) gload(first + (i + 2) * step);
        }

        // 16 output blocks of 16 (query x head) rows x 16 pools
        f32x4_t acc[4][4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int pr = 16 * cb + c16;
          const bf16x8_t B0 = as_bf16x8(kb[pr * 8 + (g ^ (pr & 7))]);
          const bf16x8_t B1 = as_bf16x8(kb[pr * 8 + ((4 + g) ^ (pr & 7))]);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            acc[rb][cb] = mfma32(A[rb][1], B1, mfma32(A[rb][0], B0, z));
          }
        }
        // epilogue: ReLU, head weights, head sum (branch-free)
        float sc[4][4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const f32x4_t x = acc[rb][cb];
            float s = w[rb][0] * fmaxf(x[0], 0.f);
            s = fmaf(w[rb][1], fmaxf(x[1], 0.f), s);
            s = fmaf(w[rb][2], fmaxf(x[2], 0.f), s);
            sc[rb][cb] = fmaf(w[rb][3], fmaxf(x[3], 0.f), s);
          }
        }
        // causal pool mask, only on tiles some query of the wave sees in part
        if (pt0 + kPT > ncmin) {
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
              if (pt0 + 16 * cb + c16 >= nc[rb]) sc[rb][cb] = NEG_INF;
        }
        consume(sc, pt0, i + 1 < nt);
        lds_barrier();
      }
    };

    if (kTwoPhase) {
      // Phase 1: each lane keeps, per query, the 8 best sampled scores of
      // its pool column (descending, in registers).  Their union holds at
      // most every sampled score, so its r-th best is at most the sample's.
      int rq[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        // r from the fraction f of the query's causal pools the sample
        // covers; 0 = no estimate (threshold stays -inf)
        const int n_full = nc[rb] / kPT, part = nc[rb] % kPT;
        const int s_q = kPT * ((n_full + kSampleStride - 1) / kSampleStride) +
                        (n_full % kSampleStride == 0 ? part : 0);
        int r = 0;
        if (nc[rb] > topk && s_q > 0) {
          const float f = (float)s_q / (float)nc[rb];
          const float x = 0.5f * (kSampleZ + sqrtf(kSampleZ * kSampleZ + 4.f * topk * f));
          r = (int)ceilf(x * x);
          if (r >= s_q || r > kSampleKeep * 16 * 3 / 4) r = 0;
        }
        rq[rb] = r;
      }
      float best[4][kSampleKeep];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int j = 0; j < kSampleKeep; ++j) best[rb][j] = NEG_INF;
      stream(0, kSampleStride, [&](float (&sc)[4][4], int, bool) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            float x = sc[rb][cb];
            if (ballot(x > best[rb][kSampleKeep - 1])) {
#pragma unroll
              for (int j = 0; j < kSampleKeep; ++j) {
                const float hi = fmaxf(best[rb][j], x);
                x = fminf(best[rb][j], x);
                best[rb][j] = hi;
              }
            }
          }
        }
      });
      // r-th best of the 16 lanes x kSampleKeep kept scores of each query:
      // the largest key v with at least r kept keys >= v, bit by bit
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        uint32_t kk[kSampleKeep];
#pragma unroll
        for (int j = 0; j < kSampleKeep; ++j) kk[j] = order_key(best[rb][j] + 0.f);
        uint32_t pre_k = 0u;
        for (int b = 31; b >= 0; --b) {
          const uint32_t cand_k = pre_k | (1u << b);
          int c = 0;
#pragma unroll
          for (int j = 0; j < kSampleKeep; ++j) c += kk[j] >= cand_k ? 1 : 0;
          c += __shfl_xor(c, 1, kWave);
          c += __shfl_xor(c, 2, kWave);
          c += __shfl_xor(c, 4, kWave);
          c += __shfl_xor(c, 8, kWave);
          if (c >= rq[rb]) pre_k = cand_k;
        }
        tau[rb] = rq[rb] > 0 ? float_below(key_to_float(pre_k)) : NEG_INF;
      }
    }

    // Phase 2 (or the exact pass): every tile; survivors of the running
    // threshold are appended to the query's list in pool order, and a list
    // that could overflow during the next tile keeps its top-k.
    stream(0, 1, [&](float (&sc)[4][4], int pt0, bool more) {
      uint64_t M[4][4];
      uint64_t any = 0;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          M[rb][cb] = ballot(sc[rb][cb] > tau[rb]);
          any |= M[rb][cb];
        }
      if (any) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            if (M[rb][cb]) {
              const uint32_t gm = (uint32_t)(M[rb][cb] >> (16 * g)) & 0xFFFFu;
              if ((gm >> c16) & 1u) {
                const int slot = __popc(gm & lane_below) + cnt[rb];
                u32x2_t e;
                e[0] = order_key(sc[rb][cb] + 0.f);  // -0 -> +0
                e[1] = (uint32_t)(pt0 + 16 * cb + c16);
                clist[rb][slot] = e;
              }
              cnt[rb] += __popc(gm);
            }
          }
        }
      }
      if (more) {
        bool fenced = false;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          uint64_t need = ballot(cnt[rb] > cap - kPT);
          if (need && !fenced) {
            __threadfence_block();  // this wave's candidate stores are visible
            fenced = true;
          }
          while (need) {
            const int L = __ffsll((long long)need) - 1;
            const int gq = L >> 4;
            need &= ~(0xFFFFull << (16 * gq));
            const int n = __shfl(cnt[rb], L, kWave);
            const int64_t base = wbase + (int64_t)(4 * rb + gq) * cap;
            const float T = select_and_compact(a.cand + base, n, topk, hist, nullptr);
            if (g == gq) {
              cnt[rb] = topk;
              tau[rb] = T;
            }
          }
        }
      }
    });

    // final selection, written straight to the output rows
    __threadfence_block();
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      for (int gq = 0; gq < 4; ++gq) {
        const int64_t qr = row_of(q0 + 16 * wave + 4 * rb + gq);
        if (qr < 0) continue;
        const int n = __shfl(cnt[rb], 16 * gq, kWave);
        const int need = min(topk, __shfl(nc[rb], 16 * gq, kWave));
        if (kTwoPhase && n < need) {  // threshold estimate too high
          if (lane == 0) a.fb_rows[atomicAdd(a.fb_count, 1u)] = (int32_t)qr;
          continue;
        }
        const int64_t base = wbase + (int64_t)(4 * rb + gq) * cap;
        int32_t* dst = a.idx_out + qr * topk;
        int filled = n;
        if (n > topk) {
          select_and_compact(a.cand + base, n, topk, hist, dst);
          filled = topk;
        } else {
          const u32x2_t* src = a.cand + base;
          for (int j0 = 0; j0 < n; j0 += 8 * kWave) {
            int32_t v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int j = j0 + i * kWave + lane;
              v[i] = j < n ? (int32_t)src[j][1] : 0;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int j = j0 + i * kWave + lane;
              if (j < n) dst[j] = v[i];
            }
          }
        }
        for (int j = filled + lane; j < topk; j += kWave) dst[j] = -1;
      }
    }
    lds_barrier();  // lds_np reuse in the next tile
  }
}

// Workgroups the device keeps resident at once (cached per device): the
// persistent grid is never larger, so no slot waits for another to finish.
int resident_index_blocks() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kIndexMaxSlots;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, indexer_topk_kernel<true>, kThreads, 0) !=
            hipSuccess ||
        cus * per <= 0) {
      (void)hipGetLastError();
      return kIndexMaxSlots;
    }
    cache[dev] = cus * per;
  }
  return cache[dev];
}

}  // namespace

hipError_t launch_index_topk(const IndexArgs& ia, hipStream_t s) {
  const IndexWorkspace L = index_ws_layout(ia.Sq, ia.Sk, ia.topk);
  char* ws = static_cast<char*>(ia.ws);
  uint16_t* kpool = reinterpret_cast<uint16_t*>(ws + L.kpool_off);
  uint32_t* fb_count = reinterpret_cast<uint32_t*>(ws + L.fb_off);
  int32_t* fb_rows = reinterpret_cast<int32_t*>(ws + L.fb_off + 256);
  const int64_t n_pools = ia.Sk / 4;
  const int64_t n_padded = index_padded_pools(ia.Sk);
  {
    const int64_t threads = n_padded * 8;
    pool_keys_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s>>>(
        ia.k_idx, kpool, n_pools, n_padded, fb_count);
  }
  KernelArgs a;
  a.q_idx = ia.q_idx;
  a.w_idx = ia.w_idx;
  a.kpool = kpool;
  a.q_pos = ia.q_pos;
  a.Sq = ia.Sq;
  a.Sk = ia.Sk;
  a.n_pools = (int)n_pools;
  a.heads = ia.heads;
  a.topk = ia.topk;
  a.cap = index_candidate_cap(ia.topk);
  a.rows = fb_rows;
  a.nrows = fb_count;
  a.fb_count = fb_count;
  a.fb_rows = fb_rows;
  a.cand = reinterpret_cast<u32x2_t*>(ws + L.cand_off);
  a.idx_out = ia.idx_out;
  int64_t slots = index_slots(ia.Sq);  // the workspace holds candidate lists for this many
  const int64_t resident = resident_index_blocks();
  if (resident < slots) slots = resident;
  indexer_topk_kernel<true><<<dim3((unsigned)slots), dim3(kThreads), 0, s>>>(a);
  // queries whose threshold estimate was too high, scored exactly
  indexer_topk_kernel<false><<<dim3((unsigned)slots), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dsa
