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
//   indexer_topk_kernel per workgroup sub-tile of 16, 32 or 64 queries (4 kRB
//                       a wave, 4 rows of query x indexer-head per query),
//                       stream the causal pool range in
//                       tiles of 64 pools staged in LDS; bf16 MFMA 16x16x32 gives
//                       the 4 head dot products of a (query, pool) pair in one
//                       lane (head weights folded into the query operand), so
//                       the weighted ReLU and the head sum are an in-register
//                       epilogue.  Each score is compared with the query's
//                       running threshold; survivors are staged in LDS and
//                       moved, in pool order, to the query's candidate list in
//                       the workspace.  When a list could overflow, the owning
//                       wave selects its exact top-k with a radix select over
//                       the order-preserving float keys and compacts it
//                       stably, raising the threshold.  The final list is
//                       already ascending in pool id.
//
// Exactness: pools are streamed in ascending id order and a candidate joins the
// list only if its score is strictly greater than the threshold score, so an
// equal score with a higher id loses exactly as the rule "ties go to the lower
// pool id" demands; compaction breaks score ties by list position, which is
// pool order.

#include <atomic>
#include <cmath>
#include <mutex>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"
#include "indexer_common.hpp"

namespace dsa {
namespace {


// ---------------------------------------------------------------------------

// Pools [n_pools, n_padded) are zero-filled so that key tiles can be loaded
// whole, without bounds predicates.
// Thread 0 also clears the indexer's counters: the fallback-list length and
// the tile queues of the two passes.
__global__ __launch_bounds__(256) void pool_keys_kernel(const uint16_t* __restrict__ k_idx,
                                                        uint16_t* __restrict__ kpool,
                                                        int64_t n_pools, int64_t n_padded,
                                                        uint32_t* __restrict__ fb_count) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t == 0) {
#pragma unroll
    for (int j = 0; j < kIndexCounters; ++j) fb_count[j] = 0u;
  }
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

constexpr int kSampleKeep = 8;   // sampled scores kept per lane and query

// Survivor-stage entries per (wave, row block) and key-ring buffers, per
// sub-tile.  The 32-query sub-tile (kRB = 2) is sized for four workgroups a CU
// (four waves a SIMD): 128 registers and 40 KB of LDS, from a two-buffer key
// ring (16 KB, loads one tile ahead) and 376-entry stages (24 KB), with the
// products of at most two column blocks live at a time.  Measured at S = 2^20
// (same ids, one block at a time then): 77.6 ms against 85.9 ms at three
// workgroups a CU (three-buffer ring, 440-entry stages, all four blocks'
// products first, 157 registers); S = 2^17: 2.01 against 2.28 ms.  (The
// three-buffer ring issues loads two tiles ahead, but the barrier's release
// fence waits for LDS-destined loads, so either ring keeps one tile in flight.)
template <int kRB>
constexpr int stage_entries() { return kRB == 2 ? 376 : kIndexStage; }
template <int kRB>
constexpr int ring_buffers() { return kRB == 2 ? 2 : kRing; }
constexpr uint32_t kTagShift = 30;               // staged pool id: query (0..3) in bits 30-31
constexpr uint32_t kPoolMask = (1u << kTagShift) - 1u;

// 8 bf16 query values times the head weight, rounded back to bf16
__device__ __forceinline__ bf16x8_t fold_weight(u32x4_t q, float w) {
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = pack_bf16x2(bf16_to_f32(q[j] & 0xFFFFu) * w, bf16_to_f32(q[j] >> 16) * w);
  return as_bf16x8(o);
}

// Two-phase pass (kTwoPhase): per query, phase 1 streams a strided sample of
// the pool tiles and takes the exact r-th best sampled score t; phase 2
// streams every tile keeping pools with score >= t, then the running top-k.
// If at least min(k, n_c) pools score >= t, every true top-k pool does (its
// score is >= the k-th best score >= t), so the result is exact; otherwise
// phase 2 is run again with a lower threshold from the same sample, and a
// query that fails that too goes to the fallback list, which the exact pass
// (!kTwoPhase: one phase, threshold from -inf) then scores.
//
// Scores: the head weight is folded into the query operand, bf16(w_h q_h),
// so w_h ReLU(q_h . k) = clamp_h(bf16(w_h q_h) . k) with clamp_h = max(., 0)
// for w_h >= 0 and min(., 0) for w_h < 0, one v_med3 against (+-inf, 0).
// For the integer indexer inputs every product and sum is exact.
//
// Survivors of the running threshold go to a per-(wave, row block) stage in
// LDS: one wave-uniform count and mbcnt give the slot, and the pool id
// carries the query (0..3) of the row block in its top bits.  Before the next
// key prefetch is issued, a stage holding 64 or more entries is moved to the
// per-query lists in HBM (stable per query, so each list stays in pool
// order).  Keeping global stores out of the scoring loop keeps the prefetch
// wait exact (loads and stores share one completion counter).
template <bool kTwoPhase, int kRB, int kHG>
__global__ __launch_bounds__(kThreads, kRB == 2 ? 4 : 2) void indexer_topk_kernel(KernelArgs a) {
  constexpr int kStage = stage_entries<kRB>();
  constexpr int kRingN = ring_buffers<kRB>();
  constexpr int kQW = 4 * kRB;        // queries per wave (kRB row blocks of 4)
  // list entries per lane the selection holds in registers: the 64-query
  // sub-tile runs one wave a SIMD beside the forward, where a selection's
  // list re-reads are exposed (S = 2^20 pipelined: 197.1 ms with 24, 202.0
  // with 8); the 16-query one (short calls, where k/n is large and lists
  // compact often) keeps 16 within 128 registers (S = 2^15, k = 512: 0.39-0.41
  // against 0.43 ms with 8); the others keep 8, which fits their registers
  // without spilling (S = 2^17: 2.20 ms against 2.34 with 24)
  constexpr int kSelectRegs = kRB == 4 ? 24 : (kRB == 1 && kHG == 1 ? 16 : 8);
  constexpr int kQTile = kWaves * kQW;  // queries per workgroup tile
  __shared__ __align__(16) u32x4_t lds_k[kRingN][kPT * 8];   // ring of (64 pools x 128 B), swizzled
  __shared__ uint32_t lds_st[kWaves][kRB][2][kStage];  // stage: [0] score bits, [1] (query tag, pool id)
  __shared__ int lds_np[kWaves];
  __shared__ uint32_t lds_fail[kWaves];
  __shared__ int lds_tile;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = uniform(tid >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int cap = a.cap;
  const int topk = a.topk;
  const float NEG_INF = -__builtin_huge_valf();
  const float POS_INF = __builtin_huge_valf();
  const int64_t nrow = kTwoPhase ? a.Sq : (int64_t)__builtin_amdgcn_readfirstlane(*a.nrows);
  const int64_t ntiles = (nrow + kQTile - 1) / kQTile;
  const uint32_t lane_tag = ((uint32_t)g << kTagShift) | (uint32_t)c16;
  // byte offsets in a key tile of this lane's two B-operand chunks of column
  // block 0 (pool c16, key chunks g and 4 + g, swizzled); block cb is 2048 B on
  const int b_off0 = c16 * 128 + ((g ^ (c16 & 7)) << 4);
  const int b_off1 = c16 * 128 + (((4 + g) ^ (c16 & 7)) << 4);
  int dma_off[2];  // byte offset in a key tile of the chunk this thread's loads bring
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = tid + kThreads * j, pr = p >> 3;
    dma_off[j] = (pr * 8 + ((p & 7) ^ (pr & 7))) * 16;
  }

  // Tiles come from a queue shared by the grid, ranked from the longest
  // causal range down (the last query tiles when q_pos is the identity): the
  // greedy order balances the uneven tile costs, retries included.  Thread 0
  // takes the next rank while the current tile is scored; the barrier at the
  // end of the tile publishes it.
  if (tid == 0) lds_tile = (int)atomicAdd(a.tile_next, 1u);
  lds_barrier();
  for (;;) {
    const int64_t rank = lds_tile;
    if (rank >= ntiles) break;
    const int64_t q0 = (kTwoPhase ? ntiles - 1 - rank : rank) * kQTile;
    auto row_of = [&](int64_t i) -> int64_t {
      if (i >= nrow) return -1;
      return kTwoPhase ? i : (int64_t)a.rows[i];
    };

    // A operands: row (4*qq + h) of row block rb and head group hg -> query
    // kQW*wave + 4*rb + qq, head 4*hg + h, weight folded in.  cl[rb][hg][h]: the
    // clamp side of the lane's query (row block rb, query g) and head 4*hg + h.
    bf16x8_t A[kRB][kHG][2];
    float cl[kRB][kHG][4];
    int nc[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
      for (int hg = 0; hg < kHG; ++hg) {
        const int64_t qr = row_of(q0 + kQW * wave + 4 * rb + (c16 >> 2));
        const int h = 4 * hg + (c16 & 3);
        const bool ok = qr >= 0 && h < a.heads;
        const uint16_t* src = a.q_idx + (qr * a.heads + h) * kDI + 8 * g;
        const float wv = ok ? bf16_to_f32(a.w_idx[qr * a.heads + h]) : 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          A[rb][hg][ks] = ok ? fold_weight(*reinterpret_cast<const u32x4_t*>(src + 32 * ks), wv)
                             : zero_bf16x8();
      }
      {
        const int64_t qr = row_of(q0 + kQW * wave + 4 * rb + g);
        const bool ok = qr >= 0;
        int64_t pos = 0;
        if (ok) {
          pos = a.q_pos ? (int64_t)a.q_pos[qr] : a.q_base + qr;
          pos = pos < 0 ? 0 : (pos >= a.Sk ? a.Sk - 1 : pos);
        }
        nc[rb] = ok ? (int)((pos + 1) >> 2) : 0;
#pragma unroll
        for (int hg = 0; hg < kHG; ++hg)
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const int hh = 4 * hg + h;
            const float wv = (ok && hh < a.heads) ? bf16_to_f32(a.w_idx[qr * a.heads + hh]) : 0.f;
            cl[rb][hg][h] = wv < 0.f ? NEG_INF : POS_INF;
          }
      }
    }
    int ncm = nc[0];
#pragma unroll
    for (int rb = 1; rb < kRB; ++rb) ncm = max(ncm, nc[rb]);
    ncm = wave_max(ncm);
    int ncmin = nc[0];
#pragma unroll
    for (int rb = 1; rb < kRB; ++rb) ncmin = min(ncmin, nc[rb]);
    ncmin = wave_min(ncmin);
    if (lane == 0) lds_np[wave] = ncm;
    lds_barrier();
    if (tid == 0) lds_tile = (int)atomicAdd(a.tile_next, 1u);  // read after the tile
    int tp = lds_np[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) tp = max(tp, lds_np[w]);
    const int ntp = (tp + kPT - 1) / kPT;   // pool tiles in the tile's causal range
    const int stride = sample_stride(ntp, topk);

    float tau[kRB], tau2[kRB];  // running thresholds, and the retry's
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) tau[rb] = tau2[rb] = NEG_INF;
    const int64_t wbase = ((int64_t)blockIdx.x * kQTile + kQW * wave) * cap;

    // Pool-key tiles go straight from HBM to LDS (buffer loads with the LDS
    // destination) through a ring of kRingN buffers, issued kRingN - 1 tiles
    // ahead of the one being scored.  (The workgroup barrier releases LDS, and
    // these loads write LDS, so the compiler waits for all of them before each
    // barrier: a tile's loads have one tile's scoring time to land.)  Lane l
    // of a load instruction writes LDS chunk
    // (base + l); its source offset is chosen so that LDS row pr, chunk ch
    // holds key chunk ch ^ (pr & 7) (the swizzle that spreads the B-operand
    // reads over the banks).  The loads are unconditional (the keys are
    // padded to whole tiles) from a per-tile resource and loop-invariant
    // per-thread offsets.
    auto dma = [&](int tile, int buf) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.kpool + (int64_t)tile * kPT * kDI), (short)0, kPT * kDI * 2, kBufferWord3);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)&lds_k[buf][kThreads * j + kWave * wave], 16,
            dma_off[j], 0, 0, 0);
    };

    // Stream pool tiles first, first+step, ... < ntp.  Per tile i: wait for
    // this thread's part of tile i and meet at the barrier (tile i is then in
    // LDS and every wave is done with tile i-1's buffer), run
    // `before_load(i)` (it may issue global stores), start tile i+kAhead, and
    // hand the tile's scores to `consume(sc, pt0)` (-inf where a pool is not
    // causal for the query).  Loads complete in order among themselves, so
    // with tile i+1's two loads younger than tile i's, "at most 2
    // outstanding" means tile i has landed, whatever the stores do.  Tile 0
    // of a stream is always loaded (in bounds: the keys are padded to >= 1
    // tile).
    constexpr int kAhead = kRingN - 1;
    // epilogue: clamp each head to the side of its weight, sum the heads
    auto head_sum = [&](const f32x4_t (&x)[kHG], int rb) -> float {
      float hs[kHG];
#pragma unroll
      for (int hg = 0; hg < kHG; ++hg) {
        const float s01 = __builtin_amdgcn_fmed3f(x[hg][0], cl[rb][hg][0], 0.f) +
                          __builtin_amdgcn_fmed3f(x[hg][1], cl[rb][hg][1], 0.f);
        const float s23 = __builtin_amdgcn_fmed3f(x[hg][2], cl[rb][hg][2], 0.f) +
                          __builtin_amdgcn_fmed3f(x[hg][3], cl[rb][hg][3], 0.f);
        hs[hg] = s01 + s23;
      }
      if constexpr (kHG == 1) return hs[0];
      else return hs[0] + hs[1];
    };
    auto stream = [&](int first, int step, auto&& before_load, auto&& consume) {
      const int nt = first < ntp ? (ntp - first + step - 1) / step : 0;
      dma(first < ntp ? first : 0, 0);
      if (kAhead == 2 && nt > 1) dma(first + step, 1);
      int buf = 0;  // buffer of tile i; tile i + kAhead goes to (buf + kAhead) mod kRingN
      for (int i = 0; i < nt; ++i) {
        const int pt0 = (first + i * step) * kPT;
        if (kAhead == 2 && i + 1 < nt) __builtin_amdgcn_s_waitcnt(kWaitVmcnt2);
        else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        lds_barrier();
        const char* kb = reinterpret_cast<const char*>(lds_k[buf]);
        before_load(i);
        if (i + kAhead < nt) dma(first + (i + kAhead) * step, buf == 0 ? kRingN - 1 : buf - 1);
        buf = buf == kRingN - 1 ? 0 : buf + 1;

        // 16 output blocks of 16 (query x head) rows x 16 pools per head group:
        // column block cb holds pools 16 cb .. 16 cb + 15 of the tile
        float sc[kRB][4];
        auto products = [&](int cb, f32x4_t (&x)[kRB][kHG]) {
          const bf16x8_t B0 = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kb + b_off0 + 2048 * cb));
          const bf16x8_t B1 = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kb + b_off1 + 2048 * cb));
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int hg = 0; hg < kHG; ++hg) {
              f32x4_t z = {0.f, 0.f, 0.f, 0.f};
              x[rb][hg] = mfma32(A[rb][hg][1], B1, mfma32(A[rb][hg][0], B0, z));
            }
        };
        if constexpr (kRB == 2) {
          // two column blocks' products live at a time (four waves a SIMD fit
          // in 128 registers): block cb + 1's products are issued before
          // block cb's epilogue, so the matrix core works on them while this
          // wave's VALU clamps and sums block cb (S = 2^20: 75.7-78.9 ms
          // against 77.2-80.7 with one block at a time, same ids)
          f32x4_t x0[kRB][kHG], x1[kRB][kHG];
          products(0, x0);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            f32x4_t (&cur)[kRB][kHG] = (cb & 1) ? x1 : x0;
            f32x4_t (&nxt)[kRB][kHG] = (cb & 1) ? x0 : x1;
            if (cb < 3) products(cb + 1, nxt);
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) sc[rb][cb] = head_sum(cur[rb], rb);
          }
        } else {
          // every block's products first, then the epilogues (one or two waves a SIMD)
          f32x4_t acc[4][kRB][kHG];
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) products(cb, acc[cb]);
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) sc[rb][cb] = head_sum(acc[cb][rb], rb);
        }
        // causal pool mask, only on tiles some query of the wave sees in part
        if (pt0 + kPT > ncmin) {
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
              if (pt0 + 16 * cb + c16 >= nc[rb]) sc[rb][cb] = NEG_INF;
        }
        consume(sc, pt0);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // a tile-0 load of an empty stream
      lds_barrier();  // every wave is done with the ring before the next stream
    };

    if (kTwoPhase) {
      // Phase 1: each lane keeps, per query, the 8 best sampled scores of
      // its pool column (descending, in registers).  Their union holds at
      // most every sampled score, so its r-th best is at most the sample's.
      int rq[2][kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        // r from the fraction f of the query's causal pools the sample
        // covers; 0 = no estimate (threshold stays -inf)
        const int n_full = nc[rb] / kPT, part = nc[rb] % kPT;
        const int s_q = kPT * ((n_full + stride - 1) / stride) +
                        (n_full % stride == 0 ? part : 0);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float z = m == 0 ? kSampleZ1 : kSampleZ2;
          int r = 0;
          if (nc[rb] > topk && s_q > 0) {
            const float f = (float)s_q / (float)nc[rb];
            const float x = 0.5f * (z + sqrtf(z * z + 4.f * topk * f));
            r = (int)ceilf(x * x);
            if (r >= s_q || r > kSampleKeep * 16 * 3 / 4) r = 0;
          }
          rq[m][rb] = r;
        }
      }
      float best[kRB][kSampleKeep];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int j = 0; j < kSampleKeep; ++j) best[rb][j] = NEG_INF;
      // Per tile and query the lane's 4 new scores are sorted (5 exchanges),
      // merged into the 8 kept ones by taking the larger of kept[4+j] and
      // new[3-j] (the top 8 of the union, in bitonic order), and the 8 are
      // sorted again by a bitonic half-cleaner network (3 x 4 exchanges).
      stream(0, stride, [](int) {}, [&](float (&sc)[kRB][4], int) {
        auto cx = [](float& hi, float& lo) {
          const float h = fmaxf(hi, lo);
          lo = fminf(hi, lo);
          hi = h;
        };
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          float n0 = sc[rb][0], n1 = sc[rb][1], n2 = sc[rb][2], n3 = sc[rb][3];
          cx(n0, n1); cx(n2, n3); cx(n0, n2); cx(n1, n3); cx(n1, n2);
          float* b = best[rb];
          b[4] = fmaxf(b[4], n3);
          b[5] = fmaxf(b[5], n2);
          b[6] = fmaxf(b[6], n1);
          b[7] = fmaxf(b[7], n0);
#pragma unroll
          for (int d = 4; d >= 1; d >>= 1)
#pragma unroll
            for (int j = 0; j < kSampleKeep; ++j)
              if ((j & d) == 0) cx(b[j], b[j + d]);
        }
      });
      // r-th best of the 16 lanes (a DPP row) x kSampleKeep kept scores of
      // each query: the largest key v with at least r kept keys >= v, bit by
      // bit from the top, for both ranks at once.  Only bits where some keys
      // of the wave differ are searched: a bit every key of the row shares is
      // the answer's too, and starting from the row's common one-bits leaves
      // each remaining test (keys >= candidate) as in the full search.
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        uint32_t kk[kSampleKeep];
        uint32_t ko = 0u, ka = 0xFFFFFFFFu;
#pragma unroll
        for (int j = 0; j < kSampleKeep; ++j) {
          kk[j] = order_key(best[rb][j] + 0.f);
          ko |= kk[j];
          ka &= kk[j];
        }
        ka = (uint32_t)row_reduce16((int)ka, [](int x, int y) { return x & y; });
        uint32_t bits = wave_or(ko ^ ka);   // wave-uniform
        const int r0 = rq[0][rb], r1 = rq[1][rb];
        uint32_t p0 = ka, p1 = ka;
        while (bits != 0u) {
          const uint32_t bit = 1u << (31 - __builtin_clz(bits));
          bits ^= bit;
          const uint32_t c0k = p0 | bit, c1k = p1 | bit;
          int c0 = 0, c1 = 0;
#pragma unroll
          for (int j = 0; j < kSampleKeep; ++j) {
            c0 += kk[j] >= c0k ? 1 : 0;
            c1 += kk[j] >= c1k ? 1 : 0;
          }
          c0 = row_sum16(c0);
          c1 = row_sum16(c1);
          if (c0 >= r0) p0 = c0k;
          if (c1 >= r1) p1 = c1k;
        }
        tau[rb] = r0 > 0 ? float_below(key_to_float(p0)) : NEG_INF;
        tau2[rb] = r1 > 0 ? float_below(key_to_float(p1)) : NEG_INF;
      }
    }

    // Phase 2 (or the exact pass): every tile; survivors of the running
    // threshold are staged, stages are flushed to the per-query lists, and a
    // list that a flush leaves within one stage of its end keeps its top-k.
    // A workgroup with a query whose threshold turned out too high runs the
    // pass once more, for those queries only, with the larger margin
    // (threshold +inf for the others); `redo` holds the wave's queries
    // (bit 4*rb + t) scored in the current attempt.
    uint32_t redo = kQW >= 32 ? 0xFFFFFFFFu : (1u << kQW) - 1u;
#pragma unroll 1
    for (int attempt = 0;; ++attempt) {
      if (attempt > 0) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          tau[rb] = ((redo >> (4 * rb + g)) & 1u) ? tau2[rb] : POS_INF;
      }
      int nst[kRB];                // staged entries per row block (wave-uniform)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) nst[rb] = 0;
      int cnt_v = 0;               // lane q < kQW: list length of wave query q = 4*rb + t

      // Entry j of stage rb (of n) is moved to the list of its query; `c` holds
      // the 4 list lengths of the row block and advances (stable per query).
      auto place = [&](int rb, int j0, int n, uint32_t fbits, uint32_t id, int (&c)[4]) {
        const bool valid = j0 + lane < n;
        const int t = (int)(id >> kTagShift);
        int pos = 0;
#pragma unroll
        for (int tq = 0; tq < 4; ++tq) {
          const bool mine = valid && t == tq;
          const uint64_t Mt = ballot(mine);
          if (mine) pos = c[tq] + mbcnt(Mt);
          c[tq] += __popcll(Mt);
        }
        if (valid) {
          u32x2_t e;
          e[0] = order_key(__uint_as_float(fbits) + 0.f);  // -0 -> +0
          e[1] = id & kPoolMask;
          a.cand[wbase + (int64_t)(4 * rb + t) * cap + pos] = e;
        }
      };
      // Move the stages flagged in fl to the lists.  The first 64 entries of
      // every flagged stage are read before any is placed, so one LDS latency
      // covers them all.
      auto flush = [&](uint32_t fl) {
        uint32_t f0[kRB], i0[kRB];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          f0[rb] = 0u;
          i0[rb] = 0u;
          if ((fl >> rb) & 1u) {
            if (lane < nst[rb]) {
              f0[rb] = lds_st[wave][rb][0][lane];
              i0[rb] = lds_st[wave][rb][1][lane];
            }
          }
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          if (!((fl >> rb) & 1u)) continue;
          const int n = nst[rb];
          int c[4];
#pragma unroll
          for (int tq = 0; tq < 4; ++tq) c[tq] = __builtin_amdgcn_readlane(cnt_v, 4 * rb + tq);
          place(rb, 0, n, f0[rb], i0[rb], c);
          for (int j0 = kWave; j0 < n; j0 += kWave) {
            const int j = j0 + lane;
            const uint32_t fb = j < n ? lds_st[wave][rb][0][j] : 0u;
            const uint32_t id = j < n ? lds_st[wave][rb][1][j] : 0u;
            place(rb, j0, n, fb, id, c);
          }
#pragma unroll
          for (int tq = 0; tq < 4; ++tq) cnt_v = lane == 4 * rb + tq ? c[tq] : cnt_v;
          nst[rb] = 0;
        }
      };

      stream(0, 1,
          [&](int i) {
            // A flush costs about one store latency, whatever its size, and a
            // wave that flushes holds up the others at the next barrier.  So
            // all 4 stages of a wave are flushed together, when one of them
            // could not take another tile's worth (4 x 64 entries), and every
            // kFlushPeriod tiles (the same tiles in every wave).
            // No stage can be within one tile of its end while the four
            // counts together are at most kStage - 256: one scalar test on
            // most tiles.  Otherwise, scalar-only tests: full = some count >
            // kStage - 256 (the sign bit of count - (kStage - 255) is clear),
            // fl = counts > 0.
            const bool period = i > 0 && (i % kFlushPeriod) == 0;
            int nsum = 0;
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) nsum += nst[rb];
            if (!period && nsum <= kStage - 4 * kWave) return;
            int neg = -1;
            uint32_t fl = 0;
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
              neg &= nst[rb] - (kStage - 4 * kWave + 1);
              fl |= ((uint32_t)(-nst[rb]) >> 31) << rb;
            }
            const bool full = neg >= 0;
            if (!(full || period) || fl == 0) return;
            flush(fl);
            bool fenced = false;
            for (uint32_t m = fl; m != 0; m &= m - 1) {
              const int rb = __builtin_ctz(m);
#pragma unroll 1
              for (int tq = 0; tq < 4; ++tq) {
                const int q = 4 * rb + tq;
                const int n = __builtin_amdgcn_readlane(cnt_v, q);
                if (n <= cap - kStage) continue;
                if (!fenced) {
                  __threadfence_block();  // this wave's list stores are visible
                  fenced = true;
                }
                // the (just flushed, empty) stage of rb holds the histogram
                const float T = select_and_compact<kSelectRegs>(a.cand + wbase + (int64_t)q * cap, n, topk,
                                                   lds_st[wave][rb][0], nullptr);
                cnt_v = lane == q ? topk : cnt_v;
#pragma unroll
                for (int r = 0; r < kRB; ++r)
                  if (r == rb && g == tq) tau[r] = T;
              }
            }
          },
          [&](float (&sc)[kRB][4], int pt0) {
            // all 16 ballots come before the first branch on one of them, so
            // no branch waits on a compare issued just before it
            uint64_t MM[kRB][4];
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
              for (int cb = 0; cb < 4; ++cb) MM[rb][cb] = ballot(sc[rb][cb] > tau[rb]);
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
              for (int cb = 0; cb < 4; ++cb) {
                const bool keep = sc[rb][cb] > tau[rb];
                const uint64_t M = MM[rb][cb];
                if (M) {
                  if (keep) {
                    const int slot = nst[rb] + mbcnt(M);
                    uint32_t* st = &lds_st[wave][rb][0][slot];
                    st[0] = __float_as_uint(sc[rb][cb]);
                    st[kStage] = (uint32_t)(pt0 + 16 * cb) + lane_tag;
                  }
                  nst[rb] += __popcll(M);
                }
              }
            }
          });

      // remaining stages, then the final selection written to the output rows
      {
        uint32_t fl = 0;
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) fl |= nst[rb] > 0 ? 1u << rb : 0u;
        if (fl) flush(fl);
      }
      __threadfence_block();
      uint32_t failed = 0;  // wave queries whose threshold was too high
#pragma unroll 1
      for (int q = 0; q < kQW; ++q) {
        if (!((redo >> q) & 1u)) continue;
        const int64_t qr = row_of(q0 + kQW * wave + q);
        if (qr < 0) continue;
        const int rb = q >> 2;
        const int n = __builtin_amdgcn_readlane(cnt_v, q);
        int ncr = nc[0];
#pragma unroll
        for (int r = 1; r < kRB; ++r) ncr = r == rb ? nc[r] : ncr;
        const int need = min(topk, __builtin_amdgcn_readlane(ncr, 16 * (q & 3)));
        if (kTwoPhase && n < need) {  // threshold estimate too high
          if (attempt == 0) {
            failed |= 1u << q;
            if (lane == 0) atomicAdd(a.fb_count + kIndexRetryCounter, 1u);
          }
          else if (lane == 0) a.fb_rows[atomicAdd(a.fb_count, 1u)] = (int32_t)qr;
          continue;
        }
        const int64_t base = wbase + (int64_t)q * cap;
        int32_t* dst = a.idx_out + qr * topk;
        int filled = n;
        if (n > topk) {
          select_and_compact<kSelectRegs>(a.cand + base, n, topk, lds_st[wave][0][0], dst);  // stages are empty
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
      if (!kTwoPhase || attempt > 0) break;
      if (lane == 0) lds_fail[wave] = failed;
      lds_barrier();
      uint32_t any_fail = 0u;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) any_fail |= lds_fail[w];
      if (any_fail == 0u) break;
      redo = failed;
    }
    lds_barrier();  // publishes lds_tile; lds_np is reused in the next tile
  }
}

// Workgroups the device keeps resident at once, and its CU count (cached per
// device): the persistent grid is never larger, so no slot waits for another
// to finish.

template <int kRB, int kHG>
Residency index_residency() {
  static std::mutex mu;
  static Residency cache[64] = {};
  int dev = 0;
  const Residency fallback{kIndexMaxSlots / 2, 2};
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fallback;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev].cus == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, indexer_topk_kernel<true, kRB, kHG>, kThreads,
                                                     0) != hipSuccess ||
        cus * per <= 0) {
      (void)hipGetLastError();
      return fallback;
    }
    cache[dev] = Residency{cus, per};
  }
  return cache[dev];
}

// Queries per wave, 4 kRB.  kRB = 4 shares each staged key tile among 64
// queries of a workgroup but needs 248 VGPRs and 81 KB of LDS: two workgroups
// a CU.  kRB = 2 is held to 128 VGPRs and 40 KB (see stage_entries), four a
// CU; kRB = 1 needs 115 VGPRs and 39 KB, also four, in half-size workgroups.
// Measured per call, same ids (kRB = 2 at three workgroups a CU, before it
// fitted four): at S = 2^20 keys 85.0 ms for kRB = 2
// against 98.3 (kRB = 4) and 106.4 (kRB = 1); at 2^17 keys 2.18 against 2.69
// and 2.49 ms; at 2^15 and 4096 queries kRB = 1 is fastest (0.46 against 0.64
// ms, 0.086 against 0.14), its grid of 16-query tiles filling the CUs evenly.
// A grid held to one workgroup a CU (CUs shared with the attention forward)
// runs best with kRB = 4 (a pipelined S = 2^20 call: 201 ms, 240 with kRB = 2).
// dsa_set_index_queries_per_wave(4, 8 or 16) overrides the choice (a tuning and
// test setting, process-wide; all give the same ids).
constexpr int64_t kIndexNarrowMaxQueries = int64_t(1) << 15;

std::atomic<int> g_queries_per_wave{0};   // 0: chosen per call

int index_queries_per_wave(const IndexArgs& ia) {
  const int forced = g_queries_per_wave.load(std::memory_order_relaxed);
  if (forced != 0) return forced;
  if (ia.max_per_cu > 0) return 16;
  return ia.Sq <= kIndexNarrowMaxQueries ? 4 : 8;
}

// Both passes with kRB row blocks (4 kRB queries) per wave.  The workspace
// holds index_slots(Sq) x kIndexQueryTile candidate lists; a workgroup of this
// variant owns kWaves x 4 kRB of them, so the grid never exceeds their count.
template <int kRB, int kHG>
void launch_passes(KernelArgs a, const IndexArgs& ia, uint32_t* fb_count, hipStream_t s) {
  constexpr int64_t qtile = (int64_t)kWaves * 4 * kRB;
  const int64_t lists = index_slots(ia.Sq) * kIndexQueryTile;
  int64_t slots = (ia.Sq + qtile - 1) / qtile;
  if (slots > lists / qtile) slots = lists / qtile;
  const Residency res = index_residency<kRB, kHG>();
  const int per_cu = ia.max_per_cu > 0 && ia.max_per_cu < res.per_cu ? ia.max_per_cu : res.per_cu;
  const int64_t resident = (int64_t)res.cus * per_cu;
  if (resident < slots) slots = resident;
  a.tile_next = fb_count + 1;
  indexer_topk_kernel<true, kRB, kHG><<<dim3((unsigned)slots), dim3(kThreads), 0, s>>>(a);
  // queries whose threshold estimate was too high twice, scored exactly.  They are
  // rare (none to a few per 2^16 rows on the workloads); when other kernels share
  // the CUs, a small grid finds free slots sooner than one workgroup per CU would.
  a.tile_next = fb_count + 2;
  const int64_t exact_slots = ia.max_per_cu > 0 && slots > kExactSharedSlots ? kExactSharedSlots : slots;
  indexer_topk_kernel<false, kRB, kHG><<<dim3((unsigned)exact_slots), dim3(kThreads), 0, s>>>(a);
}

}  // namespace

bool set_index_queries_per_wave(int qpw) {
  if (qpw != 0 && qpw != 4 && qpw != 8 && qpw != 16) return false;
  g_queries_per_wave.store(qpw, std::memory_order_relaxed);
  return true;
}

hipError_t launch_index_topk(const IndexArgs& ia, hipStream_t s) {
  const IndexWorkspace L = index_ws_layout(ia.Sq, ia.Sk, ia.topk);
  char* ws = static_cast<char*>(ia.ws);
  uint16_t* kpool = reinterpret_cast<uint16_t*>(ws + L.kpool_off);
  uint32_t* fb_count = reinterpret_cast<uint32_t*>(ws + L.fb_off);  // kIndexCounters counters
  int32_t* fb_rows = reinterpret_cast<int32_t*>(ws + L.fb_off + 256);
  const int64_t n_pools = ia.Sk / 4;
  const int64_t n_padded = index_padded_pools(ia.Sk);
  {
    // with the pooled keys already in the workspace only the counters are cleared
    const int64_t threads = ia.pooled ? 1 : n_padded * 8;
    pool_keys_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s>>>(
        ia.k_idx, kpool, n_pools, ia.pooled ? 0 : n_padded, fb_count);
  }
  KernelArgs a;
  a.q_idx = ia.q_idx;
  a.w_idx = ia.w_idx;
  a.kpool = kpool;
  a.kpool8 = nullptr;
  a.q_pos = ia.q_pos;
  a.q_base = ia.q_base;
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
  a.tile_next = nullptr;
  if (ia.heads > 4) {
    // 5 to 8 indexer heads: two groups of 4 heads per query, 16-query sub-tile
    launch_passes<1, 2>(a, ia, fb_count, s);
  } else {
    switch (index_queries_per_wave(ia)) {
      case 4: launch_passes<1, 1>(a, ia, fb_count, s); break;
      case 8: launch_passes<2, 1>(a, ia, fb_count, s); break;
      default: launch_passes<4, 1>(a, ia, fb_count, s); break;
    }
  }
  return hipGetLastError();
}

}  // namespace dsa
