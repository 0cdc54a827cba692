// Lightning indexer with a fused per-query top-k on the 32x32 MFMA layout
// (gfx950): fp8 (OCP e4m3) operands on v_mfma_f32_32x32x64_f8f6f4.
//
// What is computed is what indexer.hip computes (pages: "SkyRL 将 GLM-5.3-Flash
// 训练上下文扩至 100 万 token", sections "模型与瓶颈" and "四块优化 1. DSA
// 真稀疏"; the precision theme of its section "4. 去掉多余 fp32"): every query
// is scored against every complete 4-token pool and keeps the top-k pools.
// The algorithm is also the same (a threshold from a strided sample of the pool
// tiles, survivors staged in LDS and moved to per-query candidate lists,
// compaction by an exact radix select, a retry with a wider margin and an
// exact pass); what differs is the tile mapping:
//
//   row block     8 queries x 4 heads = the 32 rows of one MFMA
//   column block  32 pools
//   lane l        for i = 0..3: the 4 head dot products of query 2i + l/32 of
//                 the row block with pool l%32 of the column block
//
// so the weighted ReLU and the head sum stay an in-register epilogue (v_med3
// against (+-inf, 0), as in indexer.hip).  One fp8 32x32x64 MFMA scores 256
// (query, pool) pairs with the whole 64-dim contraction: half the matrix-core
// cycles of bf16 per pair, and half the key bytes per pool (64 B).
//
// Precision: the pooled keys and the folded queries w*q are rounded to e4m3;
// the dot products accumulate in fp32.  For integer indexer
// inputs in [-3, 3] every value is exact in e4m3 (w*q is an integer in
// [-9, 9], a pooled key a multiple of 1/4 in [-3, 3]) and every partial sum is
// exact in fp32, so the selection equals the exact ranking.

#include <cmath>
#include <mutex>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"
#include "indexer_common.hpp"

namespace dsa {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kKeep32 = 4;        // sampled scores kept per lane and query (32 lanes share one)
constexpr int kSelectRegs = 8;    // list entries per lane the selection holds in registers
constexpr int kStage32 = 640;     // stage entries per (wave, row block of 8 queries)
constexpr int kTileWorst = 8 * kPT;  // most entries one pool tile adds to a stage
constexpr uint32_t kTag32Shift = 29;   // staged pool id: query (0..7) of the row block in bits 29-31
constexpr uint32_t kPool32Mask = (1u << kTag32Shift) - 1u;

constexpr int kRowBytes = 64;     // a pooled key: 64 e4m3 values

// ---------------------------------------------------------------------------
// Pooled keys in fp8: kpool8[p] = e4m3(mean of k_idx[4p..4p+3]), 64 bytes a
// pool; pools [n_pools, n_padded) are zero.  Thread 0 also clears the
// indexer's counters.  One thread per 8 dims of a pool.

__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__global__ __launch_bounds__(256) void pool_keys_fp8_kernel(const uint16_t* __restrict__ k_idx,
                                                            uint8_t* __restrict__ kpool,
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
  u32x2_t o = {0u, 0u};
  if (p < n_pools) {
    const uint16_t* src = k_idx + (4 * p) * kDI + c * 8;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll
    for (int tok = 0; tok < 4; ++tok) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + tok * kDI);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += bf16_to_f32(v[j] & 0xFFFFu);
        acc[2 * j + 1] += bf16_to_f32(v[j] >> 16);
      }
    }
    o[0] = pack_fp8x4(acc[0] * 0.25f, acc[1] * 0.25f, acc[2] * 0.25f, acc[3] * 0.25f);
    o[1] = pack_fp8x4(acc[4] * 0.25f, acc[5] * 0.25f, acc[6] * 0.25f, acc[7] * 0.25f);
  }
  *reinterpret_cast<u32x2_t*>(kpool + p * kDI + c * 8) = o;
}

// ---------------------------------------------------------------------------
// Operands.  The k index of the contraction is the indexer dim: lane half h
// holds dims 32h..32h+31 of its row (A) or column (B), 32 e4m3 bytes.  A and B
// place a dim in the same (half, byte) slot, which is all the contraction
// needs.

// w * q of one (query, head) row for this lane's dims, rounded to e4m3
__device__ __forceinline__ void fold_row(const uint16_t* qrow, float w, bool ok, int h, i32x8_t& A) {
  i32x8_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4_t v = ok ? *reinterpret_cast<const u32x4_t*>(qrow + 32 * h + 8 * j) : u32x4_t{0u, 0u, 0u, 0u};
    r[2 * j] = (int)pack_fp8x4(bf16_to_f32(v[0] & 0xFFFFu) * w, bf16_to_f32(v[0] >> 16) * w,
                               bf16_to_f32(v[1] & 0xFFFFu) * w, bf16_to_f32(v[1] >> 16) * w);
    r[2 * j + 1] = (int)pack_fp8x4(bf16_to_f32(v[2] & 0xFFFFu) * w, bf16_to_f32(v[2] >> 16) * w,
                                   bf16_to_f32(v[3] & 0xFFFFu) * w, bf16_to_f32(v[3] >> 16) * w);
  }
  A = r;
}

// ---------------------------------------------------------------------------
// Key tiles in LDS: 64 pools, row-major, XOR-swizzled in 16-byte chunks so that
// the B-operand reads (8 lanes reading 16 bytes each at a time) hit distinct
// banks: 4 chunks a pool, chunk ch of pool pr at (ch ^ ((pr >> 1) & 3)).

__device__ __forceinline__ int phys_chunk(int pr, int ch) { return ch ^ ((pr >> 1) & 3); }

// The lane's B operand of one column block: pool pr of the tile, dims of lane
// half h.  `off_lo` / `off_hi` are the byte offsets of its two chunks for
// pr = lane % 32 (b_offsets); column block 1 (pr + 32) is 2048 bytes on, with
// the same swizzle.
__device__ __forceinline__ void b_offsets(int pr, int h, int& off_lo, int& off_hi) {
  off_lo = (pr * 4 + phys_chunk(pr, 2 * h)) * 16;
  off_hi = (pr * 4 + phys_chunk(pr, 2 * h + 1)) * 16;
}

__device__ __forceinline__ void read_b(const char* kb, int off_lo, int off_hi, i32x8_t& B) {
  const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(kb + off_lo);
  const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(kb + off_hi);
  i32x8_t r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  B = r;
}

// The MFMA builtin sits in a plain (non-template) device function: in the host
// pass, a gfx950-only builtin inside a template would fail the template's
// substitution and silently drop the kernel's host stub.
__device__ __forceinline__ f32x16_t mma32(i32x8_t a, i32x8_t b) {
  const f32x16_t z = {};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// The kernel.  kNRB row blocks (8 kNRB queries) a wave, 4 waves a workgroup.
// Per-lane query state is indexed [rb][i]: the lane's query 2i + h of row
// block rb, h = lane / 32 (wave query 8 rb + 2i + h).

template <bool kTwoPhase, int kNRB>
__device__ __forceinline__ void indexer32_body(const KernelArgs& a) {
  constexpr int kQW = 8 * kNRB;              // queries per wave
  constexpr int kQTile = kWaves * kQW;       // queries per workgroup tile
  constexpr int kChunks = kRowBytes * kPT / 16;   // 16-byte chunks per key tile
  constexpr int kDma = kChunks / kThreads;                // DMA loads per thread per tile
  __shared__ __align__(16) u32x4_t lds_k[kRing][kChunks];
  __shared__ uint32_t lds_st[kWaves][kNRB][2][kStage32];   // stage: [0] score bits, [1] (tag, pool id)
  __shared__ int lds_np[kWaves];
  __shared__ uint32_t lds_fail[kWaves];
  __shared__ int lds_tile;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = uniform(tid >> 6);
  const int h = lane >> 5;
  const int c = lane & 31;
  const int cap = a.cap;
  const int topk = a.topk;
  const float NEG_INF = -__builtin_huge_valf();
  const float POS_INF = __builtin_huge_valf();
  const int64_t nrow = kTwoPhase ? a.Sq : (int64_t)__builtin_amdgcn_readfirstlane(*a.nrows);
  const int64_t ntiles = (nrow + kQTile - 1) / kQTile;
  int b_lo, b_hi;     // B-operand chunk offsets of column block 0
  b_offsets(c, h, b_lo, b_hi);
  // staged pool id: pool | (query of the row block) << kTag32Shift; the lane's
  // part (pool c, lane half h) here, the tile's and the query pair's part
  // (wave-uniform) added per staged block
  const uint32_t lane_tag = (uint32_t)c | ((uint32_t)h << kTag32Shift);
  int dma_off[kDma];  // byte offset in a key tile of the chunk this thread's loads bring
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int L = tid + kThreads * j;
    const int per = kRowBytes / 16;
    const int pr = L / per, pc = L % per;
    // physical chunk pc of pool pr holds logical chunk ch with phys_chunk(pr, ch) == pc;
    // the swizzle is an involution for fixed pr
    dma_off[j] = pr * kRowBytes + phys_chunk(pr, pc) * 16;
  }

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

    // A operands: row c of row block rb -> query 8 rb + c/4, head c%4, weight folded in
    i32x8_t A[kNRB];
    float cl[kNRB][4][4];
    int nc[kNRB][4];
#pragma unroll
    for (int rb = 0; rb < kNRB; ++rb) {
      {
        const int64_t qr = row_of(q0 + kQW * wave + 8 * rb + (c >> 2));
        const int hd = c & 3;
        const bool ok = qr >= 0 && hd < a.heads;
        const uint16_t* src = a.q_idx + ((ok ? qr : 0) * a.heads + (ok ? hd : 0)) * kDI;
        const float wv = ok ? bf16_to_f32(a.w_idx[qr * a.heads + hd]) : 0.f;
        fold_row(src, wv, ok, h, A[rb]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t qr = row_of(q0 + kQW * wave + 8 * rb + 2 * i + h);
        const bool ok = qr >= 0;
        int64_t pos = 0;
        if (ok) {
          pos = a.q_pos ? (int64_t)a.q_pos[qr] : a.q_base + qr;
          pos = pos < 0 ? 0 : (pos >= a.Sk ? a.Sk - 1 : pos);
        }
        nc[rb][i] = ok ? (int)((pos + 1) >> 2) : 0;
#pragma unroll
        for (int hd = 0; hd < 4; ++hd) {
          const float wv = (ok && hd < a.heads) ? bf16_to_f32(a.w_idx[qr * a.heads + hd]) : 0.f;
          cl[rb][i][hd] = wv < 0.f ? NEG_INF : POS_INF;
        }
      }
    }
    int ncm = 0, ncmin = 1 << 30;
#pragma unroll
    for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ncm = max(ncm, nc[rb][i]);
        ncmin = min(ncmin, nc[rb][i]);
      }
    ncm = wave_max(ncm);
    ncmin = wave_min(ncmin);
    if (lane == 0) lds_np[wave] = ncm;
    lds_barrier();
    if (tid == 0) lds_tile = (int)atomicAdd(a.tile_next, 1u);  // read after the tile
    int tp = lds_np[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) tp = max(tp, lds_np[w]);
    const int ntp = (tp + kPT - 1) / kPT;   // pool tiles in the tile's causal range
    const int stride = sample_stride(ntp, topk);

    float tau[kNRB][4], tau2[kNRB][4];  // running thresholds, and the retry's
#pragma unroll
    for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) tau[rb][i] = tau2[rb][i] = NEG_INF;
    const int64_t wbase = ((int64_t)blockIdx.x * kQTile + kQW * wave) * cap;

    // key tiles: buffer loads with an LDS destination, a ring of kRing buffers,
    // two tiles ahead (as in indexer.hip)
    auto dma = [&](int tile, int buf) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.kpool8 + (int64_t)tile * kPT * kRowBytes), (short)0, kPT * kRowBytes,
          kBufferWord3);
#pragma unroll
      for (int j = 0; j < kDma; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)&lds_k[buf][kThreads * j + kWave * wave], 16,
            dma_off[j], 0, 0, 0);
    };

    // Stream pool tiles first, first+step, ... < ntp and hand each tile's scores
    // sc[rb][cb][i] to `consume` (-inf where a pool is not causal for the query).
    auto stream = [&](int first, int step, auto&& before_load, auto&& consume) {
      const int nt = first < ntp ? (ntp - first + step - 1) / step : 0;
      dma(first < ntp ? first : 0, 0);
      if (nt > 1) dma(first + step, 1);
      int buf = 0, lbuf = 2;
      for (int it = 0; it < nt; ++it) {
        const int pt0 = (first + it * step) * kPT;
        if (it + 1 < nt) __builtin_amdgcn_s_waitcnt(kWaitVmcnt2);
        else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        lds_barrier();
        const char* kb = reinterpret_cast<const char*>(lds_k[buf]);
        before_load(it);
        if (it + 2 < nt) dma(first + (it + 2) * step, lbuf);
        buf = buf == kRing - 1 ? 0 : buf + 1;
        lbuf = lbuf == kRing - 1 ? 0 : lbuf + 1;

        // both column blocks' operands read and both products issued before the
        // first epilogue, which then runs while the second product is in flight
        float sc[kNRB][2][4];
        i32x8_t Bc[2];
        read_b(kb, b_lo, b_hi, Bc[0]);
        read_b(kb + 2048, b_lo, b_hi, Bc[1]);
        f32x16_t xs[kNRB][2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int rb = 0; rb < kNRB; ++rb) xs[rb][cb] = mma32(A[rb], Bc[cb]);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
          for (int rb = 0; rb < kNRB; ++rb) {
            const f32x16_t x = xs[rb][cb];
            // epilogue: clamp each head to the side of its weight, sum the heads
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float s01 = __builtin_amdgcn_fmed3f(x[4 * i + 0], cl[rb][i][0], 0.f) +
                                __builtin_amdgcn_fmed3f(x[4 * i + 1], cl[rb][i][1], 0.f);
              const float s23 = __builtin_amdgcn_fmed3f(x[4 * i + 2], cl[rb][i][2], 0.f) +
                                __builtin_amdgcn_fmed3f(x[4 * i + 3], cl[rb][i][3], 0.f);
              sc[rb][cb][i] = s01 + s23;
            }
          }
        }
        // causal pool mask, only on tiles some query of the wave sees in part
        if (pt0 + kPT > ncmin) {
#pragma unroll
          for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (pt0 + 32 * cb + c >= nc[rb][i]) sc[rb][cb][i] = NEG_INF;
        }
        consume(sc, pt0);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // a tile-0 load of an empty stream
      lds_barrier();  // every wave is done with the ring before the next stream
    };

    if (kTwoPhase) {
      // Phase 1: each lane keeps, per query, the kKeep32 best sampled scores of
      // its pool column (descending, in registers); the 32 lanes of a lane half
      // share a query.
      int rq[2][kNRB][4];
#pragma unroll
      for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = nc[rb][i];
          const int n_full = n / kPT, part = n % kPT;
          const int s_q = kPT * ((n_full + stride - 1) / stride) +
                          (n_full % stride == 0 ? part : 0);
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const float z = m == 0 ? kSampleZ1 : kSampleZ2;
            int r = 0;
            if (n > topk && s_q > 0) {
              const float f = (float)s_q / (float)n;
              const float x = 0.5f * (z + sqrtf(z * z + 4.f * topk * f));
              r = (int)ceilf(x * x);
              if (r >= s_q || r > kKeep32 * 32 * 3 / 4) r = 0;
            }
            rq[m][rb][i] = r;
          }
        }
      float best[kNRB][4][kKeep32];
#pragma unroll
      for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < kKeep32; ++j) best[rb][i][j] = NEG_INF;
      // per tile and query the lane's 2 new scores are sorted, merged into the 4
      // kept ones by taking the larger of kept[2+j] and new[1-j] (the top 4 of
      // the union, in bitonic order), and the 4 sorted by a half-cleaner network
      stream(0, stride, [](int) {}, [&](float (&sc)[kNRB][2][4], int) {
        auto cx = [](float& hi, float& lo) {
          const float t = fmaxf(hi, lo);
          lo = fminf(hi, lo);
          hi = t;
        };
#pragma unroll
        for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float n0 = sc[rb][0][i], n1 = sc[rb][1][i];
            cx(n0, n1);
            float* b = best[rb][i];
            b[2] = fmaxf(b[2], n1);
            b[3] = fmaxf(b[3], n0);
            cx(b[0], b[2]);
            cx(b[1], b[3]);
            cx(b[0], b[1]);
            cx(b[2], b[3]);
          }
      });
      // r-th best of the 32 lanes x kKeep32 kept scores of each query: the
      // largest key v with at least r kept keys >= v, bit by bit from the top,
      // for both ranks at once; the counts of both lane halves (two queries)
      // come from one ballot per kept score.  Only bits where some keys of the
      // wave differ are searched: a bit every key shares is the answer's too,
      // and starting from the common one-bits leaves each remaining test as in
      // the full search.
#pragma unroll
      for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t kk[kKeep32];
          uint32_t ko = 0u, ka = 0xFFFFFFFFu;
#pragma unroll
          for (int j = 0; j < kKeep32; ++j) {
            kk[j] = order_key(best[rb][i][j] + 0.f);
            ko |= kk[j];
            ka &= kk[j];
          }
          ka = wave_and(ka);                 // wave-uniform
          uint32_t bits = wave_or(ko) ^ ka;
          const int r0 = rq[0][rb][i], r1 = rq[1][rb][i];
          uint32_t p0 = ka, p1 = ka;
          while (bits != 0u) {
            const uint32_t bit = 1u << (31 - __builtin_clz(bits));
            bits ^= bit;
            const uint32_t c0k = p0 | bit, c1k = p1 | bit;
            int lo0 = 0, hi0 = 0, lo1 = 0, hi1 = 0;
#pragma unroll
            for (int j = 0; j < kKeep32; ++j) {
              const uint64_t M0 = ballot(kk[j] >= c0k);
              const uint64_t M1 = ballot(kk[j] >= c1k);
              lo0 += __popc((uint32_t)M0);
              hi0 += __popc((uint32_t)(M0 >> 32));
              lo1 += __popc((uint32_t)M1);
              hi1 += __popc((uint32_t)(M1 >> 32));
            }
            if ((h ? hi0 : lo0) >= r0) p0 = c0k;
            if ((h ? hi1 : lo1) >= r1) p1 = c1k;
          }
          tau[rb][i] = r0 > 0 ? float_below(key_to_float(p0)) : NEG_INF;
          tau2[rb][i] = r1 > 0 ? float_below(key_to_float(p1)) : NEG_INF;
        }
    }

    // Phase 2 (or the exact pass): every tile; survivors of the running
    // threshold are staged, stages are flushed to the per-query lists, and a
    // list that a flush leaves within one stage of its end keeps its top-k.
    // `redo` holds the wave's queries (bit 8 rb + t) scored in this attempt.
    uint32_t redo = kQW >= 32 ? 0xFFFFFFFFu : (1u << kQW) - 1u;
#pragma unroll 1
    for (int attempt = 0;; ++attempt) {
      if (attempt > 0) {
#pragma unroll
        for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            tau[rb][i] = ((redo >> (8 * rb + 2 * i + h)) & 1u) ? tau2[rb][i] : POS_INF;
      }
      int nst[kNRB];               // staged entries per row block (wave-uniform)
#pragma unroll
      for (int rb = 0; rb < kNRB; ++rb) nst[rb] = 0;
      int cnt_v = 0;               // lane q < kQW: list length of wave query q = 8 rb + t

      // Entry j of stage rb (of n) is moved to the list of its query; `cq` holds
      // the 8 list lengths of the row block and advances (stable per query).
      auto place = [&](int rb, int j0, int n, uint32_t fbits, uint32_t id, int (&cq)[8]) {
        const bool valid = j0 + lane < n;
        const int t = (int)(id >> kTag32Shift);
        int pos = 0;
#pragma unroll
        for (int tq = 0; tq < 8; ++tq) {
          const bool mine = valid && t == tq;
          const uint64_t Mt = ballot(mine);
          if (mine) pos = cq[tq] + mbcnt(Mt);
          cq[tq] += __popcll(Mt);
        }
        if (valid) {
          u32x2_t e;
          e[0] = order_key(__uint_as_float(fbits) + 0.f);  // -0 -> +0
          e[1] = id & kPool32Mask;
          a.cand[wbase + (int64_t)(8 * rb + t) * cap + pos] = e;
        }
      };
      auto flush = [&](uint32_t fl) {
#pragma unroll
        for (int rb = 0; rb < kNRB; ++rb) {
          if (!((fl >> rb) & 1u)) continue;
          const int n = nst[rb];
          int cq[8];
#pragma unroll
          for (int tq = 0; tq < 8; ++tq) cq[tq] = __builtin_amdgcn_readlane(cnt_v, 8 * rb + tq);
          for (int j0 = 0; j0 < n; j0 += kWave) {
            const int j = j0 + lane;
            const uint32_t fb = j < n ? lds_st[wave][rb][0][j] : 0u;
            const uint32_t id = j < n ? lds_st[wave][rb][1][j] : 0u;
            place(rb, j0, n, fb, id, cq);
          }
#pragma unroll
          for (int tq = 0; tq < 8; ++tq) cnt_v = lane == 8 * rb + tq ? cq[tq] : cnt_v;
          nst[rb] = 0;
        }
      };

      stream(0, 1,
          [&](int it) {
            // all stages of a wave are flushed together when one of them could
            // not take another tile's worth, and every kFlushPeriod tiles
            const bool period = it > 0 && (it % kFlushPeriod) == 0;
            bool full = false;
            uint32_t fl = 0;
#pragma unroll
            for (int rb = 0; rb < kNRB; ++rb) {
              full |= nst[rb] > kStage32 - kTileWorst;
              fl |= (nst[rb] > 0 ? 1u : 0u) << rb;
            }
            if (!(full || period) || fl == 0) return;
            flush(fl);
            bool fenced = false;
            for (uint32_t mm = fl; mm != 0; mm &= mm - 1) {
              const int rb = __builtin_ctz(mm);
#pragma unroll 1
              for (int tq = 0; tq < 8; ++tq) {
                const int q = 8 * rb + tq;
                const int n = __builtin_amdgcn_readlane(cnt_v, q);
                if (n <= cap - kStage32) continue;
                if (!fenced) {
                  __threadfence_block();  // this wave's list stores are visible
                  fenced = true;
                }
                // the (just flushed, empty) stage of rb holds the histogram
                const float T = select_and_compact<kSelectRegs>(a.cand + wbase + (int64_t)q * cap, n, topk,
                                                   lds_st[wave][rb][0], nullptr);
                cnt_v = lane == q ? topk : cnt_v;
#pragma unroll
                for (int r = 0; r < kNRB; ++r)
#pragma unroll
                  for (int i = 0; i < 4; ++i)
                    if (r == rb && 2 * i + h == tq) tau[r][i] = T;
              }
            }
          },
          [&](float (&sc)[kNRB][2][4], int pt0) {
            uint64_t MM[kNRB][2][4];
#pragma unroll
            for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
              for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) MM[rb][cb][i] = ballot(sc[rb][cb][i] > tau[rb][i]);
#pragma unroll
            for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
              for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const uint64_t M = MM[rb][cb][i];
                  if (M) {
                    if (sc[rb][cb][i] > tau[rb][i]) {
                      const int slot = nst[rb] + mbcnt(M);
                      uint32_t* st = &lds_st[wave][rb][0][slot];
                      st[0] = __float_as_uint(sc[rb][cb][i]);
                      st[kStage32] = ((uint32_t)(pt0 + 32 * cb) + ((uint32_t)i << (kTag32Shift + 1))) | lane_tag;
                    }
                    nst[rb] += __popcll(M);
                  }
                }
          });

      // remaining stages, then the final selection written to the output rows
      {
        uint32_t fl = 0;
#pragma unroll
        for (int rb = 0; rb < kNRB; ++rb) fl |= nst[rb] > 0 ? 1u << rb : 0u;
        if (fl) flush(fl);
      }
      __threadfence_block();
      uint32_t failed = 0;  // wave queries whose threshold was too high
#pragma unroll 1
      for (int q = 0; q < kQW; ++q) {
        if (!((redo >> q) & 1u)) continue;
        const int64_t qr = row_of(q0 + kQW * wave + q);
        if (qr < 0) continue;
        const int n = __builtin_amdgcn_readlane(cnt_v, q);
        // complete pools of query q: nc of its (rb, i) in lane half q & 1
        int ncq = 0;
#pragma unroll
        for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (8 * rb + 2 * i == (q & ~1)) ncq = __builtin_amdgcn_readlane(nc[rb][i], 32 * (q & 1));
        const int need = min(topk, ncq);
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
            for (int u = 0; u < 8; ++u) {
              const int j = j0 + u * kWave + lane;
              v[u] = j < n ? (int32_t)src[j][1] : 0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int j = j0 + u * kWave + lane;
              if (j < n) dst[j] = v[u];
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

// The kernels are plain functions around the templated body (in the host pass a
// kernel template of this size lost its host stub).  fp8: one row block of 8
// queries a wave (32 queries a workgroup), held to 128 registers so that four
// workgroups share a CU (four waves a SIMD; 32 KB of LDS each).  Measured at
// S = 2^20 (same ids): 62.7 ms, against 76.1 ms at three waves a SIMD, 91.9 ms
// with 16 queries a wave at two waves a SIMD, and 105.5 ms with 8 queries a
// wave at two.  Each extra wave a SIMD hides more of the others' dependency
// chains (MFMA results before the epilogue, ballots before branches).
constexpr int kNRB32 = 1;
__global__ __launch_bounds__(kThreads, 4) void indexer32_fp8_kernel(KernelArgs a) {
  indexer32_body<true, kNRB32>(a);
}
__global__ __launch_bounds__(kThreads, 4) void indexer32_fp8_exact_kernel(KernelArgs a) {
  indexer32_body<false, kNRB32>(a);
}

// Workgroups the device keeps resident at once, and its CU count (cached per device).
Residency index32_residency() {
  static std::mutex mu;
  static Residency cache[64] = {};
  int dev = 0;
  const Residency fallback{kIndexMaxSlots / 2, 2};
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fallback;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev].cus == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, indexer32_fp8_kernel, kThreads, 0) !=
            hipSuccess ||
        cus * per <= 0) {
      (void)hipGetLastError();
      return fallback;
    }
    cache[dev] = Residency{cus, per};
  }
  return cache[dev];
}

void launch32_passes(KernelArgs a, const IndexArgs& ia, uint32_t* fb_count, hipStream_t s) {
  constexpr int64_t qtile = (int64_t)kWaves * 8 * kNRB32;   // the kernels' query tile
  const int64_t lists = index_slots(ia.Sq) * kIndexQueryTile;
  int64_t slots = (ia.Sq + qtile - 1) / qtile;
  if (slots > lists / qtile) slots = lists / qtile;
  const Residency res = index32_residency();
  const int per_cu = ia.max_per_cu > 0 && ia.max_per_cu < res.per_cu ? ia.max_per_cu : res.per_cu;
  const int64_t resident = (int64_t)res.cus * per_cu;
  if (resident < slots) slots = resident;
  a.tile_next = fb_count + 1;
  indexer32_fp8_kernel<<<dim3((unsigned)slots), dim3(kThreads), 0, s>>>(a);
  a.tile_next = fb_count + 2;
  const int64_t exact_slots = ia.max_per_cu > 0 && slots > kExactSharedSlots ? kExactSharedSlots : slots;
  indexer32_fp8_exact_kernel<<<dim3((unsigned)exact_slots), dim3(kThreads), 0, s>>>(a);
}

}  // namespace

hipError_t launch_index_topk_fp8(const IndexArgs& ia, hipStream_t s) {
  const IndexWorkspace L = index_ws_layout(ia.Sq, ia.Sk, ia.topk);
  char* ws = static_cast<char*>(ia.ws);
  uint8_t* kpool = reinterpret_cast<uint8_t*>(ws + L.kpool_off);   // 64 bytes a pool
  uint32_t* fb_count = reinterpret_cast<uint32_t*>(ws + L.fb_off);
  int32_t* fb_rows = reinterpret_cast<int32_t*>(ws + L.fb_off + 256);
  const int64_t n_pools = ia.Sk / 4;
  const int64_t n_padded = index_padded_pools(ia.Sk);
  {
    const int64_t threads = ia.pooled ? 1 : n_padded * 8;
    pool_keys_fp8_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s>>>(
        ia.k_idx, kpool, n_pools, ia.pooled ? 0 : n_padded, fb_count);
  }
  KernelArgs a;
  a.q_idx = ia.q_idx;
  a.w_idx = ia.w_idx;
  a.kpool = nullptr;
  a.kpool8 = kpool;
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
  launch32_passes(a, ia, fb_count, s);
  return hipGetLastError();
}

}  // namespace dsa
