// Host-side launchers of the DSA kernels (internal to the library).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// ---- indexer + top-k -------------------------------------------------------
constexpr int kIndexQueryTile = 64;     // queries per workgroup sub-tile
constexpr int kIndexPoolTile = 64;      // pools per LDS-staged key tile
constexpr int kIndexMaxSlots = 512;     // workgroups owning candidate lists (2 per CU x 256 CUs)
constexpr int kMaxTopk = 2048;
constexpr int kMaxIndexHeads = 8;       // indexer heads: one or two groups of 4 per query
constexpr int kMaxHeads = 64;           // attention heads: groups of 16, one wave each
// device counters at the head of the fallback region: [0] fallback-list
// length (rows the exact pass scores), [1] and [2] the tile queues of the
// two-phase and the exact pass, [3] rows whose first threshold kept fewer
// than min(k, n_c) pools (scored again with the wider margin)
constexpr int kIndexCounters = 4;
constexpr int kIndexRetryCounter = 3;

// Survivors of the running threshold are staged in LDS per (wave, row block
// of 4 queries) and moved to the per-query lists in HBM when a stage is
// within one pool tile's worst case (4 queries x 64 pools) of its end, and
// at a fixed period.
constexpr int kIndexStage = 440;

// per-query candidate capacity (multiple of 64): a list is compacted to topk
// entries when a flush leaves it within one stage of the end, so each
// compaction absorbs about 2*topk survivors
inline int index_candidate_cap(int topk) {
  int c = 3 * topk;
  if (c < topk + 384) c = topk + 384;
  c += kIndexStage;
  return (c + 63) / 64 * 64;
}

inline int64_t index_slots(int64_t Sq) {
  int64_t tiles = (Sq + kIndexQueryTile - 1) / kIndexQueryTile;
  return tiles < kIndexMaxSlots ? tiles : kIndexMaxSlots;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// pooled keys are stored padded to whole pool tiles (at least one tile)
inline int64_t index_padded_pools(int64_t Sk) {
  const int64_t n = Sk / 4;
  const int64_t t = (n + kIndexPoolTile - 1) / kIndexPoolTile;
  return (t > 0 ? t : 1) * kIndexPoolTile;
}

struct IndexWorkspace {
  size_t kpool_off, cand_off, fb_off, total;
};

// pooled keys | counters (256 B), fallback rows | candidate lists.  The pooled
// keys and the counters sit at offsets that depend on Sk only, so the query
// chunks of a pipelined call (each laid out for its own rows in the call's
// workspace) share them, and the counters of the last chunk are where
// dsa_index_topk_stats reads them for the whole call's shape.
inline IndexWorkspace index_ws_layout(int64_t Sq, int64_t Sk, int topk) {
  IndexWorkspace w;
  const size_t cand = (size_t)index_slots(Sq) * kIndexQueryTile * index_candidate_cap(topk);
  w.kpool_off = 0;
  w.fb_off = align256((size_t)index_padded_pools(Sk) * 64 * 2);
  w.cand_off = w.fb_off + 256 + align256((size_t)Sq * 4);
  w.total = w.cand_off + align256(cand * 8);
  return w;
}

struct IndexArgs {
  const uint16_t* q_idx;
  const uint16_t* k_idx;
  const uint16_t* w_idx;
  const int32_t* q_pos;
  int64_t q_base;          // position of row 0 when q_pos is NULL
  int64_t Sq, Sk;
  int heads, topk, q_chunk;
  int32_t* idx_out;
  void* ws;
  int max_per_cu;          // > 0: at most this many resident workgroups per CU
  bool pooled;             // the workspace already holds the pooled keys of k_idx
};

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t s);
// The same selection on fp8 (e4m3) operands, 32x32x64 MFMA; same workspace layout.
hipError_t launch_index_topk_fp8(const IndexArgs& a, hipStream_t s);

// Process-wide override of the indexer's workgroup sub-tile (queries per wave 4, 8 or 16;
// 0 = chosen per call).  Returns false for other values.
bool set_index_queries_per_wave(int qpw);

// ---- sparse attention --------------------------------------------------------
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;      // bwd only
  const uint16_t* dout;   // bwd only
  const float* lse_in;    // bwd only
  const int32_t* idx;
  const int32_t* q_pos;
  int64_t q_base;         // fwd: position of row 0 when q_pos is NULL
  int64_t Sq, Sk;
  int heads, topk;
  float scale;
  uint16_t* out;          // fwd: O;  bwd: dq
  float* lse_out;         // fwd only
  uint16_t* dk;           // bwd only
  uint16_t* dv;           // bwd only
  void* ws;               // bwd only
  bool fwd_shared;        // fwd: the launch shares the CUs with the indexer (lean schedule)
  bool fwd_hold;          // fwd, shared: at most one forward wave a SIMD (beside a bf16 indexer wave)
};

// Backward workspace: per (row, head) a 16-byte record (LSE in log2 units,
// Delta, position); the per-pool selection counts,
// turned into list offsets by a scan; the scan's block sums; and the query
// rows that selected each pool (an inverse of the idx lists).
constexpr int kScanBlock = 4096;

inline int64_t bwd_pools(int64_t Sk) { return (Sk + 3) / 4; }

// The inverse lists are built per (chunk of query rows, slice of pools): a
// workgroup counts its chunk's entries of its slice in LDS.  Chunks hold at
// least kInvRows rows; their number is capped so that the per-chunk counts
// (chunks x pools int32) stay within kInvCounts.
constexpr int kInvSlice = 16384;            // pools per slice (64 KiB of LDS counters)
constexpr int kInvRows = 256;               // fewest rows per chunk
constexpr int64_t kInvCounts = 1 << 22;     // most chunk counts kept (16 MiB)

inline int64_t bwd_chunks(int64_t Sq, int64_t Sk) {
  const int64_t np = bwd_pools(Sk);
  int64_t c = (Sq + kInvRows - 1) / kInvRows;
  const int64_t cap = kInvCounts / (np > 0 ? np : 1);
  if (c > cap) c = cap;
  return c > 0 ? c : 1;
}

struct BwdWorkspace {
  size_t delta_off, count_off, bsum_off, list_off, chunk_off, total;
};

inline BwdWorkspace bwd_ws_layout(int64_t Sq, int64_t Sk, int heads, int topk) {
  BwdWorkspace w;
  const int64_t np = bwd_pools(Sk);
  const int64_t nb = (np + kScanBlock - 1) / kScanBlock;
  w.delta_off = 0;
  w.count_off = align256((size_t)Sq * heads * 16);
  w.bsum_off = w.count_off + align256((size_t)np * 4);
  w.list_off = w.bsum_off + align256((size_t)nb * 4);
  w.chunk_off = w.list_off + align256((size_t)Sq * (topk + 1) * 4);
  w.total = w.chunk_off + align256((size_t)bwd_chunks(Sq, Sk) * np * 4);
  return w;
}

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_bwd(const AttnArgs& a, hipStream_t s);

// Allocation-free backward: the largest workspace its device-resident scratch
// array holds, and that array's device address on the current device (looked
// up once per device).
constexpr size_t kBwdScratchBytes = size_t(96) << 20;
hipError_t bwd_scratch_address(void** out);

}  // namespace dsa
