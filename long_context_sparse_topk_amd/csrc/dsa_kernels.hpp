// Host-side launchers of the DSA kernels (internal to the library).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// ---- indexer + top-k -------------------------------------------------------
constexpr int kIndexQueryTile = 64;     // queries per workgroup sub-tile
constexpr int kIndexPoolTile = 64;      // pools per LDS-staged key tile
constexpr int kIndexMaxSlots = 1024;    // resident workgroups owning candidate buffers
constexpr int kMaxTopk = 2048;

// per-query candidate capacity (multiple of 64, >= topk + one pool tile)
inline int index_candidate_cap(int topk) {
  int c = 2 * topk;
  if (c < topk + kIndexPoolTile) c = topk + kIndexPoolTile;
  return (c + 63) / 64 * 64;
}

inline int64_t index_slots(int64_t Sq) {
  int64_t tiles = (Sq + kIndexQueryTile - 1) / kIndexQueryTile;
  return tiles < kIndexMaxSlots ? tiles : kIndexMaxSlots;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct IndexWorkspace {
  size_t kpool_off, key_off, pool_off, total;
};

inline IndexWorkspace index_ws_layout(int64_t Sq, int64_t Sk, int topk) {
  IndexWorkspace w;
  const int64_t n_pools = Sk / 4;
  const size_t cand = (size_t)index_slots(Sq) * kIndexQueryTile * index_candidate_cap(topk);
  w.kpool_off = 0;
  w.key_off = align256((size_t)(n_pools > 0 ? n_pools : 1) * 64 * 2);
  w.pool_off = w.key_off + align256(cand * 4);
  w.total = w.pool_off + align256(cand * 4);
  return w;
}

struct IndexArgs {
  const uint16_t* q_idx;
  const uint16_t* k_idx;
  const uint16_t* w_idx;
  const int32_t* q_pos;
  int64_t Sq, Sk;
  int heads, topk, q_chunk;
  int32_t* idx_out;
  void* ws;
};

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t s);

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
  int64_t Sq, Sk;
  int heads, topk;
  float scale;
  uint16_t* out;          // fwd: O;  bwd: dq
  float* lse_out;         // fwd only
  uint16_t* dk;           // bwd only
  uint16_t* dv;           // bwd only
  void* ws;               // bwd only
};

inline size_t bwd_ws_bytes(int64_t Sk) { return align256((size_t)Sk * 128 * 4) * 2; }

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_bwd(const AttnArgs& a, hipStream_t s);

}  // namespace dsa
