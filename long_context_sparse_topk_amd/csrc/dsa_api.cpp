// C ABI of the DSA layer: argument validation, workspace sizing and launches.
//
// Validation runs on the host before any HIP call and reports a specific
// status; a shape the kernels do not implement is an error, never a silent
// change of algorithm (the failure mode the SkyRL news item describes in
// "四块优化 1. DSA 真稀疏": a fused sparse kernel that rejected the shape and
// quietly fell back to dense attention).

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "dsa.h"
#include "dsa_kernels.hpp"

#define DSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_ptr(const void* p, const char* name, size_t align) {
  if (p == nullptr) return fail(DSA_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(DSA_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return DSA_OK;
}

constexpr int64_t kMaxSeq = (int64_t)1 << 31;

int check_seq(int64_t Sq, int64_t Sk, const int32_t* q_pos) {
  if (Sq < 1 || Sk < 1) return fail(DSA_INVALID_ARG, "Sq=%lld Sk=%lld must be >= 1", (long long)Sq, (long long)Sk);
  if (Sq >= kMaxSeq || Sk >= kMaxSeq)
    return fail(DSA_UNSUPPORTED_SHAPE, "Sq=%lld Sk=%lld must be < 2^31", (long long)Sq, (long long)Sk);
  if (q_pos == nullptr && Sq > Sk)
    return fail(DSA_INVALID_ARG, "q_pos is NULL (identity positions) but Sq=%lld > Sk=%lld",
                (long long)Sq, (long long)Sk);
  if (q_pos != nullptr && !aligned(q_pos, 4)) return fail(DSA_INVALID_ARG, "q_pos is not 4-byte aligned");
  return DSA_OK;
}

int check_attn_shape(int64_t Sq, int64_t Sk, int32_t heads, int32_t head_dim, int32_t pool,
                     int32_t topk, float scale, const int32_t* q_pos) {
  int st = check_seq(Sq, Sk, q_pos);
  if (st) return st;
  if (head_dim != 128) return fail(DSA_UNSUPPORTED_SHAPE, "head_dim=%d (supported: 128)", head_dim);
  if (heads < 1 || heads > dsa::kMaxHeads)
    return fail(DSA_UNSUPPORTED_SHAPE, "heads=%d (supported: 1..%d)", heads, dsa::kMaxHeads);
  if (pool != 4) return fail(DSA_UNSUPPORTED_SHAPE, "pool=%d (supported: 4)", pool);
  if (topk < 1 || topk > dsa::kMaxTopk)
    return fail(DSA_UNSUPPORTED_SHAPE, "topk=%d (supported: 1..%d)", topk, dsa::kMaxTopk);
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(DSA_INVALID_ARG, "scale must be finite and > 0");
  return DSA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

int check_index_shape(int64_t Sq, int64_t Sk, int32_t idx_heads, int32_t idx_dim, int32_t pool,
                      int32_t topk, int32_t q_chunk, const int32_t* q_pos, size_t ws_bytes) {
  int st = check_seq(Sq, Sk, q_pos);
  if (st) return st;
  if (idx_dim != 64) return fail(DSA_UNSUPPORTED_SHAPE, "idx_dim=%d (supported: 64)", idx_dim);
  if (idx_heads < 1 || idx_heads > dsa::kMaxIndexHeads)
    return fail(DSA_UNSUPPORTED_SHAPE, "idx_heads=%d (supported: 1..%d)", idx_heads, dsa::kMaxIndexHeads);
  if (pool != 4) return fail(DSA_UNSUPPORTED_SHAPE, "pool=%d (supported: 4)", pool);
  if (topk < 1 || topk > dsa::kMaxTopk)
    return fail(DSA_UNSUPPORTED_SHAPE, "topk=%d (supported: 1..%d)", topk, dsa::kMaxTopk);
  if (q_chunk < 1) return fail(DSA_INVALID_ARG, "q_chunk=%d must be >= 1", q_chunk);
  const size_t need = dsa::index_ws_layout(Sq, Sk, topk).total;
  if (ws_bytes < need)
    return fail(DSA_WORKSPACE_TOO_SMALL, "ws_bytes=%zu < %zu", ws_bytes, need);
  return DSA_OK;
}

// Query chunks of the pipelined indexer + forward: about one per 2^17 query
// rows, at most kPipeChunks.  Row r at position r costs the indexer about r
// pool scores, so the rows below b cost a share (b / Sq)^2 of its work.  The
// first chunk's indexer overlaps nothing and gets a share w_1 = f / n of it
// (f of an equal share); the others split the rest evenly, w_c = w_1 + (1 -
// w_1)(c - 1) / (n - 1); boundary c sits at Sq * sqrt(w_c), on a multiple of
// the indexer's 64-query tile.  With the bf16 indexer the chain of indexer
// chunks is the longer one, and its first chunk runs at the full-GPU rate, so
// f = 1.05 (S = 2^20, six chunks: 180.2-181.1 ms for f in 1.0-1.1 against
// 184.4 at 0.95 and 185.7 at 0.75, and 184-186 from 1.3 up); with the fp8
// indexer f = 0.75 (176.9 ms against 178.0 at 1.0).
constexpr int kPipeChunks = 6;
constexpr int64_t kPipeRowsPerChunk = (int64_t)1 << 17;

int pipe_chunks(int64_t Sq) {
  const int64_t n = Sq / kPipeRowsPerChunk;
  return n < 1 ? 1 : (n > kPipeChunks ? kPipeChunks : (int)n);
}

int64_t pipe_bound(int64_t Sq, int c, int n, double first_share) {
  if (c <= 0) return 0;
  if (c >= n) return Sq;
  const double w1 = first_share / (double)n;
  const double w = w1 + (1.0 - w1) * (double)(c - 1) / (double)(n - 1);
  const double x = (double)Sq * std::sqrt(w);
  int64_t b = (int64_t)std::llround(x / dsa::kIndexQueryTile) * dsa::kIndexQueryTile;
  return b < 0 ? 0 : (b > Sq ? Sq : b);
}

// The pipelined call's events, created on first use per host thread and device
// and reused by every later call of that thread: no runtime object is made on the
// hot path, and calls from different threads never share an event (a wait takes
// the state of the event's latest record, so sharing one across threads could
// order a stream after another thread's work).  They live until the process ends.
constexpr int kMaxDevices = 64;

hipError_t pipe_events(int dev, hipEvent_t** out) {
  thread_local hipEvent_t events[kMaxDevices][kPipeChunks + 1] = {};
  thread_local bool made[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!made[dev]) {
    for (int c = 0; c <= kPipeChunks; ++c) {
      const hipError_t e = hipEventCreateWithFlags(&events[dev][c], hipEventDisableTiming);
      if (e != hipSuccess) {
        for (int j = 0; j < c; ++j) (void)hipEventDestroy(events[dev][j]);
        return e;
      }
    }
    made[dev] = true;
  }
  *out = events[dev];
  return hipSuccess;
}

}  // namespace

DSA_EXPORT int dsa_version(void) { return 100; }

DSA_EXPORT const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_INVALID_ARG: return "invalid argument";
    case DSA_UNSUPPORTED_SHAPE: return "unsupported shape";
    case DSA_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DSA_HIP_ERROR: return "HIP error";
    default: return "unknown status";
  }
}

DSA_EXPORT const char* dsa_last_error(void) { return g_err; }

// ---------------------------------------------------------------------------

DSA_EXPORT size_t dsa_index_topk_ws_bytes(int64_t Sq, int64_t Sk, int32_t idx_heads,
                                          int32_t idx_dim, int32_t pool, int32_t topk,
                                          int32_t q_chunk) {
  (void)idx_heads; (void)idx_dim; (void)pool; (void)q_chunk;
  if (Sq < 1 || Sk < 1 || topk < 1 || topk > dsa::kMaxTopk) return 0;
  return dsa::index_ws_layout(Sq, Sk, topk).total;
}

DSA_EXPORT int dsa_index_topk(const void* q_idx, const void* k_idx, const void* w_idx,
                              const int32_t* q_pos, int64_t Sq, int64_t Sk, int32_t idx_heads,
                              int32_t idx_dim, int32_t pool, int32_t topk, int32_t q_chunk,
                              int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  int st;
  if ((st = check_ptr(q_idx, "q_idx", 16))) return st;
  if ((st = check_ptr(k_idx, "k_idx", 16))) return st;
  if ((st = check_ptr(w_idx, "w_idx", 2))) return st;
  if ((st = check_ptr(idx_out, "idx_out", 4))) return st;
  if ((st = check_ptr(ws, "ws", 256))) return st;
  if ((st = check_index_shape(Sq, Sk, idx_heads, idx_dim, pool, topk, q_chunk, q_pos, ws_bytes)))
    return st;

  (void)hipGetLastError();
  dsa::IndexArgs a{};
  a.q_idx = static_cast<const uint16_t*>(q_idx);
  a.k_idx = static_cast<const uint16_t*>(k_idx);
  a.w_idx = static_cast<const uint16_t*>(w_idx);
  a.q_pos = q_pos;
  a.Sq = Sq;
  a.Sk = Sk;
  a.heads = idx_heads;
  a.topk = topk;
  a.q_chunk = q_chunk;
  a.idx_out = idx_out;
  a.ws = ws;
  return hip_status(dsa::launch_index_topk(a, stream), "dsa_index_topk launch");
}

DSA_EXPORT int dsa_index_topk_fp8(const void* q_idx, const void* k_idx, const void* w_idx,
                                  const int32_t* q_pos, int64_t Sq, int64_t Sk, int32_t idx_heads,
                                  int32_t idx_dim, int32_t pool, int32_t topk, int32_t q_chunk,
                                  int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  int st;
  if ((st = check_ptr(q_idx, "q_idx", 16))) return st;
  if ((st = check_ptr(k_idx, "k_idx", 16))) return st;
  if ((st = check_ptr(w_idx, "w_idx", 2))) return st;
  if ((st = check_ptr(idx_out, "idx_out", 4))) return st;
  if ((st = check_ptr(ws, "ws", 256))) return st;
  if ((st = check_index_shape(Sq, Sk, idx_heads, idx_dim, pool, topk, q_chunk, q_pos, ws_bytes)))
    return st;
  if (idx_heads > 4)
    return fail(DSA_UNSUPPORTED_SHAPE, "idx_heads=%d (the fp8 indexer supports 1..4)", idx_heads);

  (void)hipGetLastError();
  dsa::IndexArgs a{};
  a.q_idx = static_cast<const uint16_t*>(q_idx);
  a.k_idx = static_cast<const uint16_t*>(k_idx);
  a.w_idx = static_cast<const uint16_t*>(w_idx);
  a.q_pos = q_pos;
  a.Sq = Sq;
  a.Sk = Sk;
  a.heads = idx_heads;
  a.topk = topk;
  a.q_chunk = q_chunk;
  a.idx_out = idx_out;
  a.ws = ws;
  return hip_status(dsa::launch_index_topk_fp8(a, stream), "dsa_index_topk_fp8 launch");
}

DSA_EXPORT int dsa_index_topk_stats(const void* ws, size_t ws_bytes, int64_t Sq, int64_t Sk,
                                    int32_t topk, uint32_t* retried_rows, uint32_t* exact_rows,
                                    hipStream_t stream) {
  g_err[0] = '\0';
  int st;
  if ((st = check_ptr(ws, "ws", 16))) return st;
  if (!retried_rows || !exact_rows) return fail(DSA_INVALID_ARG, "retried_rows and exact_rows must not be NULL");
  if (Sq < 1 || Sk < 1 || topk < 1 || topk > dsa::kMaxTopk)
    return fail(DSA_UNSUPPORTED_SHAPE, "Sq=%lld Sk=%lld topk=%d", (long long)Sq, (long long)Sk, topk);
  const dsa::IndexWorkspace L = dsa::index_ws_layout(Sq, Sk, topk);
  if (ws_bytes < L.total) return fail(DSA_WORKSPACE_TOO_SMALL, "ws_bytes=%zu < %zu", ws_bytes, L.total);
  uint32_t c[dsa::kIndexCounters];
  const char* src = static_cast<const char*>(ws) + L.fb_off;
  if ((st = hip_status(hipMemcpyAsync(c, src, sizeof(c), hipMemcpyDeviceToHost, stream),
                       "dsa_index_topk_stats copy")))
    return st;
  if ((st = hip_status(hipStreamSynchronize(stream), "dsa_index_topk_stats synchronize"))) return st;
  *exact_rows = c[0];
  *retried_rows = c[dsa::kIndexRetryCounter];
  return DSA_OK;
}

DSA_EXPORT int dsa_set_index_queries_per_wave(int32_t queries_per_wave) {
  g_err[0] = '\0';
  if (!dsa::set_index_queries_per_wave(queries_per_wave))
    return fail(DSA_INVALID_ARG, "queries_per_wave=%d (supported: 0, 4, 8, 16)", queries_per_wave);
  return DSA_OK;
}

DSA_EXPORT int dsa_sparse_attn_fwd(const void* q, const void* k, const void* v, const int32_t* idx,
                                   const int32_t* q_pos, int64_t Sq, int64_t Sk, int32_t heads,
                                   int32_t head_dim, int32_t pool, int32_t topk, float scale,
                                   void* out, float* lse, hipStream_t stream) {
  g_err[0] = '\0';
  int st;
  if ((st = check_ptr(q, "q", 16))) return st;
  if ((st = check_ptr(k, "k", 16))) return st;
  if ((st = check_ptr(v, "v", 16))) return st;
  if ((st = check_ptr(idx, "idx", 4))) return st;
  if ((st = check_ptr(out, "out", 16))) return st;
  if ((st = check_ptr(lse, "lse", 4))) return st;
  if ((st = check_attn_shape(Sq, Sk, heads, head_dim, pool, topk, scale, q_pos))) return st;

  (void)hipGetLastError();
  dsa::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.idx = idx;
  a.q_pos = q_pos;
  a.Sq = Sq;
  a.Sk = Sk;
  a.heads = heads;
  a.topk = topk;
  a.scale = scale;
  a.out = static_cast<uint16_t*>(out);
  a.lse_out = lse;
  return hip_status(dsa::launch_attn_fwd(a, stream), "dsa_sparse_attn_fwd launch");
}

// Indexer + top-k and the sparse attention forward over query chunks on two
// streams: the indexer of chunk c+1 runs on `stream` while the forward of
// chunk c runs on `aux_stream`.  The indexer is bound by MFMA and VALU issue,
// the forward by the memory fabric, so the two share the CUs: the indexer of
// every chunk after the first keeps one workgroup per CU, which leaves each
// CU the LDS and registers for forward waves beside it.  Every chunk runs the
// same kernels on its rows, so the results equal the two separate calls bit
// for bit.
DSA_EXPORT size_t dsa_index_attn_fwd_ws_bytes(int64_t Sq, int64_t Sk, int32_t idx_heads,
                                              int32_t idx_dim, int32_t pool, int32_t topk,
                                              int32_t q_chunk) {
  return dsa_index_topk_ws_bytes(Sq, Sk, idx_heads, idx_dim, pool, topk, q_chunk);
}

namespace {

// The pipelined call with the bf16 or the fp8 indexer.  Indexer chunks after the
// first share the CUs with the forward: the bf16 indexer keeps one workgroup a
// CU there (its 64-query sub-tile), the fp8 one two (its 32-query workgroups
// hold 128 registers a wave; measured at S = 2^20: 190 ms with two, 260 with
// one, 214 with three).
int index_attn_fwd(const void* q_idx, const void* k_idx, const void* w_idx, const void* q,
                   const void* k, const void* v, const int32_t* q_pos, int64_t Sq, int64_t Sk,
                   int32_t idx_heads, int32_t idx_dim, int32_t heads, int32_t head_dim,
                   int32_t pool, int32_t topk, int32_t q_chunk, float scale, int32_t* idx_out,
                   void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream,
                   hipStream_t aux_stream, bool fp8) {
  g_err[0] = '\0';
  int st;
  if ((st = check_ptr(q_idx, "q_idx", 16))) return st;
  if ((st = check_ptr(k_idx, "k_idx", 16))) return st;
  if ((st = check_ptr(w_idx, "w_idx", 2))) return st;
  if ((st = check_ptr(q, "q", 16))) return st;
  if ((st = check_ptr(k, "k", 16))) return st;
  if ((st = check_ptr(v, "v", 16))) return st;
  if ((st = check_ptr(idx_out, "idx_out", 4))) return st;
  if ((st = check_ptr(out, "out", 16))) return st;
  if ((st = check_ptr(lse, "lse", 4))) return st;
  if ((st = check_ptr(ws, "ws", 256))) return st;
  if ((st = check_index_shape(Sq, Sk, idx_heads, idx_dim, pool, topk, q_chunk, q_pos, ws_bytes)))
    return st;
  if ((st = check_attn_shape(Sq, Sk, heads, head_dim, pool, topk, scale, q_pos))) return st;
  if (fp8 && idx_heads > 4)
    return fail(DSA_UNSUPPORTED_SHAPE, "idx_heads=%d (the fp8 indexer supports 1..4)", idx_heads);

  const int n = aux_stream == stream ? 1 : pipe_chunks(Sq);
  // events: one per chunk (indexer done) and one for the forward stream's end
  hipEvent_t* ev = nullptr;
  if (n > 1) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = pipe_events(dev, &ev);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return hip_status(e, "dsa_index_attn_fwd: events");
    }
  }
  (void)hipGetLastError();
  hipError_t err = hipSuccess;
  auto note = [&](hipError_t e) {
    if (err == hipSuccess && e != hipSuccess) err = e;
  };
  const auto* qi = static_cast<const uint16_t*>(q_idx);
  const auto* wi = static_cast<const uint16_t*>(w_idx);
  const auto* qq = static_cast<const uint16_t*>(q);
  auto* oo = static_cast<uint16_t*>(out);
  bool pooled = false;  // the workspace holds the pooled keys (chunks run in order on `stream`)
  for (int c = 0; c < n && err == hipSuccess; ++c) {
    const double f = fp8 ? 0.75 : 1.05;
    const int64_t r0 = pipe_bound(Sq, c, n, f), r1 = pipe_bound(Sq, c + 1, n, f);
    if (r1 <= r0) continue;
    dsa::IndexArgs ia{};
    ia.q_idx = qi + r0 * idx_heads * idx_dim;
    ia.k_idx = static_cast<const uint16_t*>(k_idx);
    ia.w_idx = wi + r0 * idx_heads;
    ia.q_pos = q_pos ? q_pos + r0 : nullptr;
    ia.q_base = q_pos ? 0 : r0;
    ia.Sq = r1 - r0;
    ia.Sk = Sk;
    ia.heads = idx_heads;
    ia.topk = topk;
    ia.q_chunk = q_chunk;
    ia.idx_out = idx_out + r0 * topk;
    ia.ws = ws;
    ia.max_per_cu = pooled ? (fp8 ? 2 : 1) : 0;   // the first chunk has the GPU to itself
    ia.pooled = pooled;
    note(fp8 ? dsa::launch_index_topk_fp8(ia, stream) : dsa::launch_index_topk(ia, stream));
    pooled = true;
    hipStream_t fs = stream;
    if (n > 1) {
      note(hipEventRecord(ev[c], stream));
      note(hipStreamWaitEvent(aux_stream, ev[c], 0));
      fs = aux_stream;
    }
    dsa::AttnArgs fa{};
    fa.q = qq + r0 * heads * head_dim;
    fa.k = static_cast<const uint16_t*>(k);
    fa.v = static_cast<const uint16_t*>(v);
    fa.idx = idx_out + r0 * topk;
    fa.q_pos = q_pos ? q_pos + r0 : nullptr;
    fa.q_base = q_pos ? 0 : r0;
    fa.Sq = r1 - r0;
    fa.Sk = Sk;
    fa.heads = heads;
    fa.topk = topk;
    fa.scale = scale;
    fa.out = oo + r0 * heads * head_dim;
    fa.lse_out = lse + r0 * heads;
    fa.fwd_shared = n > 1 && c + 1 < n;   // the last chunk's forward runs after the indexer
    fa.fwd_hold = fa.fwd_shared && !fp8;  // beside the 64-query bf16 sub-tile (240 registers a wave)
    note(dsa::launch_attn_fwd(fa, fs));
  }
  if (n > 1) {
    // `stream` waits for the last forward chunk, so the caller can wait on it alone
    note(hipEventRecord(ev[n], aux_stream));
    note(hipStreamWaitEvent(stream, ev[n], 0));
  }
  return hip_status(err, fp8 ? "dsa_index_attn_fwd_fp8 launch" : "dsa_index_attn_fwd launch");
}

}  // namespace

DSA_EXPORT int dsa_index_attn_fwd(const void* q_idx, const void* k_idx, const void* w_idx,
                                  const void* q, const void* k, const void* v,
                                  const int32_t* q_pos, int64_t Sq, int64_t Sk,
                                  int32_t idx_heads, int32_t idx_dim, int32_t heads,
                                  int32_t head_dim, int32_t pool, int32_t topk, int32_t q_chunk,
                                  float scale, int32_t* idx_out, void* out, float* lse, void* ws,
                                  size_t ws_bytes, hipStream_t stream, hipStream_t aux_stream) {
  return index_attn_fwd(q_idx, k_idx, w_idx, q, k, v, q_pos, Sq, Sk, idx_heads, idx_dim, heads,
                        head_dim, pool, topk, q_chunk, scale, idx_out, out, lse, ws, ws_bytes,
                        stream, aux_stream, false);
}

DSA_EXPORT int dsa_index_attn_fwd_fp8(const void* q_idx, const void* k_idx, const void* w_idx,
                                      const void* q, const void* k, const void* v,
                                      const int32_t* q_pos, int64_t Sq, int64_t Sk,
                                      int32_t idx_heads, int32_t idx_dim, int32_t heads,
                                      int32_t head_dim, int32_t pool, int32_t topk,
                                      int32_t q_chunk, float scale, int32_t* idx_out, void* out,
                                      float* lse, void* ws, size_t ws_bytes, hipStream_t stream,
                                      hipStream_t aux_stream) {
  return index_attn_fwd(q_idx, k_idx, w_idx, q, k, v, q_pos, Sq, Sk, idx_heads, idx_dim, heads,
                        head_dim, pool, topk, q_chunk, scale, idx_out, out, lse, ws, ws_bytes,
                        stream, aux_stream, true);
}

DSA_EXPORT size_t dsa_sparse_attn_bwd_ws_bytes(int64_t Sq, int64_t Sk, int32_t heads,
                                               int32_t head_dim, int32_t topk) {
  if (Sq < 1 || Sk < 1 || head_dim != 128 || heads < 1 || heads > dsa::kMaxHeads || topk < 1 ||
      topk > dsa::kMaxTopk)
    return 0;
  return dsa::bwd_ws_layout(Sq, Sk, heads, topk).total;
}

namespace {

int check_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
              const float* lse, const int32_t* idx, const int32_t* q_pos, int64_t Sq, int64_t Sk,
              int32_t heads, int32_t head_dim, int32_t pool, int32_t topk, float scale, void* dq,
              void* dk, void* dv) {
  int st;
  if ((st = check_ptr(q, "q", 16))) return st;
  if ((st = check_ptr(k, "k", 16))) return st;
  if ((st = check_ptr(v, "v", 16))) return st;
  if ((st = check_ptr(out, "out", 16))) return st;
  if ((st = check_ptr(dout, "dout", 16))) return st;
  if ((st = check_ptr(lse, "lse", 4))) return st;
  if ((st = check_ptr(idx, "idx", 4))) return st;
  if ((st = check_ptr(dq, "dq", 16))) return st;
  if ((st = check_ptr(dk, "dk", 16))) return st;
  if ((st = check_ptr(dv, "dv", 16))) return st;
  if ((st = check_attn_shape(Sq, Sk, heads, head_dim, pool, topk, scale, q_pos))) return st;
  // the inverted selection lists are indexed with 32-bit offsets
  if (Sq * (int64_t)(topk + 1) >= kMaxSeq)
    return fail(DSA_UNSUPPORTED_SHAPE, "Sq*(topk+1)=%lld must be < 2^31",
                (long long)(Sq * (int64_t)(topk + 1)));
  return DSA_OK;
}

dsa::AttnArgs bwd_args(const void* q, const void* k, const void* v, const void* out,
                       const void* dout, const float* lse, const int32_t* idx,
                       const int32_t* q_pos, int64_t Sq, int64_t Sk, int32_t heads, int32_t topk,
                       float scale, void* dq, void* dk, void* dv, void* ws) {
  dsa::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse_in = lse;
  a.idx = idx;
  a.q_pos = q_pos;
  a.Sq = Sq;
  a.Sk = Sk;
  a.heads = heads;
  a.topk = topk;
  a.scale = scale;
  a.out = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.ws = ws;
  return a;
}

}  // namespace

DSA_EXPORT int dsa_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                                   const void* dout, const float* lse, const int32_t* idx,
                                   const int32_t* q_pos, int64_t Sq, int64_t Sk, int32_t heads,
                                   int32_t head_dim, int32_t pool, int32_t topk, float scale,
                                   void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  g_err[0] = '\0';
  int st;
  if ((st = check_bwd(q, k, v, out, dout, lse, idx, q_pos, Sq, Sk, heads, head_dim, pool, topk,
                      scale, dq, dk, dv)))
    return st;
  if ((st = check_ptr(ws, "ws", 256))) return st;
  const size_t need = dsa::bwd_ws_layout(Sq, Sk, heads, topk).total;
  if (ws_bytes < need) return fail(DSA_WORKSPACE_TOO_SMALL, "ws_bytes=%zu < %zu", ws_bytes, need);

  (void)hipGetLastError();
  const dsa::AttnArgs a = bwd_args(q, k, v, out, dout, lse, idx, q_pos, Sq, Sk, heads, topk, scale,
                                   dq, dk, dv, ws);
  return hip_status(dsa::launch_attn_bwd(a, stream), "dsa_sparse_attn_bwd launch");
}

DSA_EXPORT int dsa_sparse_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                                           const void* out, const void* dout, const float* lse,
                                           const int32_t* idx, const int32_t* q_pos, int64_t Sq,
                                           int64_t Sk, int32_t heads, int32_t head_dim,
                                           int32_t pool, int32_t topk, float scale, void* dq,
                                           void* dk, void* dv, hipStream_t stream) {
  g_err[0] = '\0';
  int st;
  if ((st = check_bwd(q, k, v, out, dout, lse, idx, q_pos, Sq, Sk, heads, head_dim, pool, topk,
                      scale, dq, dk, dv)))
    return st;
  const size_t need = dsa::bwd_ws_layout(Sq, Sk, heads, topk).total;
  if (need > dsa::kBwdScratchBytes)
    return fail(DSA_UNSUPPORTED_SHAPE,
                "the workspace this shape needs (%zu bytes) exceeds the allocation-free "
                "scratch (%zu bytes); use dsa_sparse_attn_bwd with a caller workspace",
                need, dsa::kBwdScratchBytes);
  void* ws = nullptr;
  const hipError_t e = dsa::bwd_scratch_address(&ws);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return hip_status(e, "dsa_sparse_attn_bwd_noalloc: scratch address");
  }
  (void)hipGetLastError();
  const dsa::AttnArgs a = bwd_args(q, k, v, out, dout, lse, idx, q_pos, Sq, Sk, heads, topk, scale,
                                   dq, dk, dv, ws);
  return hip_status(dsa::launch_attn_bwd(a, stream), "dsa_sparse_attn_bwd_noalloc launch");
}
