/*
 * dsa.h -- C ABI of one DeepSeek-Sparse-Attention (DSA) layer on MI355X (gfx950).
 *
 * The layer, as the source pages describe it:
 *   - an indexer scores every causal query against pools of 4 consecutive
 *     key tokens, so selection cost is quadratic while attention reads about
 *     2048 keys per query ("SkyRL 将 GLM-5.3-Flash 训练上下文扩至 100 万 token",
 *     section "模型与瓶颈");
 *   - the top-k pools are kept as an int32 pool-index list, and GLM-5.3-Flash
 *     attends 2051 keys (not 2048) with no positional encoding (same page,
 *     section "四块优化 1. DSA 真稀疏"); the indexer is scored in query chunks
 *     so its score matrix never exists in full (same section, and the Anyscale
 *     blog "How Lila Sciences and Anyscale Scaled GLM-5.3-Flash Training...",
 *     lessons paragraph);
 *   - attention over the selected keys accumulates softmax blockwise with a
 *     running max and sum, which equals the one-shot softmax (lesson "128K
 *     的序列,激活放在哪?", section "改进二:Ring Attention / 上下文并行").
 *
 * Readings where the pages are silent (the whole library follows them):
 *   - pool key = mean of the 4 token keys; a pool is a candidate for the query
 *     at position i only when complete: p < floor((i+1)/4);
 *   - score(i,p) = sum_h w[i,h] * max(0, q_idx[i,h,:] . kpool[p,:]);
 *   - top-k: descending score, equal scores go to the lower pool id, -0 = +0;
 *   - keys(i) = tokens of the selected pools plus the query's own incomplete
 *     pool (positions 4*floor((i+1)/4) .. i), so at most 4k+3 keys;
 *   - softmax(scale * q.k) over keys(i) with one K/V head shared by all heads
 *     (MQA); LSE in natural log.
 *
 * Conventions common to every entry point:
 *   - Every tensor is dense, row-major and contiguous in device memory.
 *     bf16 tensors are passed as raw 16-bit bfloat16 values.  Every device
 *     pointer except q_pos must be 16-byte aligned; q_pos 4-byte aligned.
 *   - q_pos: NULL means query row r sits at position r (then Sq <= Sk);
 *     otherwise q_pos[r] is the global position of row r, 0 <= q_pos[r] < Sk,
 *     in any order.  q_pos lives in device memory and is read by the kernels
 *     (its range is the caller's contract; out-of-range values are clamped
 *     to [0, Sk-1] on the device so no access leaves the buffers).
 *   - Pool ids are global: pool p holds tokens 4p..4p+3.
 *   - All work is enqueued on `stream` (NULL = the default stream); calls
 *     return without synchronising.  Inputs must stay valid until the stream
 *     has executed the call.
 *   - The caller allocates and owns every buffer, including workspaces; the
 *     library allocates no device memory, keeps no state between calls
 *     beyond what dsa_set_index_queries_per_wave sets and the pipelined
 *     call's reusable events, never writes its inputs and overwrites its
 *     outputs completely.  Calls
 *     from several host threads are safe; two calls that share an output or
 *     workspace buffer on different streams race.
 *   - Arguments are validated on the host before any HIP call.  Unsupported
 *     shapes return DSA_UNSUPPORTED_SHAPE: there is no fallback path (dense or
 *     otherwise).  No exception crosses the ABI and nothing is printed;
 *     dsa_last_error() gives the detail text of the calling thread's last
 *     failure.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum dsa_status {
  DSA_OK = 0,
  DSA_INVALID_ARG = 1,          /* null or misaligned pointer, bad count      */
  DSA_UNSUPPORTED_SHAPE = 2,    /* shape outside what the kernels implement   */
  DSA_WORKSPACE_TOO_SMALL = 3,  /* ws_bytes below the matching *_ws_bytes()   */
  DSA_HIP_ERROR = 4             /* a kernel launch failed (hipGetLastError)   */
};

/* Library version, major*10000 + minor*100 + patch. */
int dsa_version(void);

/* Static text for a status code; never NULL. */
const char* dsa_status_string(int status);

/* Detail of the calling thread's last failed call ("" if none). The string
 * is owned by the library and valid until the thread's next call. */
const char* dsa_last_error(void);

/* ---------------------------------------------------------------------------
 * Indexer + top-k pool selection.
 *
 * Computes, for every query row r at position i, the top `topk` complete
 * pools by indexer score (readings above) and writes their ids ascending to
 * idx_out[r, 0..m), m = min(topk, floor((i+1)/4)), then -1 to idx_out[r, m..topk).
 * Scores never reach device memory: the kernel keeps them on chip and only
 * streams candidate pool ids whose score beats a running per-query threshold.
 * Scoring is done in fp32 from bf16 operands: the pooled keys are rounded to
 * bf16 and each head weight is folded into its query as bf16(w * q), so that
 * w * ReLU(q . k) is computed as a clamp of bf16(w * q) . k to the side of
 * the weight's sign.  For integer indexer inputs in [-3, 3] every value is
 * exact, so results equal the exact real-number ranking; for other inputs,
 * scores carry those two bf16 roundings and near-ties may rank differently.
 *
 *   q_idx   [Sq, idx_heads, idx_dim] bf16   indexer queries
 *   k_idx   [Sk, idx_dim]            bf16   indexer keys (one per token)
 *   w_idx   [Sq, idx_heads]          bf16   per-query head weights
 *   q_pos   [Sq] int32 or NULL              see conventions
 *   idx_out [Sq, topk]               int32  output
 *   ws      workspace of ws_bytes >= dsa_index_topk_ws_bytes(...) bytes
 *
 * Supported: idx_dim == 64, 1 <= idx_heads <= 8, pool == 4,
 * 1 <= topk <= 2048, q_chunk >= 1, 1 <= Sq, 1 <= Sk < 2^31.  (The MFMA tile
 * holds 4 heads of each query; 5 to 8 heads take two such groups.  topk is
 * capped at 2048 pools (8195 keys a query, four times the pages' 2051)
 * because the workspace keeps, for every query in flight (up to 512 x 64), a
 * candidate list of about 3*topk + 440 entries of 8 bytes: 1.7 GB at 2048,
 * growing linearly with topk.)
 * q_chunk is the query chunk of the pages' indexer, there a bound on the
 * memory of materialised score rows.  No score row leaves the chip here, so
 * the chunk bounds nothing: it is validated (>= 1) and otherwise unused; the
 * kernel scores sub-tiles of 32 queries (16 when Sq <= 2^15) and the result
 * depends neither on q_chunk nor on the sub-tile.  The workspace (see
 * dsa_index_topk_ws_bytes) holds the pooled keys and fixed-size candidate
 * lists for at most 512 x 64 queries in flight.
 */
size_t dsa_index_topk_ws_bytes(int64_t Sq, int64_t Sk, int32_t idx_heads, int32_t idx_dim,
                               int32_t pool, int32_t topk, int32_t q_chunk);

int dsa_index_topk(const void* q_idx, const void* k_idx, const void* w_idx,
                   const int32_t* q_pos, int64_t Sq, int64_t Sk, int32_t idx_heads,
                   int32_t idx_dim, int32_t pool, int32_t topk, int32_t q_chunk,
                   int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Indexer + top-k on fp8 operands (opt-in variant).
 *
 * The same selection as dsa_index_topk, with the same arguments, workspace
 * (dsa_index_topk_ws_bytes) and output, computed on the gfx950 fp8 matrix
 * cores: the pooled keys and the folded queries bf16(w * q) are rounded to
 * OCP e4m3 (fp8) instead of bf16, and one v_mfma_f32_32x32x64_f8f6f4 scores 8
 * queries x 4 heads against 32 pools over the whole 64-dim contraction (half
 * the matrix-core time and half the key bytes of the bf16 path per pair).
 * Dot products accumulate in fp32.  The precision theme of the pages (SkyRL
 * news item, section "4. 去掉多余 fp32") is the motivation; the reading is
 * that the selection may be computed on e4m3 operands.  For integer indexer
 * inputs in [-3, 3] every operand is exact in e4m3 (w * q is an integer in
 * [-9, 9], a pooled key a multiple of 1/4 in [-3, 3]), so the ids equal the
 * exact ranking and dsa_index_topk's ids bit for bit; other inputs carry the
 * e4m3 rounding (3 mantissa bits; magnitudes above 448 saturate) and may rank
 * differently.
 *
 * Supported: as dsa_index_topk, with 1 <= idx_heads <= 4.
 */
int dsa_index_topk_fp8(const void* q_idx, const void* k_idx, const void* w_idx,
                       const int32_t* q_pos, int64_t Sq, int64_t Sk, int32_t idx_heads,
                       int32_t idx_dim, int32_t pool, int32_t topk, int32_t q_chunk,
                       int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Selection statistics of the last indexer launch that used `ws` (for the
 * pipelined calls, that of their last query chunk), read after the work
 * already enqueued on `stream` (the call synchronises the stream): the rows
 * whose first sampled threshold kept fewer than min(topk, n_c) pools and
 * were scored again with the wider margin (*retried_rows), and the rows that
 * failed that too and were scored by the exact pass (*exact_rows).  This is
 * the check that a call ran the fast path (the lessons paragraph of "How Lila
 * Sciences and Anyscale Scaled GLM-5.3-Flash Training..." asks to confirm that
 * every layer runs the kernel one expects): on the integer workloads no row
 * needs the exact pass.  Sq, Sk and topk are the launch's (they fix
 * the workspace layout); ws_bytes must be at least
 * dsa_index_topk_ws_bytes(...) for them.  The two outputs are host pointers.
 * Errors: DSA_INVALID_ARG (NULL or misaligned pointer), DSA_UNSUPPORTED_SHAPE,
 * DSA_WORKSPACE_TOO_SMALL, DSA_HIP_ERROR (copy or synchronisation failed). */
int dsa_index_topk_stats(const void* ws, size_t ws_bytes, int64_t Sq, int64_t Sk, int32_t topk,
                         uint32_t* retried_rows, uint32_t* exact_rows, hipStream_t stream);

/* Tuning override of the indexer's workgroup sub-tile, process-wide: 4, 8 or
 * 16 queries per wave (16-, 32- or 64-query sub-tiles) for every later
 * indexer launch, or 0 to let each call choose by its query count (the
 * default).  The ids do not depend on it; it exists so that tests can run
 * every sub-tile.  Takes effect for calls made after it returns; returns
 * DSA_INVALID_ARG for other values. */
int dsa_set_index_queries_per_wave(int32_t queries_per_wave);

/* ---------------------------------------------------------------------------
 * Sparse attention forward.
 *
 * For every query row r at position i and head h:
 *   O[r,h]   = sum_{j in keys(i)} softmax_j(scale * q[r,h].k[j]) * v[j]
 *   lse[r,h] = log sum_{j in keys(i)} exp(scale * q[r,h].k[j])
 * keys(i) = tokens 4p..4p+3 of every id p in idx[r,:] with 0 <= p <
 * floor((i+1)/4), plus positions 4*floor((i+1)/4) .. i.  Ids outside that
 * range (the -1 padding included) are skipped; ids must be distinct.
 * Accumulation is fp32 with a running max (online softmax); O is rounded to
 * bf16 (nearest even).
 *
 *   q   [Sq, heads, head_dim] bf16      k, v [Sk, head_dim] bf16 (shared)
 *   idx [Sq, topk] int32                q_pos [Sq] int32 or NULL
 *   out [Sq, heads, head_dim] bf16      lse [Sq, heads] fp32
 *
 * Supported: head_dim == 128, 1 <= heads <= 64, pool == 4,
 * 1 <= topk <= 2048, 1 <= Sq, 1 <= Sk < 2^31.  scale must be finite and > 0.
 * (Heads go in groups of 16, one wave per query row and group.)
 */
int dsa_sparse_attn_fwd(const void* q, const void* k, const void* v, const int32_t* idx,
                        const int32_t* q_pos, int64_t Sq, int64_t Sk, int32_t heads,
                        int32_t head_dim, int32_t pool, int32_t topk, float scale,
                        void* out, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Indexer + top-k followed by the sparse attention forward, pipelined.
 *
 * Computes exactly what dsa_index_topk followed by dsa_sparse_attn_fwd on its
 * idx_out compute (the same kernels, so idx_out, out and lse are equal bit
 * for bit), with the work split into contiguous chunks of query rows: the
 * indexer of chunk c+1 runs on `stream` while the forward of chunk c runs on
 * `aux_stream`.  The indexer is bound by matrix and vector issue, the forward
 * by the memory fabric, so the two overlap on the CUs.  The pages score the
 * indexer in query chunks to bound its memory (SkyRL news item, section
 * "四块优化 1. DSA 真稀疏"); here the chunks exist to overlap the two stages.
 *
 * Arguments are those of the two calls: the indexer's (q_idx, k_idx, w_idx,
 * idx_heads, idx_dim, q_chunk, ws, ws_bytes >= dsa_index_attn_fwd_ws_bytes())
 * and the forward's (q, k, v, heads, head_dim, scale, out, lse); q_pos, Sq,
 * Sk, pool and topk are shared, idx_out receives the selection.  Every
 * supported-shape rule of both calls applies.
 *
 * Streams: work is enqueued on `stream` and `aux_stream` (which must belong
 * to the same device), and before returning the call makes `stream` wait
 * for everything it enqueued on `aux_stream`: the caller orders later work,
 * or synchronises, on `stream` alone.  The forward of a chunk starts after
 * that chunk's indexer on `stream`, so it also sees all earlier work of
 * `stream`; earlier work of `aux_stream` stays ordered before it.  With
 * aux_stream == stream the two stages run one after the other on `stream`.
 * The call orders the two streams with events that the library creates once
 * per host thread and device (at most 7) and reuses on later calls; it
 * allocates no device memory.
 * Chunks: about one per 2^17 query rows, at most 6; the first holds 3/4 of
 * an equal share of the indexer work, the others equal shares.
 */
size_t dsa_index_attn_fwd_ws_bytes(int64_t Sq, int64_t Sk, int32_t idx_heads, int32_t idx_dim,
                                   int32_t pool, int32_t topk, int32_t q_chunk);

int dsa_index_attn_fwd(const void* q_idx, const void* k_idx, const void* w_idx, const void* q,
                       const void* k, const void* v, const int32_t* q_pos, int64_t Sq,
                       int64_t Sk, int32_t idx_heads, int32_t idx_dim, int32_t heads,
                       int32_t head_dim, int32_t pool, int32_t topk, int32_t q_chunk,
                       float scale, int32_t* idx_out, void* out, float* lse, void* ws,
                       size_t ws_bytes, hipStream_t stream, hipStream_t aux_stream);

/* The same pipelined call with the fp8 indexer (dsa_index_topk_fp8) in place of
 * the bf16 one: the same arguments, workspace and streams; idx_out, out and lse
 * equal those of dsa_index_topk_fp8 followed by dsa_sparse_attn_fwd bit for
 * bit.  Supported: as dsa_index_attn_fwd, with 1 <= idx_heads <= 4. */
int dsa_index_attn_fwd_fp8(const void* q_idx, const void* k_idx, const void* w_idx, const void* q,
                           const void* k, const void* v, const int32_t* q_pos, int64_t Sq,
                           int64_t Sk, int32_t idx_heads, int32_t idx_dim, int32_t heads,
                           int32_t head_dim, int32_t pool, int32_t topk, int32_t q_chunk,
                           float scale, int32_t* idx_out, void* out, float* lse, void* ws,
                           size_t ws_bytes, hipStream_t stream, hipStream_t aux_stream);

/* ---------------------------------------------------------------------------
 * Sparse attention backward.
 *
 * Gradients of L = sum(dout * O) for the forward above, with
 *   P = exp(scale * q.k - lse),  Delta[r,h] = sum_d dout[r,h,d] * O[r,h,d],
 *   dS = P * (dout.v - Delta),
 *   dq[r,h] = scale * sum_j dS_j k[j]
 *   dk[j]   = scale * sum_{r,h} dS q[r,h],  dv[j] = sum_{r,h} P dout[r,h]
 * All sums are fp32; dq, dk and dv are rounded to bf16 (nearest even) and
 * overwritten completely (0 for keys no row attends).  For dq, Delta is taken
 * from `out` (the forward's bf16 O); for dk and dv it is summed in fp32 over
 * the row's keys as sum_j P_j (dout . v[j]), which is the same quantity
 * without the rounding of O to bf16 (dk sums many rows' dS, so that rounding
 * would add up there).  P and dS enter the dk and dv products as a bf16 value
 * plus its bf16 rounding remainder, which keeps their fp32 precision.  dq is computed per
 * query row; dk and dv per pool of 4 keys, over the query rows whose key set
 * holds the pool, found by inverting idx in the workspace (counting per
 * chunk of rows in LDS, no global atomics).  A pool's rows are summed in
 * ascending row order, so dq, dk and dv are bitwise reproducible: the same
 * inputs give the same bits on every call.  (A row that repeats an id, which
 * the layer does not allow, contributes once to that pool's dk and dv.)
 *
 *   q, out, dout [Sq, heads, head_dim] bf16   k, v [Sk, head_dim] bf16
 *   lse [Sq, heads] fp32 (from the forward)   idx, q_pos as in the forward
 *   dq [Sq, heads, head_dim] bf16             dk, dv [Sk, head_dim] bf16
 *   ws  workspace of ws_bytes >= dsa_sparse_attn_bwd_ws_bytes(...) bytes
 *       (Delta, per-pool offsets, the inverted lists and per-chunk pool
 *       counts: about 4 * (Sq * (heads + topk + 1) + Sk / 4) bytes plus at
 *       most 16 MiB)
 *
 * Supported: as the forward, and Sq * (topk + 1) < 2^31.  Returns 0 bytes
 * for arguments outside that.
 */
size_t dsa_sparse_attn_bwd_ws_bytes(int64_t Sq, int64_t Sk, int32_t heads, int32_t head_dim,
                                    int32_t topk);

int dsa_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, const int32_t* idx,
                        const int32_t* q_pos, int64_t Sq, int64_t Sk, int32_t heads,
                        int32_t head_dim, int32_t pool, int32_t topk, float scale,
                        void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Sparse attention backward without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving or
 * training loops that forbid allocation).
 *
 * Computes exactly what dsa_sparse_attn_bwd computes, with the same
 * arguments less ws and ws_bytes, and allocates nothing: its workspace is a
 * 96 MiB (100,663,296-byte) array in device memory that the library holds
 * on every GPU it runs on until the process ends (its device address is
 * looked up once per device, on the first call there).  Shapes whose
 * workspace, dsa_sparse_attn_bwd_ws_bytes(...), exceeds 96 MiB return
 * DSA_UNSUPPORTED_SHAPE before any HIP call (S = 131,072 with 4 heads and
 * topk 128 needs 88.6 MiB).  All calls on one GPU share that array: two
 * calls whose executions overlap on one GPU (different streams, or several
 * host threads) race and give wrong gradients; order them on one stream.
 */
int dsa_sparse_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                                const void* dout, const float* lse, const int32_t* idx,
                                const int32_t* q_pos, int64_t Sq, int64_t Sk, int32_t heads,
                                int32_t head_dim, int32_t pool, int32_t topk, float scale,
                                void* dq, void* dk, void* dv, hipStream_t stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* DSA_H_ */
