// Sparse attention backward (gfx950).
//
// Gradients of sum(dO * O) for the sparse forward.  The pages train through
// this layer ("SkyRL 将 GLM-5.3-Flash 训练上下文扩至 100 万 token", section "2. 激活
// 重算与 Offload" recomputes it in backward); the formulas are those of softmax
// attention:
//   P  = exp(scale * q.k - lse)          (recomputed from the saved LSE)
//   dS = P * (dO.v - Delta),   Delta = sum_d dO * O
//   dq = scale * dS K,   dk = scale * dS^T q,   dv = P^T dO
//
// Two passes, neither with atomics on the gradients:
//
//   dq pass (query-major): one wave per (query row, group of 16 heads), four
//     waves per workgroup, 32 keys per tile, gathered from the row's idx list.
//     Also saves Delta.
//       S^T  = K . Q^T,  dP^T = V . dO^T          MFMA 16x16x32, keys as M
//       dQ^T += K^T dS^T                           MFMA 16x16x32, K^T read from LDS
//
//   dk/dv pass (pool-major): the idx lists are inverted first (count per
//     pool, scan, scatter of the query rows), then one workgroup per pool of
//     4 keys walks the rows that selected it, 16 (row, head) pairs per step
//     (16/H whole rows when H <= 16, else 16 heads of one row):
//       S  = Q . K^T,  dP = dO . V^T                MFMA 16x16x32, (row, head) as M,
//                                                   the pool's keys as N (4 of 16)
//       dK[key, dim] += dS^T Q,  dV += P^T dO       MFMA 16x16x16, (row, head) as k
//     The S output layout of the first product is the A-operand layout of the
//     second, so P and dS go from registers straight into it; Q and dO are
//     read transposed from LDS (ds_read_b64_tr_b16).  Every key is written
//     once, in bf16 (0 for keys no row attends).
//   A pool's rows are listed in ascending order and each wave sums a fixed
//   block of them, so dk and dv are bitwise reproducible.
//
// Rows staged through LDS (K in the dq pass, Q and dO in the dk/dv pass) are
// gathered 16 lanes per 256-byte row, so that the four lanes of a quad read
// one contiguous segment, and the MFMA operands are read back from LDS: a
// gather whose quads read four different rows (the MFMA operand order) stays
// below ~9.5 TB/s even from L2.  S = 2^17 backward 9.3-9.4 -> 8.5-8.8 ms,
// zig-zag share 5.2-5.4 -> 4.8-5.0 ms, same gradients.  V of the dq pass, an
// MFMA operand only, stays in the operand order (staging it too gained
// nothing).

#include <mutex>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {
namespace {

constexpr int kD = 128;
constexpr int kRows = 4;
constexpr int kKStride = 136;

// ---------------------------------------------------------------------------
// dq pass

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  const int32_t* idx;
  const int32_t* q_pos;
  int64_t Sq, Sk;
  int H, HG, topk;         // heads, groups of 16 heads
  float scale, scale_log2;
  uint16_t* dq;
  float* stats;            // per (row, head): lse * log2(e), Delta, position (bits), 0
};

__device__ __forceinline__ int clamp_pos(const int32_t* q_pos, int64_t r, int64_t Sk) {
  int64_t pos = r;
  if (q_pos) {
    pos = q_pos[r];
    pos = pos < 0 ? 0 : (pos >= Sk ? Sk - 1 : pos);
  }
  return (int)pos;
}

__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(BwdArgs a) {
  __shared__ __align__(16) uint16_t lds_k[kRows][32 * kKStride];
  __shared__ int2 lds_info[kRows][2][8];

  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int64_t item = (int64_t)blockIdx.x * kRows + wave;   // (row, head group)
  const int64_t r = item / a.HG;
  if (r >= a.Sq) return;
  const int h0 = 16 * (int)(item - r * a.HG);                 // first head of the group
  const int g = lane >> 4;
  const int c16 = lane & 15;

  const int pos = clamp_pos(a.q_pos, r, a.Sk);
  const int nc = (pos + 1) >> 2;
  const int part = (pos + 1) & 3;
  const int32_t* irow = a.idx + r * a.topk;

  int np = 0;
  for (int j0 = 0; j0 < a.topk; j0 += kWave) {
    const int j = j0 + lane;
    const uint64_t M = ballot(j < a.topk && irow[j] >= 0);
    if (M) np = j0 + 64 - __clzll((long long)M);
  }
  const int nps = np + (part > 0 ? 1 : 0);
  const int ntile = (nps + 7) >> 3;

  // B operands with head h0 + c16: Q^T, dO^T; Delta from O
  const int hd = h0 + c16;
  const bool hv = hd < a.H;
  bf16x8_t QB[4], DB[4];
  float delta = 0.f;
  {
    const int64_t off = (r * a.H + hd) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      QB[ks] = hv ? load_bf16x8(a.q + off + 32 * ks) : zero_bf16x8();
      if (hv) {
        const u32x4_t d = *reinterpret_cast<const u32x4_t*>(a.dout + off + 32 * ks);
        const u32x4_t o = *reinterpret_cast<const u32x4_t*>(a.o + off + 32 * ks);
        DB[ks] = as_bf16x8(d);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          delta = fmaf(bf16_to_f32(d[j] & 0xFFFFu), bf16_to_f32(o[j] & 0xFFFFu), delta);
          delta = fmaf(bf16_to_f32(d[j] >> 16), bf16_to_f32(o[j] >> 16), delta);
        }
      } else {
        DB[ks] = zero_bf16x8();
      }
    }
  }
  delta += __shfl_xor(delta, 16, kWave);
  delta += __shfl_xor(delta, 32, kWave);
  const float lse2 = hv ? a.lse[r * a.H + hd] * kLog2e : 0.f;
  // Delta from the bf16 O serves this pass's dS.  The key loop also sums
  // P_j dP_j = dO . (sum_j P_j V_j), Delta from the fp32 output the forward
  // rounded; that value goes to the record that the dk/dv pass reads.
  float dsum = 0.f;

  f32x4_t dqa[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) dqa[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint16_t* kt = lds_k[wave];

  // The K/V rows of the next tile are in flight while a tile is computed (two
  // register buffers, the loop unrolled by two); its slot ids are loaded one
  // step earlier still, so no wait on them drains the tile in flight.  Loads
  // past the last tile read the query's own key row.  Slot info is double
  // buffered in LDS.
  struct Buf {
    u32x4_t KR[8];
    bf16x8_t VA[2][4];
  };
  // slot ids of tile t: lane j (mod 8) reads id 8t + j, clamped into the row
  auto load_ids = [&](int t) -> int {
    const int ps = 8 * t + (lane & 7);
    const int cps = ps < np ? ps : (np > 0 ? np - 1 : 0);
    return irow[cps];
  };
  auto set_info = [&](int t, int id) {
    int2* info = lds_info[wave][t & 1];
    if (lane < 8) {
      const int ps = 8 * t + lane;
      int base = pos, nv = 0;
      if (ps < np) {
        if (id >= 0 && id < nc) {
          base = 4 * id;
          nv = 4;
        }
      } else if (ps == np && part > 0) {
        base = 4 * nc;
        nv = part;
      }
      info[lane] = make_int2(base, nv);
    }
  };
  auto load_kv = [&](int t, Buf& B) {
    const int2* info = lds_info[wave][t & 1];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int2 in = info[4 * kb + (c16 >> 2)];
      const int off = c16 & 3;
      const int64_t key = off < in.y ? in.x + off : pos;
      const uint16_t* vsrc = a.v + key * kD + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) B.VA[kb][ks] = load_bf16x8(vsrc + 32 * ks);
    }
    // K rows (staged through LDS): 16 lanes per 256-byte row, slot j, key offset g
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int2 in = info[j];
      const int64_t key = g < in.y ? in.x + g : pos;
      B.KR[j] = *reinterpret_cast<const u32x4_t*>(a.k + key * kD + 8 * c16);
    }
  };
  auto compute = [&](int t, const Buf& B) {
    const int2* info = lds_info[wave][t & 1];
    // K rows go to LDS: read back as the A operand of S, and transposed for dQ
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<u32x4_t*>(kt + (4 * j + g) * kKStride + 8 * c16) = B.KR[j];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float ds[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* ksrc = kt + (16 * kb + c16) * kKStride + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s = mfma32(as_bf16x8(*reinterpret_cast<const u32x4_t*>(ksrc + 32 * ks)), QB[ks], s);
        dp = mfma32(B.VA[kb][ks], DB[ks], dp);
      }
      const int nv = info[4 * kb + g].y;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float pp = (hv && rr < nv) ? exp2f(s[rr] * a.scale_log2 - lse2) : 0.f;
        ds[4 * kb + rr] = pp * (dp[rr] - delta);
        dsum = fmaf(pp, dp[rr], dsum);
      }
    }
    u32x4_t dsb;
    dsb[0] = pack_bf16x2(ds[0], ds[1]);
    dsb[1] = pack_bf16x2(ds[2], ds[3]);
    dsb[2] = pack_bf16x2(ds[4], ds[5]);
    dsb[3] = pack_bf16x2(ds[6], ds[7]);
    const bf16x8_t DSB = as_bf16x8(dsb);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();

    // dQ^T[dim, head] += K^T[dim, key] dS^T[key, head]; the A operand holds
    // keys 4g..4g+3 then 16+4g..16+4g+3 (the keys of this lane's dS values)
    const uint16_t* k0 = kt + 4 * g * kKStride + tr_offset(c16, kKStride);
    const uint16_t* k1 = k0 + 16 * kKStride;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const u32x2_t lo = __builtin_bit_cast(u32x2_t, read_tr(k0 + 16 * db));
      const u32x2_t hi = __builtin_bit_cast(u32x2_t, read_tr(k1 + 16 * db));
      const u32x4_t ka = {lo[0], lo[1], hi[0], hi[1]};
      dqa[db] = mfma32(as_bf16x8(ka), DSB, dqa[db]);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };

  Buf B0, B1;
  int id = load_ids(0);
  if (ntile > 0) {
    const int id0 = id;
    id = load_ids(1);
    set_info(0, id0);
    load_kv(0, B0);
  }
  for (int t = 0; t < ntile; t += 2) {
    {
      const int idt = id;
      id = load_ids(t + 2);
      set_info(t + 1, idt);
      load_kv(t + 1, B1);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(t, B0);
    if (t + 1 >= ntile) break;
    {
      const int idt = id;
      id = load_ids(t + 3);
      set_info(t + 2, idt);
      load_kv(t + 2, B0);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(t + 1, B1);
  }

  dsum += __shfl_xor(dsum, 16, kWave);
  dsum += __shfl_xor(dsum, 32, kWave);
  if (hv && g == 0) {
    f32x4_t rec = {lse2, dsum, __int_as_float(pos), 0.f};
    reinterpret_cast<f32x4_t*>(a.stats)[r * a.H + hd] = rec;
  }
  if (hv) {
    uint16_t* dst = a.dq + (r * a.H + hd) * kD + 4 * g;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      u32x2_t o;
      o[0] = pack_bf16x2(dqa[db][0] * a.scale, dqa[db][1] * a.scale);
      o[1] = pack_bf16x2(dqa[db][2] * a.scale, dqa[db][3] * a.scale);
      *reinterpret_cast<u32x2_t*>(dst + 16 * db) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// inverse of the idx lists: for every pool, the query rows that attend it
// (selected pools, plus the row's own incomplete pool)

// Inverse of the idx lists: for every pool, the query rows whose key set
// holds it, as one array `list` with the rows of pool p at
// [end[p-1], end[p]).  The rows are split into chunks and the pools into
// slices of kInvSlice; one workgroup per (chunk, slice) counts, and later
// places, its chunk's rows of its slice's pools in LDS, so no global atomics
// are needed:
//   inv_count_kernel         cnt[c][p] = rows of chunk c holding pool p
//   inv_chunk_prefix_kernel  cnt[c][p] = rows of p in chunks before c; offs[p] = total
//   scan kernels             offs[p] = end of p's rows (inclusive scan)
//   inv_place_kernel         list[start(p) + cnt[c][p] + rank in chunk] = row,
//                            rows of a pool in ascending order
struct InvArgs {
  const int32_t* idx;
  const int32_t* q_pos;
  int64_t Sq, Sk;
  int topk;
  int64_t np;              // pools
  int64_t chunk_rows;      // rows per chunk
  int64_t chunks;
  int nslices;
  int32_t* cnt;            // [chunks][np]
  int32_t* offs;           // [np]
  int32_t* list;
};

// One thread per pool: per-chunk counts -> exclusive prefix over the
// chunks; the pool's total to offs.
__global__ __launch_bounds__(256) void inv_chunk_prefix_kernel(InvArgs a) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= a.np) return;
  int32_t* col = a.cnt + p;
  int s = 0;
  int64_t c = 0;
  for (; c + 8 <= a.chunks; c += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = col[(c + u) * a.np];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      col[(c + u) * a.np] = s;
      s += v[u];
    }
  }
  for (; c < a.chunks; ++c) {
    const int v = col[c * a.np];
    col[c * a.np] = s;
    s += v;
  }
  a.offs[p] = s;
}

// Both passes walk a chunk's rows in blocks of up to 32, whose entries (k + 1
// a row) the 1024 threads read at once, kInvPer at most a thread, into
// registers, and mark each entry's row in its pool's 32-bit mask.  A pool
// counts the rows of its mask (a row holding a pool twice, against the
// layer's requirement of distinct ids, counts once), and the placement gives
// an entry the slot h[pool] + (rows of the mask before its own), so the rows of
// a pool are listed in ascending order and the dk/dv pass sums them in an
// order fixed by the inputs: dk and dv are bitwise reproducible.  Whichever of
// a pool's entries first takes its mask (an exchange with 0) moves the count
// or h[pool] on.  The barriers order LDS only: list stores need not land
// before the next block.  (S = 2^17, k = 128: count 0.11 ms, placement 0.22,
// as with the unordered placement by LDS atomics.)
constexpr int kInvThreads = 1024;
constexpr int kInvBlockRows = 32;
constexpr int kInvPer = 8;

__device__ __forceinline__ int inv_block_rows(int topk) {
  const int r = kInvThreads * kInvPer / (topk + 1);
  return r < 1 ? 1 : (r > kInvBlockRows ? kInvBlockRows : r);
}

// This thread's entries of rows [b0, b1) whose pool lies in [p0, p1),
// row-major from entry threadIdx.x in strides of kInvThreads, as
// (pool - p0) << 5 | (row - b0), else -1.  Entry j < topk of row r (position
// i, nc = floor((i+1)/4) complete pools) is pool idx[r][j] if 0 <= idx[r][j] <
// nc; entry topk is the row's own incomplete pool nc if (i+1) % 4 != 0.  The
// loads use in-bounds clamped indices and are issued unconditionally, so that
// they are in flight together.
template <bool kPos>
__device__ __forceinline__ void block_entries(const InvArgs& a, int64_t b0, int64_t b1, int p0, int p1,
                                              int (&ent)[kInvPer]) {
  const int per = a.topk + 1;
  const int step_r = kInvThreads / per, step_j = kInvThreads % per;
  int64_t rr[kInvPer];
  int jj[kInvPer], id[kInvPer], ps[kInvPer];
  int64_t r = b0 + (int)threadIdx.x / per;
  int j = (int)threadIdx.x % per;
#pragma unroll
  for (int u = 0; u < kInvPer; ++u) {
    rr[u] = r;
    jj[u] = j;
    const int64_t rc = r < b1 ? r : b1 - 1;
    id[u] = a.idx[rc * a.topk + (j < a.topk ? j : a.topk - 1)];
    ps[u] = kPos ? a.q_pos[rc] : (int)rc;
    r += step_r;
    j += step_j;
    const bool wrap = j >= per;
    j = wrap ? j - per : j;
    r += wrap ? 1 : 0;
  }
#pragma unroll
  for (int u = 0; u < kInvPer; ++u) {
    const int pos = kPos ? (ps[u] < 0 ? 0 : (ps[u] >= a.Sk ? (int)(a.Sk - 1) : ps[u])) : ps[u];
    const int nc = (pos + 1) >> 2;
    int p;
    if (jj[u] < a.topk) p = (id[u] >= 0 && id[u] < nc) ? id[u] : -1;
    else p = ((pos + 1) & 3) ? nc : -1;
    ent[u] = (rr[u] < b1 && p >= p0 && p < p1) ? ((p - p0) << 5) | (int)(rr[u] - b0) : -1;
  }
}

// kPlace = false: h[pool] += rows of the chunk holding the pool; true: list the
// rows at h[pool] onwards, ascending.
template <bool kPos, bool kPlace>
__device__ __forceinline__ void walk_chunk(const InvArgs& a, int32_t* h, uint32_t* msk, int64_t r0,
                                           int64_t r1, int p0, int p1) {
  const int rows = inv_block_rows(a.topk);
  for (int64_t b0 = r0; b0 < r1; b0 += rows) {
    const int64_t b1 = min(b0 + rows, r1);
    int ent[kInvPer];
    block_entries<kPos>(a, b0, b1, p0, p1, ent);
#pragma unroll
    for (int u = 0; u < kInvPer; ++u)
      if (ent[u] >= 0) atomicOr(&msk[ent[u] >> 5], 1u << (ent[u] & 31));
    lds_barrier();
    if (kPlace) {
#pragma unroll
      for (int u = 0; u < kInvPer; ++u)
        if (ent[u] >= 0) {
          const int i = ent[u] >> 5, rb = ent[u] & 31;
          a.list[h[i] + __popc(msk[i] & ((1u << rb) - 1u))] = (int32_t)(b0 + rb);
        }
      lds_barrier();
    }
#pragma unroll
    for (int u = 0; u < kInvPer; ++u)
      if (ent[u] >= 0) {
        const int i = ent[u] >> 5;
        const uint32_t m = atomicExch(&msk[i], 0u);   // one of the pool's entries takes the mask
        if (m != 0u) h[i] += __popc(m);
      }
    lds_barrier();
  }
}

template <bool kPlace>
__device__ __forceinline__ void inv_pass(const InvArgs& a, int32_t* h, uint32_t* msk) {
  const int64_t c = blockIdx.x / a.nslices;
  const int p0 = (int)(blockIdx.x % a.nslices) * kInvSlice;
  const int p1 = (int)min((int64_t)p0 + kInvSlice, a.np);
  const int32_t* pre = a.cnt + c * a.np;
  for (int i = threadIdx.x; i < p1 - p0; i += kInvThreads) {
    const int p = p0 + i;
    // placement: start of p's rows + earlier chunks' rows of p
    h[i] = kPlace ? (p > 0 ? a.offs[p - 1] : 0) + pre[p] : 0;
    msk[i] = 0u;
  }
  lds_barrier();
  const int64_t r0 = c * a.chunk_rows;
  const int64_t r1 = min(r0 + a.chunk_rows, a.Sq);
  if (a.q_pos) walk_chunk<true, kPlace>(a, h, msk, r0, r1, p0, p1);
  else walk_chunk<false, kPlace>(a, h, msk, r0, r1, p0, p1);
  if (!kPlace) {
    int32_t* dst = a.cnt + c * a.np + p0;
    for (int i = threadIdx.x; i < p1 - p0; i += kInvThreads) dst[i] = h[i];
  }
}

__global__ __launch_bounds__(kInvThreads) void inv_count_kernel(InvArgs a) {
  __shared__ int32_t h[kInvSlice];
  __shared__ uint32_t msk[kInvSlice];
  inv_pass<false>(a, h, msk);
}

__global__ __launch_bounds__(kInvThreads) void inv_place_kernel(InvArgs a) {
  __shared__ int32_t h[kInvSlice];
  __shared__ uint32_t msk[kInvSlice];
  inv_pass<true>(a, h, msk);
}

// Inclusive scan of n counts in place, in blocks of kScanBlock: block sums,
// an exclusive scan of the block sums (one workgroup), then each block's
// local scan.
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_w, int& total) {
  // 1024 threads: wave scans, then a scan of the 16 wave totals
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(x, o, kWave);
    if (lane >= o) x += t;
  }
  if (lane == kWave - 1) lds_w[w] = x;
  __syncthreads();
  if (w == 0) {
    int y = lane < 16 ? lds_w[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int t = __shfl_up(y, o, kWave);
      if (lane >= o) y += t;
    }
    if (lane < 16) lds_w[16 + lane] = y;
  }
  __syncthreads();
  total = lds_w[31];
  const int before = w > 0 ? lds_w[16 + w - 1] : 0;
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(1024) void scan_block_sums_kernel(const int32_t* __restrict__ c,
                                                               int32_t* __restrict__ bsum, int64_t n) {
  __shared__ int lds_w[32];
  const int64_t base = (int64_t)blockIdx.x * kScanBlock;
  int v = 0;
#pragma unroll
  for (int i = 0; i < kScanBlock / 1024; ++i) {
    const int64_t j = base + i * 1024 + threadIdx.x;
    v += j < n ? c[j] : 0;
  }
  int total;
  (void)block_exclusive_scan(v, lds_w, total);
  if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

__global__ __launch_bounds__(1024) void scan_sums_kernel(int32_t* __restrict__ bsum, int64_t nb) {
  __shared__ int lds_w[32];
  int carry = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += 1024) {
    const int64_t j = b0 + threadIdx.x;
    const int v = j < nb ? bsum[j] : 0;
    int total;
    const int ex = block_exclusive_scan(v, lds_w, total);
    if (j < nb) bsum[j] = carry + ex;
    carry += total;
  }
}

// Writes the inclusive scan (each element: the sum up to and including it).
__global__ __launch_bounds__(1024) void scan_apply_kernel(int32_t* __restrict__ c,
                                                          const int32_t* __restrict__ bsum, int64_t n) {
  __shared__ int lds_w[32];
  const int64_t base = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * (kScanBlock / 1024);
  int v[kScanBlock / 1024];
  int s = 0;
#pragma unroll
  for (int i = 0; i < kScanBlock / 1024; ++i) {
    v[i] = base + i < n ? c[base + i] : 0;
    s += v[i];
  }
  int total;
  int ex = block_exclusive_scan(s, lds_w, total) + bsum[blockIdx.x];
#pragma unroll
  for (int i = 0; i < kScanBlock / 1024; ++i) {
    ex += v[i];
    if (base + i < n) c[base + i] = ex;
  }
}

// ---------------------------------------------------------------------------
// dk/dv pass

struct KvArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const f32x4_t* stats;    // per (row, head): lse * log2(e), Delta, position (bits), 0
  const int32_t* offs;     // per pool: end of its rows in `list` (start = end of the previous)
  const int32_t* list;
  int64_t Sk;
  int H;
  float scale, scale_log2;
  uint16_t* dk;
  uint16_t* dv;
};

constexpr int kKvWaves = 4;
constexpr int kTStride = 136;   // LDS row stride (bf16) of the Q / dO tiles

// Operands of one step (16 (row, head) pairs): the A lanes' Q and dO
// chunks, and the record of each D-layout pair.
struct KvStep {
  u32x4_t q[4], d[4];
  f32x4_t st[4];
};

__global__ __launch_bounds__(kKvWaves * kWave, 2) void attn_bwd_dkdv_kernel(KvArgs a) {
  __shared__ __align__(16) uint16_t lds_q[kKvWaves][16 * kTStride];
  __shared__ __align__(16) uint16_t lds_do[kKvWaves][16 * kTStride];
  __shared__ __align__(16) float lds_red[kKvWaves][2][8][kD];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = uniform(tid >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int64_t p = blockIdx.x;
  const int beg = p > 0 ? a.offs[p - 1] : 0;
  const int n = a.offs[p] - beg;
  const int64_t key0 = 4 * p;
  const int nkeys = a.Sk - key0 < 4 ? (int)(a.Sk - key0) : 4;
  // A step holds 16 (row, head) pairs: with H <= 16, qpc = 16/H whole rows
  // (nrh = qpc*H pairs used); with H > 16, heads 16c..16c+15 of one row, the
  // row's cpr = ceil(H/16) groups in consecutive steps.
  const int H = a.H;
  const bool wide = H > 16;
  const int qpc = wide ? 1 : 16 / H;
  const int nrh = wide ? 16 : qpc * H;
  const int cpr = wide ? (H + 15) / 16 : 1;
  // pair c of step s: the row's index in the chunk and its head; valid within H
  auto pair_of = [&](int s, int c, int& j, int& h) -> bool {
    if (wide) {
      j = s / cpr;
      h = 16 * (s - j * cpr) + c;
      return h < H;
    }
    j = s * qpc + c / H;
    h = c % H;
    return c < nrh;
  };

  // K, V of the pool as B operands: B[dim 8g + j (+32 ks)][column c16].  Columns
  // 0-3 and 4-7 both hold the pool's keys 0-3 (zero past nkeys), 8-15 are zero.
  // The dK/dV products take P and dS as bf16 operands; to keep their fp32
  // precision each value v goes in as two bf16 parts, hi = bf16(v) in the
  // row of columns 0-3 and lo = bf16(v - hi) in the row of columns 4-7, and
  // the two output rows of a key are summed at the end.
  const int kcol = c16 & 3;
  const bool lo_lane = c16 >= 4 && c16 < 8;
  bf16x8_t KB[4], VB[4];
  {
    const bool kv = c16 < 8 && kcol < nkeys;
    const int64_t off = (key0 + kcol) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      KB[ks] = kv ? load_bf16x8(a.k + off + 32 * ks) : zero_bf16x8();
      VB[ks] = kv ? load_bf16x8(a.v + off + 32 * ks) : zero_bf16x8();
    }
  }
  f32x4_t adk[8], adv[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    adk[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    adv[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  uint16_t* tq = lds_q[wave];
  uint16_t* tdo = lds_do[wave];
  const int64_t kpos = key0 + kcol;  // key of this lane's D column
  const int toff = 4 * g * kTStride + tr_offset(c16, kTStride);

  // This wave's rows: a contiguous block of the pool's list, read 64 entries
  // at a time (one per lane) and handed out by shuffles, 16/H rows per step.
  const int per = (n + kKvWaves - 1) / kKvWaves;
  const int r0 = min(n, wave * per), r1 = min(n, r0 + per);

  // rows lst (lane j: entry j of the chunk), step s of the chunk, chunk length m
  auto load_step = [&](int lst, int s, int m, KvStep& o) {
    // Q and dO rows, 16 lanes per 256-byte (row, head) row: load j brings
    // pair 4j + g, 16-byte chunk c16
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int jp, hp;
      const bool vp = pair_of(s, 4 * j + g, jp, hp) && jp < m;
      const int64_t rp = __shfl(lst, jp & 63, kWave);
      const int64_t poff = ((vp ? rp : 0) * H + (vp ? hp : 0)) * kD + 8 * c16;
      o.q[j] = vp ? *reinterpret_cast<const u32x4_t*>(a.q + poff) : u32x4_t{0u, 0u, 0u, 0u};
      o.d[j] = vp ? *reinterpret_cast<const u32x4_t*>(a.dout + poff) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {                        // D lanes: pairs 4g + i
      int jd, hdd;
      const bool vr = pair_of(s, 4 * g + i, jd, hdd) && jd < m;
      const int64_t rd = __shfl(lst, jd & 63, kWave);
      o.st[i] = vr ? a.stats[(vr ? rd : 0) * H + (vr ? hdd : 0)] : f32x4_t{0.f, 0.f, __int_as_float(-1), 0.f};
    }
  };

  for (int base = r0; base < r1; base += kWave) {
    const int m = min(kWave, r1 - base);
    const int lst = lane < m ? a.list[beg + base + lane] : 0;
    const int nsteps = wide ? m * cpr : (m + qpc - 1) / qpc;
    KvStep cur, nxt;
    load_step(lst, 0, m, cur);
    for (int s = 0; s < nsteps; ++s) {
      if (s + 1 < nsteps) load_step(lst, s + 1, m, nxt);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<u32x4_t*>(tq + (4 * j + g) * kTStride + 8 * c16) = cur.q[j];
        *reinterpret_cast<u32x4_t*>(tdo + (4 * j + g) * kTStride + 8 * c16) = cur.d[j];
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // A operands from the tiles: pair c16, dims 8g + 32ks
      f32x4_t sv = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4_t qa = *reinterpret_cast<const u32x4_t*>(tq + c16 * kTStride + 8 * g + 32 * ks);
        const u32x4_t da = *reinterpret_cast<const u32x4_t*>(tdo + c16 * kTStride + 8 * g + 32 * ks);
        sv = mfma32(as_bf16x8(qa), KB[ks], sv);
        dp = mfma32(as_bf16x8(da), VB[ks], dp);
      }
      // lane holds S[(row, head) 4g+i][key c16]
      float pv[4], dsv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = c16 < 8 && kcol < nkeys && kpos <= (int64_t)__float_as_int(cur.st[i][2]);
        pv[i] = ok ? exp2f(sv[i] * a.scale_log2 - cur.st[i][0]) : 0.f;
        dsv[i] = pv[i] * (dp[i] - cur.st[i][1]);
      }
      // A operands of the 16x16x16 products: A[column c16][(row, head) 4g+j],
      // the bf16 value in columns 0-3 and its rounding remainder in 4-7
      u32x2_t pa, dsa;
      pa[0] = pack_bf16x2(pv[0], pv[1]);
      pa[1] = pack_bf16x2(pv[2], pv[3]);
      dsa[0] = pack_bf16x2(dsv[0], dsv[1]);
      dsa[1] = pack_bf16x2(dsv[2], dsv[3]);
      if (lo_lane) {
        pa[0] = pack_bf16x2(pv[0] - bf16_to_f32(pa[0] & 0xFFFFu), pv[1] - bf16_to_f32(pa[0] >> 16));
        pa[1] = pack_bf16x2(pv[2] - bf16_to_f32(pa[1] & 0xFFFFu), pv[3] - bf16_to_f32(pa[1] >> 16));
        dsa[0] = pack_bf16x2(dsv[0] - bf16_to_f32(dsa[0] & 0xFFFFu), dsv[1] - bf16_to_f32(dsa[0] >> 16));
        dsa[1] = pack_bf16x2(dsv[2] - bf16_to_f32(dsa[1] & 0xFFFFu), dsv[3] - bf16_to_f32(dsa[1] >> 16));
      }
      const s16x4_t PA = as_s16x4(pa), DSA = as_s16x4(dsa);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // B operands B[(row, head) 4g+j][dim 16db+c16] by transposed reads: lane s
      // of the group supplies (row 4g + s/4, dims 16db + 4(s%4) .. +3)
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const s16x4_t QT = read_tr(tq + toff + 16 * db);
        const s16x4_t DT = read_tr(tdo + toff + 16 * db);
        adk[db] = mfma16(DSA, QT, adk[db]);
        adv[db] = mfma16(PA, DT, adv[db]);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      cur = nxt;
    }
  }

  // adk[db]: lane holds row 4g+i, dim 16db+c16 of the product: the bf16 parts of
  // key i in g == 0, the remainders of key i in g == 1
  if (g < 2) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lds_red[wave][0][4 * g + i][16 * db + c16] = adk[db][i];
        lds_red[wave][1][4 * g + i][16 * db + c16] = adv[db][i];
      }
  }
  __syncthreads();
  // 256 threads x 4 consecutive values = 2 x 4 keys x 128 dims
  {
    const int which = tid >> 7;            // 0: dk, 1: dv
    const int key = (tid >> 5) & 3;
    const int d0 = (tid & 31) * 4;
    if (key < nkeys) {
      float v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kKvWaves; ++w)
          acc += lds_red[w][which][key][d0 + e] + lds_red[w][which][4 + key][d0 + e];
        v4[e] = which == 0 ? acc * a.scale : acc;
      }
      u32x2_t o;
      o[0] = pack_bf16x2(v4[0], v4[1]);
      o[1] = pack_bf16x2(v4[2], v4[3]);
      uint16_t* dst = (which == 0 ? a.dk : a.dv) + (key0 + key) * kD + d0;
      *reinterpret_cast<u32x2_t*>(dst) = o;
    }
  }
}

}  // namespace

hipError_t launch_attn_bwd(const AttnArgs& x, hipStream_t s) {
  const BwdWorkspace L = bwd_ws_layout(x.Sq, x.Sk, x.heads, x.topk);
  char* ws = static_cast<char*>(x.ws);
  float* stats = reinterpret_cast<float*>(ws + L.delta_off);
  int32_t* offs = reinterpret_cast<int32_t*>(ws + L.count_off);
  int32_t* bsum = reinterpret_cast<int32_t*>(ws + L.bsum_off);
  int32_t* list = reinterpret_cast<int32_t*>(ws + L.list_off);
  const int64_t np = bwd_pools(x.Sk);
  const int64_t nb = (np + kScanBlock - 1) / kScanBlock;

  // inverse of the idx lists
  InvArgs ia;
  ia.idx = x.idx;
  ia.q_pos = x.q_pos;
  ia.Sq = x.Sq;
  ia.Sk = x.Sk;
  ia.topk = x.topk;
  ia.np = np;
  ia.chunk_rows = (x.Sq + bwd_chunks(x.Sq, x.Sk) - 1) / bwd_chunks(x.Sq, x.Sk);
  ia.chunks = (x.Sq + ia.chunk_rows - 1) / ia.chunk_rows;   // <= bwd_chunks: fits the workspace
  ia.nslices = (int)((np + kInvSlice - 1) / kInvSlice);
  ia.cnt = reinterpret_cast<int32_t*>(ws + L.chunk_off);
  ia.offs = offs;
  ia.list = list;
  const unsigned inv_blocks = (unsigned)(ia.chunks * ia.nslices);
  inv_count_kernel<<<dim3(inv_blocks), dim3(kInvThreads), 0, s>>>(ia);
  inv_chunk_prefix_kernel<<<dim3((unsigned)((np + 255) / 256)), dim3(256), 0, s>>>(ia);
  scan_block_sums_kernel<<<dim3((unsigned)nb), dim3(1024), 0, s>>>(offs, bsum, np);
  scan_sums_kernel<<<dim3(1), dim3(1024), 0, s>>>(bsum, nb);
  scan_apply_kernel<<<dim3((unsigned)nb), dim3(1024), 0, s>>>(offs, bsum, np);
  inv_place_kernel<<<dim3(inv_blocks), dim3(kInvThreads), 0, s>>>(ia);

  // dq (and Delta)
  BwdArgs a;
  a.q = x.q;
  a.k = x.k;
  a.v = x.v;
  a.o = x.o;
  a.dout = x.dout;
  a.lse = x.lse_in;
  a.idx = x.idx;
  a.q_pos = x.q_pos;
  a.Sq = x.Sq;
  a.Sk = x.Sk;
  a.H = x.heads;
  a.HG = (x.heads + 15) / 16;
  a.topk = x.topk;
  a.scale = x.scale;
  a.scale_log2 = x.scale * kLog2e;
  a.dq = x.out;
  a.stats = stats;
  const int64_t blocks = (x.Sq * a.HG + kRows - 1) / kRows;
  attn_bwd_dq_kernel<<<dim3((unsigned)blocks), dim3(kRows * kWave), 0, s>>>(a);

  // dk, dv
  KvArgs kv;
  kv.q = x.q;
  kv.k = x.k;
  kv.v = x.v;
  kv.dout = x.dout;
  kv.stats = reinterpret_cast<const f32x4_t*>(stats);
  kv.offs = offs;
  kv.list = list;
  kv.Sk = x.Sk;
  kv.H = x.heads;
  kv.scale = x.scale;
  kv.scale_log2 = x.scale * kLog2e;
  kv.dk = x.dk;
  kv.dv = x.dv;
  attn_bwd_dkdv_kernel<<<dim3((unsigned)np), dim3(kKvWaves * kWave), 0, s>>>(kv);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the workspace is a file-scope device array, one copy
// per GPU, that lives until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in symbol): its
// device address is looked up once per device with hipGetSymbolAddress and
// that address is what the kernels receive.  Nothing in the workspace has to
// start at zero (every pass writes what a later pass reads), so it is not
// cleared.  All calls on one GPU share the array: calls that overlap on a GPU
// (on different streams) race.

namespace {
static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];

constexpr int kScratchDevices = 64;
}  // namespace

hipError_t bwd_scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kScratchDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace dsa
