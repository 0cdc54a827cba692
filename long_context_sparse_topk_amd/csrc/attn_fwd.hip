// Sparse attention forward over the selected pools (gfx950).
//
// What is computed (pages: "SkyRL 将 GLM-5.3-Flash 训练上下文扩至 100 万 token",
// sections "模型与瓶颈" and "四块优化 1. DSA 真稀疏"; online softmax: lesson
// "128K 的序列,激活放在哪?", section "改进二:Ring Attention / 上下文并行"):
// each query attends, with no positional encoding, to the tokens of its
// selected pools plus its own incomplete pool, all heads sharing one K/V head.
// The softmax is accumulated tile by tile with a running max and sum.
//
// Mapping: one wave per (query row, group of 16 heads), four waves per
// workgroup; the groups of one row are neighbouring waves, so their K/V
// gathers meet in the same caches.  A tile is 8 pool slots = 32 keys.  Every
// gathered K/V row is a contiguous 256-byte segment and every selected pool a
// contiguous 1 KiB segment of K (and of V).
//   S^T[key, head] = K[key, :] . Q[head, :]      MFMA 16x16x32, keys as M
//   O^T[dim, head] += V^T[dim, key] P^T[key, head]
// V goes through LDS to be read transposed; the K rows go straight into MFMA
// A-operand registers, or through LDS as well for key sets the caches hold
// (kStagedMaxKeys).  With keys as M and heads as N, each lane owns one head,
// so the online-softmax rescale is a per-lane scalar.
//
// Gather lane order: in the MFMA operand order the four lanes of a quad read
// four different rows, and such a gather stays below ~9.5 TB/s even when
// every row hits in L2; with 16 lanes reading one 256-byte row (a quad reads
// one contiguous 64-byte segment) the same gather reaches ~26 TB/s from L2
// and ~8% more from beyond it (a probe gathering random rows of 0.5 MB to
// 256 MB tables).  V, which is staged through LDS anyway, is loaded in the
// row-contiguous order: S = 2^20 141.6 -> 139.4 ms, S = 2^15 3.6 -> 2.6 ms,
// S = 2^12 0.147 -> 0.105 ms, same outputs.  K is staged the same way when
// the key set is small (kStagedMaxKeys below); at S = 2^20 the extra LDS
// round trip costs more than the row-contiguous order gains.

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {
namespace {

constexpr int kD = 128;
constexpr int kRows = 4;        // query rows (waves) per workgroup
constexpr int kVStride = 136;   // LDS row stride (elements) of the V tile
constexpr float kLazyLog2 = 8.f;  // log2 of the largest P before the reference max moves
// Up to this many keys (K and V together at most 64 MiB) the forward stages
// K through LDS too: S = 2^15 2.71 -> 2.31-2.33 ms, S = 2^12 0.102-0.105 ->
// 0.093-0.095, S = 2^17 3.50-3.57 -> 3.40-3.41; at 2^18 keys (the zig-zag
// share) it changes nothing, and at S = 2^20, where the fabric below L2
// binds, it costs about 1% (139.0 against 137.9-138.2 ms), so larger key sets
// load K straight into MFMA registers.
constexpr int64_t kStagedMaxKeys = int64_t(1) << 17;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  const int32_t* q_pos;
  int64_t q_base;  // position of row 0 when q_pos is NULL
  int64_t Sq, Sk;
  int H, HG, topk;         // heads, groups of 16 heads
  float scale_log2;
  uint16_t* out;
  float* lse;
};

// Pool slot ps of a row: slots [0, np) are idx entries, slot np is the query's
// own incomplete pool.  Returns the first key and the number of valid keys.
__device__ __forceinline__ int2 slot_info(const int32_t* irow, int ps, int np, int nc, int part,
                                          int pos) {
  int base = pos, nv = 0;
  if (ps < np) {
    const int p = irow[ps];
    if (p >= 0 && p < nc) {
      base = 4 * p;
      nv = 4;
    }
  } else if (ps == np && part > 0) {
    base = 4 * nc;
    nv = part;
  }
  return make_int2(base, nv);
}

// kKStaged: K rows go through LDS as well (gathered 16 lanes per row, read
// back as the MFMA operand), for key sets the caches hold (kStagedMaxKeys).
// kHold (shared schedule only): the kernel claims 272 of a SIMD's 512
// registers, so at most one forward wave sits on a SIMD and a 240-register
// indexer wave always finds room beside it.  Without the hold the shared
// forward (184 registers) puts two waves on SIMDs the indexer has not reached
// yet, and the indexer's workgroups of a new chunk wait for them: pipelined
// S = 2^20 step 186.6-186.8 ms with the hold against 189.1-189.7 without.
// The fp8 indexer's shared chunks keep two 128-register workgroups a CU,
// which a held forward wave would not fit beside (215 against 178 ms), so
// they use the unheld instance.
template <bool kPrefetch, bool kKStaged, bool kHold>
__global__ __launch_bounds__(256) void attn_fwd_kernel(FwdArgs a) {
  // an empty asm that clobbers v231 makes the allocation 232 VGPRs (+ 40 AGPRs)
  if constexpr (kHold) asm volatile("" ::: "v231");
  __shared__ __align__(16) uint16_t lds_v[kRows][32 * kVStride];
  __shared__ __align__(16) uint16_t lds_k[kRows][kKStaged ? 32 * kVStride : 8];
  __shared__ int2 lds_info[kRows][kPrefetch ? 2 : 1][8];  // slot info, double buffered when prefetching

  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int64_t item = (int64_t)blockIdx.x * kRows + wave;   // (row, head group)
  const int64_t r = item / a.HG;
  if (r >= a.Sq) return;
  const int h0 = 16 * (int)(item - r * a.HG);                 // first head of the group
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const float NEG_INF = -__builtin_huge_valf();

  int64_t pos64 = a.q_pos ? (int64_t)a.q_pos[r] : a.q_base + r;
  pos64 = pos64 < 0 ? 0 : (pos64 >= a.Sk ? a.Sk - 1 : pos64);
  const int pos = (int)pos64;
  const int nc = (pos + 1) >> 2;
  const int part = (pos + 1) & 3;
  const int32_t* irow = a.idx + r * a.topk;

  // pool slots to visit: up to the last non-negative id, then the own pool
  int np = 0;
  for (int j0 = 0; j0 < a.topk; j0 += kWave) {
    const int j = j0 + lane;
    const uint64_t M = ballot(j < a.topk && irow[j] >= 0);
    if (M) np = j0 + 64 - __clzll((long long)M);
  }
  const int nps = np + (part > 0 ? 1 : 0);
  const int ntile = (nps + 7) >> 3;

  const int hd = h0 + c16;   // this lane's head
  const bool hv = hd < a.H;
  bf16x8_t QB[4];
  {
    const uint16_t* src = a.q + (r * a.H + hd) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) QB[ks] = hv ? load_bf16x8(src + 32 * ks) : zero_bf16x8();
  }

  f32x4_t acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m2 = NEG_INF, lsum = 0.f;
  uint16_t* vt = lds_v[wave];
  uint16_t* kt = lds_k[wave];

  // Two schedules.  kPrefetch (the kernel has the GPU to itself): the K/V
  // rows of the next tile are in flight while a tile is computed, with two
  // register buffers and the loop unrolled by two; loads past the last tile
  // read the query's own key row (no valid key there), so every step issues
  // its 16 loads.  Otherwise (the kernel shares the CUs with the indexer): one
  // tile's 16 loads at a time, which keeps the wave at 176 registers so that
  // it fits beside an indexer wave on a SIMD and leaves that wave the issue
  // slots.  Slot info is double buffered in LDS.
  struct Buf {
    bf16x8_t KA[kKStaged ? 1 : 2][4];
    u32x4_t KR[kKStaged ? 8 : 1];
    u32x4_t VR[8];
  };
  // slot ids of tile t: lane j (mod 8) reads id 8t + j, clamped into the row
  // so the load is unconditional (ids at or past np are not used)
  auto load_ids = [&](int t) -> int {
    const int ps = 8 * t + (lane & 7);
    const int cps = ps < np ? ps : (np > 0 ? np - 1 : 0);
    return irow[cps];
  };
  // slot info of tile t from its id (lanes < 8), as slot_info computes it
  auto set_info = [&](int t, int id) {
    int2* info = lds_info[wave][kPrefetch ? (t & 1) : 0];
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
  // the 16 K/V row loads of tile t (after its slot info is in LDS)
  auto load_kv = [&](int t, Buf& B) {
    const int2* info = lds_info[wave][kPrefetch ? (t & 1) : 0];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if constexpr (!kKStaged) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int2 in = info[4 * kb + (c16 >> 2)];
        const int off = c16 & 3;
        const int64_t key = off < in.y ? in.x + off : pos;
        const uint16_t* ks_src = a.k + key * kD + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) B.KA[kb][ks] = load_bf16x8(ks_src + 32 * ks);
      }
    }
    // V (and staged K) rows: 16 lanes per 256-byte row (slot j, key offset
    // g), so that the lanes of a quad read one contiguous segment
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int2 in = info[j];
      const int64_t key = g < in.y ? in.x + g : pos;
      if constexpr (kKStaged) B.KR[j] = *reinterpret_cast<const u32x4_t*>(a.k + key * kD + 8 * c16);
      B.VR[j] = *reinterpret_cast<const u32x4_t*>(a.v + key * kD + 8 * c16);
    }
  };
  auto compute = [&](int t, const Buf& B) {
    const int2* info = lds_info[wave][kPrefetch ? (t & 1) : 0];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (kKStaged) *reinterpret_cast<u32x4_t*>(kt + (4 * j + g) * kVStride + 8 * c16) = B.KR[j];
      *reinterpret_cast<u32x4_t*>(vt + (4 * j + g) * kVStride + 8 * c16) = B.VR[j];
    }
    if constexpr (kKStaged) {
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    f32x4_t S[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      S[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint16_t* ksrc = kt + (16 * kb + c16) * kVStride + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if constexpr (kKStaged)
          S[kb] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4_t*>(ksrc + 32 * ks)), QB[ks], S[kb]);
        else
          S[kb] = mfma32(B.KA[kb][ks], QB[ks], S[kb]);
      }
    }

    // lane holds keys 16*kb + 4*g + rr (pool slot 4*kb + g, offset rr) of head c16
    float lg[8];
    float tmax = NEG_INF;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int nv = info[4 * kb + g].y;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float x = rr < nv ? S[kb][rr] * a.scale_log2 : NEG_INF;
        lg[4 * kb + rr] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    // The reference m2 of a head moves only when a logit exceeds it by more
    // than kLazyLog2 (or on its first finite logit), so P <= 2^kLazyLog2 and
    // the rescale of O and the sum, skipped by the whole wave when no head
    // moves, runs a few times per row instead of on most tiles (S = 2^15
    // 2.77 -> 2.62-2.66 ms, S = 2^17 3.52-3.65 -> 3.38-3.51 ms; outputs
    // within one bf16 ulp of the rescale on every new maximum).  The
    // exponentials are bare v_exp_f32: a P below 2^-126 of the reference
    // flushes to zero.
    const bool move = tmax > m2 + kLazyLog2;
    if (ballot(move)) {
      const float mref = move ? tmax : m2;
      const float alpha = mref == m2 ? 1.f : __builtin_amdgcn_exp2f(m2 - mref);  // 0 from -inf
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= alpha;
      m2 = mref;
    }
    const float ms = m2 == NEG_INF ? 0.f : m2;
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = __builtin_amdgcn_exp2f(lg[j] - ms);
      psum += p[j];
    }
    lsum += psum;

    u32x4_t pb;
    pb[0] = pack_bf16x2(p[0], p[1]);
    pb[1] = pack_bf16x2(p[2], p[3]);
    pb[2] = pack_bf16x2(p[4], p[5]);
    pb[3] = pack_bf16x2(p[6], p[7]);
    const bf16x8_t PB = as_bf16x8(pb);

    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // V^T operand: row = dim 16*db + c16, k slot j -> key 4g+j (j<4) or
    // 16+4g+(j-4), read transposed from the [key][dim] tile
    const uint16_t* v0 = vt + 4 * g * kVStride + tr_offset(c16, kVStride);
    const uint16_t* v1 = v0 + 16 * kVStride;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const u32x2_t lo = __builtin_bit_cast(u32x2_t, read_tr(v0 + 16 * db));
      const u32x2_t hi = __builtin_bit_cast(u32x2_t, read_tr(v1 + 16 * db));
      const u32x4_t va = {lo[0], lo[1], hi[0], hi[1]};
      acc[db] = mfma32(as_bf16x8(va), PB, acc[db]);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };

  if constexpr (kPrefetch) {
    // ids are loaded one step before the K/V loads that use them, so no wait
    // for them drains the tile in flight
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
  } else {
    // one tile at a time: its 16 loads are issued together, then waited on
    Buf B;
    for (int t = 0; t < ntile; ++t) {
      if (lane < 8) lds_info[wave][kPrefetch ? (t & 1) : 0][lane] = slot_info(irow, 8 * t + lane, np, nc, part, pos);
      load_kv(t, B);
      __builtin_amdgcn_sched_barrier(0);
      compute(t, B);
    }
  }

  float lt = lsum + __shfl_xor(lsum, 16, kWave);
  lt += __shfl_xor(lt, 32, kWave);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (hv) {
    uint16_t* dst = a.out + (r * a.H + hd) * kD + 4 * g;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      u32x2_t o;
      o[0] = pack_bf16x2(acc[db][0] * inv, acc[db][1] * inv);
      o[1] = pack_bf16x2(acc[db][2] * inv, acc[db][3] * inv);
      *reinterpret_cast<u32x2_t*>(dst + 16 * db) = o;
    }
    if (g == 0) a.lse[r * a.H + hd] = lt > 0.f ? (m2 + log2f(lt)) * kLn2 : NEG_INF;
  }
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& x, hipStream_t s) {
  FwdArgs a;
  a.q = x.q;
  a.k = x.k;
  a.v = x.v;
  a.idx = x.idx;
  a.q_pos = x.q_pos;
  a.q_base = x.q_base;
  a.Sq = x.Sq;
  a.Sk = x.Sk;
  a.H = x.heads;
  a.HG = (x.heads + 15) / 16;
  a.topk = x.topk;
  a.scale_log2 = x.scale * kLog2e;
  a.out = x.out;
  a.lse = x.lse_out;
  const int64_t blocks = (x.Sq * a.HG + kRows - 1) / kRows;
  if (x.fwd_shared && x.fwd_hold)
    attn_fwd_kernel<false, false, true><<<dim3((unsigned)blocks), dim3(kRows * kWave), 0, s>>>(a);
  else if (x.fwd_shared)
    attn_fwd_kernel<false, false, false><<<dim3((unsigned)blocks), dim3(kRows * kWave), 0, s>>>(a);
  else if (x.Sk <= kStagedMaxKeys)
    attn_fwd_kernel<true, true, false><<<dim3((unsigned)blocks), dim3(kRows * kWave), 0, s>>>(a);
  else
    attn_fwd_kernel<true, false, false><<<dim3((unsigned)blocks), dim3(kRows * kWave), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dsa
