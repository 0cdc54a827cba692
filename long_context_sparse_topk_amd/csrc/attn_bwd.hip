// Sparse attention backward (gfx950).
//
// Gradients of sum(dO * O) for the sparse forward.  The pages train through
// this layer ("SkyRL 将 GLM-5.3-Flash 训练上下文扩至 100 万 token", section "2. 激活
// 重算与 Offload" recomputes it in backward); the formulas are those of softmax
// attention:
//   P  = exp(scale * q.k - lse)          (recomputed from the saved LSE)
//   dS = P * (dO.v - Delta),   Delta = sum_d dO * O
//   dq = scale * dS K    (one query row per wave, written directly)
//   dk += scale * dS^T q,  dv += P^T dO   (fp32 atomics into the workspace)
//
// Mapping: one wave per query row, four rows per workgroup, 32 keys per tile.
//   S^T  = K . Q^T,  dP^T = V . dO^T          MFMA 16x16x32, keys as M
//   dQ^T += K^T dS^T                           MFMA 16x16x32, K^T read from LDS
//   dK[key, dim] = dS[key, head] Q[head, dim]  MFMA 16x16x16, heads as k
//   dV[key, dim] = P[key, head] dO[head, dim]  MFMA 16x16x16
// dS and P are transposed through LDS (1 KiB each per tile and wave).
// Kernels: zero the fp32 accumulators, the row kernel, convert to bf16.

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {
namespace {

constexpr int kD = 128;
constexpr int kRows = 4;
constexpr int kKStride = 136;

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
  int H, topk;
  float scale, scale_log2;
  uint16_t* dq;
  float* dk_ws;
  float* dv_ws;
};

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

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) reinterpret_cast<f32x4_t*>(p)[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ a,
                                                      const float* __restrict__ b,
                                                      uint16_t* __restrict__ oa,
                                                      uint16_t* __restrict__ ob, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4_t x = reinterpret_cast<const f32x4_t*>(a)[i];
  const f32x4_t y = reinterpret_cast<const f32x4_t*>(b)[i];
  u32x2_t px, py;
  px[0] = pack_bf16x2(x[0], x[1]);
  px[1] = pack_bf16x2(x[2], x[3]);
  py[0] = pack_bf16x2(y[0], y[1]);
  py[1] = pack_bf16x2(y[2], y[3]);
  reinterpret_cast<u32x2_t*>(oa)[i] = px;
  reinterpret_cast<u32x2_t*>(ob)[i] = py;
}

__global__ __launch_bounds__(256) void attn_bwd_kernel(BwdArgs a) {
  __shared__ __align__(16) uint16_t lds_k[kRows][32 * kKStride];
  __shared__ __align__(16) uint16_t lds_ds[kRows][32 * 16];
  __shared__ __align__(16) uint16_t lds_p[kRows][32 * 16];
  __shared__ int2 lds_info[kRows][8];

  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int64_t r = (int64_t)blockIdx.x * kRows + wave;
  if (r >= a.Sq) return;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const float NEG_INF = -__builtin_huge_valf();

  int64_t pos64 = r;
  if (a.q_pos) {
    pos64 = a.q_pos[r];
    pos64 = pos64 < 0 ? 0 : (pos64 >= a.Sk ? a.Sk - 1 : pos64);
  }
  const int pos = (int)pos64;
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

  // B operands with head c16: Q^T, dO^T; Delta from O
  const bool hv = c16 < a.H;
  bf16x8_t QB[4], DB[4];
  float delta = 0.f;
  {
    const int64_t off = (r * a.H + c16) * kD + 8 * g;
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
  const float lse2 = hv ? a.lse[r * a.H + c16] * kLog2e : 0.f;

  // B operands of the 16x16x16 products: [k = head 4g+j][n = dim 16db+c16]
  s16x4_t QH[8], DH[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    u32x2_t qv, dv;
    uint32_t qe[4], de[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 4 * g + j;
      const int64_t off = (r * a.H + h) * kD + 16 * db + c16;
      qe[j] = h < a.H ? a.q[off] : 0u;
      de[j] = h < a.H ? a.dout[off] : 0u;
    }
    qv[0] = qe[0] | (qe[1] << 16);
    qv[1] = qe[2] | (qe[3] << 16);
    dv[0] = de[0] | (de[1] << 16);
    dv[1] = de[2] | (de[3] << 16);
    QH[db] = as_s16x4(qv);
    DH[db] = as_s16x4(dv);
  }

  f32x4_t dqa[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) dqa[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint16_t* kt = lds_k[wave];
  uint16_t* dst_ds = lds_ds[wave];
  uint16_t* dst_p = lds_p[wave];
  int2* info = lds_info[wave];

  for (int t = 0; t < ntile; ++t) {
    if (lane < 8) info[lane] = slot_info(irow, 8 * t + lane, np, nc, part, pos);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();

    bf16x8_t KA[2][4], VA[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int2 in = info[4 * kb + (c16 >> 2)];
      const int off = c16 & 3;
      const int64_t key = off < in.y ? in.x + off : pos;
      const uint16_t* ksrc = a.k + key * kD + 8 * g;
      const uint16_t* vsrc = a.v + key * kD + 8 * g;
      uint16_t* kdst = kt + (16 * kb + c16) * kKStride + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(ksrc + 32 * ks);
        KA[kb][ks] = as_bf16x8(kv);
        *reinterpret_cast<u32x4_t*>(kdst + 32 * ks) = kv;
        VA[kb][ks] = load_bf16x8(vsrc + 32 * ks);
      }
    }

    float p[8], ds[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s = mfma32(KA[kb][ks], QB[ks], s);
        dp = mfma32(VA[kb][ks], DB[ks], dp);
      }
      const int nv = info[4 * kb + g].y;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float pp = (hv && rr < nv) ? exp2f(s[rr] * a.scale_log2 - lse2) : 0.f;
        p[4 * kb + rr] = pp;
        ds[4 * kb + rr] = pp * (dp[rr] - delta);
      }
    }

    // dS^T and P^T (head c16, keys pi(g, j)) -> LDS as [key][head]
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
      dst_ds[key * 16 + c16] = (uint16_t)f32_to_bf16_bits(ds[j]);
      dst_p[key * 16 + c16] = (uint16_t)f32_to_bf16_bits(p[j]);
    }
    u32x4_t dsb;
    dsb[0] = pack_bf16x2(ds[0], ds[1]);
    dsb[1] = pack_bf16x2(ds[2], ds[3]);
    dsb[2] = pack_bf16x2(ds[4], ds[5]);
    dsb[3] = pack_bf16x2(ds[6], ds[7]);
    const bf16x8_t DSB = as_bf16x8(dsb);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();

    // dQ^T[dim, head] += K^T[dim, key] dS^T[key, head]
    const uint16_t* k0 = kt + (4 * g) * kKStride + c16;
    const uint16_t* k1 = kt + (16 + 4 * g) * kKStride + c16;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      u32x4_t ka;
      ka[0] = (uint32_t)k0[0 * kKStride + 16 * db] | ((uint32_t)k0[1 * kKStride + 16 * db] << 16);
      ka[1] = (uint32_t)k0[2 * kKStride + 16 * db] | ((uint32_t)k0[3 * kKStride + 16 * db] << 16);
      ka[2] = (uint32_t)k1[0 * kKStride + 16 * db] | ((uint32_t)k1[1 * kKStride + 16 * db] << 16);
      ka[3] = (uint32_t)k1[2 * kKStride + 16 * db] | ((uint32_t)k1[3 * kKStride + 16 * db] << 16);
      dqa[db] = mfma32(as_bf16x8(ka), DSB, dqa[db]);
    }

    // dK, dV rows of this tile: D[key 4g+rr][dim 16db+c16] per key block kb
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const s16x4_t Ads = *reinterpret_cast<const s16x4_t*>(dst_ds + (16 * kb + c16) * 16 + 4 * g);
      const s16x4_t Ap = *reinterpret_cast<const s16x4_t*>(dst_p + (16 * kb + c16) * 16 + 4 * g);
      const int2 in = info[4 * kb + g];
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        const f32x4_t dk = mfma16(Ads, QH[db], z);
        const f32x4_t dv = mfma16(Ap, DH[db], z);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          if (rr < in.y) {
            const int64_t off = (int64_t)(in.x + rr) * kD + 16 * db + c16;
            unsafeAtomicAdd(a.dk_ws + off, a.scale * dk[rr]);
            unsafeAtomicAdd(a.dv_ws + off, dv[rr]);
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  if (hv) {
    uint16_t* dst = a.dq + (r * a.H + c16) * kD + 4 * g;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      u32x2_t o;
      o[0] = pack_bf16x2(dqa[db][0] * a.scale, dqa[db][1] * a.scale);
      o[1] = pack_bf16x2(dqa[db][2] * a.scale, dqa[db][3] * a.scale);
      *reinterpret_cast<u32x2_t*>(dst + 16 * db) = o;
    }
  }
}

}  // namespace

hipError_t launch_attn_bwd(const AttnArgs& x, hipStream_t s) {
  char* ws = static_cast<char*>(x.ws);
  float* dk_ws = reinterpret_cast<float*>(ws);
  float* dv_ws = reinterpret_cast<float*>(ws + align256((size_t)x.Sk * kD * 4));
  const int64_t n4 = x.Sk * kD / 4;
  const unsigned eb = (unsigned)((n4 + 255) / 256);
  zero_f32_kernel<<<dim3(eb), dim3(256), 0, s>>>(dk_ws, n4);
  zero_f32_kernel<<<dim3(eb), dim3(256), 0, s>>>(dv_ws, n4);

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
  a.topk = x.topk;
  a.scale = x.scale;
  a.scale_log2 = x.scale * kLog2e;
  a.dq = x.out;
  a.dk_ws = dk_ws;
  a.dv_ws = dv_ws;
  const int64_t blocks = (x.Sq + kRows - 1) / kRows;
  attn_bwd_kernel<<<dim3((unsigned)blocks), dim3(kRows * kWave), 0, s>>>(a);
  to_bf16_kernel<<<dim3(eb), dim3(256), 0, s>>>(dk_ws, dv_ws, x.dk, x.dv, n4);
  return hipGetLastError();
}

}  // namespace dsa
