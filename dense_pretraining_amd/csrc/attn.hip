// Causal multi-query attention on gfx950, forward and backward.
//
// The architecture list on vpshk.cn (Q&A section) gives multi-query attention;
// next-token training (imeisheng.com, section "预训练") makes it causal. Per
// batch row and query head h (KV head g = h*G/H):
//   S = q k^T / sqrt(D), masked to key <= query position, P = softmax(S), o = P v.
//
// MI355X design:
//  * All n_rep = H/G query heads of one KV head are flattened into one row
//    space r = t * n_rep + (h - g*n_rep), t = r / n_rep. A 128-row block then
//    spans ~128/n_rep positions of every head, so one LDS-staged K/V tile is
//    shared by all heads and the causal diagonal is only ~13 positions wide
//    at H = 10 instead of 128.
//  * 32x32x16 bf16 MFMA. The score tile is computed transposed, S^T = K Q^T,
//    so each lane owns one query (lane % 32) and 16 of the 32 keys: the row
//    sum is lane-local, and the probabilities are already laid out as the
//    B operand of O^T += V^T P^T (the keys a lane holds are paired with the
//    matching V^T entries when V^T is read from LDS). No P round trip via LDS.
//  * QK norm bounds every score: |q|, |k| <= sqrt(D) after the per-head
//    RMSNorm, so |s| <= sqrt(D). exp(s - sqrt(D)) lies in [e^{-2 sqrt(D)}, 1],
//    so a fixed shift replaces the running maximum of online softmax.
//  * Backward without atomics: a dQ pass over query blocks (which also forms
//    Delta = rowsum(dO * O)), then a dK/dV pass over key blocks that sums all
//    heads' contributions in registers.
// Float storage (check mode) runs the same code with 32x32x2 f32 MFMAs.
#include "common.h"
#include "kernels.h"

namespace nc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------ fragments
// An operand fragment: 8 consecutive k-slots of one lane.
template <typename T> struct F8;
template <> struct F8<bf16> { bf16x8 v; };
template <> struct F8<float> { float v[8]; };

__device__ __forceinline__ void mma32(f32x16& c, const F8<bf16>& a, const F8<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16& c, const F8<float>& a, const F8<float>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[s], b.v[s], c, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ F8<T> ld_row8(const T* p);
template <> __device__ __forceinline__ F8<bf16> ld_row8<bf16>(const bf16* p) {
  F8<bf16> f; f.v = *reinterpret_cast<const bf16x8*>(p); return f;
}
template <> __device__ __forceinline__ F8<float> ld_row8<float>(const float* p) {
  F8<float> f;
  float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w; f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}
// 4 elements from p0 then 4 from p1.
template <typename T> __device__ __forceinline__ F8<T> ld_split8(const T* p0, const T* p1);
template <> __device__ __forceinline__ F8<bf16> ld_split8<bf16>(const bf16* p0, const bf16* p1) {
  uint2 a = *reinterpret_cast<const uint2*>(p0), b = *reinterpret_cast<const uint2*>(p1);
  uint4 u = make_uint4(a.x, a.y, b.x, b.y);
  F8<bf16> f; f.v = *reinterpret_cast<bf16x8*>(&u); return f;
}
template <> __device__ __forceinline__ F8<float> ld_split8<float>(const float* p0, const float* p1) {
  float4 a = *reinterpret_cast<const float4*>(p0), b = *reinterpret_cast<const float4*>(p1);
  F8<float> f;
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w; f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}
template <typename T> __device__ __forceinline__ F8<T> pack8(const float* v);
template <> __device__ __forceinline__ F8<bf16> pack8<bf16>(const float* v) {
  F8<bf16> f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = (bf16)v[i];
  return f;
}
template <> __device__ __forceinline__ F8<float> pack8<float>(const float* v) {
  F8<float> f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = v[i];
  return f;
}
// Global fragment: 8 consecutive elements (zero if !ok).
template <typename T> __device__ __forceinline__ F8<T> gld8(const T* p, bool ok) {
  if (ok) return ld_row8<T>(p);
  float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  return pack8<T>(z);
}

// Operand fragment X[r][k0a..k0a+3 | k0b..k0b+3] for row r = r0 + lane % 16,
// read from an LDS tile stored k-major (xt[k * LD + r], rows contiguous).
// bf16 uses the gfx950 transposing LDS read: inside each 16-lane group,
// source lane j reads 4 consecutive rows at k-row k0 + j/4 and the hardware
// hands lane i the 4 k values of row r0 + i. Float (check mode) reads the 8
// values one by one.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <typename T> __device__ __forceinline__ F8<T> ld_tr8(const T* xt, int LD, int k0a, int k0b, int r0, int lane);
template <> __device__ __forceinline__ F8<bf16> ld_tr8<bf16>(const bf16* xt, int LD, int k0a, int k0b, int r0,
                                                             int lane) {
  const int j = lane & 15;
  const int c = r0 + 4 * (j & 3);
  v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)const_cast<bf16*>(xt + (k0a + (j >> 2)) * LD + c));
  v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)const_cast<bf16*>(xt + (k0b + (j >> 2)) * LD + c));
  uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  uint4 u = make_uint4(ua.x, ua.y, ub.x, ub.y);
  F8<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, u);
  return f;
}
template <> __device__ __forceinline__ F8<float> ld_tr8<float>(const float* xt, int LD, int k0a, int k0b, int r0,
                                                               int lane) {
  const int r = r0 + (lane & 15);
  F8<float> f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f.v[s] = xt[(k0a + s) * LD + r];
    f.v[4 + s] = xt[(k0b + s) * LD + r];
  }
  return f;
}

// 2^x with the bare hardware instruction. Every argument here lies in
// [-2 sqrt(D) log2(e) - log2(T), 1], far from the range where the library
// exp2f needs its denormal rescaling.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// r / n for 0 <= r < 2^24 without an integer division.
struct DivN {
  int n;
  float inv;
  __device__ __forceinline__ int q(int r) const {
    int x = (int)((float)r * inv);
    x -= (x * n > r) ? 1 : 0;
    x += ((x + 1) * n <= r) ? 1 : 0;
    return x;
  }
};

// ------------------------------------------------------------ tile staging
// Row-major tile [ROWS][D] -> LDS [ROWS][LD]; the row addresses come from a
// function (nullptr = zero row).
template <typename T, int ROWS, int D>
struct RowTile {
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int LD = D + VE;
  static constexpr int N = ROWS * D / VE;
  static constexpr int PER = (N + 255) / 256;
  uint4 r[PER];
  template <typename AddrF>
  __device__ __forceinline__ void load(AddrF addr, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int u = tid + 256 * i;
      r[i] = make_uint4(0, 0, 0, 0);
      if (u < N) {
        int row = u / (D / VE), c = u % (D / VE);
        const T* p = addr(row);
        if (p) r[i] = *reinterpret_cast<const uint4*>(p + c * VE);
      }
    }
  }
  __device__ __forceinline__ void store(T* s, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int u = tid + 256 * i;
      if (u < N) {
        int row = u / (D / VE), c = u % (D / VE);
        *reinterpret_cast<uint4*>(s + row * LD + c * VE) = r[i];
      }
    }
  }
};

// Key index held in accumulator slot v by lane half lh (C layout of a 32x32
// MFMA: rows 8*(v/4) + 4*lh + v%4).
__device__ __forceinline__ int crow(int v, int lh) { return 8 * (v >> 2) + 4 * lh + (v & 3); }

struct AttnGeom {
  int B, T, H, G, D, n_rep;
  long ld_qk, ld_v, ld_o, ld_dq;
  int q_off_k;  // column of K head 0 inside the qk rows (H*D)
  float inv_rep;
};

// ============================================================ forward
template <typename T, int D>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(AttnGeom g, const T* __restrict__ qk,
                                                          const T* __restrict__ vsrc, T* __restrict__ o,
                                                          float* __restrict__ lse) {
  constexpr int BKV = 64;
  using KT = RowTile<T, BKV, D>;
  constexpr int LD = KT::LD;
  __shared__ __align__(16) T ks[2][BKV * LD];
  __shared__ __align__(16) T vs[2][BKV * LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lh = lane >> 5, l32 = lane & 31;
  const int g16 = (lane >> 4) & 1;
  const int nrows = g.T * g.n_rep;
  const int nqb = (nrows + 127) / 128;
  const int per = g.G * g.B;
  const int qb = nqb - 1 - (int)(blockIdx.x / per);  // longest query blocks first
  const int kvh = blockIdx.x % per % g.G, b = blockIdx.x % per / g.G;
  const int R0 = qb * 128;
  const long tok0 = (long)b * g.T;
  const DivN dv{g.n_rep, g.inv_rep};

  const int rq = R0 + 32 * wave + l32;
  const bool qok = rq < nrows;
  const int tq = qok ? dv.q(rq) : 0;
  const int hq = kvh * g.n_rep + (qok ? rq - tq * g.n_rep : 0);
  const int w_last = min(nrows - 1, R0 + 32 * wave + 31);
  const int t_wmax = dv.q(w_last);
  const int t_wmin = dv.q(min(nrows - 1, R0 + 32 * wave));
  const bool wfull = R0 + 32 * wave + 31 < nrows;
  const int t_bmax = dv.q(min(nrows - 1, R0 + 127));
  const int nkt = t_bmax / BKV + 1;

  // Q as the B operand of S^T = K Q^T: lane holds d = 16*s + 8*lh + (0..7) of its query.
  F8<T> qf[D / 16];
  const T* qrow = qk + (tok0 + tq) * g.ld_qk + (long)hq * D;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qf[s] = gld8<T>(qrow + 16 * s + 8 * lh, qok);

  const T* kbase = qk + tok0 * g.ld_qk + g.q_off_k + (long)kvh * D;
  const T* vbase = vsrc + tok0 * g.ld_v + (long)kvh * D;

  KT kl, vl;
  auto kaddr = [&](int kt) {
    return [=](int row) -> const T* {
      int key = kt * BKV + row;
      return key < g.T ? kbase + (long)key * g.ld_qk : nullptr;
    };
  };
  auto vaddr = [&](int kt) {
    return [=](int row) -> const T* {
      int key = kt * BKV + row;
      return key < g.T ? vbase + (long)key * g.ld_v : nullptr;
    };
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  float lsum = 0.f;
  const float c1 = kLog2e / sqrtf((float)D);
  const float m0 = sqrtf((float)D) * kLog2e;  // fixed shift: |s| <= sqrt(D)

  kl.load(kaddr(0), tid);
  vl.load(vaddr(0), tid);
  kl.store(ks[0], tid);
  vl.store(vs[0], tid);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) {
      kl.load(kaddr(kt + 1), tid);
      vl.load(vaddr(kt + 1), tid);
    }
    const T* sk = ks[kt & 1];
    const T* sv = vs[kt & 1];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kb = kt * BKV + 32 * sub;
      if (kb > t_wmax) continue;
      f32x16 sacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        F8<T> kf = ld_row8<T>(sk + (32 * sub + l32) * LD + 16 * s + 8 * lh);
        mma32(sacc, kf, qf[s]);
      }
      float p[16];
      if (wfull && kb + 31 <= t_wmin) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          p[v] = fast_exp2(sacc[v] * c1 - m0);
          lsum += p[v];
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          int key = kb + crow(v, lh);
          float e = fast_exp2(sacc[v] * c1 - m0);
          p[v] = (qok && key <= tq) ? e : 0.f;
          lsum += p[v];
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        F8<T> pf = pack8<T>(p + 8 * kk);
        const int k0 = 32 * sub + 16 * kk + 4 * lh;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          F8<T> vf = ld_tr8<T>(sv, LD, k0, k0 + 8, 32 * dt + 16 * g16, lane);
          mma32(oacc[dt], vf, pf);
        }
      }
    }
    if (more) {
      kl.store(ks[(kt + 1) & 1], tid);
      vl.store(vs[(kt + 1) & 1], tid);
    }
    __syncthreads();
  }

  lsum += __shfl_xor(lsum, 32, 64);
  if (qok) {
    const float inv = 1.f / lsum;
    T* orow = o + (tok0 + tq) * g.ld_o + (long)hq * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        T* dst = orow + 32 * dt + 8 * j + 4 * lh;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = from_f32<T>(oacc[dt][4 * j + i] * inv);
      }
    if (lh == 0) lse[(tok0 + tq) * g.H + hq] = (m0 + log2f(lsum)) / kLog2e;
  }
}

// ============================================================ backward: dQ pass (+ Delta)
template <typename T, int D>
__global__ void __launch_bounds__(256, 2) attn_bwd_dq_kernel(AttnGeom g, const T* __restrict__ qk,
                                                             const T* __restrict__ vsrc, const T* __restrict__ o,
                                                             const T* __restrict__ dO, const float* __restrict__ lse,
                                                             float* __restrict__ delta, T* __restrict__ dq) {
  constexpr int BKV = 64;
  using KT = RowTile<T, BKV, D>;
  constexpr int LD = KT::LD;
  __shared__ __align__(16) T ks[2][BKV * LD];
  __shared__ __align__(16) T vs[2][BKV * LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lh = lane >> 5, l32 = lane & 31;
  const int g16 = (lane >> 4) & 1;
  const int nrows = g.T * g.n_rep;
  const int nqb = (nrows + 127) / 128;
  const int per = g.G * g.B;
  const int qb = nqb - 1 - (int)(blockIdx.x / per);
  const int kvh = blockIdx.x % per % g.G, b = blockIdx.x % per / g.G;
  const int R0 = qb * 128;
  const long tok0 = (long)b * g.T;
  const DivN dv{g.n_rep, g.inv_rep};

  const int rq = R0 + 32 * wave + l32;
  const bool qok = rq < nrows;
  const int tq = qok ? dv.q(rq) : 0;
  const int hq = kvh * g.n_rep + (qok ? rq - tq * g.n_rep : 0);
  const int t_wmax = dv.q(min(nrows - 1, R0 + 32 * wave + 31));
  const int t_wmin = dv.q(min(nrows - 1, R0 + 32 * wave));
  const bool wfull = R0 + 32 * wave + 31 < nrows;
  const int t_bmax = dv.q(min(nrows - 1, R0 + 127));
  const int nkt = t_bmax / BKV + 1;

  const long qi = (tok0 + tq) * g.H + hq;
  F8<T> qf[D / 16], df[D / 16];
  const T* qrow = qk + (tok0 + tq) * g.ld_qk + (long)hq * D;
  const T* drow = dO + (tok0 + tq) * g.ld_o + (long)hq * D;
  const T* orow = o + (tok0 + tq) * g.ld_o + (long)hq * D;
  float dsum = 0.f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = gld8<T>(qrow + 16 * s + 8 * lh, qok);
    df[s] = gld8<T>(drow + 16 * s + 8 * lh, qok);
    F8<T> of = gld8<T>(orow + 16 * s + 8 * lh, qok);
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum += to_f32(df[s].v[e]) * to_f32(of.v[e]);
  }
  dsum += __shfl_xor(dsum, 32, 64);
  const float dlt = dsum;
  if (qok && lh == 0) delta[qi] = dlt;
  const float lse2 = qok ? lse[qi] * kLog2e : 0.f;
  const float c1 = kLog2e / sqrtf((float)D);

  const T* kbase = qk + tok0 * g.ld_qk + g.q_off_k + (long)kvh * D;
  const T* vbase = vsrc + tok0 * g.ld_v + (long)kvh * D;
  KT kl, vl;
  auto kaddr = [&](int kt) {
    return [=](int row) -> const T* {
      int key = kt * BKV + row;
      return key < g.T ? kbase + (long)key * g.ld_qk : nullptr;
    };
  };
  auto vaddr = [&](int kt) {
    return [=](int row) -> const T* {
      int key = kt * BKV + row;
      return key < g.T ? vbase + (long)key * g.ld_v : nullptr;
    };
  };

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) dqacc[i][v] = 0.f;

  kl.load(kaddr(0), tid);
  vl.load(vaddr(0), tid);
  kl.store(ks[0], tid);
  vl.store(vs[0], tid);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) {
      kl.load(kaddr(kt + 1), tid);
      vl.load(vaddr(kt + 1), tid);
    }
    const T* sk = ks[kt & 1];
    const T* sv = vs[kt & 1];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kb = kt * BKV + 32 * sub;
      if (kb > t_wmax) continue;
      f32x16 sacc, pacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) { sacc[v] = 0.f; pacc[v] = 0.f; }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        F8<T> kf = ld_row8<T>(sk + (32 * sub + l32) * LD + 16 * s + 8 * lh);
        mma32(sacc, kf, qf[s]);
        F8<T> vf = ld_row8<T>(sv + (32 * sub + l32) * LD + 16 * s + 8 * lh);
        mma32(pacc, vf, df[s]);
      }
      float ds[16];
      if (wfull && kb + 31 <= t_wmin) {
#pragma unroll
        for (int v = 0; v < 16; ++v) ds[v] = fast_exp2(sacc[v] * c1 - lse2) * (pacc[v] - dlt);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          int key = kb + crow(v, lh);
          float p = fast_exp2(sacc[v] * c1 - lse2);
          ds[v] = (qok && key <= tq) ? p * (pacc[v] - dlt) : 0.f;
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        F8<T> sf = pack8<T>(ds + 8 * kk);
        const int k0 = 32 * sub + 16 * kk + 4 * lh;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          F8<T> kf = ld_tr8<T>(sk, LD, k0, k0 + 8, 32 * dt + 16 * g16, lane);
          mma32(dqacc[dt], kf, sf);
        }
      }
    }
    if (more) {
      kl.store(ks[(kt + 1) & 1], tid);
      vl.store(vs[(kt + 1) & 1], tid);
    }
    __syncthreads();
  }

  if (qok) {
    const float sc = 1.f / sqrtf((float)D);
    T* out = dq + (tok0 + tq) * g.ld_dq + (long)hq * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[32 * dt + 8 * j + 4 * lh + i] = from_f32<T>(dqacc[dt][4 * j + i] * sc);
  }
}

// ============================================================ backward: dK/dV pass
// Block: 128 keys (4 waves x 32). Query rows of all heads sharing the KV head
// stream through LDS in tiles of 32 flattened rows, with each row's position,
// LSE and Delta staged beside them.
template <typename T, int D>
__global__ void __launch_bounds__(256, 1) attn_bwd_dkdv_kernel(AttnGeom g, const T* __restrict__ qk,
                                                               const T* __restrict__ vsrc, const T* __restrict__ dO,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ delta, T* __restrict__ dk,
                                                               T* __restrict__ dv, long ld_dkv) {
  constexpr int BQ = 32;
  using QT = RowTile<T, BQ, D>;
  constexpr int LD = QT::LD;
  __shared__ __align__(16) T qs[2][BQ * LD];
  __shared__ __align__(16) T ds_[2][BQ * LD];
  __shared__ float sl[2][BQ], sd[2][BQ];
  __shared__ int st[2][BQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lh = lane >> 5, l32 = lane & 31;
  const int g16 = (lane >> 4) & 1;
  const int per = g.G * g.B;
  const int kblk = (int)(blockIdx.x / per);  // key block 0 sees every query row: first
  const int kvh = blockIdx.x % per % g.G, b = blockIdx.x % per / g.G;
  const long tok0 = (long)b * g.T;
  const int kb0 = kblk * 128;
  const int key = kb0 + 32 * wave + l32;  // this lane's key
  const bool kok = key < g.T;
  const int kw0 = kb0 + 32 * wave;
  const DivN dvn{g.n_rep, g.inv_rep};

  // own K and V rows as B operands (lane: key, 8 consecutive d)
  F8<T> kf[D / 16], vf[D / 16];
  const T* krow = qk + (tok0 + (kok ? key : 0)) * g.ld_qk + g.q_off_k + (long)kvh * D;
  const T* vrow = vsrc + (tok0 + (kok ? key : 0)) * g.ld_v + (long)kvh * D;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kf[s] = gld8<T>(krow + 16 * s + 8 * lh, kok);
    vf[s] = gld8<T>(vrow + 16 * s + 8 * lh, kok);
  }

  const int nrows = g.T * g.n_rep;
  const int r_start = (kb0 * g.n_rep) / BQ * BQ;
  const int ntiles = r_start < nrows ? (nrows - r_start + BQ - 1) / BQ : 0;
  auto qaddr = [&](int tile) {
    return [=](int row) -> const T* {
      int r = r_start + tile * BQ + row;
      if (r >= nrows) return nullptr;
      int t = dvn.q(r), h = kvh * g.n_rep + (r - t * g.n_rep);
      return qk + (tok0 + t) * g.ld_qk + (long)h * D;
    };
  };
  auto daddr = [&](int tile) {
    return [=](int row) -> const T* {
      int r = r_start + tile * BQ + row;
      if (r >= nrows) return nullptr;
      int t = dvn.q(r), h = kvh * g.n_rep + (r - t * g.n_rep);
      return dO + (tok0 + t) * g.ld_o + (long)h * D;
    };
  };
  // per-row staging of (lse * log2 e, Delta, position) by threads < BQ
  float pl = 0.f, pd = 0.f;
  int pt = -1;
  auto stats_load = [&](int tile) {
    if (tid < BQ) {
      int r = r_start + tile * BQ + tid;
      pl = 0.f;
      pd = 0.f;
      pt = -1;
      if (r < nrows) {
        int t = dvn.q(r), h = kvh * g.n_rep + (r - t * g.n_rep);
        long i = (tok0 + t) * g.H + h;
        pl = lse[i] * kLog2e;
        pd = delta[i];
        pt = t;
      }
    }
  };
  auto stats_store = [&](int buf) {
    if (tid < BQ) {
      sl[buf][tid] = pl;
      sd[buf][tid] = pd;
      st[buf][tid] = pt;
    }
  };

  QT ql, dl;
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) { dkacc[i][v] = 0.f; dvacc[i][v] = 0.f; }
  const float c1 = kLog2e / sqrtf((float)D);

  if (ntiles > 0) {
    ql.load(qaddr(0), tid);
    dl.load(daddr(0), tid);
    stats_load(0);
    ql.store(qs[0], tid);
    dl.store(ds_[0], tid);
    stats_store(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const bool more = it + 1 < ntiles;
    const int buf = it & 1;
    if (more) {
      ql.load(qaddr(it + 1), tid);
      dl.load(daddr(it + 1), tid);
      stats_load(it + 1);
    }
    const int rq0 = r_start + it * BQ;
    const int t_tmax = dvn.q(min(nrows - 1, rq0 + BQ - 1));
    if (t_tmax >= kw0) {
      f32x16 sacc, pacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) { sacc[v] = 0.f; pacc[v] = 0.f; }
      const T* sq = qs[buf];
      const T* sdo = ds_[buf];
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        F8<T> qa = ld_row8<T>(sq + l32 * LD + 16 * s + 8 * lh);
        mma32(sacc, qa, kf[s]);
        F8<T> da = ld_row8<T>(sdo + l32 * LD + 16 * s + 8 * lh);
        mma32(pacc, da, vf[s]);
      }
      // sacc[v] = S[query crow(v,lh)][key l32]
      float p[16], dsv[16];
      const bool full = kok && rq0 + BQ <= nrows && dvn.q(rq0) >= kw0 + 31;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q0 = 8 * j + 4 * lh;
        const float4 l4 = *reinterpret_cast<const float4*>(&sl[buf][q0]);
        const float4 d4 = *reinterpret_cast<const float4*>(&sd[buf][q0]);
        const float la[4] = {l4.x, l4.y, l4.z, l4.w}, da[4] = {d4.x, d4.y, d4.z, d4.w};
        int4 t4 = make_int4(0, 0, 0, 0);
        if (!full) t4 = *reinterpret_cast<const int4*>(&st[buf][q0]);
        const int ta[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = 4 * j + i;
          float pv = fast_exp2(sacc[v] * c1 - la[i]);
          if (!full) pv = (kok && key <= ta[i]) ? pv : 0.f;
          p[v] = pv;
          dsv[v] = pv * (pacc[v] - da[i]);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        F8<T> pf = pack8<T>(p + 8 * kk);
        F8<T> sf = pack8<T>(dsv + 8 * kk);
        const int k0 = 16 * kk + 4 * lh;
#pragma unroll
        for (int dti = 0; dti < D / 32; ++dti) {
          F8<T> da = ld_tr8<T>(sdo, LD, k0, k0 + 8, 32 * dti + 16 * g16, lane);
          mma32(dvacc[dti], da, pf);
          F8<T> qa = ld_tr8<T>(sq, LD, k0, k0 + 8, 32 * dti + 16 * g16, lane);
          mma32(dkacc[dti], qa, sf);
        }
      }
    }
    if (more) {
      ql.store(qs[buf ^ 1], tid);
      dl.store(ds_[buf ^ 1], tid);
      stats_store(buf ^ 1);
    }
    __syncthreads();
  }

  if (kok) {
    const float sc = 1.f / sqrtf((float)D);
    T* ko = dk + (tok0 + key) * ld_dkv + (long)kvh * D;
    T* vo = dv + (tok0 + key) * ld_dkv + (long)kvh * D;
#pragma unroll
    for (int dti = 0; dti < D / 32; ++dti)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        int d = 32 * dti + crow(v, lh);
        ko[d] = from_f32<T>(dkacc[dti][v] * sc);
        vo[d] = from_f32<T>(dvacc[dti][v]);
      }
  }
}

// Unmasked (query, key) pairs of causal attention over all heads and rows.
double causal_pairs(const AttnGeom& g) { return (double)g.B * g.H * g.T * (g.T + 1.0) / 2.0; }

template <typename T, int D>
nc_status attn_fwd_impl(const AttnGeom& g, const T* qk, const T* v, T* o, float* lse, hipStream_t st) {
  int nqb = (g.T * g.n_rep + 127) / 128;
  const double tok = (double)g.B * g.T, es = sizeof(T);
  // S = Q K^T and O = P V: 4 D flops per pair
  ProfScope prof(NC_NAME(T, "attn_fwd"), 4.0 * D * causal_pairs(g),
                 es * tok * D * (2.0 * g.H + 2.0 * g.G) + 4.0 * tok * g.H, st);
  hipLaunchKernelGGL((attn_fwd_kernel<T, D>), dim3(nqb * g.G * g.B), dim3(256), 0, st, g, qk, v, o, lse);
  NC_LAUNCH_CHECK("attn_fwd");
  return NC_OK;
}

template <typename T, int D>
nc_status attn_bwd_impl(const AttnGeom& g, const T* qk, const T* v, const T* o, const T* dO, const float* lse,
                        float* delta, T* dq, T* dk, T* dv, long ld_dkv, hipStream_t st) {
  int nqb = (g.T * g.n_rep + 127) / 128;
  const double tok = (double)g.B * g.T, es = sizeof(T);
  {
    // recompute S, then dP = dO V^T and dQ = dS K: 6 D flops per pair
    ProfScope prof(NC_NAME(T, "attn_bwd_dq"), 6.0 * D * causal_pairs(g),
                   es * tok * D * (4.0 * g.H + 2.0 * g.G) + 8.0 * tok * g.H, st);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D>), dim3(nqb * g.G * g.B), dim3(256), 0, st, g, qk, v, o, dO, lse,
                       delta, dq);
    NC_LAUNCH_CHECK("attn_bwd_dq");
  }
  int nkb = (g.T + 127) / 128;
  // recompute S and dP, then dV = P^T dO and dK = dS^T Q: 8 D flops per pair
  ProfScope prof(NC_NAME(T, "attn_bwd_dkdv"), 8.0 * D * causal_pairs(g),
                 es * tok * D * (2.0 * g.H + 4.0 * g.G) + 8.0 * tok * g.H, st);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D>), dim3(nkb * g.G * g.B), dim3(256), 0, st, g, qk, v, dO, lse,
                     delta, dk, dv, ld_dkv);
  NC_LAUNCH_CHECK("attn_bwd_dkdv");
  return NC_OK;
}

AttnGeom make_geom(const AttnArgs& a) {
  AttnGeom g;
  g.B = a.B; g.T = a.T; g.H = a.H; g.G = a.G; g.D = a.D; g.n_rep = a.H / a.G;
  g.ld_qk = a.ld_qk; g.ld_v = a.ld_v; g.ld_o = a.ld_o; g.ld_dq = a.ld_dq;
  g.q_off_k = a.H * a.D;
  g.inv_rep = 1.0f / (float)g.n_rep;
  return g;
}

}  // namespace

template <typename T>
nc_status attn_fwd(const AttnArgs& a, const T* qk, const T* v, T* o, float* lse, hipStream_t st) {
  AttnGeom g = make_geom(a);
  if (a.D == 128) return attn_fwd_impl<T, 128>(g, qk, v, o, lse, st);
  if (a.D == 64) return attn_fwd_impl<T, 64>(g, qk, v, o, lse, st);
  return NC_ERR_UNSUPPORTED;
}

template <typename T>
nc_status attn_bwd(const AttnArgs& a, const T* qk, const T* v, const T* o, const T* dO, const float* lse,
                   float* delta, T* dq, T* dk, T* dv, long ld_dkv, hipStream_t st) {
  AttnGeom g = make_geom(a);
  if (a.D == 128) return attn_bwd_impl<T, 128>(g, qk, v, o, dO, lse, delta, dq, dk, dv, ld_dkv, st);
  if (a.D == 64) return attn_bwd_impl<T, 64>(g, qk, v, o, dO, lse, delta, dq, dk, dv, ld_dkv, st);
  return NC_ERR_UNSUPPORTED;
}

template nc_status attn_fwd<bf16>(const AttnArgs&, const bf16*, const bf16*, bf16*, float*, hipStream_t);
template nc_status attn_fwd<float>(const AttnArgs&, const float*, const float*, float*, float*, hipStream_t);
template nc_status attn_bwd<bf16>(const AttnArgs&, const bf16*, const bf16*, const bf16*, const bf16*, const float*,
                                  float*, bf16*, bf16*, bf16*, long, hipStream_t);
template nc_status attn_bwd<float>(const AttnArgs&, const float*, const float*, const float*, const float*,
                                   const float*, float*, float*, float*, float*, long, hipStream_t);

}  // namespace nc
