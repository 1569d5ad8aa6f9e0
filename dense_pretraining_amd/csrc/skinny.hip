// Products with few rows: y = epilogue(x W^T) for the one-row-per-sequence
// activations of a decode step (M = batch, typically <= 64).
//
// At M = 64 a weight matrix is read once and each of its bytes feeds only
// 64 multiply-adds, so the kernel streams W from HBM and the layout choices
// are about keeping enough of it in flight:
//  * block tile: 32 output columns x all (up to 64) rows, 4 waves; the K range
//    of a block is cut into 64-wide steps dealt to the waves in turn, so the
//    four waves read neighbouring 128-byte pieces of the same W rows;
//  * fragments load straight from global memory into the 32x32 MFMA operand
//    layout (W rows as the A operand, x rows as the B operand), next step's
//    fragments in flight while the current step multiplies;
//  * the waves' partial tiles meet in LDS; when K is split over blocks (to
//    reach about one block per CU) each block writes float32 partial sums and
//    a small second kernel adds them in split order (so the result does not
//    depend on timing) and applies the epilogue. A kernel boundary is the
//    cheap way to make the partials visible across the XCDs' separate L2
//    caches: a device-scope release inside the kernel writes back the whole
//    L2 and costs more than the second launch.
//  * a parameter-free RMSNorm of the input rows folds into the epilogue:
//    N(x) W^T = diag(1/rms(x)) (x W^T), with the sums of squares gathered from
//    the x fragments already loaded.
// Epilogues: plain store (+ residual), ReLU^2, or the softcapped logit maximum
// of each row over the tile's columns (ties to the lowest column) for greedy
// decoding; a second small kernel picks the row maximum over the tiles.
#include "common.h"
#include "frag.h"
#include "kernels.h"

namespace nc {
namespace {

constexpr int kSkBN = 32;       // output columns per block
constexpr int kSkKC = 64;       // k per wave step (four 16-wide MFMA steps)
// Blocks aimed for when splitting K. Half the CUs: a decode step at depth 20
// (64 rows) ran 10 % faster than with 256 (W1 no longer splits, so it needs
// no finishing pass; Wo and W2 take 4 splits instead of 7); 64 and 512 were
// slower, 128 to 160 a plateau.
constexpr int kSkTarget = 128;
constexpr int kSkFin = 8;       // partials loaded at once by the finishing kernel

struct SkinnyArgs {
  const void* x;
  long ldx;
  const void* w;  // [N][K], row stride K
  void* y;
  long ldy;
  const void* res;  // optional residual, [M][ldres]
  long ldres;
  float2* cand;  // softcap-argmax epilogue: [M][ntn] (value, column as int bits)
  float* part;   // [nsplit][M][N] partial sums, then [nsplit][M] sums of squares
  int M, N, K, kper, nsplit, ntn;
  int norm;
  float eps, cap;
};

template <typename T> __device__ __forceinline__ float sumsq8(const F8<T>& f);
template <> __device__ __forceinline__ float sumsq8<bf16>(const F8<bf16>& f) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = (float)f.v[i];
    s += v * v;
  }
  return s;
}
template <> __device__ __forceinline__ float sumsq8<float>(const F8<float>& f) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += f.v[i] * f.v[i];
  return s;
}

__device__ __forceinline__ bool better(float a, int ia, float b, int ib) { return b > a || (b == a && ib < ia); }

// Output-tile geometry shared by the product and finishing kernels: thread
// tid of 256 owns row r and CPT consecutive columns from c0 of a BM x 32 tile.
template <int MT>
struct TileMap {
  static constexpr int BM = 32 * MT;
  static constexpr int TPR = 256 / BM;      // threads per row
  static constexpr int CPT = kSkBN / TPR;   // columns per thread
};

// Epilogue of one thread's CPT columns of row m (v = raw sums, ssum = the row's
// sum of squares when a.norm). Whole rows (TPR lanes) take the same path.
template <typename T, int MT, int EPI>
__device__ __forceinline__ void skinny_epilogue(const SkinnyArgs& a, int nt, int m, int n, const float* v, float ssum,
                                                int tid) {
  using Map = TileMap<MT>;
  constexpr int CPT = Map::CPT, TPR = Map::TPR;
  const bool cok = n < a.N;  // N % 8 == 0: a thread's columns are all in or all out
  const float rs = a.norm ? 1.f / sqrtf(ssum / (float)a.K + a.eps) : 1.f;
  if constexpr (EPI == kSkinnyArgmax) {
    float best = -INFINITY;
    int bi = 0x7fffffff;
    if (cok) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const float zc = a.cap * tanhf(v[c] * rs / a.cap);
        if (zc > best) {  // columns rise with c: the first maximum is kept
          best = zc;
          bi = n + c;
        }
      }
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) {
      const float ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(best, bi, ov, oi)) {
        best = ov;
        bi = oi;
      }
    }
    if (tid % TPR == 0) a.cand[(long)m * a.ntn + nt] = make_float2(best, __int_as_float(bi));
  } else {
    if (!cok) return;
    const T* res = static_cast<const T*>(a.res);
    T* y = static_cast<T*>(a.y) + (long)m * a.ldy + n;
#pragma unroll
    for (int c = 0; c < CPT; c += 4) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = v[c + e] * rs;
        if constexpr (EPI == kSkinnyReluSq) {
          const float q = __builtin_amdgcn_fmed3f(o[e], 0.f, 3.402823466e38f);  // max(o, 0), one instruction
          o[e] = q * q;
        }
      }
      if (res) {
        float rr[4];
        load4<T>(res + (long)m * a.ldres + n + c, rr);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] += rr[e];
      }
      store4<T>(y + c, o);
    }
  }
}

template <typename T, int MT, int EPI>
__global__ void __launch_bounds__(256) skinny_kernel(SkinnyArgs a) {
  using Map = TileMap<MT>;
  constexpr int BM = Map::BM, BN = kSkBN, TPR = Map::TPR, CPT = Map::CPT;
  constexpr int LDR = BN + 4;  // LDS row stride (floats)
  __shared__ __align__(16) float red[4][BM * LDR];
  __shared__ float ssr[4][BM];

  const int tid = threadIdx.x, lane = tid & 63, lh = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt = blockIdx.x, mt = blockIdx.y, z = blockIdx.z;
  const int n0 = nt * BN, m0 = mt * BM;
  const int kb = z * a.kper;
  const int ke = min(a.K, kb + a.kper);
  const T* x = static_cast<const T*>(a.x);
  const T* w = static_cast<const T*>(a.w);

  // Rows past N (of W) or M (of x) read the last real row instead: their
  // products land in output rows / columns that are never stored, so the
  // loads need no guard.
  const T* wrow = w + (long)min(n0 + l32, a.N - 1) * a.K + 8 * lh;
  const T* xrow[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) xrow[i] = x + (long)min(m0 + 32 * i + l32, a.M - 1) * a.ldx + 8 * lh;

  f32x16 acc[MT];
  float ss[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    ss[i] = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  }

  struct Fr {
    F8<T> w[4];
    F8<T> x[MT][4];
  };
  auto load = [&](int k, Fr& f) {
#pragma unroll
    for (int s = 0; s < 4; ++s) f.w[s] = ld_row8<T>(wrow + k + 16 * s);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) f.x[i][s] = ld_row8<T>(xrow[i] + k + 16 * s);
  };
  auto use = [&](const Fr& f) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < MT; ++i) mma32(acc[i], f.w[s], f.x[i][s]);
    if (a.norm) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int s = 0; s < 4; ++s) ss[i] += sumsq8<T>(f.x[i][s]);
    }
  };
  // this wave's steps start at k0 and lie 4 * kSkKC apart; the prefetch of
  // the step after the last one repeats the last address (a cache hit), so
  // every iteration issues the same loads and waits only for the older ones
  const int k0 = kb + kSkKC * wave;
  const int nst = k0 < ke ? (ke - k0 + 4 * kSkKC - 1) / (4 * kSkKC) : 0;
  if (nst > 0) {
    Fr cur, nxt;
    load(k0, cur);
    for (int i = 0; i < nst; ++i) {
      load(k0 + 4 * kSkKC * (i + 1 < nst ? i + 1 : i), nxt);
      use(cur);
      cur = nxt;
    }
  }

  // C[n][m] of this wave (lane: m = l32, n = 8j + 4lh + 0..3) -> red[wave][m][n]
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    ss[i] += __shfl_xor(ss[i], 32, 64);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(&red[wave][(32 * i + l32) * LDR + 8 * j + 4 * lh]) =
          make_float4(acc[i][4 * j], acc[i][4 * j + 1], acc[i][4 * j + 2], acc[i][4 * j + 3]);
    if (lh == 0) ssr[wave][32 * i + l32] = ss[i];
  }
  __syncthreads();

  const int r = tid / TPR, c0 = (tid % TPR) * CPT;
  const int m = m0 + r, n = n0 + c0;
  if (m >= a.M) return;  // whole rows (groups of TPR lanes) leave together
  float v[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c)
    v[c] = red[0][r * LDR + c0 + c] + red[1][r * LDR + c0 + c] + red[2][r * LDR + c0 + c] + red[3][r * LDR + c0 + c];
  const float ssum = a.norm ? ssr[0][r] + ssr[1][r] + ssr[2][r] + ssr[3][r] : 0.f;

  if constexpr (EPI != kSkinnyPartial) {
    if (a.nsplit == 1) {
      skinny_epilogue<T, MT, EPI>(a, nt, m, n, v, ssum, tid);
      return;
    }
  }
  // split K: this block's float32 partial sums, added up by skinny_finish_kernel
  if (n < a.N) {
    float* dst = a.part + ((long)z * a.M + m) * a.N + n;
#pragma unroll
    for (int c = 0; c < CPT; c += 4) *reinterpret_cast<float4*>(dst + c) = make_float4(v[c], v[c + 1], v[c + 2], v[c + 3]);
  }
  if (a.norm && tid % TPR == 0) a.part[(long)a.nsplit * a.M * a.N + (long)z * a.M + m] = ssum;
}

// Split-K finish: the partial sums of each output in split order (so the
// result does not depend on timing), then the epilogue. Same tile geometry
// as the product kernel.
template <typename T, int MT, int EPI>
__global__ void __launch_bounds__(256) skinny_finish_kernel(SkinnyArgs a) {
  using Map = TileMap<MT>;
  constexpr int TPR = Map::TPR, CPT = Map::CPT;
  const int tid = threadIdx.x, nt = blockIdx.x;
  const int m = blockIdx.y * Map::BM + tid / TPR, n = nt * kSkBN + (tid % TPR) * CPT;
  if (m >= a.M) return;
  float v[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) v[c] = 0.f;
  // groups of kSkFin splits: their loads are issued together, then added in order
  if (n < a.N)
    for (int z0 = 0; z0 < a.nsplit; z0 += kSkFin) {
      float4 p[kSkFin][CPT / 4];
#pragma unroll
      for (int u = 0; u < kSkFin; ++u)
        if (z0 + u < a.nsplit) {
          const float* src = a.part + ((long)(z0 + u) * a.M + m) * a.N + n;
#pragma unroll
          for (int c = 0; c < CPT / 4; ++c) p[u][c] = *reinterpret_cast<const float4*>(src + 4 * c);
        }
#pragma unroll
      for (int u = 0; u < kSkFin; ++u)
        if (z0 + u < a.nsplit)
#pragma unroll
          for (int c = 0; c < CPT / 4; ++c) {
            v[4 * c] += p[u][c].x;
            v[4 * c + 1] += p[u][c].y;
            v[4 * c + 2] += p[u][c].z;
            v[4 * c + 3] += p[u][c].w;
          }
    }
  float ssum = 0.f;
  if (a.norm) {
    const float* ssp = a.part + (long)a.nsplit * a.M * a.N;
    for (int zz = 0; zz < a.nsplit; ++zz) ssum += ssp[(long)zz * a.M + m];
  }
  skinny_epilogue<T, MT, EPI>(a, nt, m, n, v, ssum, tid);
}

// out[m] = the column of the largest candidate of row m (ties: lowest column).
__global__ void __launch_bounds__(256) argmax_cand_kernel(const float2* __restrict__ cand, int ntn,
                                                          int32_t* __restrict__ out) {
  __shared__ float wv[4];
  __shared__ int wi[4];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int t = tid; t < ntn; t += 256) {
    const float2 c = cand[(long)m * ntn + t];
    if (better(best, bi, c.x, __float_as_int(c.y))) {
      best = c.x;
      bi = __float_as_int(c.y);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better(best, bi, ov, oi)) {
      best = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    wv[wave] = best;
    wi[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(best, bi, wv[w], wi[w])) {
        best = wv[w];
        bi = wi[w];
      }
    out[m] = bi;
  }
}

}  // namespace

SkinnyPlan skinny_plan(int M, int N, int K) {
  SkinnyPlan p;
  p.mt = M <= 32 ? 1 : 2;
  const int bm = 32 * p.mt;
  p.nmt = (M + bm - 1) / bm;
  p.ntn = (N + kSkBN - 1) / kSkBN;
  const long tiles = (long)p.nmt * p.ntn;
  long s = (kSkTarget + tiles - 1) / tiles;
  const long smax = K / (2 * kSkKC);  // at least two 64-wide steps per split
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  p.kper = (int)(((K + s - 1) / s + kSkKC - 1) / kSkKC * kSkKC);
  p.nsplit = (K + p.kper - 1) / p.kper;
  return p;
}

size_t skinny_part_elems(int M, int N, int K) {
  const SkinnyPlan p = skinny_plan(M, N, K);
  return (size_t)p.nsplit * M * ((size_t)N + 1);
}

int skinny_col_tiles(int N) { return (N + kSkBN - 1) / kSkBN; }

template <typename T>
nc_status gemm_skinny(const T* x, long ldx, const T* w, int M, int N, int K, bool norm, float eps, int epi, T* y,
                      long ldy, const T* res, long ldres, float cap, float2* cand, float* part, size_t part_elems,
                      hipStream_t st) {
  if (M < 1 || N < 1 || K < 1) return NC_ERR_SHAPE;
  if (K % kSkKC != 0 || N % 8 != 0 || ldx % 8 != 0) return NC_ERR_UNSUPPORTED;
  if (epi == kSkinnyArgmax ? cand == nullptr
                           : epi != kSkinnyPartial && (y == nullptr || ldy % 8 != 0 || (res && ldres % 8 != 0)))
    return NC_ERR_INVALID_ARG;
  const SkinnyPlan p = skinny_plan(M, N, K);
  if ((p.nsplit > 1 || epi == kSkinnyPartial) && (part == nullptr || part_elems < skinny_part_elems(M, N, K)))
    return NC_ERR_WORKSPACE;
  SkinnyArgs a{x, ldx, w, y, ldy, res, ldres, cand, part, M, N, K, p.kper, p.nsplit, p.ntn, norm ? 1 : 0, eps, cap};
  const double out_bytes = epi == kSkinnyArgmax    ? 8.0 * M * p.ntn
                           : epi == kSkinnyPartial ? 4.0 * p.nsplit * M * (N + 1.0)
                                                   : sizeof(T) * (double)M * N * (res ? 2.0 : 1.0);
  ProfScope prof(NC_NAME(T, "gemm_skinny"), 2.0 * M * N * K, sizeof(T) * ((double)N * K + (double)M * K) + out_bytes,
                 st);
  dim3 grid(p.ntn, p.nmt, p.nsplit);
#define NC_SK(MT, E)                                                                                            \
  do {                                                                                                           \
    hipLaunchKernelGGL((skinny_kernel<T, MT, E>), grid, dim3(256), 0, st, a);                                    \
    if (E != kSkinnyPartial && p.nsplit > 1)                                                                     \
      hipLaunchKernelGGL((skinny_finish_kernel<T, MT, E == kSkinnyPartial ? kSkinnyStore : E>), dim3(p.ntn, p.nmt), \
                         dim3(256), 0, st, a);                                                                   \
  } while (0)
#define NC_SK_EPI(MT)                                     \
  do {                                                    \
    if (epi == kSkinnyStore) NC_SK(MT, kSkinnyStore);     \
    else if (epi == kSkinnyReluSq) NC_SK(MT, kSkinnyReluSq); \
    else if (epi == kSkinnyArgmax) NC_SK(MT, kSkinnyArgmax); \
    else NC_SK(MT, kSkinnyPartial);                       \
  } while (0)
  if (p.mt == 1) NC_SK_EPI(1);
  else NC_SK_EPI(2);
#undef NC_SK_EPI
#undef NC_SK
  NC_LAUNCH_CHECK("gemm_skinny");
  return NC_OK;
}

nc_status argmax_cand(const float2* cand, int M, int ntn, int32_t* out, hipStream_t st) {
  ProfScope prof("argmax_cand", 0, 8.0 * M * ntn + 4.0 * M, st);
  hipLaunchKernelGGL(argmax_cand_kernel, dim3(M), dim3(256), 0, st, cand, ntn, out);
  NC_LAUNCH_CHECK("argmax_cand");
  return NC_OK;
}

#define NC_INST(T)                                                                                                \
  template nc_status gemm_skinny<T>(const T*, long, const T*, int, int, int, bool, float, int, T*, long, const T*, \
                                    long, float, float2*, float*, size_t, hipStream_t);
NC_INST(bf16)
NC_INST(float)
#undef NC_INST

}  // namespace nc
