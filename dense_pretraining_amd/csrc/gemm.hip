// GEMM entry points of the block and the unembedding, built on gemm.h.
#include "gemm.h"
#include "kernels.h"

namespace nc {

namespace {
constexpr int kCUs = 256;  // MI355X compute units; one GEMM workgroup fills one

// Number of splits of the reduction (token) axis for a weight gradient, and
// the rows each split covers (a multiple of the tile depth). Every split
// writes a float32 partial tile that is read back once, so the smallest count
// is taken whose workgroups fill the GPU's rounds (the last round at least 90 %
// busy), with at most 16 splits of at least 512 rows.
void dw_split(int M, int N, int K, int bk, int bmn, int& nsplit, int& kper) {
  const long tiles = (long)((N + bmn - 1) / bmn) * ((K + bmn - 1) / bmn);
  int maxs = M / 512;
  maxs = maxs < 1 ? 1 : (maxs > 16 ? 16 : maxs);
  int s = 1;
  for (; s < maxs; ++s) {
    const long blocks = tiles * s;
    const long rounds = (blocks + kCUs - 1) / kCUs;
    if (blocks * 10 >= rounds * kCUs * 9) break;
  }
  kper = ((M + s - 1) / s + bk - 1) / bk * bk;
  nsplit = (M + kper - 1) / kper;
}
}  // namespace

size_t gemm_dw_partial_elems(int M, int N, int K) {
  int ns, kp;
  dw_split(M, N, K, GemmTile<float>::BK, GemmTile<float>::BM, ns, kp);
  int ns2, kp2;
  dw_split(M, N, K, GemmTile<bf16>::BK, GemmTile<bf16>::BM, ns2, kp2);
  int s = ns > ns2 ? ns : ns2;
  return s > 1 ? (size_t)s * N * K : 0;
}

// The epilogues address a 256 x 256 tile through 32-bit byte offsets from its
// origin (the unembedding: its 8 column panels of M rows each), which must
// stay inside one buffer record.
bool tile_span_ok(long row_stride_elems, size_t es) {
  return row_stride_elems >= 0 && 256L * row_stride_elems * (long)es < (long)kDmaRecords;
}

// Builds the store epilogue for y (ld N) with or without the residual and
// hands it to launch.
template <typename T, bool Relu, bool Track, typename Launch>
nc_status with_store_epi(T* y, const T* res, int M, int N, const float* sa, const float* sb, uint32_t* amax,
                         Launch&& launch) {
  if (res) {
    EpiStore<T, Relu, Track, true> e{y, N, res, M, N};
    e.sa = sa;
    e.sb = sb;
    e.amax = amax;
    return launch(e);
  }
  EpiStore<T, Relu, Track, false> e{y, N, nullptr, M, N};
  e.sa = sa;
  e.sb = sb;
  e.amax = amax;
  return launch(e);
}

template <typename T>
nc_status gemm_xwt(const T* x, const T* w, T* y, const T* res, int M, int N, int K, bool relu_sq_out,
                   hipStream_t st) {
  if (!tile_span_ok(N, sizeof(T))) return NC_ERR_UNSUPPORTED;
  GemmShape s{x, w, K, K, M, N, K, K, 1};
  const double es = sizeof(T);
  ProfScope prof(relu_sq_out ? NC_NAME(T, "gemm_fwd_relusq") : NC_NAME(T, "gemm_fwd"), 2.0 * M * N * K,
                 es * ((double)M * K + (double)N * K + (double)M * N * (res ? 2 : 1)), st);
  auto launch = [&](const auto& e) { return launch_gemm<T, kKc, kKc>(s, e, st); };
  if (relu_sq_out) return with_store_epi<T, true, false>(y, res, M, N, nullptr, nullptr, nullptr, launch);
  return with_store_epi<T, false, false>(y, res, M, N, nullptr, nullptr, nullptr, launch);
}

template <typename T>
nc_status gemm_xwt_axpby(const T* x, const T* w, T* y, const T* res, int M, int N, int K, float alpha, float beta,
                         hipStream_t st, int batch, long x_batch, long w_batch, long y_batch) {
  if (!tile_span_ok(N, sizeof(T))) return NC_ERR_UNSUPPORTED;
  GemmShape s{x, w, K, K, M, N, K, K, 1};
  s.batch = batch;
  s.a_batch = x_batch;
  s.b_batch = w_batch;
  const double es = sizeof(T);
  ProfScope prof(NC_NAME(T, "gemm_ns"), 2.0 * M * N * K * batch,
                 es * batch * ((double)M * K + (double)N * K + (double)M * N * (res ? 2 : 1)), st);
  if (!res) {
    EpiAxpby<T, false> e{y, N, nullptr, M, N, alpha, 0.f, y_batch, 0};
    return launch_gemm<T, kKc, kKc>(s, e, st);
  }
  EpiAxpby<T, true> e{y, N, res, M, N, alpha, beta, y_batch, y_batch};
  return launch_gemm<T, kKc, kKc>(s, e, st);
}

nc_status gemm_fp8(const uint8_t* xq, const uint8_t* wq, const float* sx, const float* sw, bf16* y, const bf16* res,
                   int M, int N, int K, bool relu_sq_out, uint32_t* amax_out, hipStream_t st) {
  if (K % 16 != 0 || !sx || !sw || !tile_span_ok(N, sizeof(bf16))) return NC_ERR_UNSUPPORTED;
  // the FP8 matrices seen as rows of K / 2 sixteen-bit pairs
  const int K2 = K / 2;
  GemmShape s{xq, wq, K2, K2, M, N, K2, K2, 1};
  ProfScope prof(relu_sq_out ? "gemm_fwd_relusq_fp8" : "gemm_fwd_fp8", 2.0 * M * N * K,
                 (double)M * K + (double)N * K + 2.0 * M * N * (res ? 2 : 1), st);
  // the ReLU^2 output is the next product's FP8 operand: its maximum is taken here
  auto launch = [&](const auto& e) { return launch_gemm_f8(s, e, st); };
  if (amax_out) {
    if (!relu_sq_out || res) return NC_ERR_UNSUPPORTED;
    EpiStore<bf16, true, true> e{y, N, nullptr, M, N};
    e.sa = sx;
    e.sb = sw;
    e.amax = amax_out;
    return launch(e);
  }
  if (relu_sq_out) return with_store_epi<bf16, true, false>(y, res, M, N, sx, sw, nullptr, launch);
  return with_store_epi<bf16, false, false>(y, res, M, N, sx, sw, nullptr, launch);
}

template <typename T>
nc_status gemm_gram(const T* x, T* a, int R, int C, hipStream_t st, int batch, long x_batch, long a_batch) {
  if (!tile_span_ok(C, sizeof(T))) return NC_ERR_UNSUPPORTED;
  // a[C,C] = x^T x for x [R,C]: both operands K-outer, the reduction over the R rows.
  GemmShape s{x, x, C, C, C, C, R, R, 1};
  s.batch = batch;
  s.a_batch = x_batch;
  s.b_batch = x_batch;
  const double es = sizeof(T);
  ProfScope prof(NC_NAME(T, "gemm_gram"), 2.0 * R * C * C * batch, es * batch * ((double)R * C + (double)C * C), st);
  EpiAxpby<T, false> e{a, C, nullptr, C, C, 1.f, 0.f, a_batch, 0};
  return launch_gemm<T, kKo, kKo>(s, e, st);
}

template <typename T>
nc_status gemm_dyw(const T* dy, const T* w, T* dx, const T* act, int M, int N, int K, hipStream_t st,
                   long dy_panel) {
  if (!tile_span_ok(K, sizeof(T))) return NC_ERR_UNSUPPORTED;
  // C[M,K] = A[M,N] * B where B(n=k_out, k=n_in) = W[n_in][k_out]: K-outer.
  GemmShape s{dy, w, N, K, M, K, N, N, 1};
  s.a_panel = dy_panel;
  const double es = sizeof(T);
  ProfScope prof(act ? NC_NAME(T, "gemm_dx_drelusq") : NC_NAME(T, "gemm_dx"), 2.0 * M * N * K,
                 es * ((double)M * N + (double)N * K + (double)M * K * (act ? 2 : 1)), st);
  if (act) {
    EpiDReluSq<T> e{dx, K, act, M, K};
    return launch_gemm<T, kKc, kKo>(s, e, st);
  }
  EpiStore<T> e{dx, K, nullptr, M, K};
  return launch_gemm<T, kKc, kKo>(s, e, st);
}

template <typename T>
nc_status gemm_dyw_scaled(const T* dy, const T* w, T* dx, const float* q, int M, int N, int K, hipStream_t st,
                          long dy_panel) {
  if (!tile_span_ok(K, sizeof(T)) || !q) return NC_ERR_UNSUPPORTED;
  GemmShape s{dy, w, N, K, M, K, N, N, 1};
  s.a_panel = dy_panel;
  const double es = sizeof(T);
  ProfScope prof(NC_NAME(T, "gemm_dx"), 2.0 * M * N * K, es * ((double)M * N + (double)N * K + (double)M * K) + 4.0 * M,
                 st);
  EpiRowScale<T> e{dx, K, q, M, K};
  return launch_gemm<T, kKc, kKo>(s, e, st);
}

template <typename T>
nc_status gemm_dw(const T* dy, const T* x, float* dw, int M, int N, int K, int accumulate, float* partial,
                  size_t partial_elems, hipStream_t st, long dy_panel) {
  if (!tile_span_ok(K, sizeof(float))) return NC_ERR_UNSUPPORTED;
  int nsplit, kper;
  dw_split(M, N, K, GemmTile<T>::BK, GemmTile<T>::BM, nsplit, kper);
  // C[N,K] = sum_m dy[m][n] x[m][k]: both operands K-outer (token axis is the reduction).
  GemmShape s{dy, x, N, K, N, K, M, kper, nsplit};
  s.a_panel = dy_panel;
  if (nsplit > 1 && (partial == nullptr || partial_elems < (size_t)nsplit * N * K)) return NC_ERR_WORKSPACE;
  EpiF32 e;
  e.ldc = K;
  e.M = N;
  e.N = K;
  if (nsplit > 1) {
    e.C = partial;
    e.split_stride = (long)N * K;
    e.accumulate = 0;
  } else {
    e.C = dw;
    e.split_stride = 0;
    e.accumulate = accumulate;
  }
  nc_status r;
  {
    const double es = sizeof(T);
    ProfScope prof(NC_NAME(T, "gemm_dw"), 2.0 * M * N * K,
                   es * ((double)M * N + (double)M * K) + 4.0 * N * K * (accumulate ? 2 : 1), st);
    r = launch_gemm<T, kKo, kKo>(s, e, st);
  }
  if (r != NC_OK || nsplit == 1) return r;
  return splitk_reduce(partial, nsplit, (size_t)N * K, dw, accumulate, st);
}

int lmhead_tiles(int N, bool bf16_storage) {
  const int bn = bf16_storage ? GemmTile<bf16>::BN : GemmTile<float>::BN;
  return (N + bn - 1) / bn;
}

template <typename T>
nc_status gemm_lmhead(const T* x, const T* w, T* z, int M, int N, int K, float cap, float* part, hipStream_t st,
                      bool grad) {
  // a tile's 8 column panels of M * kPanel elements are addressed with 32-bit
  // offsets, the panel stride through a 24-bit multiply
  if (!tile_span_ok(M, sizeof(T)) || (long)M * kPanel * 8 * (long)sizeof(T) >= (long)kDmaRecords ||
      (long)M * kPanel >= (1L << 24))
    return NC_ERR_UNSUPPORTED;
  GemmShape s{x, w, K, K, M, N, K, K, 1};
  ProfScope prof(NC_NAME(T, "gemm_lmhead_softcap"), 2.0 * M * N * K,
                 sizeof(T) * ((double)M * K + (double)N * K + (double)M * N) + 4.0 * M * lmhead_tiles(N, is_bf16<T>()),
                 st);
  const float k2 = (float)(2.8853900817779268 / cap);
  if (grad) {
    EpiSoftcap<T, GemmTile<T>::BM, GemmTile<T>::BN, true> e{z, M * kPanel, cap, k2, part, lmhead_tiles(N, is_bf16<T>()),
                                                         M, N};
    e.kc = (float)(-2.0 * cap * 1.4426950408889634);
    return launch_gemm<T, kKc, kKc>(s, e, st);
  }
  EpiSoftcap<T, GemmTile<T>::BM, GemmTile<T>::BN> e{z, M * kPanel, cap, k2, part, lmhead_tiles(N, is_bf16<T>()), M, N};
  return launch_gemm<T, kKc, kKc>(s, e, st);
}

#define NC_INST(T)                                                                                            \
  template nc_status gemm_xwt<T>(const T*, const T*, T*, const T*, int, int, int, bool, hipStream_t);        \
  template nc_status gemm_xwt_axpby<T>(const T*, const T*, T*, const T*, int, int, int, float, float,          \
                                       hipStream_t, int, long, long, long);                                   \
  template nc_status gemm_gram<T>(const T*, T*, int, int, hipStream_t, int, long, long);                       \
  template nc_status gemm_dyw<T>(const T*, const T*, T*, const T*, int, int, int, hipStream_t, long);         \
  template nc_status gemm_dw<T>(const T*, const T*, float*, int, int, int, int, float*, size_t, hipStream_t,  \
                                long);                                                                        \
  template nc_status gemm_dyw_scaled<T>(const T*, const T*, T*, const float*, int, int, int, hipStream_t, long); \
  template nc_status gemm_lmhead<T>(const T*, const T*, T*, int, int, int, float, float*, hipStream_t, bool);
NC_INST(bf16)
NC_INST(float)
#undef NC_INST

}  // namespace nc
