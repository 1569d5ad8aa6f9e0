// The optimizer step: AdamW for the embedding and the unembedding, Muon for
// every block matrix (the page on vpshk.cn, Q&A "卡帕西亲自揭秘背后技术",
// names Muon + AdamW; imeisheng.com, section "预训练", assigns Muon to the
// matrices and AdamW to the embedding and unembedding). Muon follows its
// published definition (K. Jordan, 2024): Nesterov momentum, then five steps
// of the quintic Newton-Schulz map X <- a X + b (X X^T) X + c (X X^T)^2 X on
// the update scaled to unit Frobenius norm, written for the wide orientation
// (a matrix with more rows than columns is transposed first) so that the
// Gram matrix is the small side squared. Here every matrix is handled in its
// tall orientation instead (a wide one is transposed on the way in and out),
// where the same map reads
//   A = X^T X,  B = b A + c A^2,  X <- a X + X B     (B is symmetric).
//
// HBM layout of the caller's optimizer state (float32, parameter layout of
// nc_param_layout): master weights [n_params]; s1 [n_params] holding AdamW's
// first moment in the embedding and unembedding ranges and Muon's momentum in
// the block matrices; s2 [2 V d] holding AdamW's second moment of the
// embedding then of the unembedding.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace nc {
namespace {

constexpr int kNormParts = 256;  // blocks per matrix of the momentum pass (partial sums of squares)
constexpr int kTile = 32;         // transposing tile of the layout kernels

template <typename T>
__global__ void __launch_bounds__(256) opt_init_kernel(const T* __restrict__ p, float* __restrict__ master,
                                                       float* __restrict__ s1, long n, float* __restrict__ s2,
                                                       long n2) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    master[i] = to_f32(p[i]);
    s1[i] = 0.f;
  }
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n2; i += (long)gridDim.x * 256) s2[i] = 0.f;
}

// AdamW on n4 groups of 4: m, v updated in place, w <- w (1 - lr wd) - lr m_hat / (sqrt(v_hat) + eps),
// p = w in the storage type. c1, c2 = 1 / (1 - beta^t).
// The optimizer's results (master weights, moments, stored parameters) are
// read again only at the next step: stored non-temporal.
typedef float opt_v4f __attribute__((ext_vector_type(4)));
typedef unsigned opt_v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_f4_stream(float* p, float a, float b, float c, float d) {
  const opt_v4f v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<opt_v4f*>(p));
}
template <typename T>
__device__ __forceinline__ void store4_stream(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 o;
    o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
    __builtin_nontemporal_store(__builtin_bit_cast(opt_v2u, o), reinterpret_cast<opt_v2u*>(p));
  } else {
    store_f4_stream(p, v[0], v[1], v[2], v[3]);
  }
}

template <typename T>
__global__ void __launch_bounds__(256) adamw_kernel(const float* __restrict__ g, float* __restrict__ w,
                                                    float* __restrict__ m, float* __restrict__ v, T* __restrict__ p,
                                                    long n4, float lr, float b1, float b2, float c1, float c2,
                                                    float eps, float decay) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    const float4 gg = reinterpret_cast<const float4*>(g)[i];
    float4 ww = reinterpret_cast<float4*>(w)[i], mm = reinterpret_cast<float4*>(m)[i],
           vv = reinterpret_cast<float4*>(v)[i];
    float ga[4] = {gg.x, gg.y, gg.z, gg.w}, wa[4] = {ww.x, ww.y, ww.z, ww.w}, ma[4] = {mm.x, mm.y, mm.z, mm.w},
          va[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ma[e] = b1 * ma[e] + (1.f - b1) * ga[e];
      va[e] = b2 * va[e] + (1.f - b2) * ga[e] * ga[e];
      wa[e] = wa[e] * decay - lr * (ma[e] * c1) / (sqrtf(va[e] * c2) + eps);
    }
    store_f4_stream(w + 4 * i, wa[0], wa[1], wa[2], wa[3]);
    store_f4_stream(m + 4 * i, ma[0], ma[1], ma[2], ma[3]);
    store_f4_stream(v + 4 * i, va[0], va[1], va[2], va[3]);
    store4_stream<T>(p + 4 * i, wa);
  }
}

// Momentum pass: mom <- mu mom + g; the update U = g + mu mom (Nesterov) or mom;
// part[block] = sum of U^2 over the block's elements (grid of kNormParts blocks).
// Matrix blockIdx.y of a batch lies ls elements after the previous one.
__global__ void __launch_bounds__(256) muon_mom_kernel(const float* __restrict__ g, float* __restrict__ mom, long n4,
                                                       long ls, float mu, int nesterov, float* __restrict__ part) {
  __shared__ float red[4];
  g += blockIdx.y * ls;
  mom += blockIdx.y * ls;
  part += blockIdx.y * kNormParts;
  float acc = 0.f;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    const float4 gg = reinterpret_cast<const float4*>(g)[i];
    float4 mm = reinterpret_cast<float4*>(mom)[i];
    mm.x = mu * mm.x + gg.x;
    mm.y = mu * mm.y + gg.y;
    mm.z = mu * mm.z + gg.z;
    mm.w = mu * mm.w + gg.w;
    reinterpret_cast<float4*>(mom)[i] = mm;
    const float u0 = nesterov ? gg.x + mu * mm.x : mm.x, u1 = nesterov ? gg.y + mu * mm.y : mm.y;
    const float u2 = nesterov ? gg.z + mu * mm.z : mm.z, u3 = nesterov ? gg.w + mu * mm.w : mm.w;
    acc += u0 * u0 + u1 * u1 + u2 * u2 + u3 * u3;
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// 1 / (|U|_F + 1e-7) from the momentum pass's partial sums, in a fixed order.
__device__ __forceinline__ float inv_frobenius(const float* part, float* sh) {
  float s = 0.f;
  for (int i = threadIdx.x; i < kNormParts; i += 256) s += part[i];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  return 1.f / (sqrtf(sh[0] + sh[1] + sh[2] + sh[3]) + 1e-7f);
}

// X = U / |U|_F, U [R][C] recomputed from g and the new momentum, when X keeps
// U's layout (a tall or square matrix): groups of 4 elements, two per thread
// and trip, 256 groups apart (each load instruction of a wave stays contiguous).
// Matrix blockIdx.y of a batch: g, mom at + y ls, its X at + y xs.
template <typename T>
__global__ void __launch_bounds__(256) muon_norm_flat_kernel(const float* __restrict__ g,
                                                             const float* __restrict__ mom, long ls, long n4, float mu,
                                                             int nesterov, const float* __restrict__ part,
                                                             T* __restrict__ X, long xs) {
  __shared__ float sh[4];
  g += blockIdx.y * ls;
  mom += blockIdx.y * ls;
  X += blockIdx.y * xs;
  const float inv = inv_frobenius(part + blockIdx.y * kNormParts, sh);
  for (long i0 = (long)blockIdx.x * 512 + threadIdx.x; i0 < n4; i0 += (long)gridDim.x * 512) {
    float4 gs[2], ms[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const long i = i0 + 256 * u < n4 ? i0 + 256 * u : i0;
      gs[u] = reinterpret_cast<const float4*>(g)[i];
      ms[u] = reinterpret_cast<const float4*>(mom)[i];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const long i = i0 + 256 * u;
      if (i >= n4) break;
      const float gv[4] = {gs[u].x, gs[u].y, gs[u].z, gs[u].w}, mv[4] = {ms[u].x, ms[u].y, ms[u].z, ms[u].w};
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (nesterov ? gv[e] + mu * mv[e] : mv[e]) * inv;
      store4<T>(X + 4 * i, v);
    }
  }
}

// The same for a wide matrix, whose X is the transpose: X[c][r] = U[r][c] / |U|_F,
// through a 32 x 32 LDS tile, 4 elements per access (R % 4 == C % 4 == 0).
// Matrix blockIdx.z of a batch.
template <typename T>
__global__ void __launch_bounds__(256) muon_norm_tr_kernel(const float* __restrict__ g, const float* __restrict__ mom,
                                                           long ls, int R, int C, float mu, int nesterov,
                                                           const float* __restrict__ part, T* __restrict__ X,
                                                           long xs) {
  __shared__ float sh[4];
  __shared__ float tile[kTile][kTile + 1];
  g += blockIdx.z * ls;
  mom += blockIdx.z * ls;
  X += blockIdx.z * xs;
  const float inv = inv_frobenius(part + blockIdx.z * kNormParts, sh);
  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  const int ty = threadIdx.x >> 3, tx = threadIdx.x & 7;  // 32 rows x 8 groups of 4 columns
  {
    const int r = r0 + ty, c = c0 + 4 * tx;
    float u[4] = {0.f, 0.f, 0.f, 0.f};
    if (r < R && c < C) {
      const long i = (long)r * C + c;
      const float4 gg = *reinterpret_cast<const float4*>(g + i), mm = *reinterpret_cast<const float4*>(mom + i);
      const float gv[4] = {gg.x, gg.y, gg.z, gg.w}, mv[4] = {mm.x, mm.y, mm.z, mm.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = nesterov ? gv[e] + mu * mv[e] : mv[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[ty][4 * tx + e] = u[e] * inv;
  }
  __syncthreads();
  {  // X [C][R]: row c0 + ty, columns r0 + 4 tx .. + 3
    const int c = c0 + ty, r = r0 + 4 * tx;
    if (r < R && c < C) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = tile[4 * tx + e][ty];
      store4<T>(X + (long)c * R + r, v);
    }
  }
}

// w <- w decay - step X, p = w in the storage type, when X keeps w's layout:
// groups of 4, two per thread and trip, 256 groups apart.
template <typename T>
__global__ void __launch_bounds__(256) muon_apply_flat_kernel(float* __restrict__ w, T* __restrict__ p, long ls,
                                                              const T* __restrict__ X, long xs, long n4, float decay,
                                                              float step) {
  w += blockIdx.y * ls;
  p += blockIdx.y * ls;
  X += blockIdx.y * xs;
  for (long i0 = (long)blockIdx.x * 512 + threadIdx.x; i0 < n4; i0 += (long)gridDim.x * 512) {
    float4 ws[2];
    float x[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const long i = i0 + 256 * u < n4 ? i0 + 256 * u : i0;
      ws[u] = reinterpret_cast<const float4*>(w)[i];
      load4<T>(X + 4 * i, x[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const long i = i0 + 256 * u;
      if (i >= n4) break;
      float nw[4] = {ws[u].x, ws[u].y, ws[u].z, ws[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) nw[e] = nw[e] * decay - step * x[u][e];
      store_f4_stream(w + 4 * i, nw[0], nw[1], nw[2], nw[3]);
      store4_stream<T>(p + 4 * i, nw);
    }
  }
}

// The same for a wide matrix: X [C][R] read transposed through a 32 x 32 tile.
template <typename T>
__global__ void __launch_bounds__(256) muon_apply_tr_kernel(float* __restrict__ w, T* __restrict__ p, long ls,
                                                            const T* __restrict__ X, long xs, int R, int C,
                                                            float decay, float step) {
  __shared__ float tile[kTile][kTile + 1];
  w += blockIdx.z * ls;
  p += blockIdx.z * ls;
  X += blockIdx.z * xs;
  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  const int ty = threadIdx.x >> 3, tx = threadIdx.x & 7;
  {  // X row c0 + ty, columns r0 + 4 tx .. + 3
    const int c = c0 + ty, r = r0 + 4 * tx;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (r < R && c < C) load4<T>(X + (long)c * R + r, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[4 * tx + e][ty] = v[e];
  }
  __syncthreads();
  const int r = r0 + ty, c = c0 + 4 * tx;
  if (r >= R || c >= C) return;
  const long i = (long)r * C + c;
  const float4 ww = *reinterpret_cast<const float4*>(w + i);
  float nw[4] = {ww.x, ww.y, ww.z, ww.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) nw[e] = nw[e] * decay - step * tile[ty][4 * tx + e];
  store_f4_stream(w + i, nw[0], nw[1], nw[2], nw[3]);
  store4_stream<T>(p + i, nw);
}

unsigned grid_of(long n, long per_block, unsigned cap) {
  const long b = (n + per_block - 1) / per_block;
  return (unsigned)(b < 1 ? 1 : (b > cap ? cap : b));
}

}  // namespace

template <typename T>
nc_status opt_init(const T* params, float* master, float* s1, size_t n, float* s2, size_t n2, hipStream_t st) {
  ProfScope prof("opt_init", 0, (double)n * (sizeof(T) + 8.0) + 4.0 * n2, st);
  hipLaunchKernelGGL((opt_init_kernel<T>), dim3(grid_of((long)n, 256, 8192)), dim3(256), 0, st, params, master, s1,
                     (long)n, s2, (long)n2);
  NC_LAUNCH_CHECK("opt_init");
  return NC_OK;
}

template <typename T>
nc_status adamw_step(const float* g, float* w, float* m, float* v, T* p, size_t n, float lr, float beta1,
                     float beta2, float eps, float wd, int step, hipStream_t st) {
  if (n % 4 != 0) return NC_ERR_UNSUPPORTED;
  const float c1 = (float)(1.0 / (1.0 - std::pow((double)beta1, (double)step)));
  const float c2 = (float)(1.0 / (1.0 - std::pow((double)beta2, (double)step)));
  ProfScope prof("adamw", 0, (double)n * (16.0 + 12.0 + sizeof(T)), st);
  hipLaunchKernelGGL((adamw_kernel<T>), dim3(grid_of((long)n / 4, 256, 8192)), dim3(256), 0, st, g, w, m, v, p,
                     (long)n / 4, lr, beta1, beta2, c1, c2, eps, 1.f - lr * wd);
  NC_LAUNCH_CHECK("adamw");
  return NC_OK;
}

size_t muon_work_bytes(int R, int C, int L, bool bf16_storage) {
  const size_t Rt = R > C ? R : C, Ct = R > C ? C : R;
  const size_t es = bf16_storage ? 2 : 4;
  return align_up(2 * L * Rt * Ct * es, 256) + align_up(2 * L * Ct * Ct * es, 256) + align_up(4 * (size_t)L * kNormParts, 256);
}

template <typename T>
nc_status muon_step(const MuonKind<T>* kinds, int nk, int L, long ls, float lr, float mu, int nesterov, float wd,
                    void* work, size_t work_bytes, hipStream_t st) {
  if (nk < 1 || L < 1 || L > 65535 || (long)nk * L > 65535 || ls % 8 != 0) return NC_ERR_UNSUPPORTED;
  // 16-byte accesses: R % 4 == C % 4 == 0, and every matrix of the batch starts 32-byte aligned
  auto al = [](const void* v) { return reinterpret_cast<uintptr_t>(v) % 32 == 0; };
  const int Rt = kinds[0].R > kinds[0].C ? kinds[0].R : kinds[0].C;  // the tall form
  const int Ct = kinds[0].R > kinds[0].C ? kinds[0].C : kinds[0].R;
  for (int k = 0; k < nk; ++k) {
    const MuonKind<T>& x = kinds[k];
    if (x.R % 4 != 0 || x.C % 4 != 0 || !al(x.g) || !al(x.mom) || !al(x.w) ||
        reinterpret_cast<uintptr_t>(x.p) % 16 != 0)
      return NC_ERR_UNSUPPORTED;
    if ((x.R > x.C ? x.R : x.C) != Rt || (x.R > x.C ? x.C : x.R) != Ct) return NC_ERR_UNSUPPORTED;
  }
  const int NL = nk * L;
  if (work_bytes < muon_work_bytes(Rt, Ct, NL, is_bf16<T>())) return NC_ERR_WORKSPACE;
  const long xs = (long)Rt * Ct, as = (long)Ct * Ct;
  const size_t es = sizeof(T);
  char* q = static_cast<char*>(work);
  T* xa = reinterpret_cast<T*>(q);
  T* xb = xa + NL * xs;
  q += align_up(2 * NL * (size_t)xs * es, 256);
  T* Ab = reinterpret_cast<T*>(q);
  T* Bb = Ab + NL * as;
  q += align_up(2 * NL * (size_t)as * es, 256);
  float* norm_part = reinterpret_cast<float*>(q);

  // kind k's matrices are batch entries k L .. k L + L - 1
  const long n4 = (long)Rt * Ct / 4;
  for (int k = 0; k < nk; ++k) {
    const MuonKind<T>& x = kinds[k];
    float* part = norm_part + (size_t)k * L * kNormParts;
    {
      ProfScope prof("muon_momentum", 0, 12.0 * 4 * n4 * L, st);
      hipLaunchKernelGGL(muon_mom_kernel, dim3(kNormParts, L), dim3(256), 0, st, x.g, x.mom, n4, ls, mu, nesterov,
                         part);
      NC_LAUNCH_CHECK("muon_momentum");
    }
    const dim3 tiles((x.C + kTile - 1) / kTile, (x.R + kTile - 1) / kTile, L);
    const dim3 flat(grid_of(n4, 512, 4096), L);
    ProfScope prof("muon_normalize", 0, (8.0 + es) * 4 * n4 * L, st);
    if (x.R < x.C)
      hipLaunchKernelGGL((muon_norm_tr_kernel<T>), tiles, dim3(256), 0, st, x.g, x.mom, ls, x.R, x.C, mu, nesterov,
                         part, xa + (long)k * L * xs, xs);
    else
      hipLaunchKernelGGL((muon_norm_flat_kernel<T>), flat, dim3(256), 0, st, x.g, x.mom, ls, n4, mu, nesterov, part,
                         xa + (long)k * L * xs, xs);
    NC_LAUNCH_CHECK("muon_normalize");
  }
  // the published coefficients (a, b, c) of the quintic map, five steps, every matrix of every kind at once
  const float a = 3.4445f, b = -4.7750f, c = 2.0315f;
  T* x = xa;
  T* xn = xb;
  for (int it = 0; it < 5; ++it) {
    NC_TRY(gemm_gram<T>(x, Ab, Rt, Ct, st, NL, xs, as));                           // A = X^T X
    NC_TRY(gemm_xwt_axpby<T>(Ab, Ab, Bb, Ab, Ct, Ct, Ct, c, b, st, NL, as, as, as));  // B = c A A^T + b A
    NC_TRY(gemm_xwt_axpby<T>(x, Bb, xn, x, Rt, Ct, Ct, 1.f, a, st, NL, xs, as, xs));  // X' = X B^T + a X
    T* t = x;
    x = xn;
    xn = t;
  }
  for (int k = 0; k < nk; ++k) {
    const MuonKind<T>& m = kinds[k];
    const float scale = m.R > m.C ? std::sqrt((float)m.R / (float)m.C) : 1.f;
    const dim3 tiles((m.C + kTile - 1) / kTile, (m.R + kTile - 1) / kTile, L);
    const dim3 flat(grid_of(n4, 512, 4096), L);
    ProfScope prof("muon_apply", 0, (8.0 + 2.0 * es) * 4 * n4 * L, st);
    if (m.R < m.C)
      hipLaunchKernelGGL((muon_apply_tr_kernel<T>), tiles, dim3(256), 0, st, m.w, m.p, ls, x + (long)k * L * xs, xs,
                         m.R, m.C, 1.f - lr * wd, lr * scale);
    else
      hipLaunchKernelGGL((muon_apply_flat_kernel<T>), flat, dim3(256), 0, st, m.w, m.p, ls, x + (long)k * L * xs, xs,
                         n4, 1.f - lr * wd, lr * scale);
    NC_LAUNCH_CHECK("muon_apply");
  }
  return NC_OK;
}

#define NC_INST(T)                                                                                                \
  template nc_status opt_init<T>(const T*, float*, float*, size_t, float*, size_t, hipStream_t);                   \
  template nc_status adamw_step<T>(const float*, float*, float*, float*, T*, size_t, float, float, float, float,   \
                                   float, int, hipStream_t);                                                       \
  template nc_status muon_step<T>(const MuonKind<T>*, int, int, long, float, float, int, float, void*, size_t,    \
                                  hipStream_t);
NC_INST(bf16)
NC_INST(float)
#undef NC_INST

}  // namespace nc
