// Row-wise HBM-bound kernels: parameter-free RMSNorm forward/backward (also
// fused with the embedding gather), the per-head QK norm + rotary embedding
// forward/backward, the softcapped cross-entropy reductions, split-K sums and
// fills. One wavefront owns one row, the row stays in registers, and the row
// statistics are reduced with cross-lane shuffles in a fixed order.
#include <utility>

#include "common.h"
#include "kernels.h"

namespace nc {
namespace {

template <typename T> constexpr int max_vecs() { return 2048 / Vec<T>::n / 64; }  // d <= 2048

// ------------------------------------------------------------ fills
__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}
__global__ void fill_f32_kernel(float* p, float v, size_t n) {
  size_t n4 = n / 4;
  float4 v4 = make_float4(v, v, v, v);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x)
    reinterpret_cast<float4*>(p)[i] = v4;
  for (size_t i = n4 * 4 + blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// ------------------------------------------------------------ RMSNorm
// N(v) = v / sqrt(mean(v^2) + eps) (no gain: the architecture list on vpshk.cn
// gives RMSNorm without learnable parameters). With GATHER, row m is the
// embedding row idx[m] (the norm that follows the token embedding). One wave
// per row; returns the lane's largest stored |y| when AMAX.
template <typename T, bool GATHER, bool AMAX>
__device__ __forceinline__ float rmsnorm_fwd_row(const T* __restrict__ x, const int32_t* __restrict__ idx, int V,
                                                 T* __restrict__ y, float* __restrict__ r, int row, int d, float eps,
                                                 uint32_t* status) {
  constexpr int VE = Vec<T>::n, MAXV = max_vecs<T>();
  const int lane = threadIdx.x & 63;
  long src_row = row;
  bool zero = false;
  if constexpr (GATHER) {
    int id = idx[row];
    if (id < 0 || id >= V) {
      zero = true;
      if (lane == 0) set_status(status, kStatusBadToken);
      id = 0;
    }
    src_row = id;
  }
  const T* src = x + src_row * d;
  const int nv = d / VE;
  float v[MAXV][VE];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < MAXV; ++c) {
    int vi = lane + 64 * c;
    if (vi < nv && !zero) {
      load16<T>(src + vi * VE, v[c]);
#pragma unroll
      for (int e = 0; e < VE; ++e) ss += v[c][e] * v[c][e];
    } else {
#pragma unroll
      for (int e = 0; e < VE; ++e) v[c][e] = 0.f;
    }
  }
  ss = wave_sum(ss);
  const float rr = 1.f / sqrtf(ss / (float)d + eps);
  T* dst = y + (long)row * d;
  float m = 0.f;
#pragma unroll
  for (int c = 0; c < MAXV; ++c) {
    int vi = lane + 64 * c;
    if (vi < nv) {
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        v[c][e] *= rr;
        if constexpr (AMAX) m = fmaxf(m, fabsf(v[c][e]));
      }
      store16<T>(dst + vi * VE, v[c]);
    }
  }
  if (lane == 0) r[row] = rr;
  return m;
}

// Four rows per block. With AMAX the block's largest stored magnitude goes
// into *amax (the per-tensor scale of an FP8 operand).
template <typename T, bool GATHER, bool AMAX = false>
__global__ void __launch_bounds__(256) rmsnorm_fwd_kernel(const T* __restrict__ x, const int32_t* __restrict__ idx,
                                                          int V, T* __restrict__ y, float* __restrict__ r, int M,
                                                          int d, float eps, uint32_t* status, uint32_t* amax) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  float m = 0.f;
  if (row < M) m = rmsnorm_fwd_row<T, GATHER, AMAX>(x, idx, V, y, r, row, d, eps, status);
  if constexpr (AMAX) {
    __shared__ float red[4];
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = to_f32(from_f32<T>(m));
    __syncthreads();
    if (threadIdx.x == 0) amax_publish(amax, fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  }
}

// dx = res + r (dy - y mean(dy y)), written in terms of the output y.
template <typename T, typename TO>
__global__ void __launch_bounds__(256) rmsnorm_bwd_kernel(const T* __restrict__ dy, const T* __restrict__ y,
                                                          const float* __restrict__ r, const T* __restrict__ res,
                                                          TO* __restrict__ dx, int M, int d) {
  constexpr int VE = Vec<T>::n, MAXV = max_vecs<T>();
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;
  const long off = (long)row * d;
  const int nv = d / VE;
  float g[MAXV][VE], yy[MAXV][VE], rs[MAXV][VE];
  float dot = 0.f;
  // all three inputs in flight before the row sum (the residual was loaded after it)
#pragma unroll
  for (int c = 0; c < MAXV; ++c) {
    int vi = lane + 64 * c;
    if (vi < nv) {
      load16<T>(dy + off + vi * VE, g[c]);
      load16<T>(y + off + vi * VE, yy[c]);
      if (res) load16<T>(res + off + vi * VE, rs[c]);
#pragma unroll
      for (int e = 0; e < VE; ++e) dot += g[c][e] * yy[c][e];
    }
  }
  dot = wave_sum(dot) / (float)d;
  const float rr = r[row];
#pragma unroll
  for (int c = 0; c < MAXV; ++c) {
    int vi = lane + 64 * c;
    if (vi < nv) {
      float o[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) o[e] = rr * (g[c][e] - yy[c][e] * dot);
      if (res) {
#pragma unroll
        for (int e = 0; e < VE; ++e) o[e] += rs[c][e];
      }
      if constexpr (sizeof(TO) == sizeof(T)) {
        store16<TO>(dx + off + vi * VE, o);
      } else {
        // float output from bf16 inputs: two 16-byte stores
        store16<TO>(dx + off + vi * VE, o);
        store16<TO>(dx + off + vi * VE + 4, o + 4);
      }
    }
  }
}

// ------------------------------------------------------------ rotary + QK norm
// Rotary embedding (architecture list on vpshk.cn): pair (i, i + D/2) of a
// head at position t turns by t * base^(-2i/D). The table is evaluated in
// double precision.
__global__ void rope_table_kernel(float* cs, float* sn, int T, int D, float base, int t0) {
  int P = D / 2;
  int n = T * P;
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < n; k += gridDim.x * blockDim.x) {
    int t = t0 + k / P, i = k % P;
    double omega = pow((double)base, -2.0 * (double)i / (double)D);
    double ang = (double)t * omega;
    cs[k] = (float)cos(ang);
    sn[k] = (float)sin(ang);
  }
}

// QK norm (parameter-free RMSNorm over each head's D values) then the
// rotation. Lane i of a head holds the pair (i, i + D/2), so the rotation is
// lane-local; D = 64 puts two heads in one wavefront.
// Each (token, head) pair takes D/8 lanes; lane j holds the rotation pairs
// 4j .. 4j+3, i.e. elements 4j.. of both halves of the head (two 8-byte
// loads), so the rotation is lane-local and the per-head norm is a reduction
// over D/8 lanes.
template <typename T, int D>
__global__ void __launch_bounds__(256) qknorm_rope_fwd_kernel(const T* __restrict__ qkv, long ld_in, T* __restrict__ qk,
                                                              long ld_out, const float* __restrict__ cs,
                                                              const float* __restrict__ sn, int M, int Tn, int nheads,
                                                              float eps, int pos0) {
  constexpr int P = D / 2, LPH = P / 4, HPB = 256 / LPH;
  const long pair = (long)blockIdx.x * HPB + threadIdx.x / LPH;
  const int j = threadIdx.x % LPH;
  if (pair >= (long)M * nheads) return;  // whole lane groups leave together
  const int m = (int)(pair / nheads), h = (int)(pair - (long)m * nheads);
  const int t = pos0 + m % Tn;
  const T* src = qkv + (long)m * ld_in + (long)h * D + 4 * j;
  float a[4], b[4];
  load4<T>(src, a);
  load4<T>(src + P, b);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) ss += a[e] * a[e] + b[e] * b[e];
  const float rr = 1.f / sqrtf(group_sum(ss, LPH) / (float)D + eps);
  const float4 c4 = *reinterpret_cast<const float4*>(cs + (long)t * P + 4 * j);
  const float4 s4 = *reinterpret_cast<const float4*>(sn + (long)t * P + 4 * j);
  const float c[4] = {c4.x, c4.y, c4.z, c4.w}, s[4] = {s4.x, s4.y, s4.z, s4.w};
  float oa[4], ob[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float ya = a[e] * rr, yb = b[e] * rr;
    oa[e] = ya * c[e] - yb * s[e];
    ob[e] = ya * s[e] + yb * c[e];
  }
  T* dst = qk + (long)m * ld_out + (long)h * D + 4 * j;
  store4<T>(dst, oa);
  store4<T>(dst + P, ob);
}

// Backward of the same map, in place on g (the gradient of the rotated,
// normed heads on entry, of the raw heads on exit).
template <typename T, int D>
__global__ void __launch_bounds__(256) qknorm_rope_bwd_kernel(const T* __restrict__ qkv, long ld_in, T* __restrict__ gr,
                                                              long ld_g, const float* __restrict__ cs,
                                                              const float* __restrict__ sn, int M, int Tn, int nheads,
                                                              float eps) {
  constexpr int P = D / 2, LPH = P / 4, HPB = 256 / LPH;
  const long pair = (long)blockIdx.x * HPB + threadIdx.x / LPH;
  const int j = threadIdx.x % LPH;
  if (pair >= (long)M * nheads) return;
  const int m = (int)(pair / nheads), h = (int)(pair - (long)m * nheads);
  const int t = m % Tn;
  const T* src = qkv + (long)m * ld_in + (long)h * D + 4 * j;
  T* g = gr + (long)m * ld_g + (long)h * D + 4 * j;
  float a[4], b[4], ga[4], gb[4];
  load4<T>(src, a);
  load4<T>(src + P, b);
  load4<T>(g, ga);
  load4<T>(g + P, gb);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) ss += a[e] * a[e] + b[e] * b[e];
  const float rr = 1.f / sqrtf(group_sum(ss, LPH) / (float)D + eps);
  const float4 c4 = *reinterpret_cast<const float4*>(cs + (long)t * P + 4 * j);
  const float4 s4 = *reinterpret_cast<const float4*>(sn + (long)t * P + 4 * j);
  const float c[4] = {c4.x, c4.y, c4.z, c4.w}, s[4] = {s4.x, s4.y, s4.z, s4.w};
  // transpose rotation, then the norm's backward: rr (u - y <u, y> / D)
  float ua[4], ub[4], dot = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ua[e] = ga[e] * c[e] + gb[e] * s[e];
    ub[e] = -ga[e] * s[e] + gb[e] * c[e];
    dot += ua[e] * a[e] + ub[e] * b[e];
  }
  dot = group_sum(dot, LPH) * rr / (float)D;  // <u, y> / D with y = x rr
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ua[e] = rr * (ua[e] - a[e] * rr * dot);
    ub[e] = rr * (ub[e] - b[e] * rr * dot);
  }
  store4<T>(g, ua);
  store4<T>(g + P, ub);
}

// ------------------------------------------------------------ cross-entropy
// Next-token cross-entropy over the softcapped logits (imeisheng.com section
// "预训练"; softcap from the architecture list). Per row: lse = log(sum of the
// unembedding epilogue's per-tile exp sums); loss term lse - z'[target], the
// target's logit recomputed here as one float32 dot product of the row's
// input with the target's weight row (the epilogue then has no per-element
// target test).
template <typename T>
__global__ void __launch_bounds__(256) xent_rows_kernel(const float* __restrict__ part, int ntiles,
                                                        const T* __restrict__ x, const T* __restrict__ w, int d,
                                                        float cap, const int32_t* __restrict__ tg, int M, int V,
                                                        float* __restrict__ lse, float* __restrict__ block_sums,
                                                        int* __restrict__ block_counts, uint32_t* status, float shift,
                                                        float* __restrict__ zt) {
  __shared__ float ws[4];
  __shared__ int wc[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float acc = 0.f;
  int cnt = 0;
  for (int k = 0; k < 8; ++k) {
    const int m = blockIdx.x * 32 + wave * 8 + k;
    if (m >= M) break;
    float s = 0.f;
    for (int t = lane; t < ntiles; t += 64) s += part[(long)m * ntiles + t];
    s = wave_sum(s);
    const float l = shift + logf(s);
    int y = tg[m];
    if (y < -1 || y >= V) {
      if (lane == 0) set_status(status, kStatusBadTarget);
      y = -1;
    }
    if (lane == 0) lse[m] = l;
    if (zt && y < 0 && lane == 0) zt[m] = 0.f;
    if (y >= 0) {
      constexpr int n = Vec<T>::n;
      float dot = 0.f;
      for (int c = n * lane; c < d; c += 64 * n) {
        float a[n], b[n];
        load16<T>(x + (long)m * d + c, a);
        load16<T>(w + (long)y * d + c, b);
#pragma unroll
        for (int e = 0; e < n; ++e) dot += a[e] * b[e];
      }
      dot = wave_sum(dot);
      const float zy = cap * tanhf(dot / cap);
      if (zt && lane == 0) zt[m] = zy;
      acc += l - zy;
      cnt += 1;
    }
  }
  if (lane == 0) {
    ws[wave] = acc;
    wc[wave] = cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    block_sums[blockIdx.x] = ((ws[0] + ws[1]) + ws[2]) + ws[3];
    block_counts[blockIdx.x] = wc[0] + wc[1] + wc[2] + wc[3];
  }
}

__global__ void __launch_bounds__(256) xent_final_kernel(const float* __restrict__ block_sums,
                                                         const int* __restrict__ block_counts, int nblocks,
                                                         float* loss, int* nv, uint32_t* status) {
  __shared__ float s[256];
  __shared__ int c[256];
  float a = 0.f;
  int n = 0;
  for (int i = threadIdx.x; i < nblocks; i += 256) {
    a += block_sums[i];
    n += block_counts[i];
  }
  s[threadIdx.x] = a;
  c[threadIdx.x] = n;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) {
      s[threadIdx.x] += s[threadIdx.x + w];
      c[threadIdx.x] += c[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int count = c[0];
    float l = count > 0 ? s[0] / (float)count : 0.f;
    if (count == 0) set_status(status, kStatusNoTargets);
    if (!isfinite(l)) set_status(status, kStatusNonFinite);
    *loss = l;
    *nv = count;
  }
}

// The softcapped cross-entropy's backward over rows (the logits are not read
// again): the unembedding stored u = exp(z' - c) (1 - (z'/c)^2) / 4 per logit,
// so dz[m][v] = 4 g / S (u[m][v] - [v = y] S (1 - (z'_y/c)^2) / 4) with
// g = dloss / Nv and S = exp(lse - c) the row's sum of exp(z' - c)
// (imeisheng.com section "预训练" for the loss; the softcap from the
// architecture list). One wave a row: lane 0 corrects the target's element of
// u (in the column-panel layout) and writes q = 4 g / S; the wave writes
// xs = q xf, the weight-gradient product's row-scaled operand. Rows without a
// target get q = 0.
template <typename T>
__global__ void __launch_bounds__(256) xent_grad_prep_kernel(T* __restrict__ u, int M, int V,
                                                             const float* __restrict__ lse,
                                                             const float* __restrict__ zt,
                                                             const int32_t* __restrict__ tg,
                                                             const int* __restrict__ nvp, float dloss, float cap,
                                                             const T* __restrict__ xf, int d, T* __restrict__ xs,
                                                             float* __restrict__ q) {
  constexpr int VE = Vec<T>::n;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (m >= M) return;
  const int y = tg[m];
  const int nv = *nvp;
  const bool valid = y >= 0 && y < V && nv > 0;
  const float S = expf(lse[m] - cap);
  const float qm = valid ? 4.f * dloss / (float)nv / S : 0.f;
  if (lane == 0) {
    q[m] = qm;
    if (valid) {
      T* p = u + (long)(y / kPanel) * M * kPanel + (long)m * kPanel + y % kPanel;
      const float w = zt[m] / cap;
      *p = from_f32<T>(to_f32(*p) - 0.25f * S * (1.f - w * w));
    }
  }
  const long off = (long)m * d;
  for (int c = VE * lane; c < d; c += 64 * VE) {
    float a[VE];
    load16<T>(xf + off + c, a);
#pragma unroll
    for (int e = 0; e < VE; ++e) a[e] *= qm;
    store16<T>(xs + off + c, a);
  }
}

// Sums the splits' partial tiles in split order (deterministic). The split
// count is a template parameter, so all of a thread's partial loads are issued
// before the first add with no per-split test; one 16-byte piece per thread.
constexpr int kMaxSplits = 16;
template <int NS>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part, size_t n4,
                                                            float* __restrict__ out, int accumulate) {
  const size_t i = blockIdx.x * (size_t)256 + threadIdx.x;
  if (i >= n4) return;
  float4 p[NS];
#pragma unroll
  for (int zz = 0; zz < NS; ++zz) p[zz] = reinterpret_cast<const float4*>(part + (size_t)zz * n4 * 4)[i];
  float4 a = accumulate ? reinterpret_cast<const float4*>(out)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int zz = 0; zz < NS; ++zz) {
    a.x += p[zz].x; a.y += p[zz].y; a.z += p[zz].z; a.w += p[zz].w;
  }
  reinterpret_cast<float4*>(out)[i] = a;
}

template <int NS>
void launch_splitk(const float* part, size_t n4, float* out, int accumulate, hipStream_t st) {
  hipLaunchKernelGGL(splitk_reduce_kernel<NS>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, part, n4, out,
                     accumulate);
}
template <int... NS>
bool launch_splitk_n(int nsplit, const float* part, size_t n4, float* out, int accumulate, hipStream_t st,
                     std::integer_sequence<int, NS...>) {
  return ((nsplit == NS + 1 ? (launch_splitk<NS + 1>(part, n4, out, accumulate, st), true) : false) || ...);
}

unsigned grid_for(size_t n, size_t per_block) {
  size_t g = (n + per_block - 1) / per_block;
  if (g > 65536) g = 65536;
  return (unsigned)(g ? g : 1);
}

}  // namespace

nc_status fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t st) {
  ProfScope prof("fill_u32", 0, 4.0 * n, st);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, st, p, v, n);
  NC_LAUNCH_CHECK("fill_u32");
  return NC_OK;
}
nc_status fill_f32(float* p, float v, size_t n, hipStream_t st) {
  ProfScope prof("fill_f32", 0, 4.0 * n, st);
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n / 4 + 1, 256)), dim3(256), 0, st, p, v, n);
  NC_LAUNCH_CHECK("fill_f32");
  return NC_OK;
}

template <typename T>
nc_status rmsnorm_fwd(const T* x, const int32_t* idx, int V, T* y, float* r, int M, int d, float eps, uint32_t* status,
                      hipStream_t st, uint32_t* amax) {
  dim3 grid((M + 3) / 4);
  ProfScope prof(idx ? NC_NAME(T, "embed_gather_rmsnorm") : NC_NAME(T, "rmsnorm_fwd"), 0,
                 2.0 * sizeof(T) * M * d + 4.0 * M + (idx ? 4.0 * M : 0.0), st);
  if (idx && amax) return NC_ERR_UNSUPPORTED;
  if (idx)
    hipLaunchKernelGGL((rmsnorm_fwd_kernel<T, true>), grid, dim3(256), 0, st, x, idx, V, y, r, M, d, eps, status,
                       amax);
  else if (amax)
    hipLaunchKernelGGL((rmsnorm_fwd_kernel<T, false, true>), grid, dim3(256), 0, st, x, idx, V, y, r, M, d, eps,
                       status, amax);
  else
    hipLaunchKernelGGL((rmsnorm_fwd_kernel<T, false>), grid, dim3(256), 0, st, x, idx, V, y, r, M, d, eps, status,
                       amax);
  NC_LAUNCH_CHECK("rmsnorm_fwd");
  return NC_OK;
}

template <typename T, typename TO>
nc_status rmsnorm_bwd(const T* dy, const T* y, const float* r, const T* res, TO* dx, int M, int d, hipStream_t st) {
  ProfScope prof(sizeof(TO) != sizeof(T) ? "rmsnorm_bwd_bf16_to_f32" : NC_NAME(T, "rmsnorm_bwd"), 0,
                 sizeof(T) * (double)M * d * (res ? 3 : 2) + sizeof(TO) * (double)M * d + 4.0 * M, st);
  hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, TO>), dim3((M + 3) / 4), dim3(256), 0, st, dy, y, r, res, dx, M, d);
  NC_LAUNCH_CHECK("rmsnorm_bwd");
  return NC_OK;
}

nc_status rope_table(float* cs, float* sn, int T, int D, float base, hipStream_t st, int t0) {
  ProfScope prof("rope_table", 0, 4.0 * T * D, st);
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for((size_t)T * D / 2, 256)), dim3(256), 0, st, cs, sn, T, D, base,
                     t0);
  NC_LAUNCH_CHECK("rope_table");
  return NC_OK;
}

template <typename T>
nc_status qknorm_rope_fwd(const T* qkv, long ld_in, T* qk, long ld_out, const float* cs, const float* sn, int M,
                          int T_, int nheads, int D, float eps, hipStream_t st, int pos0) {
  ProfScope prof(NC_NAME(T, "qknorm_rope_fwd"), 0, 2.0 * sizeof(T) * M * nheads * D, st);
  const long pairs = (long)M * nheads;
  if (D == 128)
    hipLaunchKernelGGL((qknorm_rope_fwd_kernel<T, 128>), dim3((unsigned)((pairs + 15) / 16)), dim3(256), 0, st, qkv,
                       ld_in, qk, ld_out, cs, sn, M, T_, nheads, eps, pos0);
  else if (D == 64)
    hipLaunchKernelGGL((qknorm_rope_fwd_kernel<T, 64>), dim3((unsigned)((pairs + 31) / 32)), dim3(256), 0, st, qkv,
                       ld_in, qk, ld_out, cs, sn, M, T_, nheads, eps, pos0);
  else
    return NC_ERR_UNSUPPORTED;
  NC_LAUNCH_CHECK("qknorm_rope_fwd");
  return NC_OK;
}

template <typename T>
nc_status qknorm_rope_bwd(const T* qkv, long ld_in, T* g, long ld_g, const float* cs, const float* sn, int M, int T_,
                          int nheads, int D, float eps, hipStream_t st) {
  ProfScope prof(NC_NAME(T, "qknorm_rope_bwd"), 0, 3.0 * sizeof(T) * M * nheads * D, st);
  const long pairs = (long)M * nheads;
  if (D == 128)
    hipLaunchKernelGGL((qknorm_rope_bwd_kernel<T, 128>), dim3((unsigned)((pairs + 15) / 16)), dim3(256), 0, st, qkv,
                       ld_in, g, ld_g, cs, sn, M, T_, nheads, eps);
  else if (D == 64)
    hipLaunchKernelGGL((qknorm_rope_bwd_kernel<T, 64>), dim3((unsigned)((pairs + 31) / 32)), dim3(256), 0, st, qkv,
                       ld_in, g, ld_g, cs, sn, M, T_, nheads, eps);
  else
    return NC_ERR_UNSUPPORTED;
  NC_LAUNCH_CHECK("qknorm_rope_bwd");
  return NC_OK;
}

size_t xent_loss_blocks(int M) { return (size_t)(M + 31) / 32; }

template <typename T>
nc_status xent_loss(const float* part, int ntiles, const T* x, const T* w, int d, float cap, const int32_t* targets,
                    int M, int V, float* lse, float* block_sums, int* block_counts, float* loss, int* nv,
                    uint32_t* status, hipStream_t st, float shift, float* zt) {
  if (d % Vec<T>::n != 0) return NC_ERR_UNSUPPORTED;
  int nb = (int)xent_loss_blocks(M);
  ProfScope prof("xent_loss", 0, 4.0 * M * ntiles + 12.0 * M + 2.0 * sizeof(T) * M * d, st);
  hipLaunchKernelGGL((xent_rows_kernel<T>), dim3(nb), dim3(256), 0, st, part, ntiles, x, w, d, cap, targets, M, V,
                     lse, block_sums, block_counts, status, shift, zt);
  NC_LAUNCH_CHECK("xent_rows");
  hipLaunchKernelGGL(xent_final_kernel, dim3(1), dim3(256), 0, st, block_sums, block_counts, nb, loss, nv, status);
  NC_LAUNCH_CHECK("xent_final");
  return NC_OK;
}

template <typename T>
nc_status xent_grad_prep(T* u, int M, int V, const float* lse, const float* zt, const int32_t* targets, const int* nv,
                         float dloss, float cap, const T* xf, int d, T* xs, float* q, hipStream_t st) {
  if (d % Vec<T>::n != 0) return NC_ERR_UNSUPPORTED;
  // rows' x read and scaled x written; the target corrections and per-row words
  ProfScope prof(NC_NAME(T, "xent_grad_prep"), 0, 2.0 * sizeof(T) * M * d + 20.0 * M, st);
  hipLaunchKernelGGL((xent_grad_prep_kernel<T>), dim3((M + 3) / 4), dim3(256), 0, st, u, M, V, lse, zt, targets, nv,
                     dloss, cap, xf, d, xs, q);
  NC_LAUNCH_CHECK("xent_grad_prep");
  return NC_OK;
}

nc_status splitk_reduce(const float* partial, int nsplit, size_t n, float* out, int accumulate, hipStream_t st) {
  if (nsplit < 1 || nsplit > kMaxSplits || n % 4 != 0) return NC_ERR_UNSUPPORTED;
  size_t n4 = n / 4;
  // one piece per thread: the grid's x dimension bounds the element count
  if ((n4 + 255) / 256 > 0x7fffffffULL) return NC_ERR_UNSUPPORTED;
  if (n4 == 0) return NC_OK;
  ProfScope prof("splitk_reduce", 0, 4.0 * n * (nsplit + (accumulate ? 2 : 1)), st);
  launch_splitk_n(nsplit, partial, n4, out, accumulate, st, std::make_integer_sequence<int, kMaxSplits>{});
  NC_LAUNCH_CHECK("splitk_reduce");
  return NC_OK;
}

#define NC_INST(T)                                                                                                  \
  template nc_status rmsnorm_fwd<T>(const T*, const int32_t*, int, T*, float*, int, int, float, uint32_t*,         \
                                    hipStream_t, uint32_t*);                                                        \
  template nc_status rmsnorm_bwd<T, T>(const T*, const T*, const float*, const T*, T*, int, int, hipStream_t);     \
  template nc_status qknorm_rope_fwd<T>(const T*, long, T*, long, const float*, const float*, int, int, int, int,   \
                                        float, hipStream_t, int);                                                   \
  template nc_status qknorm_rope_bwd<T>(const T*, long, T*, long, const float*, const float*, int, int, int, int,   \
                                        float, hipStream_t);                                                        \
  template nc_status xent_grad_prep<T>(T*, int, int, const float*, const float*, const int32_t*, const int*, float, \
                                       float, const T*, int, T*, float*, hipStream_t);                                 \
  template nc_status xent_loss<T>(const float*, int, const T*, const T*, int, float, const int32_t*, int, int,      \
                                  float*, float*, int*, float*, int*, uint32_t*, hipStream_t, float, float*);
NC_INST(bf16)
NC_INST(float)
#undef NC_INST

}  // namespace nc
