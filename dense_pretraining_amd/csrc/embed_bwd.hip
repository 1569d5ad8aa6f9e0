// Deterministic embedding-gradient scatter: dWte[v] = sum of de[m] over the
// positions m with idx[m] = v (the untied token embedding of the architecture
// list on vpshk.cn; its gradient is a sum of rows, one per occurrence), where
// de = N_bwd(dx0) is the backward of the parameter-free norm that follows the
// embedding: de = r (dx0 - x0 mean(dx0 x0)). The norm backward is folded into
// the window sums: they read each sorted position's dx0 and x0 rows once, take
// the row's dot product dx0 . x0 over the block, and add de = r dx0 - b x0
// (b = r mean(dx0 x0)) to the run, so de never reaches memory.
//
// No floating-point atomics: the positions are first sorted by (id, m) with a
// counting sort whose within-id ranks are computed exactly (chunk histograms,
// a prefix over chunks, and an in-chunk rank count), then fixed windows of 64
// sorted positions each sum their runs in order. A run that crosses a window
// boundary (a frequent id: with Zipf-distributed tokens the top id holds
// ~14% of all positions) leaves one partial per window, and the partials are
// added in window order by the block that owns the segment's first crossing.
#include "common.h"
#include "kernels.h"

namespace nc {
namespace {

constexpr int kChunk = 1024;  // tokens per histogram chunk
constexpr int kWin = 64;      // sorted positions per summation window

__global__ void __launch_bounds__(256) eb_hist_kernel(const int32_t* __restrict__ idx, int M, int V,
                                                      int* __restrict__ hist) {
  int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  int v = idx[m];
  if (v < 0 || v >= V) return;
  atomicAdd(&hist[(long)(m / kChunk) * V + v], 1);
}

// Per id: exclusive prefix of the chunk histograms over chunks (in place) and
// the id's total count into seg[v].
__global__ void __launch_bounds__(256) eb_colscan_kernel(int* __restrict__ hist, int nchunks, int V,
                                                         int* __restrict__ seg) {
  int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= V) return;
  int run = 0;
  // eight chunks' loads in flight at a time (a rolled loop would wait for each)
  int c = 0;
  for (; c + 8 <= nchunks; c += 8) {
    int h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = hist[(long)(c + j) * V + v];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hist[(long)(c + j) * V + v] = run;
      run += h[j];
    }
  }
  for (; c < nchunks; ++c) {
    long i = (long)c * V + v;
    int h = hist[i];
    hist[i] = run;
    run += h;
  }
  seg[v] = run;
}

// Exclusive scan of seg[0..V) in place, seg[V] = total (one block of 1024).
// Thread t owns the contiguous slice [t per, t per + per); with per <= 64 (a
// multiple of 4) the slice is held in registers, read and written four at a time.
constexpr int kScanPer = 64;
__global__ void __launch_bounds__(1024) eb_scan_kernel(int* __restrict__ seg, int V) {
  __shared__ int sums[1024];
  const int t = threadIdx.x;
  const int per = (V + 1023) / 1024;
  const int b = t * per, e = min(V, b + per);
  if (per <= kScanPer && per % 4 == 0 && V % 4 == 0) {
    int4 x[kScanPer / 4];
#pragma unroll
    for (int j = 0; j < kScanPer / 4; ++j)
      x[j] = b + 4 * j < e ? reinterpret_cast<const int4*>(seg + b)[j] : make_int4(0, 0, 0, 0);
    int s = 0;
#pragma unroll
    for (int j = 0; j < kScanPer / 4; ++j) s += (x[j].x + x[j].y) + (x[j].z + x[j].w);
    sums[t] = s;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int y = (t >= off) ? sums[t - off] : 0;
      __syncthreads();
      sums[t] += y;
      __syncthreads();
    }
    int run = (t > 0) ? sums[t - 1] : 0;
#pragma unroll
    for (int j = 0; j < kScanPer / 4; ++j) {
      int4 o;
      o.x = run; run += x[j].x;
      o.y = run; run += x[j].y;
      o.z = run; run += x[j].z;
      o.w = run; run += x[j].w;
      if (b + 4 * j < e) reinterpret_cast<int4*>(seg + b)[j] = o;
    }
    if (t == 1023) seg[V] = sums[1023];
    return;
  }
  int s = 0;
  for (int i = b; i < e; ++i) s += seg[i];
  sums[t] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 thread sums
  for (int off = 1; off < 1024; off <<= 1) {
    int x = (t >= off) ? sums[t - off] : 0;
    __syncthreads();
    sums[t] += x;
    __syncthreads();
  }
  int run = (t > 0) ? sums[t - 1] : 0;
  for (int i = b; i < e; ++i) {
    int c = seg[i];
    seg[i] = run;
    run += c;
  }
  if (t == 1023) seg[V] = sums[1023];
}

// Stable placement: rank of m among equal ids earlier in its chunk.
__global__ void __launch_bounds__(256) eb_place_kernel(const int32_t* __restrict__ idx, int M, int V,
                                                       const int* __restrict__ hist, const int* __restrict__ seg,
                                                       int* __restrict__ perm, int* __restrict__ sid) {
  __shared__ int ids[kChunk];
  const int c = blockIdx.x, t = threadIdx.x;
  const int base = c * kChunk;
  const int n = min(kChunk, M - base);
  for (int j = t; j < kChunk; j += 256) {
    int v = -1;
    if (j < n) {
      v = idx[base + j];
      if (v < 0 || v >= V) v = -1;
    }
    ids[j] = v;
  }
  __syncthreads();
  int my[4], rank[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    my[k] = ids[t + 256 * k];
    rank[k] = 0;
  }
  for (int j = 0; j < n; ++j) {
    int v = ids[j];
#pragma unroll
    for (int k = 0; k < 4; ++k) rank[k] += (j < t + 256 * k && v == my[k]) ? 1 : 0;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int j = t + 256 * k;
    if (j < n && my[k] >= 0) {
      int v = my[k];
      int dst = seg[v] + hist[(long)c * V + v] + rank[k];
      perm[dst] = base + j;
      sid[dst] = v;
    }
  }
}

// 16 bytes of T as float values.
template <typename T>
__device__ __forceinline__ void unpack16(const uint4& u, float* out) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    out[0] = __uint_as_float(u.x); out[1] = __uint_as_float(u.y);
    out[2] = __uint_as_float(u.z); out[3] = __uint_as_float(u.w);
  }
}

// Window sums of de = r dx - (r mean(dx x)) x over the sorted positions.
// Thread t owns the VE consecutive columns of 16-byte group t (d <= 256 VE).
// A window's positions, ids and norm scales r are staged in LDS first, with
// whether its first run began before the window and its last run goes on
// past it. The rows of kBatch positions are in flight while the previous
// batch is summed; their dot products dx . x are summed per wave and then
// over the four waves in order (double-buffered, one barrier per batch), and
// each position's de is added to its run. A run inside the window goes to
// its dWte row, stored outright over the zero-filled row unless accumulating;
// a run crossing an edge goes to the window's spill slot (0: the window's
// first run, 1: its last).
constexpr int kBatch = 4;
template <typename T>
__global__ void __launch_bounds__(256) eb_window_kernel(const T* __restrict__ dx, const T* __restrict__ x,
                                                        const float* __restrict__ r, int d,
                                                        const int* __restrict__ seg, const int* __restrict__ perm,
                                                        const int* __restrict__ sid, int V, int accumulate,
                                                        float* __restrict__ dwte, float* __restrict__ spill) {
  constexpr int VE = Vec<T>::n;
  __shared__ int spos[kWin], sids[kWin];
  __shared__ float sr[kWin];
  __shared__ float red[2][4][kBatch];
  __shared__ int cont[2];  // first run began before the window, last run goes on past it
  const int w = blockIdx.x;
  const int nvalid = seg[V];
  const int p0 = w * kWin;
  if (p0 >= nvalid) return;  // the whole block leaves together
  const int n = min(kWin, nvalid - p0);
  if (threadIdx.x < n) {
    const int m = perm[p0 + threadIdx.x];
    spos[threadIdx.x] = m;
    sids[threadIdx.x] = sid[p0 + threadIdx.x];
    sr[threadIdx.x] = r[m];
  }
  if (threadIdx.x == 64) cont[0] = p0 > 0 && sid[p0 - 1] == sid[p0];
  if (threadIdx.x == 65) cont[1] = p0 + n < nvalid && sid[p0 + n] == sid[p0 + n - 1];
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = VE * threadIdx.x;  // first column of this thread's group
  const bool on = c < d;
  const float inv_d = 1.f / (float)d;
  const int v_first = sids[0], v_last = sids[n - 1];
  const bool c_first = cont[0], c_last = cont[1];
  auto flush = [&](int v, const float* a) {
    const bool inside = !((v == v_first && c_first) || (v == v_last && c_last));
    float* o = inside ? dwte + (long)v * d + c : spill + (long)(2 * w + (v == v_first ? 0 : 1)) * d + c;
    const bool add = inside && accumulate;
#pragma unroll
    for (int q = 0; q < VE; q += 4) {
      float4 y = add ? *reinterpret_cast<const float4*>(o + q) : make_float4(0.f, 0.f, 0.f, 0.f);
      y.x += a[q]; y.y += a[q + 1]; y.z += a[q + 2]; y.w += a[q + 3];
      *reinterpret_cast<float4*>(o + q) = y;
    }
  };
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
  int cur = v_first;
  uint4 nd[kBatch], nx[kBatch];  // the next batch's chunks, in flight
  auto fetch = [&](int b0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      nd[i] = nx[i] = make_uint4(0u, 0u, 0u, 0u);
      if (on && b0 + i < n) {
        const long ro = (long)spos[b0 + i] * d + c;
        nd[i] = *reinterpret_cast<const uint4*>(dx + ro);
        nx[i] = *reinterpret_cast<const uint4*>(x + ro);
      }
    }
  };
  fetch(0);
  int par = 0;
  for (int b0 = 0; b0 < n; b0 += kBatch, par ^= 1) {
    float gx[kBatch][VE], xx[kBatch][VE], dot[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      unpack16<T>(nd[i], gx[i]);
      unpack16<T>(nx[i], xx[i]);
    }
    if (b0 + kBatch < n) fetch(b0 + kBatch);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) t += gx[i][e] * xx[i][e];
      dot[i] = wave_sum(t);
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) red[par][wv][i] = dot[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (b0 + i >= n) break;
      const int v = sids[b0 + i];
      if (v != cur) {
        if (on) flush(cur, acc);
        cur = v;
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[e] = 0.f;
      }
      const float tot = red[par][0][i] + red[par][1][i] + red[par][2][i] + red[par][3][i];
      const float ka = sr[b0 + i], kb = ka * tot * inv_d;
      if (on) {
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[e] += ka * gx[i][e] - kb * xx[i][e];
      }
    }
  }
  if (on) flush(cur, acc);
}

// Segments spanning windows: block w owns the segment whose first crossed
// boundary is w * kWin and adds its window partials in window order.
__global__ void __launch_bounds__(256) eb_fixup_kernel(int d, const int* __restrict__ seg, const int* __restrict__ sid,
                                                       int V, float* __restrict__ dwte,
                                                       const float* __restrict__ spill) {
  const int w = blockIdx.x + 1;
  const int b = w * kWin;
  const int nvalid = seg[V];
  if (b >= nvalid) return;
  const int v = sid[b];
  if (sid[b - 1] != v) return;
  const int s = seg[v], e = seg[v + 1];
  if (s / kWin + 1 != w) return;
  const int d4 = d / 4;
  const int w0 = s / kWin, w1 = (e - 1) / kWin;
  for (int c4 = threadIdx.x; c4 < d4; c4 += 256) {
    float4 tot = make_float4(0.f, 0.f, 0.f, 0.f);
    // eight windows' partials loaded before they are added (in window order)
    int ww = w0;
    for (; ww + 8 <= w1 + 1; ww += 8) {
      float4 x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int slot = (s <= (ww + j) * kWin) ? 0 : 1;
        x[j] = reinterpret_cast<const float4*>(spill + (long)(2 * (ww + j) + slot) * d)[c4];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        tot.x += x[j].x; tot.y += x[j].y; tot.z += x[j].z; tot.w += x[j].w;
      }
    }
    for (; ww <= w1; ++ww) {
      const int slot = (s <= ww * kWin) ? 0 : 1;
      const float4 x = reinterpret_cast<const float4*>(spill + (long)(2 * ww + slot) * d)[c4];
      tot.x += x.x; tot.y += x.y; tot.z += x.z; tot.w += x.w;
    }
    float4* o = reinterpret_cast<float4*>(dwte + (long)v * d) + c4;
    float4 x = *o;
    x.x += tot.x; x.y += tot.y; x.z += tot.z; x.w += tot.w;
    *o = x;
  }
}

}  // namespace

size_t embed_sort_bytes(int M, int V, int d) {
  size_t nch = (size_t)(M + kChunk - 1) / kChunk;
  size_t nwin = (size_t)(M + kWin - 1) / kWin;
  size_t b = 0;
  b += align_up(nch * V * sizeof(int), 256);
  b += align_up((size_t)(V + 1) * sizeof(int), 256);
  b += 2 * align_up((size_t)M * sizeof(int), 256);
  b += align_up(nwin * 2 * d * sizeof(float), 256);
  return b;
}

EmbedSortBufs embed_sort_carve(void* base, int M, int V, int d) {
  size_t nch = (size_t)(M + kChunk - 1) / kChunk;
  char* p = static_cast<char*>(base);
  EmbedSortBufs b;
  b.hist = reinterpret_cast<int*>(p); p += align_up(nch * V * sizeof(int), 256);
  b.seg = reinterpret_cast<int*>(p); p += align_up((size_t)(V + 1) * sizeof(int), 256);
  b.perm = reinterpret_cast<int*>(p); p += align_up((size_t)M * sizeof(int), 256);
  b.sid = reinterpret_cast<int*>(p); p += align_up((size_t)M * sizeof(int), 256);
  b.spill = reinterpret_cast<float*>(p);
  return b;
}

template <typename T>
nc_status embed_bwd(const int32_t* idx, const T* x0, const float* r0, const T* dx0, float* dwte, int M, int V, int d,
                    int accumulate, const EmbedSortBufs& b, hipStream_t st) {
  if (d % Vec<T>::n != 0 || d > 256 * Vec<T>::n) return NC_ERR_UNSUPPORTED;
  const int nch = (M + kChunk - 1) / kChunk;
  const int nwin = (M + kWin - 1) / kWin;
  NC_TRY(fill_u32(reinterpret_cast<uint32_t*>(b.hist), 0u, (size_t)nch * V, st));
  if (!accumulate) NC_TRY(fill_f32(dwte, 0.f, (size_t)V * d, st));
  const double es = sizeof(T);
  {
    ProfScope prof("embed_sort", 0, 4.0 * M * 5 + 8.0 * nch * V, st);
    hipLaunchKernelGGL(eb_hist_kernel, dim3((M + 255) / 256), dim3(256), 0, st, idx, M, V, b.hist);
    NC_LAUNCH_CHECK("eb_hist");
    hipLaunchKernelGGL(eb_colscan_kernel, dim3((V + 255) / 256), dim3(256), 0, st, b.hist, nch, V, b.seg);
    NC_LAUNCH_CHECK("eb_colscan");
    hipLaunchKernelGGL(eb_scan_kernel, dim3(1), dim3(1024), 0, st, b.seg, V);
    NC_LAUNCH_CHECK("eb_scan");
    hipLaunchKernelGGL(eb_place_kernel, dim3(nch), dim3(256), 0, st, idx, M, V, b.hist, b.seg, b.perm, b.sid);
    NC_LAUNCH_CHECK("eb_place");
  }
  {
    // counted: dx0 and x0 rows once, r, positions and ids. The distinct ids'
    // dWte rows and the spill slots it writes are unknown to the host and
    // left out, so the rate is a lower bound.
    ProfScope prof(NC_NAME(T, "embed_window_sum"), 0, 2.0 * es * M * d + 12.0 * M, st);
    hipLaunchKernelGGL((eb_window_kernel<T>), dim3(nwin), dim3(256), 0, st, dx0, x0, r0, d, b.seg, b.perm, b.sid,
                       V, accumulate, dwte, b.spill);
    NC_LAUNCH_CHECK("eb_window");
  }
  if (nwin > 1) {
    ProfScope prof("embed_fixup", 0, 0, st);
    hipLaunchKernelGGL(eb_fixup_kernel, dim3(nwin - 1), dim3(256), 0, st, d, b.seg, b.sid, V, dwte, b.spill);
    NC_LAUNCH_CHECK("eb_fixup");
  }
  return NC_OK;
}

template nc_status embed_bwd<bf16>(const int32_t*, const bf16*, const float*, const bf16*, float*, int, int, int, int,
                                   const EmbedSortBufs&, hipStream_t);
template nc_status embed_bwd<float>(const int32_t*, const float*, const float*, const float*, float*, int, int, int,
                                    int, const EmbedSortBufs&, hipStream_t);

}  // namespace nc
