// Deterministic embedding-gradient scatter: dWte[v] = sum of de[m] over the
// positions m with idx[m] = v (the untied token embedding of the architecture
// list on vpshk.cn; its gradient is a sum of rows, one per occurrence).
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
  for (int c = 0; c < nchunks; ++c) {
    long i = (long)c * V + v;
    int h = hist[i];
    hist[i] = run;
    run += h;
  }
  seg[v] = run;
}

// Exclusive scan of seg[0..V) in place, seg[V] = total (one block of 1024).
__global__ void __launch_bounds__(1024) eb_scan_kernel(int* __restrict__ seg, int V) {
  __shared__ int sums[1024];
  const int t = threadIdx.x;
  const int per = (V + 1023) / 1024;
  const int b = t * per, e = min(V, b + per);
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

// Window sums. Thread t owns float4 column groups t, t+256, ...
__global__ void __launch_bounds__(256) eb_window_kernel(const float* __restrict__ de, int d,
                                                        const int* __restrict__ seg, const int* __restrict__ perm,
                                                        const int* __restrict__ sid, int V, float* __restrict__ dwte,
                                                        float* __restrict__ spill) {
  const int w = blockIdx.x;
  const int nvalid = seg[V];
  const int p0 = w * kWin;
  if (p0 >= nvalid) return;
  const int p1 = min(p0 + kWin, nvalid);
  const int d4 = d / 4;
  for (int c4 = threadIdx.x; c4 < d4; c4 += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int cur = sid[p0];
    for (int p = p0; p < p1; ++p) {
      const int v = sid[p];
      if (v != cur) {
        // flush run of `cur` (it ended inside the window)
        const int s = seg[cur], e = seg[cur + 1];
        if (s >= p0 && e <= p1) {
          float4* o = reinterpret_cast<float4*>(dwte + (long)cur * d) + c4;
          float4 x = *o;
          x.x += acc.x; x.y += acc.y; x.z += acc.z; x.w += acc.w;
          *o = x;
        } else {
          reinterpret_cast<float4*>(spill + (long)(2 * w + (s <= p0 ? 0 : 1)) * d)[c4] = acc;
        }
        cur = v;
        acc = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      const float4 x = reinterpret_cast<const float4*>(de + (long)perm[p] * d)[c4];
      acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
    }
    const int s = seg[cur], e = seg[cur + 1];
    if (s >= p0 && e <= p1) {
      float4* o = reinterpret_cast<float4*>(dwte + (long)cur * d) + c4;
      float4 x = *o;
      x.x += acc.x; x.y += acc.y; x.z += acc.z; x.w += acc.w;
      *o = x;
    } else {
      reinterpret_cast<float4*>(spill + (long)(2 * w + (s <= p0 ? 0 : 1)) * d)[c4] = acc;
    }
  }
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
  for (int c4 = threadIdx.x; c4 < d4; c4 += 256) {
    float4 tot = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int ww = s / kWin; ww <= (e - 1) / kWin; ++ww) {
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
  size_t nwin = (size_t)(M + kWin - 1) / kWin;
  char* p = static_cast<char*>(base);
  EmbedSortBufs b;
  b.hist = reinterpret_cast<int*>(p); p += align_up(nch * V * sizeof(int), 256);
  b.seg = reinterpret_cast<int*>(p); p += align_up((size_t)(V + 1) * sizeof(int), 256);
  b.perm = reinterpret_cast<int*>(p); p += align_up((size_t)M * sizeof(int), 256);
  b.sid = reinterpret_cast<int*>(p); p += align_up((size_t)M * sizeof(int), 256);
  b.spill = reinterpret_cast<float*>(p);
  return b;
}

nc_status embed_scatter(const int32_t* idx, const float* de, float* dwte, int M, int V, int d, int accumulate,
                        const EmbedSortBufs& b, hipStream_t st) {
  const int nch = (M + kChunk - 1) / kChunk;
  const int nwin = (M + kWin - 1) / kWin;
  NC_TRY(fill_u32(reinterpret_cast<uint32_t*>(b.hist), 0u, (size_t)nch * V, st));
  if (!accumulate) NC_TRY(fill_f32(dwte, 0.f, (size_t)V * d, st));
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
  ProfScope prof("embed_window_sum", 0, 4.0 * M * d + 8.0 * M + 4.0 * (double)d * M, st);
  hipLaunchKernelGGL(eb_window_kernel, dim3(nwin), dim3(256), 0, st, de, d, b.seg, b.perm, b.sid, V, dwte, b.spill);
  NC_LAUNCH_CHECK("eb_window");
  }
  if (nwin > 1) {
    ProfScope prof("embed_fixup", 0, 0, st);
    hipLaunchKernelGGL(eb_fixup_kernel, dim3(nwin - 1), dim3(256), 0, st, d, b.seg, b.sid, V, dwte, b.spill);
    NC_LAUNCH_CHECK("eb_fixup");
  }
  return NC_OK;
}

}  // namespace nc
