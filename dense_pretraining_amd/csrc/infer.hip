// Greedy generation with a key/value cache: the kernels that only inference
// needs. The pages describe an inference engine that keeps keys and values in
// a cache and runs a prefill pass and then decode steps (imeisheng.com,
// feature list and the end of section "预训练"; geoz.com.cn, sections
// "推理与部署" and "高效推理引擎与交互界面").
//
// Cache layout, per layer l and sequence b: K at [l][0][b][pos][G*D] and V at
// [l][1][b][pos][G*D], positions 0 .. capacity-1; K is stored after QK norm
// and rotation, exactly as attention consumes it.
#include "common.h"
#include "kernels.h"

namespace nc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// cache[b][pos0 + t] = src row (b * Tsrc + t), for the K and V column blocks.
template <typename T>
__global__ void __launch_bounds__(256) kv_store_kernel(const T* __restrict__ k, long ldk, const T* __restrict__ v,
                                                       long ldv, T* __restrict__ ck, T* __restrict__ cv, int B,
                                                       int Tsrc, int pos0, int cap, int GD) {
  constexpr int VE = 16 / sizeof(T);
  const int per_row = GD / VE;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)B * Tsrc * per_row) return;
  const int c = (int)(i % per_row);
  const long r = i / per_row;
  const int b = (int)(r / Tsrc), t = (int)(r % Tsrc);
  const long dst = ((long)b * cap + pos0 + t) * GD + (long)c * VE;
  *reinterpret_cast<uint4*>(ck + dst) = *reinterpret_cast<const uint4*>(k + r * ldk + (long)c * VE);
  *reinterpret_cast<uint4*>(cv + dst) = *reinterpret_cast<const uint4*>(v + r * ldv + (long)c * VE);
}

// out[b] = the lowest v with c tanh(z[b][v] / c) maximal.
__global__ void __launch_bounds__(256) argmax_softcap_kernel(const float* __restrict__ z, long ldz, int V, float cap,
                                                             int32_t* __restrict__ out) {
  __shared__ float wv[4];
  __shared__ int wi[4];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float best = -INFINITY;
  int bi = V;
  for (int v = tid; v < V; v += 256) {
    const float zz = cap * tanhf(z[(long)b * ldz + v] / cap);
    if (zz > best) {  // v grows: the first maximum of this thread is kept
      best = zz;
      bi = v;
    }
  }
  auto better = [](float a, int ia, float c, int ic) { return c > a || (c == a && ic < ia); };
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(best, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
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
    out[b] = bi;
  }
}

// y = act(sum_z part[z]) (+ res): the split partials in a fixed order.
template <typename T, typename TO>
__global__ void __launch_bounds__(256) splitk_act_kernel(const float* __restrict__ part, int nsplit, long n4,
                                                         TO* __restrict__ y, const T* __restrict__ res, int relu_sq) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int zz = 0; zz < nsplit; ++zz) {
      const float4 p = reinterpret_cast<const float4*>(part + (long)zz * n4 * 4)[i];
      a.x += p.x; a.y += p.y; a.z += p.z; a.w += p.w;
    }
    float v[4] = {a.x, a.y, a.z, a.w};
    if (relu_sq) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float r = fmaxf(v[e], 0.f);
        v[e] = r * r;
      }
    }
    if (res) {
      float rr[4];
      load4<T>(res + 4 * i, rr);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += rr[e];
    }
    store4<TO>(y + 4 * i, v);
  }
}

__global__ void iota_i32_kernel(int32_t* __restrict__ out, int n, int start, int step) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = start + i * step;
}

}  // namespace

template <typename T>
nc_status kv_store(const T* k, long ldk, const T* v, long ldv, T* ck, T* cv, int B, int Tsrc, int pos0, int cap,
                   int GD, hipStream_t st) {
  const long n = (long)B * Tsrc * (GD / (16 / (int)sizeof(T)));
  ProfScope prof(NC_NAME(T, "kv_store"), 0, 4.0 * sizeof(T) * B * Tsrc * GD, st);
  hipLaunchKernelGGL((kv_store_kernel<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, k, ldk, v, ldv, ck, cv,
                     B, Tsrc, pos0, cap, GD);
  NC_LAUNCH_CHECK("kv_store");
  return NC_OK;
}

nc_status argmax_softcap(const float* z, long ldz, int B, int V, float cap, int32_t* out, hipStream_t st) {
  ProfScope prof("argmax_softcap", 0, 4.0 * B * V, st);
  hipLaunchKernelGGL(argmax_softcap_kernel, dim3(B), dim3(256), 0, st, z, ldz, V, cap, out);
  NC_LAUNCH_CHECK("argmax_softcap");
  return NC_OK;
}

template <typename T>
nc_status splitk_act(const float* part, int nsplit, int M, int N, void* y, bool y_f32, const T* res, bool relu_sq,
                     hipStream_t st) {
  const long n4 = (long)M * N / 4;
  const long nb = (n4 + 255) / 256;
  const unsigned grid = (unsigned)(nb < 4096 ? nb : 4096);
  ProfScope prof("splitk_act", 0, 4.0 * M * N * nsplit + (y_f32 ? 4.0 : (double)sizeof(T)) * M * N, st);
  if (y_f32)
    hipLaunchKernelGGL((splitk_act_kernel<T, float>), dim3(grid), dim3(256), 0, st, part, nsplit, n4,
                       static_cast<float*>(y), res, relu_sq ? 1 : 0);
  else
    hipLaunchKernelGGL((splitk_act_kernel<T, T>), dim3(grid), dim3(256), 0, st, part, nsplit, n4, static_cast<T*>(y),
                       res, relu_sq ? 1 : 0);
  NC_LAUNCH_CHECK("splitk_act");
  return NC_OK;
}

nc_status iota_i32(int32_t* out, int n, int start, int step, hipStream_t st) {
  hipLaunchKernelGGL(iota_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, out, n, start, step);
  NC_LAUNCH_CHECK("iota");
  return NC_OK;
}

#define NC_INST(T)                                                                                              \
  template nc_status kv_store<T>(const T*, long, const T*, long, T*, T*, int, int, int, int, int, hipStream_t); \
  template nc_status splitk_act<T>(const float*, int, int, int, void*, bool, const T*, bool, hipStream_t);
NC_INST(bf16)
NC_INST(float)
#undef NC_INST

}  // namespace nc
