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

// One (sequence, head) per LPH = D/8 lanes; lane j holds elements 4j.. of
// both halves of the head, so the rotation pairs (i, i + D/2) are lane-local.
template <typename T, int D>
__global__ void __launch_bounds__(256) qkv_finish_kernel(const float* __restrict__ part, int nsplit, int B, int d,
                                                         int H, int G, float eps, const float* __restrict__ cs,
                                                         const float* __restrict__ sn, T* __restrict__ q, long ldq,
                                                         T* __restrict__ ck, T* __restrict__ cv, int pos, int cap) {
  constexpr int P = D / 2, LPH = P / 4, HPB = 256 / LPH, U = 4;
  const int NH = H + 2 * G;
  const long QKV = (long)NH * D;
  const long pair = (long)blockIdx.x * HPB + threadIdx.x / LPH;
  const int j = threadIdx.x % LPH;
  if (pair >= (long)B * NH) return;  // whole lane groups leave together
  const int b = (int)(pair / NH), h = (int)(pair - (long)b * NH);

  // split-K sum in split order, loads of U splits in flight together
  float a[4] = {0.f, 0.f, 0.f, 0.f}, c[4] = {0.f, 0.f, 0.f, 0.f};
  const float* src = part + (long)b * QKV + (long)h * D + 4 * j;
  const long zs = (long)B * QKV;
  for (int z0 = 0; z0 < nsplit; z0 += U) {
    float4 pa[U], pb[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (z0 + u < nsplit) {
        pa[u] = *reinterpret_cast<const float4*>(src + (z0 + u) * zs);
        pb[u] = *reinterpret_cast<const float4*>(src + (z0 + u) * zs + P);
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (z0 + u < nsplit) {
        a[0] += pa[u].x; a[1] += pa[u].y; a[2] += pa[u].z; a[3] += pa[u].w;
        c[0] += pb[u].x; c[1] += pb[u].y; c[2] += pb[u].z; c[3] += pb[u].w;
      }
  }
  // the block's input RMSNorm, applied to the product: N(x) W^T = (x W^T) / rms(x)
  const float* ssp = part + (long)nsplit * zs;
  float ss = 0.f;
  for (int zz = 0; zz < nsplit; ++zz) ss += ssp[(long)zz * B + b];
  const float rs = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] *= rs;
    c[e] *= rs;
  }
  const long GD = (long)G * D;
  if (h >= H + G) {  // value head: stored as is
    T* dst = cv + ((long)b * cap + pos) * GD + (long)(h - H - G) * D + 4 * j;
    store4<T>(dst, a);
    store4<T>(dst + P, c);
    return;
  }
  float sq = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) sq += a[e] * a[e] + c[e] * c[e];
  const float rr = 1.f / sqrtf(group_sum(sq, LPH) / (float)D + eps);
  const float4 c4 = *reinterpret_cast<const float4*>(cs + 4 * j);
  const float4 s4 = *reinterpret_cast<const float4*>(sn + 4 * j);
  const float co[4] = {c4.x, c4.y, c4.z, c4.w}, si[4] = {s4.x, s4.y, s4.z, s4.w};
  float oa[4], ob[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float ya = a[e] * rr, yb = c[e] * rr;
    oa[e] = ya * co[e] - yb * si[e];
    ob[e] = ya * si[e] + yb * co[e];
  }
  T* dst = h < H ? q + (long)b * ldq + (long)h * D + 4 * j
                 : ck + ((long)b * cap + pos) * GD + (long)(h - H) * D + 4 * j;
  store4<T>(dst, oa);
  store4<T>(dst + P, ob);
}

}  // namespace

template <typename T>
nc_status qkv_finish(const float* part, int nsplit, int B, int d, int H, int G, int D, float eps, const float* cs,
                     const float* sn, T* q, long ldq, T* ck, T* cv, int pos, int cap, hipStream_t st) {
  const long pairs = (long)B * (H + 2 * G);
  ProfScope prof(NC_NAME(T, "qkv_finish"), 0,
                 4.0 * nsplit * pairs * D + sizeof(T) * (double)pairs * D, st);
  if (D == 128)
    hipLaunchKernelGGL((qkv_finish_kernel<T, 128>), dim3((unsigned)((pairs + 15) / 16)), dim3(256), 0, st, part, nsplit,
                       B, d, H, G, eps, cs, sn, q, ldq, ck, cv, pos, cap);
  else if (D == 64)
    hipLaunchKernelGGL((qkv_finish_kernel<T, 64>), dim3((unsigned)((pairs + 31) / 32)), dim3(256), 0, st, part, nsplit,
                       B, d, H, G, eps, cs, sn, q, ldq, ck, cv, pos, cap);
  else
    return NC_ERR_UNSUPPORTED;
  NC_LAUNCH_CHECK("qkv_finish");
  return NC_OK;
}

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

#define NC_INST(T)                                                                                                 \
  template nc_status kv_store<T>(const T*, long, const T*, long, T*, T*, int, int, int, int, int, hipStream_t);    \
  template nc_status qkv_finish<T>(const float*, int, int, int, int, int, int, float, const float*, const float*, T*, \
                                   long, T*, T*, int, int, hipStream_t);
NC_INST(bf16)
NC_INST(float)
#undef NC_INST

}  // namespace nc
