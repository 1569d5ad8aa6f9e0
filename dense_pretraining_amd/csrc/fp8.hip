// FP8 E4M3 operands of the forward products, one scale per tensor (the page
// on pomoai.com says the newest nanochat trains with FP8 and gives no
// recipe): a = max |v| over the tensor, q = E4M3(clip(fp32(v * fp32(448 / a)),
// -448, 448)) with round to nearest even (v_cvt_pk_fp8_f32, gfx950's OCP E4M3),
// dequantisation scale s = fp32(a / 448); a = 0 gives 1 for both.
//
// The activations' maxima come from the kernels that write them (RMSNorm,
// attention, the W1 epilogue), so an activation costs one pass here: read the
// bf16 tensor, write its codes. The weights take an amax pass first; the four
// of a block go through each pass in one launch.
#include "common.h"
#include "kernels.h"

namespace nc {
namespace {

constexpr int kQuantUnroll = 4;  // 16-byte loads in flight per thread

template <typename T>
__global__ void __launch_bounds__(256) amax_kernel(Fp8Tab<T> t, uint32_t* __restrict__ amax) {
  const int k = blockIdx.y;
  const T* __restrict__ x = t.x[k];
  const long n8 = t.n8[k];
  __shared__ float red[4];
  float m = 0.f;
  for (long b = (long)blockIdx.x * 256 * kQuantUnroll + threadIdx.x; b < n8; b += (long)gridDim.x * 256 * kQuantUnroll) {
    float v[kQuantUnroll][8];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const long i = b + 256 * u;
      if (i < n8) load16<T>(x + 8 * i, v[u]);
      else
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[u][e]));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) amax_publish(amax + (long)k * kAmaxWords, fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
}

__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <typename T>
__global__ void __launch_bounds__(256) quant_fp8_kernel(Fp8Tab<T> t, const uint32_t* __restrict__ amax,
                                                        float* __restrict__ scale) {
  const int k = blockIdx.y;
  const T* __restrict__ x = t.x[k];
  uint8_t* __restrict__ q = t.q[k];
  const long n8 = t.n8[k];
  const float a = amax_read(amax + (long)k * kAmaxWords);
  const float inv = a > 0.f ? 448.f / a : 1.f;
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[k] = a > 0.f ? a / 448.f : 1.f;
  for (long b = (long)blockIdx.x * 256 * kQuantUnroll + threadIdx.x; b < n8; b += (long)gridDim.x * 256 * kQuantUnroll) {
    float v[kQuantUnroll][8];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u)
      if (b + 256 * u < n8) load16<T>(x + 8 * (b + 256 * u), v[u]);
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const long i = b + 256 * u;
      if (i < n8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = fminf(fmaxf(v[u][e] * inv, -448.f), 448.f);
        *reinterpret_cast<uint2*>(q + 8 * i) =
            make_uint2(pack4_fp8(v[u][0], v[u][1], v[u][2], v[u][3]), pack4_fp8(v[u][4], v[u][5], v[u][6], v[u][7]));
      }
    }
  }
}

// Blocks along x: enough to cover the largest tensor once, at most 8 per CU.
dim3 tab_grid(long n8max, int count) {
  const long per = 256L * kQuantUnroll;
  long b = (n8max + per - 1) / per;
  b = b < 1 ? 1 : (b > 2048 ? 2048 : b);
  return dim3((unsigned)b, (unsigned)count);
}

template <typename T>
nc_status check_tab(const Fp8Tab<T>& t, int count, long* n8max, double* elems) {
  if (count < 1 || count > kFp8TabMax) return NC_ERR_INVALID_ARG;
  *n8max = 0;
  *elems = 0;
  for (int k = 0; k < count; ++k) {
    if (t.n8[k] < 0 || (t.n8[k] > 0 && !t.x[k])) return NC_ERR_INVALID_ARG;
    *n8max = t.n8[k] > *n8max ? t.n8[k] : *n8max;
    *elems += 8.0 * t.n8[k];
  }
  return NC_OK;
}

}  // namespace

template <typename T>
nc_status fp8_amax(const Fp8Tab<T>& t, int count, uint32_t* amax, hipStream_t st) {
  long n8max;
  double elems;
  NC_TRY(check_tab(t, count, &n8max, &elems));
  ProfScope prof("fp8_amax", 0, sizeof(T) * elems, st);
  hipLaunchKernelGGL((amax_kernel<T>), tab_grid(n8max, count), dim3(256), 0, st, t, amax);
  NC_LAUNCH_CHECK("amax");
  return NC_OK;
}

template <typename T>
nc_status fp8_quantize(const Fp8Tab<T>& t, int count, const uint32_t* amax, float* scale, hipStream_t st) {
  long n8max;
  double elems;
  NC_TRY(check_tab(t, count, &n8max, &elems));
  for (int k = 0; k < count; ++k)
    if (t.n8[k] > 0 && !t.q[k]) return NC_ERR_INVALID_ARG;
  ProfScope prof("quantize_fp8", 0, (sizeof(T) + 1.0) * elems, st);
  hipLaunchKernelGGL((quant_fp8_kernel<T>), tab_grid(n8max, count), dim3(256), 0, st, t, amax, scale);
  NC_LAUNCH_CHECK("quant_fp8");
  return NC_OK;
}

template nc_status fp8_amax<bf16>(const Fp8Tab<bf16>&, int, uint32_t*, hipStream_t);
template nc_status fp8_quantize<bf16>(const Fp8Tab<bf16>&, int, const uint32_t*, float*, hipStream_t);

}  // namespace nc
