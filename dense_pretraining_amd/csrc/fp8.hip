// FP8 E4M3 operands of the forward products, one scale per tensor (the page
// on pomoai.com says the newest nanochat trains with FP8 and gives no
// recipe): a = max |v| over the tensor, q = E4M3(clip(fp32(v * fp32(448 / a)),
// -448, 448)) with round to nearest even (v_cvt_pk_fp8_f32, gfx950's OCP E4M3),
// dequantisation scale s = fp32(a / 448); a = 0 gives 1 for both.
#include "common.h"
#include "kernels.h"

namespace nc {
namespace {

template <typename T>
__global__ void __launch_bounds__(256) amax_kernel(const T* __restrict__ x, long n8, uint32_t* __restrict__ out) {
  __shared__ float red[4];
  float m = 0.f;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    float v[8];
    load16<T>(x + 8 * i, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  // the bits of non-negative floats order like the floats: the maximum does not depend on the order
  if (threadIdx.x == 0) atomicMax(out, __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <typename T>
__global__ void __launch_bounds__(256) quant_fp8_kernel(const T* __restrict__ x, long n8,
                                                        const uint32_t* __restrict__ amax, uint8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
  const float a = __uint_as_float(*amax);
  const float inv = a > 0.f ? 448.f / a : 1.f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = a > 0.f ? a / 448.f : 1.f;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    float v[8];
    load16<T>(x + 8 * i, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = fminf(fmaxf(v[e] * inv, -448.f), 448.f);
    *reinterpret_cast<uint2*>(q + 8 * i) = make_uint2(pack4_fp8(v[0], v[1], v[2], v[3]), pack4_fp8(v[4], v[5], v[6], v[7]));
  }
}

unsigned grid8(long n8) {
  const long b = (n8 + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 4096 ? 4096 : b));
}

}  // namespace

template <typename T>
nc_status quantize_fp8(const T* x, long n, uint8_t* q, float* scale, uint32_t* amax, hipStream_t st) {
  if (n % 8 != 0) return NC_ERR_UNSUPPORTED;
  const long n8 = n / 8;
  ProfScope prof("quantize_fp8", 0, (2.0 * sizeof(T) + 1.0) * n, st);
  NC_TRY(fill_u32(amax, 0u, 1, st));
  hipLaunchKernelGGL((amax_kernel<T>), dim3(grid8(n8)), dim3(256), 0, st, x, n8, amax);
  NC_LAUNCH_CHECK("amax");
  hipLaunchKernelGGL((quant_fp8_kernel<T>), dim3(grid8(n8)), dim3(256), 0, st, x, n8, amax, q, scale);
  NC_LAUNCH_CHECK("quant_fp8");
  return NC_OK;
}

template nc_status quantize_fp8<bf16>(const bf16*, long, uint8_t*, float*, uint32_t*, hipStream_t);

}  // namespace nc
