// MFMA operand fragments shared by the attention and few-row product kernels.
//
// A 32x32 MFMA (32x32x16 bf16, or eight 32x32x2 f32 steps for float storage)
// takes, per lane, 8 consecutive k-slots of row (lane % 32) of each operand:
// k = 8 * (lane / 32) + 0..7 within a 16-wide k step.
#pragma once
#include "common.h"

namespace nc {
namespace {

// An operand fragment: 8 consecutive k-slots of one lane.
template <typename T> struct F8;
template <> struct F8<bf16> { bf16x8 v; };
template <> struct F8<float> { float v[8]; };

__device__ __forceinline__ void mma32(f32x16& c, const F8<bf16>& a, const F8<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16& c, const F8<float>& a, const F8<float>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[s], b.v[s], c, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ F8<T> ld_row8(const T* p);
template <> __device__ __forceinline__ F8<bf16> ld_row8<bf16>(const bf16* p) {
  F8<bf16> f; f.v = *reinterpret_cast<const bf16x8*>(p); return f;
}
template <> __device__ __forceinline__ F8<float> ld_row8<float>(const float* p) {
  F8<float> f;
  float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w; f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}
// 4 elements from p0 then 4 from p1.
template <typename T> __device__ __forceinline__ F8<T> ld_split8(const T* p0, const T* p1);
template <> __device__ __forceinline__ F8<bf16> ld_split8<bf16>(const bf16* p0, const bf16* p1) {
  uint2 a = *reinterpret_cast<const uint2*>(p0), b = *reinterpret_cast<const uint2*>(p1);
  uint4 u = make_uint4(a.x, a.y, b.x, b.y);
  F8<bf16> f; f.v = *reinterpret_cast<bf16x8*>(&u); return f;
}
template <> __device__ __forceinline__ F8<float> ld_split8<float>(const float* p0, const float* p1) {
  float4 a = *reinterpret_cast<const float4*>(p0), b = *reinterpret_cast<const float4*>(p1);
  F8<float> f;
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w; f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}
template <typename T> __device__ __forceinline__ F8<T> pack8(const float* v);
template <> __device__ __forceinline__ F8<bf16> pack8<bf16>(const float* v) {
  F8<bf16> f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = (bf16)v[i];
  return f;
}
template <> __device__ __forceinline__ F8<float> pack8<float>(const float* v) {
  F8<float> f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = v[i];
  return f;
}
// Global fragment: 8 consecutive elements (zero if !ok).
template <typename T> __device__ __forceinline__ F8<T> gld8(const T* p, bool ok) {
  if (ok) return ld_row8<T>(p);
  float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  return pack8<T>(z);
}

}  // namespace
}  // namespace nc
