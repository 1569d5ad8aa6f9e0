// Shared device helpers for the gfx950 kernels: storage types, conversions,
// wavefront reductions, the sticky device status word, launch checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/nc.h"

namespace nc {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kWave = 64;

// Status bits of the device status word (first 4 bytes of every scratch or
// workspace buffer). Bits are only ever OR-ed in; they stay set until cleared.
enum : uint32_t {
  kStatusBadToken = 1u << 0,    // an input token id outside [0, vocab)
  kStatusBadTarget = 1u << 1,   // a target outside [-1, vocab)
  kStatusNonFinite = 1u << 2,   // the loss is not finite
  kStatusNoTargets = 1u << 3,   // every target is ignored (-1)
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Elements per 16-byte vector of a storage type.
template <typename T> struct Vec { static constexpr int n = 16 / sizeof(T); };

// Load / store 16 bytes as float values.
template <typename T> __device__ __forceinline__ void load16(const T* p, float* out);
template <> __device__ __forceinline__ void load16<bf16>(const bf16* p, float* out) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void load16<float>(const float* p, float* out) {
  float4 u = *reinterpret_cast<const float4*>(p);
  out[0] = u.x; out[1] = u.y; out[2] = u.z; out[3] = u.w;
}

template <typename T> __device__ __forceinline__ void store16(T* p, const float* in);
template <> __device__ __forceinline__ void store16<bf16>(bf16* p, const float* in) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (bf16)in[i];
  *reinterpret_cast<bf16x8*>(p) = v;
}
template <> __device__ __forceinline__ void store16<float>(float* p, const float* in) {
  *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
}

// 4 consecutive elements (8 bytes of bf16, 16 of float).
template <typename T>
__device__ __forceinline__ void store4(T* p, const float* v);
template <> __device__ __forceinline__ void store4<bf16>(bf16* p, const float* v) {
  bf16x4 o;
  o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
  *reinterpret_cast<bf16x4*>(p) = o;
}
template <> __device__ __forceinline__ void store4<float>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <typename T>
__device__ __forceinline__ void load4(const T* p, float* v);
template <> __device__ __forceinline__ void load4<bf16>(const bf16* p, float* v) {
  uint2 u = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
}
template <> __device__ __forceinline__ void load4<float>(const float* p, float* v) {
  float4 u = *reinterpret_cast<const float4*>(p);
  v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int m = width >> 1; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// Running maximum magnitude of a tensor, kept as the bits of non-negative
// floats: those order like the floats, so unsigned atomic maxima reach the
// same words whatever the order of the calls. The maximum is spread over
// kAmaxStripes words kAmaxStride words (128 bytes) apart; a block publishes
// into the stripe of its index, so that thousands of blocks do not queue on
// one address, and the reader takes the largest stripe. Callers pass the
// maximum of the values they stored, in the storage type's rounding (which is
// monotonic: the rounded maximum is the maximum of the rounded values).
constexpr int kAmaxStripes = 64, kAmaxStride = 32;
constexpr int kAmaxWords = kAmaxStripes * kAmaxStride;  // uint32 words per tensor
__device__ __forceinline__ void amax_publish(uint32_t* amax, float m) {
  atomicMax(amax + (blockIdx.x % kAmaxStripes) * kAmaxStride, __float_as_uint(m));
}
// Lane 0 of each wave publishes the wave's maximum; nothing waits for the atomic.
__device__ __forceinline__ void amax_publish_wave(float m, uint32_t* amax) {
  m = wave_max(m);
  if ((threadIdx.x & (kWave - 1)) == 0) amax_publish(amax, m);
}
// The tensor's maximum, read by a whole wave (lane i reads stripe i).
__device__ __forceinline__ float amax_read(const uint32_t* amax) {
  static_assert(kAmaxStripes == kWave, "one stripe per lane");
  return wave_max(__uint_as_float(amax[(threadIdx.x & (kWave - 1)) * kAmaxStride]));
}

__device__ __forceinline__ void set_status(uint32_t* status, uint32_t bits) {
  if (status) atomicOr(status, bits);
}

// The unembedding logits (and their gradient, written in place) are stored in
// column panels of kPanel: element (m, v) of the [M, V] matrix at
// (v / kPanel) * M * kPanel + m * kPanel + v % kPanel. A k-tile of the input-grad
// GEMM (k = v) is then one contiguous block, instead of 64-byte pieces of rows
// that lie V * 2 bytes apart.
constexpr int kPanel = 32;
inline size_t logit_elems(long M, long V) { return (size_t)M * (size_t)((V + kPanel - 1) / kPanel * kPanel); }

// ---------------------------------------------------------------- direct-to-LDS loads
// buffer_load_* ... lds (gfx950) writes lane i's data at the LDS address in
// M0 plus i times the access size, whatever the source address. A buffer
// resource with a 2 GiB record turns any offset at or past kDmaOOB into a
// zero read, so out-of-range lanes need no branch.
constexpr unsigned kDmaRecords = 0x7ffffff0u;  // buffer record size (bytes)
constexpr unsigned kDmaOOB = 0x7ffffff0u;      // offset that reads as zero
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)kDmaRecords, 0x00020000);
}

// Ring barrier: this wave's loads older than the newest N have landed in
// LDS and its LDS reads are done (s_waitcnt vmcnt(N) lgkmcnt(0)), then all
// waves meet. A plain s_barrier: __syncthreads() would also drain the loads
// that are meant to stay in flight.
template <int N>
__device__ __forceinline__ void ring_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Records the HIP error text for nc_last_hip_error and maps it to a status.
nc_status record_hip_error(hipError_t e, const char* where);

#define NC_LAUNCH_CHECK(where)                                        \
  do {                                                                \
    hipError_t e_ = hipGetLastError();                                \
    if (e_ != hipSuccess) return ::nc::record_hip_error(e_, where);   \
  } while (0)

#define NC_TRY(...)                          \
  do {                                       \
    nc_status s_ = (__VA_ARGS__);            \
    if (s_ != NC_OK) return s_;              \
  } while (0)

}  // namespace nc
