// Tiled MFMA GEMM for gfx950: C[m][n] = sum_k A(m,k) * B(n,k), fp32 accumulate.
//
// Every linear layer of the block and the unembedding (bias-free linears and
// untied unembedding from the architecture list on vpshk.cn) is one of three
// shapes of this kernel:
//   forward     y  = x W^T   A = x  [M,K] (K contiguous), B = W  [N,K] (K contiguous)
//   input grad  dx = dy W    A = dy [M,K] (K contiguous), B = W  [K,N] (K outer)
//   weight grad dW = dy^T x  A = dy [K,M] (K outer),      B = x  [K,N] (K outer)
// Both operands are staged in LDS as [row][k] so that each lane's MFMA
// fragment (8 consecutive k of one row) is one 16-byte LDS read; a K-outer
// operand is transposed while it is written to LDS.
//
// Block tile 128 x 128 (x BK), 256 threads = 4 wavefronts in a 2 x 2 grid,
// each owning 64 x 64 of C as 4 x 4 MFMA tiles of 16 x 16. bf16 storage uses
// v_mfma_f32_16x16x32_bf16 (BK = 64); float storage (check mode) uses eight
// v_mfma_f32_16x16x4_f32 per 32-wide k chunk (BK = 32). The MFMA's first
// source is the B fragment so that each lane ends up holding 4 consecutive
// columns of one row of C (lane l: row l%16, columns 4*(l/16)..+3).
// Tiles are walked in groups of 8 M-tiles, and each XCD (workgroups are
// dispatched round-robin over the 8 XCDs) gets a contiguous range of the
// walk, so that tiles sharing operand rows share an L2.
#pragma once

#include "common.h"

namespace nc {

enum OperandLayout { kKc = 0, kKo = 1 };

struct Identity {
  static constexpr bool active = false;
  __device__ __forceinline__ float operator()(float x) const { return x; }
};
// a = max(u, 0)^2: the ReLU^2 activation applied while an operand is loaded.
struct ReluSq {
  static constexpr bool active = true;
  __device__ __forceinline__ float operator()(float x) const {
    float r = fmaxf(x, 0.f);
    return r * r;
  }
};

template <typename T> struct GemmTile;
template <> struct GemmTile<bf16> {
  static constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;
};
template <> struct GemmTile<float> {
  static constexpr int BM = 128, BN = 128, BK = 32, LDK = BK + 4;
};

struct GemmShape {
  const void* A;
  const void* B;
  long lda, ldb;
  int M, N, K;
  int k_split;  // K range handled by one split (multiple of BK), K if unsplit
  int n_split;
};

// ---------------------------------------------------------------- tile walk

__device__ __forceinline__ void gemm_tile_coords(int tiles_m, int tiles_n, int& tm, int& tn, int& z) {
  int nb = gridDim.x;
  int pid = blockIdx.x;
  // contiguous range per XCD
  int xcd = pid & 7, local = pid >> 3;
  int per = nb >> 3, rem = nb & 7;
  int p = xcd * per + min(xcd, rem) + local;
  int per_split = tiles_m * tiles_n;
  z = p / per_split;
  int r = p - z * per_split;
  const int GM = 8;
  int group = r / (GM * tiles_n);
  int first_m = group * GM;
  int gm = min(tiles_m - first_m, GM);
  int in_group = r - group * GM * tiles_n;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// ---------------------------------------------------------------- loaders

// Global -> register stage of one operand tile (ROWS x BK), then -> LDS.
template <typename T, int Layout, int ROWS, typename Tr>
struct OperandLoader {
  static constexpr int BK = GemmTile<T>::BK;
  static constexpr int LDK = GemmTile<T>::LDK;
  static constexpr int VE = Vec<T>::n;  // elements per 16 B
  // Kc: ROWS * (BK / VE) vectors; Ko: (BK / 4) k-groups x (ROWS / VE) row vectors, 4 loads each
  static constexpr int NLOAD = 4;
  uint4 r[NLOAD];

  __device__ __forceinline__ void load(const T* __restrict__ g, long ld, int row0, int nrows, int k0, int kend,
                                       int tid) {
    if constexpr (Layout == kKc) {
      constexpr int VPR = BK / VE;  // vectors per row (8)
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) {
        int v = tid + 256 * i;
        int row = v / VPR, kv = v % VPR;
        int gr = row0 + row, gk = k0 + kv * VE;
        if (gr < nrows && gk < kend)
          r[i] = *reinterpret_cast<const uint4*>(g + (long)gr * ld + gk);
        else
          r[i] = make_uint4(0, 0, 0, 0);
      }
    } else {
      constexpr int NKG = BK / 4;  // k groups of 4 lines
      int kg = tid % NKG, rv = tid / NKG;
      int gr = row0 + rv * VE;
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) {
        int gk = k0 + kg * 4 + i;
        if (gk < kend && gr < nrows)
          r[i] = *reinterpret_cast<const uint4*>(g + (long)gk * ld + gr);
        else
          r[i] = make_uint4(0, 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void transform() {
    if constexpr (Tr::active) {
      Tr tr;
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) {
        float f[VE];
        load16<T>(reinterpret_cast<const T*>(&r[i]), f);
#pragma unroll
        for (int e = 0; e < VE; ++e) f[e] = tr(f[e]);
        store16<T>(reinterpret_cast<T*>(&r[i]), f);
      }
    }
  }

  __device__ __forceinline__ void store(T* __restrict__ s, int tid) {
    if constexpr (Layout == kKc) {
      constexpr int VPR = BK / VE;
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) {
        int v = tid + 256 * i;
        int row = v / VPR, kv = v % VPR;
        *reinterpret_cast<uint4*>(s + row * LDK + kv * VE) = r[i];
      }
    } else {
      constexpr int NKG = BK / 4;
      int kg = tid % NKG, rv = tid / NKG;
      if constexpr (sizeof(T) == 2) {
        // r[kk] holds rows rv*8 + 0..7 of k-line kk; write 4 k values per row.
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          int sh = (i & 1) * 16;
          uint32_t e0 = (w0[i >> 1] >> sh) & 0xffffu, e1 = (w1[i >> 1] >> sh) & 0xffffu;
          uint32_t e2 = (w2[i >> 1] >> sh) & 0xffffu, e3 = (w3[i >> 1] >> sh) & 0xffffu;
          uint2 o = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
          *reinterpret_cast<uint2*>(s + (rv * 8 + i) * LDK + kg * 4) = o;
        }
      } else {
        const float* f0 = reinterpret_cast<const float*>(&r[0]);
        const float* f1 = reinterpret_cast<const float*>(&r[1]);
        const float* f2 = reinterpret_cast<const float*>(&r[2]);
        const float* f3 = reinterpret_cast<const float*>(&r[3]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<float4*>(s + (rv * 4 + i) * LDK + kg * 4) = make_float4(f0[i], f1[i], f2[i], f3[i]);
        }
      }
    }
  }
};

// ---------------------------------------------------------------- MFMA core

template <typename T> struct Frag;
template <> struct Frag<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void read(const bf16* s) { v = *reinterpret_cast<const bf16x8*>(s); }
};
template <> struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void read(const float* s) {
    float4 a = *reinterpret_cast<const float4*>(s);
    float4 b = *reinterpret_cast<const float4*>(s + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

__device__ __forceinline__ void mfma_acc(f32x4& c, const Frag<bf16>& b, const Frag<bf16>& a) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.v, a.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mfma_acc(f32x4& c, const Frag<float>& b, const Frag<float>& a) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(b.v[s], a.v[s], c, 0, 0, 0);
}

// Per-lane view of the finished tile handed to an epilogue.
struct TileAcc {
  f32x4 c[4][4];  // c[i][j][v] = C[row(i)][col(j) + v]
};

template <typename T, int LA, int LB, typename TrA, typename TrB, typename Epi>
__global__ void __launch_bounds__(256, 2) gemm_kernel(GemmShape s, Epi epi) {
  using Cfg = GemmTile<T>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, LDK = Cfg::LDK;
  __shared__ __align__(16) T smem[2][(BM + BN) * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int tiles_m = (s.M + BM - 1) / BM, tiles_n = (s.N + BN - 1) / BN;
  int tm, tn, z;
  gemm_tile_coords(tiles_m, tiles_n, tm, tn, z);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = z * s.k_split;
  const int kend = min(s.K, kbeg + s.k_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  const T* __restrict__ A = static_cast<const T*>(s.A);
  const T* __restrict__ B = static_cast<const T*>(s.B);
  OperandLoader<T, LA, BM, TrA> la;
  OperandLoader<T, LB, BN, TrB> lb;

  TileAcc acc;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.c[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int frow = lane & 15, fk = (lane >> 4) * 8;

  if (nk > 0) {
    la.load(A, s.lda, m0, s.M, kbeg, kend, tid);
    lb.load(B, s.ldb, n0, s.N, kbeg, kend, tid);
    la.transform();
    lb.transform();
    la.store(smem[0], tid);
    lb.store(smem[0] + BM * LDK, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(A, s.lda, m0, s.M, kbeg + (kt + 1) * BK, kend, tid);
      lb.load(B, s.ldb, n0, s.N, kbeg + (kt + 1) * BK, kend, tid);
    }
    const T* sa = smem[kt & 1];
    const T* sb = sa + BM * LDK;
#pragma unroll
    for (int kc = 0; kc < BK; kc += 32) {
      Frag<T> fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i].read(sa + (wm + 16 * i + frow) * LDK + kc + fk);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j].read(sb + (wn + 16 * j + frow) * LDK + kc + fk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mfma_acc(acc.c[i][j], fb[j], fa[i]);
    }
    if (more) {
      la.transform();
      lb.transform();
      la.store(smem[(kt + 1) & 1], tid);
      lb.store(smem[(kt + 1) & 1] + BM * LDK, tid);
    }
    __syncthreads();
  }

  epi(acc, m0 + wm + frow, n0 + wn + (lane >> 4) * 4, z, lane, wave, reinterpret_cast<float*>(&smem[0][0]));
}

// ---------------------------------------------------------------- epilogues
// Called with row_base = first row of this lane (add 16*i), col_base = first
// of its 4 columns (add 16*j). `red` is LDS scratch usable after a barrier.

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

// C = acc (+ residual). Output in the storage type.
template <typename T>
struct EpiStore {
  T* C;
  long ldc;
  const T* res;  // optional residual, same layout as C
  long ldr;
  int M, N;
  __device__ __forceinline__ void operator()(TileAcc& a, int row_base, int col_base, int, int, int, float*) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = row_base + 16 * i;
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int col = col_base + 16 * j;
        if (col >= N) continue;
        float v[4] = {a.c[i][j][0], a.c[i][j][1], a.c[i][j][2], a.c[i][j][3]};
        if (res) {
          float r[4];
          load4<T>(res + (long)row * ldr + col, r);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += r[e];
        }
        store4<T>(C + (long)row * ldc + col, v);
      }
    }
  }
};

// du = acc * 2 max(u, 0): input grad of the ReLU^2 activation.
template <typename T>
struct EpiDReluSq {
  T* C;
  long ldc;
  const T* u;
  long ldu;
  int M, N;
  __device__ __forceinline__ void operator()(TileAcc& a, int row_base, int col_base, int, int, int, float*) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = row_base + 16 * i;
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int col = col_base + 16 * j;
        if (col >= N) continue;
        float uu[4], v[4];
        load4<T>(u + (long)row * ldu + col, uu);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = a.c[i][j][e] * 2.f * fmaxf(uu[e], 0.f);
        store4<T>(C + (long)row * ldc + col, v);
      }
    }
  }
};

// float32 output: a weight gradient (store or accumulate) or, with several
// K splits, the split's partial tile at C + z * split_stride.
struct EpiF32 {
  float* C;
  long ldc;
  long split_stride;
  int accumulate;
  int M, N;
  __device__ __forceinline__ void operator()(TileAcc& a, int row_base, int col_base, int z, int, int, float*) const {
    float* base = C + (long)z * split_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = row_base + 16 * i;
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int col = col_base + 16 * j;
        if (col >= N) continue;
        float* p = base + (long)row * ldc + col;
        float4 v = make_float4(a.c[i][j][0], a.c[i][j][1], a.c[i][j][2], a.c[i][j][3]);
        if (accumulate) {
          float4 o = *reinterpret_cast<float4*>(p);
          v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
        }
        *reinterpret_cast<float4*>(p) = v;
      }
    }
  }
};

// Unembedding epilogue: z' = c tanh(z / c) (the logit softcap of the
// architecture list), stored in the storage type; per row, the sum of
// exp(z') over this tile's 128 columns goes to part[row * n_tiles + tile]
// (|z'| <= c, so no running maximum is needed in float32); the float32 z'
// of the target column goes to zt[row].
template <typename T>
struct EpiSoftcap {
  T* Z;
  long ldz;
  float cap;
  const int32_t* targets;
  float* part;
  float* zt;
  int n_tiles;
  int M, N;
  __device__ __forceinline__ void operator()(TileAcc& a, int row_base, int col_base, int, int lane, int wave,
                                             float* red) const {
    const float two_over_c = 2.f / cap;
    float rowsum[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = row_base + 16 * i;
      rowsum[i] = 0.f;
      int tgt = (row < M) ? targets[row] : -1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int col = col_base + 16 * j;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // c tanh(x/c) = c - 2c / (exp(2x/c) + 1)
          float ex = __expf(a.c[i][j][e] * two_over_c);
          v[e] = cap - 2.f * cap / (ex + 1.f);
        }
        if (row < M && col < N) {
          store4<T>(Z + (long)row * ldz + col, v);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            rowsum[i] += __expf(v[e]);
            if (col + e == tgt) zt[row] = v[e];
          }
        }
      }
      // sum over the 4 lane groups holding the other columns of this row
      rowsum[i] += __shfl_xor(rowsum[i], 16, 64);
      rowsum[i] += __shfl_xor(rowsum[i], 32, 64);
    }
    __syncthreads();  // operand LDS is free now
    const int wn_idx = wave & 1, wm = (wave >> 1) * 64;
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wn_idx * 128 + wm + 16 * i + lane] = rowsum[i];
    }
    __syncthreads();
    int tid = threadIdx.x;
    if (tid < 128) {
      int row = (row_base - wm - (lane & 15)) + tid;  // block's first row + tid
      (void)row;
    }
    if (tid < 128) {
      int block_row0 = row_base - (wave >> 1) * 64 - (lane & 15);
      int row = block_row0 + tid;
      int tile = (col_base - (wave & 1) * 64 - (lane >> 4) * 4) / 128;
      if (row < M) part[(long)row * n_tiles + tile] = red[tid] + red[128 + tid];
    }
  }
};

// ---------------------------------------------------------------- launcher

template <typename T, int LA, int LB, typename TrA, typename TrB, typename Epi>
nc_status launch_gemm(const GemmShape& s, const Epi& epi, hipStream_t stream) {
  using Cfg = GemmTile<T>;
  int tiles_m = (s.M + Cfg::BM - 1) / Cfg::BM, tiles_n = (s.N + Cfg::BN - 1) / Cfg::BN;
  long blocks = (long)tiles_m * tiles_n * s.n_split;
  if (blocks <= 0) return NC_OK;
  hipLaunchKernelGGL((gemm_kernel<T, LA, LB, TrA, TrB, Epi>), dim3((unsigned)blocks), dim3(256), 0, stream, s, epi);
  NC_LAUNCH_CHECK("gemm");
  return NC_OK;
}

}  // namespace nc
