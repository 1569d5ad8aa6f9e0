// Tiled MFMA GEMM for gfx950: C[m][n] = sum_k A(m,k) * B(n,k), fp32 accumulate.
//
// Every linear layer of the block and the unembedding (bias-free linears and
// untied unembedding from the architecture list on vpshk.cn) is one of three
// shapes of this kernel:
//   forward     y  = x W^T   A = x  [M,K] (K contiguous), B = W  [N,K] (K contiguous)
//   input grad  dx = dy W    A = dy [M,K] (K contiguous), B = W  [K,N] (K outer)
//   weight grad dW = dy^T x  A = dy [K,M] (K outer),      B = x  [K,N] (K outer)
// A K-contiguous operand is staged in LDS as [row][k] and each lane's MFMA
// fragment (8 consecutive k of one row) is one 16-byte LDS read. A K-outer
// operand is copied to LDS as it lies in memory, [k][row], and the fragment
// is gathered with two gfx950 transposing LDS reads (ds_read_b64_tr_b16), so
// neither layout costs a register transpose.
//
// bf16: block tile 256 x 256 x 64, 256 threads = 4 wavefronts in a 2 x 2
// grid, each owning 128 x 128 of C as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16
// (256 fp32 accumulators per lane, kept in AGPRs). Per 16-deep k step a wave
// reads 8 fragments (8 KB) for 16 MFMAs, 64 B of LDS per CU clock at full
// MFMA rate. Float storage (check mode) runs the same code on 128 x 128 x 32
// tiles with eight 32x32x2 f32 MFMAs per fragment pair.
// The MFMA's first source is the B fragment, so each lane ends up holding
// one row of C and runs of 4 consecutive columns.
// Tiles are walked in groups of 8 M-tiles, and each XCD (workgroups are
// dispatched round-robin over the 8 XCDs) gets a contiguous range of the
// walk, so that tiles sharing operand rows share an L2.
#pragma once

#include <utility>

#include <type_traits>

#include "common.h"

namespace nc {

enum OperandLayout { kKc = 0, kKo = 1 };

template <typename T> struct GemmTile;
template <> struct GemmTile<bf16> {
  static constexpr int BM = 256, BN = 256, BK = 32, WTM = 4, WTN = 4;
};
template <> struct GemmTile<float> {
  static constexpr int BM = 128, BN = 128, BK = 32, WTM = 2, WTN = 2;
};

struct GemmShape {
  const void* A;
  const void* B;
  long lda, ldb;
  int M, N, K;
  int k_split;  // K range handled by one split (multiple of BK), K if unsplit
  int n_split;
  // A in column panels of kPanel (the unembedding logits): element (r, c) of
  // the stored [R, C] matrix at (c / kPanel) * a_panel + r * kPanel + c % kPanel;
  // 0 = plain row-major with stride lda.
  long a_panel = 0;
  // independent products of the same shape: problem b reads A + b * a_batch
  // and B + b * b_batch (elements); the epilogue sees b in EpiCtx::batch
  int batch = 1;
  long a_batch = 0, b_batch = 0;
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
  // groups of GM M-tiles, walked M-fastest. An XCD's 32 concurrent tiles then
  // span about 32 / GM N-tiles, so an A panel (a block of activation rows) is
  // fetched by about tiles_n GM / 32 XCDs. GM = 3 measured best over 1, 2, 4,
  // 6, 8 and 16 on the depth-20 step (8: 2.3 ms slower, 16: 5 ms slower).
  const int GM = 3;
  int group = r / (GM * tiles_n);
  int first_m = group * GM;
  int gm = min(tiles_m - first_m, GM);
  int in_group = r - group * GM * tiles_n;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// ---------------------------------------------------------------- fragments

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void mfma32(f32x16& c, const Frag<bf16>& b, const Frag<bf16>& a) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b.v, a.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mfma32(f32x16& c, const Frag<float>& b, const Frag<float>& a) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(b.v[s], a.v[s], c, 0, 0, 0);
}

// 8 consecutive k of one row from a [row][k] tile.
template <typename T> __device__ __forceinline__ Frag<T> frag_row(const T* p);
template <> __device__ __forceinline__ Frag<bf16> frag_row<bf16>(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
template <> __device__ __forceinline__ Frag<float> frag_row<float>(const float* p) {
  Frag<float> f;
  float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w; f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}

typedef short gemm_v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) gemm_v4i16 gemm_lds_v4i16;

// Row r0 + lane%16, k = k0 .. k0+7, from a [k][row] tile (row stride LD).
// Transposing read: inside each 16-lane group, source lane j points at k row
// k0 + j/4, rows r0 + 4*(j%4) .. +3, and lane i receives the 4 k values of
// row r0 + i (layout measured on the device).
template <typename T> __device__ __forceinline__ Frag<T> frag_col(const T* xt, int LD, int k0, int r0, int lane);
template <> __device__ __forceinline__ Frag<bf16> frag_col<bf16>(const bf16* xt, int LD, int k0, int r0, int lane) {
  const int j = lane & 15;
  const bf16* p = xt + (k0 + (j >> 2)) * LD + r0 + 4 * (j & 3);
  gemm_v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((gemm_lds_v4i16*)const_cast<bf16*>(p));
  gemm_v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((gemm_lds_v4i16*)const_cast<bf16*>(p + 4 * LD));
  uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  uint4 u = make_uint4(ua.x, ua.y, ub.x, ub.y);
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, u);
  return f;
}
template <> __device__ __forceinline__ Frag<float> frag_col<float>(const float* xt, int LD, int k0, int r0,
                                                                    int lane) {
  const int r = r0 + (lane & 15);
  Frag<float> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = xt[(k0 + s) * LD + r];
  return f;
}

// ---------------------------------------------------------------- loaders

// One operand tile (ROWS x BK) : global -> registers -> LDS.
template <typename T, int Layout, int ROWS>
struct OperandLoader {
  static constexpr int BK = GemmTile<T>::BK;
  static constexpr int VE = Vec<T>::n;  // elements per 16 B
  // LDS row stride: [row][k] rows of BK + 16 B; [k][row] rows of ROWS + 32 B
  static constexpr int LD = Layout == kKc ? BK + VE : ROWS + 2 * VE;
  static constexpr int SIZE = Layout == kKc ? ROWS * LD : BK * LD;
  static constexpr int NV = ROWS * BK / VE;
  static constexpr int NLOAD = NV / 256;
  static_assert(NV % 256 == 0, "tile must split evenly over 256 threads");
  uint4 r[NLOAD];

  __device__ __forceinline__ void load(const T* __restrict__ g, long ld, int row0, int nrows, int k0, int kend,
                                       int tid, long panel) {
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const int v = tid + 256 * i;
      if constexpr (Layout == kKc) {
        constexpr int VPR = BK / VE;
        const int row = v / VPR, kv = v % VPR;
        const int gr = row0 + row, gk = k0 + kv * VE;
        const long a = panel ? (long)(gk / kPanel) * panel + (long)gr * kPanel + gk % kPanel : (long)gr * ld + gk;
        r[i] = (gr < nrows && gk < kend) ? *reinterpret_cast<const uint4*>(g + a) : make_uint4(0, 0, 0, 0);
      } else {
        constexpr int VPL = ROWS / VE;
        const int kl = v / VPL, rv = v % VPL;
        const int gk = k0 + kl, gr = row0 + rv * VE;
        const long a = panel ? (long)(gr / kPanel) * panel + (long)gk * kPanel + gr % kPanel : (long)gk * ld + gr;
        r[i] = (gk < kend && gr < nrows) ? *reinterpret_cast<const uint4*>(g + a) : make_uint4(0, 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void store(T* __restrict__ s, int tid) const {
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const int v = tid + 256 * i;
      if constexpr (Layout == kKc) {
        constexpr int VPR = BK / VE;
        *reinterpret_cast<uint4*>(s + (v / VPR) * LD + (v % VPR) * VE) = r[i];
      } else {
        constexpr int VPL = ROWS / VE;
        *reinterpret_cast<uint4*>(s + (v / VPL) * LD + (v % VPL) * VE) = r[i];
      }
    }
  }

  // Fragment of tile row `row` (0..ROWS), k = k0..k0+7, for this lane
  // (row = base + lane % 32 in the caller).
  __device__ __forceinline__ static Frag<T> frag(const T* s, int row_base, int k0, int lane) {
    if constexpr (Layout == kKc) {
      return frag_row<T>(s + (row_base + (lane & 31)) * LD + k0);
    } else {
      return frag_col<T>(s, LD, k0, row_base + 16 * ((lane >> 4) & 1), lane);
    }
  }
};

// ---------------------------------------------------------------- kernel

template <typename T>
struct TileAcc {
  static constexpr int WTM = GemmTile<T>::WTM, WTN = GemmTile<T>::WTN;
  // c[i][j][4*g + e] = C[m_base + 32 i][n_base + 32 j + 8 g + e]
  f32x16 c[WTM][WTN];
};

// ---------------------------------------------------------------- epilogues
// The accumulators leave through LDS: each wave owns a 32-row x (32*WTN)
// float32 slab (16-byte chunks XOR-swizzled by row, so both the column-wise
// writes and the row-wise reads are conflict-free). Phase 1 runs in the
// accumulator layout, where a lane holds one row and runs of 4 columns
// (epi.pre may transform the values and keep per-row state); phase 2 reads
// the slab back so that 16 consecutive lanes cover 64 consecutive columns of
// one row, and epi.post writes 4 values per lane: each store instruction
// fills whole 128-byte lines of 4 rows instead of touching 32 rows.

struct EpiCtx {
  int m0, n0;     // block tile origin
  int wm, wn;     // wave sub-tile origin inside the block tile
  int z;          // K split
  int lane, wave;
  float* red;     // LDS scratch beside the slabs (2 * BM floats)
  int batch;      // problem index of a batched launch
  float scale = 1.f;  // FP8 products: the operands' scale product, read once per tile
};

// A store-phase group of 4 values: its row and first column, the parts of
// them that are the same in every lane (ru rows and cu columns past the
// lane's first group), and off, the group's byte offset in a row-major
// output from its 32-row block's first row and the wave's first column
// (kDmaOOB for a column at or past N): the store phase's offsets are the
// same 16 values in every row block, so they are formed once per tile.
struct EpiPos {
  int row, col, ru, cu, off;
};

// The dequantisation scale product of an FP8 epilogue (members sa, sb), 1 otherwise.
template <typename Epi, typename = void>
struct EpiScaled { static constexpr bool value = false; };
template <typename Epi>
struct EpiScaled<Epi, std::void_t<decltype(Epi::sa)>> { static constexpr bool value = true; };
template <typename Epi>
__device__ __forceinline__ float epi_scale(const Epi& e) {
  if constexpr (EpiScaled<Epi>::value) return e.sa ? *e.sa * *e.sb : 1.f;
  else return 1.f;
}


// A wave's LDS instructions execute in order, and the compiler keeps the slab
// writes and reads (lane-dependent addresses it cannot tell apart) in program
// order, so no fence is needed between the two phases.

// Epilogues that can report the largest stored magnitude (kTracksMax).
template <typename Epi, typename = void>
struct EpiTracksMax { static constexpr bool value = false; };
template <typename Epi>
struct EpiTracksMax<Epi, std::void_t<decltype(Epi::kTracksMax)>> { static constexpr bool value = Epi::kTracksMax; };

// Epilogues whose store phase only rounds to bf16 and stores (kPacked; no
// second input): staged_epilogue_packed below.
template <typename Epi, typename = void>
struct EpiPacked { static constexpr bool value = false; };
template <typename Epi>
struct EpiPacked<Epi, std::void_t<decltype(Epi::kPacked)>> {
  static constexpr bool value = Epi::kPacked && Epi::kOutBytes == 2;
};

typedef int epi_v2i __attribute__((ext_vector_type(2)));
typedef int epi_v4i __attribute__((ext_vector_type(4)));

// The staged epilogue of a kPacked epilogue: phase 1 applies epi.pre and
// rounds to bf16 in the accumulator layout, so the slab holds bf16 (32 rows
// of 128 columns, 8 KB a wave) and phase 2 moves half the bytes of the
// float32 slab through LDS. A phase-2 lane reads 8 consecutive columns (one
// 16-byte chunk) of a row, 16 lanes cover the wave's 128 columns of one row,
// and epi.store8 writes the chunk with one 16-byte store. Slab row r, chunk c
// sits at byte 256 r + 16 (c ^ (r & 15)): a phase-1 write (the two lane
// halves fill the two 8-byte halves of one chunk of rows 0..31) and a phase-2
// read (4 rows of 16 chunks) each spread over all banks. Every output column
// count is a multiple of 8 (checked by the launchers), so a chunk lies wholly
// inside or wholly outside the matrix.
template <int WTM, int WTN, typename Epi, bool Scaled>
__device__ __forceinline__ void staged_epilogue_packed(f32x16 (&c)[WTM][WTN], const Epi& epi, const EpiCtx& x,
                                                       float* slab_f) {
  static_assert(WTN == 4, "a slab row is the wave's 128 columns: 16 chunks of 8 bf16");
  static_assert(!EpiTracksMax<Epi>::value, "maximum tracking keeps the float32 slab");
  const int lane = x.lane, lr = lane & 31, h = lane >> 5;
  const int r0 = x.m0 + x.wm, c0 = x.n0 + x.wn;
  char* const slab = reinterpret_cast<char*>(slab_f);
  // phase 1: lane (lr, h) writes half h of chunk 4j + g of row lr
  char* const w1 = slab + 256 * lr + 8 * h;
  const int s1 = lr & 15;
  // phase 2: row 4 it + lane / 16, chunk lane % 16, whose slot
  // (lane % 16) ^ (lane / 16) ^ 4 (it % 4) is one of four per-lane bases
  const char* r2[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) r2[t] = slab + 256 * (lane >> 4) + 16 * (((lane & 15) ^ (lane >> 4)) ^ (4 * t));
  const int cq = 8 * (lane & 15);  // the lane's first store-phase column past c0
  // store offsets from the wave's 32-row block origin, the same in every block
  int goff[8];
  {
    const unsigned ld = (unsigned)epi.out_ld(), lrow = lane >> 4;
#pragma unroll
    for (int it = 0; it < 8; ++it)
      goff[it] = c0 + cq < epi.N ? (int)((__umul24(4 * it + lrow, ld) + (unsigned)cq) * 2u) : (int)kDmaOOB;
  }
  typename Epi::RowState rs[WTM];
#pragma unroll
  for (int i = 0; i < WTM; ++i) epi.row_begin(rs[i], r0 + 32 * i + lr);
#pragma unroll
  for (int i = 0; i < WTM; ++i) {
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4] = {c[i][j][4 * g], c[i][j][4 * g + 1], c[i][j][4 * g + 2], c[i][j][4 * g + 3]};
        if constexpr (Scaled) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= x.scale;
        }
        const int row = r0 + 32 * i + lr, col = c0 + 32 * j + 8 * g + 4 * h;
        epi.pre(rs[i], row, col, v);
        bf16x4 o;
        o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
        *reinterpret_cast<uint2*>(w1 + 16 * ((4 * j + g) ^ s1)) = __builtin_bit_cast(uint2, o);
      }
    epi.row_end(rs[i], x, i);
    uint4 q[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) q[it] = *reinterpret_cast<const uint4*>(r2[it & 3] + 1024 * it);
#pragma unroll
    for (int it = 0; it < 8; ++it)
      epi.store8(x, EpiPos{r0 + 32 * i + 4 * it + (lane >> 4), c0 + cq, 32 * i + 4 * it, 0, goff[it]}, q[it]);
  }
}

// Scaled: multiply the accumulators by x.scale first (FP8 products only; a
// multiply per element costs about a microsecond of a tile's epilogue).
template <int WTM, int WTN, typename Epi, bool Scaled = false>
__device__ __forceinline__ void staged_epilogue(f32x16 (&c)[WTM][WTN], const Epi& epi, const EpiCtx& x,
                                                float* slab) {
  if constexpr (EpiPacked<Epi>::value) {
    staged_epilogue_packed<WTM, WTN, Epi, Scaled>(c, epi, x, slab);
    return;
  }
  constexpr int NCH = 8 * WTN;  // 16-byte chunks per slab row
  constexpr bool kMax = EpiTracksMax<Epi>::value;
  constexpr int kReadBatch = (kMax || !std::is_empty<typename Epi::RowState>::value) ? 4 : 8;
  const int lane = x.lane, lr = lane & 31, h = lane >> 5;
  const int r0 = x.m0 + x.wm, c0 = x.n0 + x.wn;
  float tmax = 0.f;
  // Slab row r, chunk c sits at slab + 4 (r NCH + (c ^ (r & 15))). A phase-1
  // write has c = 8j + 2g + h with h the lane's bit 0, so c ^ (r & 15) is
  // (8j + 2g) ^ s1 for a per-lane s1; a phase-2 read has r = 4 it + lane / 16
  // and c = lane % 16 + 16 k, so its address is one of four per-lane bases
  // (it mod 4) plus a constant.
  float* const w1 = slab + 4 * lr * NCH;
  const int s1 = (lr & 15) ^ h;
  const float* r2[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    r2[t] = slab + 4 * ((lane >> 4) * NCH + (((lane & 15) ^ (lane >> 4)) ^ (4 * t)));
  // the store phase's byte offsets (EpiPos::off), one per group of a row
  // block; a row past M is left to the row block's buffer record
  int goff[8][NCH / 16];
  {
    const unsigned ld = (unsigned)epi.out_ld(), lrow = lane >> 4, lcol = 4 * (lane & 15);
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
      for (int k = 0; k < NCH / 16; ++k)
        goff[it][k] = c0 + (int)lcol + 64 * k < epi.N
                          ? (int)((__umul24(4 * it + lrow, ld) + lcol + 64 * k) * Epi::kOutBytes)
                          : (int)kDmaOOB;
  }
  // every row's state first: whatever it loads is in flight before the first store
  typename Epi::RowState rs[WTM];
#pragma unroll
  for (int i = 0; i < WTM; ++i) epi.row_begin(rs[i], r0 + 32 * i + lr);
#pragma unroll
  for (int i = 0; i < WTM; ++i) {
    // the slab's other inputs (residual, activation) are fetched first, in
    // the phase-2 layout, so that their latency hides behind phase 1
    typename Epi::Aux aux[8][NCH / 16];
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
      for (int k = 0; k < NCH / 16; ++k)
        aux[it][k] = epi.load_aux(x, EpiPos{r0 + 32 * i + 4 * it + (lane >> 4), c0 + 4 * ((lane & 15) + 16 * k),
                                            32 * i + 4 * it, 64 * k, goff[it][k]});
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4] = {c[i][j][4 * g], c[i][j][4 * g + 1], c[i][j][4 * g + 2], c[i][j][4 * g + 3]};
        if constexpr (Scaled) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= x.scale;
        }
        const int cc = 8 * j + 2 * g + h;
        epi.pre(rs[i], r0 + 32 * i + lr, c0 + 4 * cc, v);
        *reinterpret_cast<float4*>(w1 + 4 * ((8 * j + 2 * g) ^ s1)) = make_float4(v[0], v[1], v[2], v[3]);
      }
    epi.row_end(rs[i], x, i);
    // a batch of the slab's reads first, then its stores: the reads overlap
    // and are waited for together, instead of one read, one wait, one store
    // at a time (half batches where the epilogue's own registers are many)
#pragma unroll
    for (int b0 = 0; b0 < 8; b0 += kReadBatch) {
      float4 q[kReadBatch][NCH / 16];
#pragma unroll
      for (int ib = 0; ib < kReadBatch; ++ib) {
        const int it = b0 + ib;
#pragma unroll
        for (int k = 0; k < NCH / 16; ++k)
          q[ib][k] = *reinterpret_cast<const float4*>(r2[it & 3] + 4 * (4 * it * NCH + 16 * k));
      }
#pragma unroll
      for (int ib = 0; ib < kReadBatch; ++ib) {
        const int it = b0 + ib, rr = 4 * it + (lane >> 4);
#pragma unroll
        for (int k = 0; k < NCH / 16; ++k) {
          const int cc = (lane & 15) + 16 * k;
          float v[4] = {q[ib][k].x, q[ib][k].y, q[ib][k].z, q[ib][k].w};
          epi.post(x, EpiPos{r0 + 32 * i + rr, c0 + 4 * cc, 32 * i + 4 * it, 64 * k, goff[it][k]}, v, aux[it][k]);
          if constexpr (kMax) epi.track(tmax, r0 + 32 * i + rr, c0 + 4 * cc, v);
        }
      }
    }
  }
  if constexpr (kMax) epi.publish(tmax);
}

// Four values of a second [M,N] input in the storage type, fetched ahead.
template <typename T> struct Aux4;
template <> struct Aux4<bf16> { uint2 u; };
template <> struct Aux4<float> { float4 u; };
template <typename T>
__device__ __forceinline__ Aux4<T> aux_load(const T* p, bool ok) {
  Aux4<T> a;
  if constexpr (sizeof(T) == 2) a.u = ok ? *reinterpret_cast<const uint2*>(p) : make_uint2(0, 0);
  else a.u = ok ? *reinterpret_cast<const float4*>(p) : make_float4(0, 0, 0, 0);
  return a;
}
template <typename T>
__device__ __forceinline__ void aux_get(const Aux4<T>& a, float* v) {
  if constexpr (sizeof(T) == 2) {
    v[0] = __uint_as_float(a.u.x << 16); v[1] = __uint_as_float(a.u.x & 0xffff0000u);
    v[2] = __uint_as_float(a.u.y << 16); v[3] = __uint_as_float(a.u.y & 0xffff0000u);
  } else {
    v[0] = a.u.x; v[1] = a.u.y; v[2] = a.u.z; v[3] = a.u.w;
  }
}
struct NoAux {};

// Branch-free epilogue I/O. A buffer resource starts at the first row of a
// wave's 32-row block and its first column, and its record ends at the
// matrix's last row, so a row at or past M is out of the record with no test
// per element: the hardware drops such stores and reads such loads as zero.
// A column at or past N has an offset past the record (EpiPos::off). With no
// branch and no address arithmetic per group, the slab reads and stores of a
// row are scheduled together instead of one read, one wait, one store at a
// time. Offsets within a row block: 32 ld es < 2^31 (every launcher checks
// 256 ld es), and the rows' factor fits 24 bits.
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const T* base, long ld, const EpiCtx& x, int M,
                                                            const EpiPos& p) {
  const int row0 = x.m0 + x.wm + (p.ru & ~31);
  const long rem = (long)(M - row0) * ld * (long)sizeof(T);
  const long rec = rem < 0 ? 0L : rem < (long)kDmaRecords ? rem : (long)kDmaRecords;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base + (long)row0 * ld + x.n0 + x.wn), (short)0,
                                           (int)rec, 0x00020000);
}
// bf16 tiles are stored non-temporal (cache policy bit nt): an output tile is
// written once and read by a later kernel, and streaming it past the caches
// made the store-heavy products 3-10 % faster (the unembedding's 8.6 GB of
// logits most).
constexpr int kStoreStream = 2;
template <typename T>
__device__ __forceinline__ void tile_store4(__amdgpu_buffer_rsrc_t rs, int off, const float* v) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 o;
    o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(epi_v2i, o), rs, off, 0, kStoreStream);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(epi_v4i, make_float4(v[0], v[1], v[2], v[3])), rs, off,
                                           0, 0);
  }
}
template <typename T>
__device__ __forceinline__ Aux4<T> tile_load4(__amdgpu_buffer_rsrc_t rs, int off) {
  Aux4<T> a;
  if constexpr (sizeof(T) == 2) a.u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
  else a.u = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  return a;
}

// Hooks of an epilogue with no per-row state and no phase-1 work.
#define NC_EPI_NO_ROW_WORK                                                          \
  struct RowState {};                                                               \
  __device__ __forceinline__ void row_begin(RowState&, int) const {}                \
  __device__ __forceinline__ void pre(RowState&, int, int, float*) const {}         \
  __device__ __forceinline__ void row_end(RowState&, const EpiCtx&, int) const {}   \
  __device__ __forceinline__ void finish(const EpiCtx&) const {}

// C = act(acc) (+ residual), act = identity or the ReLU^2 activation
// max(x, 0)^2. Output in the storage type. With TrackMax, the largest stored
// |C| goes into the striped maximum at amax (an FP8 operand's scale). The
// residual is a compile-time choice (HasRes): a residual load waited for after
// the slab's first store makes the compiler drain every store in flight (one
// counter covers loads and stores, and it cannot assume they retire in
// order), so an epilogue without one must carry no loads at all.
template <typename T, bool ReluSqOut = false, bool TrackMax = false, bool HasRes = false>
struct EpiStore {
  struct RowState {};
  __device__ __forceinline__ void row_begin(RowState&, int) const {}
  __device__ __forceinline__ void row_end(RowState&, const EpiCtx&, int) const {}
  __device__ __forceinline__ void finish(const EpiCtx&) const {}
  T* C;
  long ldc;
  const T* res;  // optional residual, C's layout (the same leading dimension: one offset serves both)
  int M, N;
  const float* sa = nullptr;  // FP8 products: the two operands' dequantisation scales, multiplied in first
  const float* sb = nullptr;
  uint32_t* amax = nullptr;   // TrackMax: the striped maximum
  static constexpr bool kTracksMax = TrackMax;
  static constexpr int kOutBytes = sizeof(T);
  // without a residual the store phase only rounds and stores (the FP8
  // operand's maximum tracking keeps the float32 slab: packed, it spilled)
  static constexpr bool kPacked = !HasRes && !TrackMax;
  __device__ __forceinline__ long out_ld() const { return ldc; }
  using Aux = std::conditional_t<HasRes, Aux4<T>, NoAux>;
  __device__ __forceinline__ Aux load_aux(const EpiCtx& x, const EpiPos& p) const {
    if constexpr (HasRes) return tile_load4<T>(block_rsrc(res, ldc, x, M, p), p.off);
    else return Aux{};
  }
  // the activation, in phase 1 (an FP8 product's scale is applied to the
  // accumulators before it)
  __device__ __forceinline__ void pre(RowState&, int, int, float* v) const {
    if constexpr (ReluSqOut) {
      // max(v, 0) as one median of three (fmaxf adds a canonicalising max per
      // element: 256 more vector instructions per thread and tile)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float r = __builtin_amdgcn_fmed3f(v[e], 0.f, 3.402823466e38f);
        v[e] = r * r;
      }
    }
  }
  __device__ __forceinline__ void post(const EpiCtx& x, const EpiPos& p, float* v, const Aux& a) const {
    if constexpr (HasRes) {
      float r[4];
      aux_get<T>(a, r);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += r[e];
    }
    tile_store4<T>(block_rsrc(C, ldc, x, M, p), p.off, v);
  }
  // kPacked: 8 rounded values of one row
  __device__ __forceinline__ void store8(const EpiCtx& x, const EpiPos& p, const uint4& q) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(epi_v4i, q), block_rsrc(C, ldc, x, M, p), p.off, 0,
                                           kStoreStream);
  }
  // the stored values before rounding
  __device__ __forceinline__ void track(float& t, int row, int col, const float* v) const {
    const float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    t = row < M && col < N ? fmaxf(t, m) : t;
  }
  __device__ __forceinline__ void publish(float t) const { amax_publish_wave(to_f32(from_f32<T>(t)), amax); }
};

// C = q[row] acc in the storage type: the unembedding's input-grad product,
// whose rows carry the softmax normaliser and the loss scale as one factor.
// The factors are loaded for every row of the wave before its first store.
template <typename T>
struct EpiRowScale {
  T* C;
  long ldc;
  const float* q;
  int M, N;
  static constexpr int kOutBytes = sizeof(T);
  // the float32 slab: packed, the per-row factor's registers spilled
  static constexpr bool kPacked = false;
  __device__ __forceinline__ long out_ld() const { return ldc; }
  struct RowState {
    float q;
  };
  __device__ __forceinline__ void row_begin(RowState& rs, int row) const { rs.q = row < M ? q[row] : 0.f; }
  __device__ __forceinline__ void pre(RowState& rs, int, int, float* v) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= rs.q;
  }
  __device__ __forceinline__ void row_end(RowState&, const EpiCtx&, int) const {}
  __device__ __forceinline__ void finish(const EpiCtx&) const {}
  using Aux = NoAux;
  __device__ __forceinline__ Aux load_aux(const EpiCtx&, const EpiPos&) const { return Aux{}; }
  __device__ __forceinline__ void post(const EpiCtx& x, const EpiPos& p, float* v, const Aux&) const {
    tile_store4<T>(block_rsrc(C, ldc, x, M, p), p.off, v);
  }
};

// y = alpha * acc + beta * res (res a compile-time choice), stored in T: the steps of the
// Newton-Schulz iteration (B = c (A A^T) + b A, X' = (X B^T) + a X).
template <typename T, bool HasRes = true>
struct EpiAxpby {
  NC_EPI_NO_ROW_WORK
  T* C;
  long ldc;
  const T* res;  // C's layout
  int M, N;
  float alpha, beta;
  long c_batch, r_batch;  // per-problem strides of C and res in a batched launch
  static constexpr int kOutBytes = sizeof(T);
  __device__ __forceinline__ long out_ld() const { return ldc; }
  using Aux = std::conditional_t<HasRes, Aux4<T>, NoAux>;
  __device__ __forceinline__ Aux load_aux(const EpiCtx& x, const EpiPos& p) const {
    if constexpr (HasRes)
      return tile_load4<T>(block_rsrc(res + x.batch * r_batch, ldc, x, M, p), p.off);
    else return Aux{};
  }
  __device__ __forceinline__ void post(const EpiCtx& x, const EpiPos& p, float* v, const Aux& a) const {
    if constexpr (HasRes) {
      float r[4];
      aux_get<T>(a, r);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = alpha * v[e] + beta * r[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] *= alpha;
    }
    tile_store4<T>(block_rsrc(C + x.batch * c_batch, ldc, x, M, p), p.off, v);
  }
};

// du = acc * 2 max(u, 0), the input gradient of a = max(u, 0)^2, from the
// stored activation a: max(u, 0) = sqrt(a).
template <typename T>
struct EpiDReluSq {
  NC_EPI_NO_ROW_WORK
  T* C;
  long ldc;
  const T* act;  // a = max(u, 0)^2 as stored by the forward pass, C's layout
  int M, N;
  static constexpr int kOutBytes = sizeof(T);
  __device__ __forceinline__ long out_ld() const { return ldc; }
  using Aux = Aux4<T>;
  __device__ __forceinline__ Aux load_aux(const EpiCtx& x, const EpiPos& p) const {
    return tile_load4<T>(block_rsrc(act, ldc, x, M, p), p.off);
  }
  // The square root is the bare hardware instruction (within 1 ulp): the
  // correctly rounded library form is about 17 vector instructions, which for
  // 256 elements a thread per tile cost several microseconds of every tile.
  __device__ __forceinline__ void post(const EpiCtx& x, const EpiPos& p, float* v, const Aux& a) const {
    float av[4];
    aux_get<T>(a, av);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= 2.f * __builtin_amdgcn_sqrtf(av[e]);
    tile_store4<T>(block_rsrc(C, ldc, x, M, p), p.off, v);
  }
};

// float32 output: a weight gradient (store or accumulate) or, with several
// K splits, the split's partial tile at C + z * split_stride.
struct EpiF32 {
  NC_EPI_NO_ROW_WORK
  float* C;
  long ldc;
  long split_stride;
  int accumulate;
  int M, N;
  static constexpr int kOutBytes = sizeof(float);
  __device__ __forceinline__ long out_ld() const { return ldc; }
  using Aux = NoAux;
  __device__ __forceinline__ Aux load_aux(const EpiCtx&, const EpiPos&) const { return Aux{}; }
  __device__ __forceinline__ void post(const EpiCtx& x, const EpiPos& p, float* v, const Aux&) const {
    const __amdgpu_buffer_rsrc_t rs = block_rsrc(C + (long)x.z * split_stride, ldc, x, M, p);
    const int off = p.off;
    if (accumulate) {
      float q[4];
      aux_get<float>(tile_load4<float>(rs, off), q);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += q[e];
    }
    tile_store4<float>(rs, off, v);
  }
};

// Unembedding epilogue: z' = c tanh(z / c) (the logit softcap of the
// architecture list), stored in the storage type; per row, the sum of
// exp(z') over this tile's BN columns goes to part[row * n_tiles + tile]
// (|z'| <= c, so no running maximum is needed in float32). The tanh and
// exponentials use the hardware exp2 and reciprocal:
// c tanh(x/c) = c - 2c / (2^(x 2 log2(e)/c) + 1).
// With Grad (the training step's head) the tile stores instead what the
// softcapped cross-entropy's gradient needs from each logit,
// u = exp(z' - c) (1 - (z'/c)^2) / 4, and the row sums are of exp(z' - c):
// then dz = 4 dloss / Nv / S (u - onehot(target) S (1 - (z'_target/c)^2) / 4),
// S the row's sum, so the backward never passes over the [M, V] matrix again
// (one element a row is corrected, 4/S goes into the products as a row
// scale). With r = 1 / (2^(2 log2(e) z / c) + 1): z' - c = -2c r and
// (1 - (z'/c)^2) / 4 = r (1 - r), so z' itself is never formed, and the factor
// comes from float32 r rather than a rounded z' (which cancels near |z'| = c).
template <typename T, int BM, int BN, bool Grad = false>
struct EpiSoftcap {
  T* Z;        // [M, N] in column panels of kPanel
  int zpanel;  // panel stride (elements): M * kPanel
  float cap;
  float k2;  // 2 log2(e) / c, computed by the host
  float* part;
  int n_tiles;
  int M, N;
  float kc = 0.f;  // Grad: -2 c log2(e)
  // the logits are stored in column panels with their own offsets
  // (EpiPos::off is not used)
  static constexpr int kOutBytes = sizeof(T);
  static constexpr bool kPacked = true;
  __device__ __forceinline__ long out_ld() const { return 0; }
  struct RowState {
    float sum;
  };
  __device__ __forceinline__ void row_begin(RowState& rs, int) const { rs.sum = 0.f; }
  // z' = c - 2c / (2^(2 log2(e) z / c) + 1) = c tanh(z / c); out-of-range
  // columns add nothing to the row's sum of exp(z')
  __device__ __forceinline__ void pre(RowState& rs, int row, int col, float* v) const {
    const float lg = 1.4426950408889634f;
    float s4 = 0.f;
    if constexpr (Grad) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float r = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(v[e] * k2) + 1.f);
        const float ex = __builtin_amdgcn_exp2f(r * kc);  // exp(z' - c) <= 1
        s4 += ex;
        v[e] = ex * (r - r * r);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = __builtin_amdgcn_exp2f(v[e] * k2);
        v[e] = cap - 2.f * cap * __builtin_amdgcn_rcpf(t + 1.f);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) s4 += __builtin_amdgcn_exp2f(v[e] * lg);
    }
    rs.sum += row < M && col < N ? s4 : 0.f;
  }
  __device__ __forceinline__ void row_end(RowState& rs, const EpiCtx& x, int i) const {
    // the other half of this row's columns sits in lane ^ 32
    const float s2 = rs.sum + __shfl_xor(rs.sum, 32, 64);
    if (x.lane < 32) x.red[(x.wn ? BM : 0) + x.wm + 32 * i + x.lane] = s2;
  }
  using Aux = NoAux;
  __device__ __forceinline__ Aux load_aux(const EpiCtx&, const EpiPos&) const { return Aux{}; }
  __device__ __forceinline__ void post(const EpiCtx& x, const EpiPos& p, float* v, const Aux&) const {
    const int row = p.row, col = p.col;
    // the tile's panels from its origin: panel (col - n0) / kPanel, row (row - m0)
    const __amdgpu_buffer_rsrc_t rs = dma_rsrc(Z + (long)(x.n0 / kPanel) * zpanel + (long)x.m0 * kPanel);
    const unsigned dc = (unsigned)(col - x.n0), dr = (unsigned)(row - x.m0);
    // panel index < 8 and zpanel < 2^24 (checked by the launcher): a 24-bit multiply
    const unsigned o = (__umul24(dc / kPanel, (unsigned)zpanel) + dr * kPanel + dc % kPanel) * (unsigned)sizeof(T);
    tile_store4<T>(rs, row < M && col < N ? (int)o : (int)kDmaOOB, v);
  }
  // kPacked: 8 columns of a row, inside one panel (8 divides kPanel)
  __device__ __forceinline__ void store8(const EpiCtx& x, const EpiPos& p, const uint4& q) const {
    const __amdgpu_buffer_rsrc_t rs = dma_rsrc(Z + (long)(x.n0 / kPanel) * zpanel + (long)x.m0 * kPanel);
    const unsigned dc = (unsigned)(p.col - x.n0), dr = (unsigned)(p.row - x.m0);
    const unsigned o = (__umul24(dc / kPanel, (unsigned)zpanel) + dr * kPanel + dc % kPanel) * (unsigned)sizeof(T);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(epi_v4i, q), rs,
                                           p.row < M && p.col < N ? (int)o : (int)kDmaOOB, 0, kStoreStream);
  }
  __device__ __forceinline__ void finish(const EpiCtx& x) const {
    __syncthreads();
    for (int r = threadIdx.x; r < BM; r += blockDim.x) {
      const int row = x.m0 + r;
      if (row < M) part[(long)row * n_tiles + x.n0 / BN] = x.red[r] + x.red[BM + r];
    }
  }
};

template <typename T, int LA, int LB, typename Epi>
__global__ void __launch_bounds__(256, 1) gemm_kernel(GemmShape s, Epi epi) {
  using Cfg = GemmTile<T>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, WTM = Cfg::WTM, WTN = Cfg::WTN;
  using LoadA = OperandLoader<T, LA, BM>;
  using LoadB = OperandLoader<T, LB, BN>;
  __shared__ __align__(16) T smem[2][LoadA::SIZE + LoadB::SIZE];

  const int tid = threadIdx.x;
  // the wave index through readfirstlane: uniform, so the epilogue's buffer
  // resources (which start at the wave's rows) stay in scalar registers
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_m = (s.M + BM - 1) / BM, tiles_n = (s.N + BN - 1) / BN;
  int tm, tn, z;
  gemm_tile_coords(tiles_m, tiles_n, tm, tn, z);
  const int bi = z / s.n_split;  // batched problem, then K split
  z -= bi * s.n_split;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = z * s.k_split;
  const int kend = min(s.K, kbeg + s.k_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  const T* __restrict__ A = static_cast<const T*>(s.A) + bi * s.a_batch;
  const T* __restrict__ B = static_cast<const T*>(s.B) + bi * s.b_batch;
  LoadA la;
  LoadB lb;

  TileAcc<T> acc;
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.f;

  const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (BN / 2);
  const int kl = 8 * (lane >> 5);  // this lane's k offset inside a 16-deep step

  if (nk > 0) {
    la.load(A, s.lda, m0, s.M, kbeg, kend, tid, s.a_panel);
    lb.load(B, s.ldb, n0, s.N, kbeg, kend, tid, 0);
    la.store(smem[0], tid);
    lb.store(smem[0] + LoadA::SIZE, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(A, s.lda, m0, s.M, kbeg + (kt + 1) * BK, kend, tid, s.a_panel);
      lb.load(B, s.ldb, n0, s.N, kbeg + (kt + 1) * BK, kend, tid, 0);
    }
    const T* sa = smem[kt & 1];
    const T* sb = sa + LoadA::SIZE;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      Frag<T> fa[WTM], fb[WTN];
#pragma unroll
      for (int i = 0; i < WTM; ++i) fa[i] = LoadA::frag(sa, wm + 32 * i, kk + kl, lane);
#pragma unroll
      for (int j = 0; j < WTN; ++j) fb[j] = LoadB::frag(sb, wn + 32 * j, kk + kl, lane);
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j) mfma32(acc.c[i][j], fb[j], fa[i]);
    }
    if (more) {
      la.store(smem[(kt + 1) & 1], tid);
      lb.store(smem[(kt + 1) & 1] + LoadA::SIZE, tid);
    }
    __syncthreads();
  }

  // operand LDS is free now: one 32 x (32 WTN) float32 slab per wave, then the row-sum scratch
  float* lds = reinterpret_cast<float*>(&smem[0][0]);
  static_assert(sizeof(smem) >= (4 * 32 * 32 * WTN + 2 * BM) * sizeof(float), "epilogue LDS");
  const EpiCtx x{m0, n0, wm, wn, z, lane, wave, lds + 4 * 32 * 32 * WTN, bi};
  staged_epilogue<WTM, WTN>(acc.c, epi, x, lds + wave * 32 * 32 * WTN);
  epi.finish(x);
}

// ---------------------------------------------------------------- bf16: direct-to-LDS pipeline
// The bf16 path streams operand tiles straight from HBM into LDS with
// buffer_load_dwordx4 ... lds (gfx950): no staging registers, so k-tiles
// t+1 .. t+4 are fetched while tile t is multiplied (5-stage LDS ring of
// 256x32 A and B tiles, 160 KB). Each load instruction of a wavefront fills 1 KB of LDS, lane i at
// byte 16*i; the 16-byte chunks are XOR-swizzled on the way in so that the
// fragment reads (b128 for K-contiguous, transposing b64 for K-outer tiles)
// hit distinct banks. Out-of-range lanes get an offset beyond the buffer
// record, which the hardware turns into zeros: ragged M/N/K need no branch.

constexpr int kDmaBK = 32;

__device__ __forceinline__ int dma_swz_row(int r) { return ((r >> 2) & 3) ^ (r & 2); }  // K-contiguous chunks
__device__ __forceinline__ int dma_swz_k(int k) { return (5 * (k & 3)) & 31; }          // K-outer chunks

template <int Layout>
struct DmaOperand {
  // tile: 256 rows x 32 k of bf16 = 16 KB; per wavefront 4 load instructions.
  static constexpr int ELEMS = 256 * kDmaBK;
  // Per-lane byte offsets of the 4 loads inside a tile (rows beyond the matrix
  // already point out of the record); they do not change from tile to tile:
  // the k advance goes into soffset (K contiguous) or the record base (K outer).
  unsigned off[4];
  int kpos[4];  // k of each load inside the tile (for the ragged last tile)
  const bf16* g;
  long ld;
  long panel;  // column-panel stride (elements) of a panelled operand, else 0
  int row0;

  __device__ __forceinline__ void init(const bf16* g_, long ld_, int row0_, int nrows, int wave, int lane,
                                       long panel_) {
    g = g_;
    ld = ld_;
    panel = panel_;
    row0 = row0_;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = 4 * wave + q;
      if constexpr (Layout == kKc) {
        // a k-tile of a panelled operand lies inside one panel: rows kPanel apart
        const long rs = panel ? kPanel : ld;
        const int row = 16 * c + (lane >> 2);  // 1 KB chunk = 16 rows of 32 k
        const int kc = (lane & 3) ^ dma_swz_row(row);
        kpos[q] = 8 * kc;
        off[q] = row0 + row < nrows ? (unsigned)(((long)row * rs + 8 * kc) * 2) : kDmaOOB;
      } else {
        const int kl = 2 * c + (lane >> 5);  // 1 KB chunk = 2 k lines of 256 rows
        const int rc = (lane & 31) ^ dma_swz_k(kl);
        kpos[q] = kl;
        // panelled: the 8 columns of chunk rc sit in panel rc / 4 of the tile
        const long o = panel ? (long)(rc >> 2) * panel + (long)kl * kPanel + 8 * (rc & 3) : (long)kl * ld + 8 * rc;
        off[q] = row0 + 8 * rc < nrows ? (unsigned)(o * 2) : kDmaOOB;
      }
    }
  }

  __device__ __forceinline__ void issue(bf16* lds, int k0, int kend, int wave) const {
    const bool full = k0 + kDmaBK <= kend;
    if constexpr (Layout == kKc) {
      // plain: the k advance goes into soffset; panelled: into the record base
      __amdgpu_buffer_rsrc_t rs = dma_rsrc(panel ? g + (long)(k0 / kPanel) * panel + (long)row0 * kPanel
                                                 : g + (long)row0 * ld);
      const unsigned so = panel ? 0u : (unsigned)(k0 * 2);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const unsigned o = (full || k0 + kpos[q] < kend) ? off[q] : kDmaOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + 512 * (4 * wave + q)), 16, o, so, 0, 0);
      }
    } else {
      __amdgpu_buffer_rsrc_t rs = dma_rsrc(panel ? g + (long)(row0 / kPanel) * panel + (long)k0 * kPanel
                                                 : g + (long)k0 * ld + row0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const unsigned o = (full || k0 + kpos[q] < kend) ? off[q] : kDmaOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + 512 * (4 * wave + q)), 16, o, 0, 0, 0);
      }
    }
  }

  // Fragment of tile row row_base + lane%32, k = kk + 8*(lane/32) .. +7.
  __device__ __forceinline__ static Frag<bf16> frag(const bf16* lds, int row_base, int kk, int lane) {
    if constexpr (Layout == kKc) {
      const int r = row_base + (lane & 31);
      const int kc = (kk >> 3) + (lane >> 5);
      return frag_row<bf16>(lds + r * kDmaBK + 8 * (kc ^ dma_swz_row(r)));
    } else {
      const int j = lane & 15;
      const int r = row_base + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      const int rc = r >> 3, half = (r >> 2) & 1;
      const int ka = kk + 8 * (lane >> 5) + (j >> 2);
      const int kb = ka + 4;
      const bf16* pa = lds + ka * 256 + 8 * (rc ^ dma_swz_k(ka)) + 4 * half;
      const bf16* pb = lds + kb * 256 + 8 * (rc ^ dma_swz_k(kb)) + 4 * half;
      gemm_v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((gemm_lds_v4i16*)const_cast<bf16*>(pa));
      gemm_v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((gemm_lds_v4i16*)const_cast<bf16*>(pb));
      uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
      uint4 u = make_uint4(ua.x, ua.y, ub.x, ub.y);
      Frag<bf16> f;
      f.v = __builtin_bit_cast(bf16x8, u);
      return f;
    }
  }
};

template <int LA, int LB>
struct DmaTile {
  using OpA = DmaOperand<LA>;
  using OpB = DmaOperand<LB>;
  static constexpr int WTM = 4, WTN = 4;
  // LDS read instructions per step (both halves): one b128 per K-contiguous
  // fragment, two transposing b64 per K-outer fragment
  static constexpr int NREADS = 2 * (WTM * (LA == kKo ? 2 : 1) + WTN * (LB == kKo ? 2 : 1));
  // The fragments of one 16-deep half of a stage.
  struct Frags {
    Frag<bf16> a[WTM], b[WTN];
  };
  __device__ __forceinline__ static void load(Frags& f, const bf16* ta, const bf16* tb, int kk, int wm, int wn,
                                              int lane) {
#pragma unroll
    for (int i = 0; i < WTM; ++i) f.a[i] = OpA::frag(ta, wm + 32 * i, kk, lane);
#pragma unroll
    for (int j = 0; j < WTN; ++j) f.b[j] = OpB::frag(tb, wn + 32 * j, kk, lane);
  }
  __device__ __forceinline__ static void mma(TileAcc<bf16>& acc, const Frags& f) {
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int j = 0; j < WTN; ++j) mfma32(acc.c[i][j], f.b[j], f.a[i]);
  }
  // FP8 E4M3 operands stored as pairs in 16-bit elements: a stage's two
  // halves together are 64 k of FP8, one 32x32x64 MFMA per sub-tile. A
  // lane's 32 bytes are its 16 of the first half then its 16 of the second,
  // the same for both operands (no block scales); each fragment is read straight
  // into the 8 registers the MFMA takes.
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  struct Frags8 {
    i32x8 a[WTM], b[WTN];
  };
  __device__ __forceinline__ static i32x8 cat32(const Frag<bf16>& lo, const Frag<bf16>& hi) {
    const i32x4 x = __builtin_bit_cast(i32x4, lo.v), y = __builtin_bit_cast(i32x4, hi.v);
    return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  __device__ __forceinline__ static void load_f8(Frags8& f, const bf16* ta, const bf16* tb, int wm, int wn,
                                                 int lane) {
#pragma unroll
    for (int i = 0; i < WTM; ++i)
      f.a[i] = cat32(OpA::frag(ta, wm + 32 * i, 0, lane), OpA::frag(ta, wm + 32 * i, 16, lane));
#pragma unroll
    for (int j = 0; j < WTN; ++j)
      f.b[j] = cat32(OpB::frag(tb, wn + 32 * j, 0, lane), OpB::frag(tb, wn + 32 * j, 16, lane));
  }
  __device__ __forceinline__ static void mma_f8(TileAcc<bf16>& acc, const Frags8& f) {
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int j = 0; j < WTN; ++j)
        acc.c[i][j] =  // zero scale operands select the unscaled v_mfma_f32_32x32x64_f8f6f4 (AGPR accumulators)
            __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc.c[i][j], 0, 0, 0, 0, 0, 0);
  }
};

// The FP8 step's schedule: one fragment read after each multiply (16
// multiplies, at most 16 reads) and one of the 8 tile loads after every other
// multiply, then a fence: a wave never stops issuing multiplies to push a
// burst of loads through the address unit.
template <bool WithLoads>
__device__ __forceinline__ void interleave_reads_with_mfma() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    // the 8 tile loads go after every other multiply: in a burst they overrun
    // the CU's texture-address queue, and a wave stalled on a load issues no
    // multiply (the queue is full for about a fifth of the cycles even so)
    if (WithLoads && (i & 1) == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one tile load
  }
  __builtin_amdgcn_sched_barrier(0);
}

// The scheduler is told to put one fragment read after every other multiply
// and one tile load after every fourth: the reads of a set stay ahead of the
// multiplies that need them (it would otherwise pull those forward), and a
// burst of loads would overrun the CU's texture-address queue, stalling the
// wave's multiplies behind it.
template <bool WithLoads>
__device__ __forceinline__ void interleave_full() {
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if ((i & 1) == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    if (WithLoads && (i & 3) == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one tile load
  }
  __builtin_amdgcn_sched_barrier(0);
}
// With a K-outer operand a step has 24 or 32 fragment reads (two transposing
// reads per fragment), and spread over all 32 multiplies the last ones were
// still in flight when the next step's barrier waited for them. They go with
// the first 16 multiplies instead (as evenly as they divide), a tile load
// after every fourth: the weight- and input-grad products ran about 1 %
// faster, while the forward products (16 reads) ran slower that way and keep
// interleave_full.
template <int NR, int I>
__device__ __forceinline__ void interleave_front_group() {
  constexpr int n = I < 16 ? (NR * (I + 1)) / 16 - (NR * I) / 16 : 0;
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
  if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);  // its LDS reads
  if constexpr ((I & 3) == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one tile load
}
template <int NR, int... I>
__device__ __forceinline__ void interleave_front_groups(std::integer_sequence<int, I...>) {
  (interleave_front_group<NR, I>(), ...);
}
template <int NR>
__device__ __forceinline__ void interleave_step() {
  if constexpr (NR > 16) {
    interleave_front_groups<NR>(std::make_integer_sequence<int, 32>{});
    __builtin_amdgcn_sched_barrier(0);
  } else {
    interleave_full<true>();
  }
}
#define NC_DMA_STEP_FULL(t, SA, SB, NA, NB, CUR, NXT)       \
  {                                                         \
    ring_barrier<24>();                                     \
    opa.issue(SA, kbeg + ((t) + 5) * kDmaBK, kend, wave);   \
    opb.issue(SB, kbeg + ((t) + 5) * kDmaBK, kend, wave);   \
    Tile::load(NXT.h0, NA, NB, 0, wm, wn, lane);            \
    Tile::load(NXT.h1, NA, NB, 16, wm, wn, lane);           \
    Tile::mma(acc, CUR.h0);                                 \
    Tile::mma(acc, CUR.h1);                                 \
    interleave_step<Tile::NREADS>();                        \
  }

// The whole ring in one inlined function whose stage arrays are __restrict__
// parameters: every LDS access inside then carries alias-scope information,
// which lets the compiler see that the reads of one stage do not depend on
// the loads still streaming into the others (it would otherwise drain them).
// Five 32 KB stages fill the 160 KB of LDS: tiles t+1 .. t+4 are in flight
// while tile t is multiplied (about 2 us of lookahead at the clock the
// matrix cores sustain), enough to ride out the operand fetches that miss L2.
// Each step waits for tile t+1 and for every wave to be done with tile t's
// stage (its fragments are all in registers by then), refills that stage with
// tile t+5, and reads all of tile t+1 into the second fragment set while
// multiplying tile t: no multiply waits for a read issued just before it, and
// with one wavefront per SIMD that is what keeps the matrix core busy. The two
// sets trade places every step, so the main loop runs ten steps a trip (five
// stages, two sets) with fixed stage names and no branch, and nothing is
// copied. Loads past the end of K read zeros, so every step is the same.
template <typename Tile>
__device__ __forceinline__ void dma_ring(TileAcc<bf16>& acc, typename Tile::OpA& opa, typename Tile::OpB& opb,
                                              bf16* __restrict__ sa0, bf16* __restrict__ sa1, bf16* __restrict__ sa2,
                                              bf16* __restrict__ sa3, bf16* __restrict__ sa4, bf16* __restrict__ sb0,
                                              bf16* __restrict__ sb1, bf16* __restrict__ sb2, bf16* __restrict__ sb3,
                                              bf16* __restrict__ sb4, int nk, int kbeg, int kend, int wave, int wm,
                                              int wn, int lane) {
  constexpr int BK = kDmaBK;
  struct Full {
    typename Tile::Frags h0, h1;
  } F, G;
  opa.issue(sa0, kbeg, kend, wave);
  opb.issue(sb0, kbeg, kend, wave);
  opa.issue(sa1, kbeg + BK, kend, wave);
  opb.issue(sb1, kbeg + BK, kend, wave);
  opa.issue(sa2, kbeg + 2 * BK, kend, wave);
  opb.issue(sb2, kbeg + 2 * BK, kend, wave);
  opa.issue(sa3, kbeg + 3 * BK, kend, wave);
  opb.issue(sb3, kbeg + 3 * BK, kend, wave);
  opa.issue(sa4, kbeg + 4 * BK, kend, wave);
  opb.issue(sb4, kbeg + 4 * BK, kend, wave);
  ring_barrier<32>();  // tile 0 has landed
  Tile::load(F.h0, sa0, sb0, 0, wm, wn, lane);
  Tile::load(F.h1, sa0, sb0, 16, wm, wn, lane);
  int kt = 0;
  for (; kt + 10 <= nk; kt += 10) {
    NC_DMA_STEP_FULL(kt, sa0, sb0, sa1, sb1, F, G);
    NC_DMA_STEP_FULL(kt + 1, sa1, sb1, sa2, sb2, G, F);
    NC_DMA_STEP_FULL(kt + 2, sa2, sb2, sa3, sb3, F, G);
    NC_DMA_STEP_FULL(kt + 3, sa3, sb3, sa4, sb4, G, F);
    NC_DMA_STEP_FULL(kt + 4, sa4, sb4, sa0, sb0, F, G);
    NC_DMA_STEP_FULL(kt + 5, sa0, sb0, sa1, sb1, G, F);
    NC_DMA_STEP_FULL(kt + 6, sa1, sb1, sa2, sb2, F, G);
    NC_DMA_STEP_FULL(kt + 7, sa2, sb2, sa3, sb3, G, F);
    NC_DMA_STEP_FULL(kt + 8, sa3, sb3, sa4, sb4, F, G);
    NC_DMA_STEP_FULL(kt + 9, sa4, sb4, sa0, sb0, G, F);
  }
  // kt is a multiple of 10: tile kt sits in stage 0 with its fragments in F
  if (kt < nk) NC_DMA_STEP_FULL(kt, sa0, sb0, sa1, sb1, F, G);
  if (kt + 1 < nk) NC_DMA_STEP_FULL(kt + 1, sa1, sb1, sa2, sb2, G, F);
  if (kt + 2 < nk) NC_DMA_STEP_FULL(kt + 2, sa2, sb2, sa3, sb3, F, G);
  if (kt + 3 < nk) NC_DMA_STEP_FULL(kt + 3, sa3, sb3, sa4, sb4, G, F);
  if (kt + 4 < nk) NC_DMA_STEP_FULL(kt + 4, sa4, sb4, sa0, sb0, F, G);
  if (kt + 5 < nk) NC_DMA_STEP_FULL(kt + 5, sa0, sb0, sa1, sb1, G, F);
  if (kt + 6 < nk) NC_DMA_STEP_FULL(kt + 6, sa1, sb1, sa2, sb2, F, G);
  if (kt + 7 < nk) NC_DMA_STEP_FULL(kt + 7, sa2, sb2, sa3, sb3, G, F);
  if (kt + 8 < nk) NC_DMA_STEP_FULL(kt + 8, sa3, sb3, sa4, sb4, F, G);
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8) | (0 << 14));
}
#undef NC_DMA_STEP_FULL

// The FP8 step has the bf16 step's shape: wait for tile t+1 and refill
// stage S (tile t's fragments, both halves, are already in CUR); read tile
// t+1 into NXT while multiplying tile t. Its 16 multiplies are each as long
// as two bf16 ones, so it places one fragment read after each multiply and
// one tile load after every other (interleave_reads_with_mfma).
#define NC_DMA_STEP_F8(t, SA, SB, NA, NB, CUR, NXT)         \
  {                                                         \
    ring_barrier<24>();                                     \
    opa.issue(SA, kbeg + ((t) + 5) * kDmaBK, kend, wave);   \
    opb.issue(SB, kbeg + ((t) + 5) * kDmaBK, kend, wave);   \
    Tile::load_f8(NXT, NA, NB, wm, wn, lane);               \
    Tile::mma_f8(acc, CUR);                                 \
    interleave_reads_with_mfma<true>();                     \
  }

template <typename Tile>
__device__ __forceinline__ void dma_ring_f8(TileAcc<bf16>& acc, typename Tile::OpA& opa, typename Tile::OpB& opb,
                                            bf16* __restrict__ sa0, bf16* __restrict__ sa1, bf16* __restrict__ sa2,
                                            bf16* __restrict__ sa3, bf16* __restrict__ sa4, bf16* __restrict__ sb0,
                                            bf16* __restrict__ sb1, bf16* __restrict__ sb2, bf16* __restrict__ sb3,
                                            bf16* __restrict__ sb4, int nk, int kbeg, int kend, int wave, int wm,
                                            int wn, int lane) {
  constexpr int BK = kDmaBK;
  typename Tile::Frags8 F, G;
  opa.issue(sa0, kbeg, kend, wave);
  opb.issue(sb0, kbeg, kend, wave);
  opa.issue(sa1, kbeg + BK, kend, wave);
  opb.issue(sb1, kbeg + BK, kend, wave);
  opa.issue(sa2, kbeg + 2 * BK, kend, wave);
  opb.issue(sb2, kbeg + 2 * BK, kend, wave);
  opa.issue(sa3, kbeg + 3 * BK, kend, wave);
  opb.issue(sb3, kbeg + 3 * BK, kend, wave);
  opa.issue(sa4, kbeg + 4 * BK, kend, wave);
  opb.issue(sb4, kbeg + 4 * BK, kend, wave);
  ring_barrier<32>();  // tile 0 has landed
  Tile::load_f8(F, sa0, sb0, wm, wn, lane);
  int kt = 0;
  for (; kt + 10 <= nk; kt += 10) {
    NC_DMA_STEP_F8(kt, sa0, sb0, sa1, sb1, F, G);
    NC_DMA_STEP_F8(kt + 1, sa1, sb1, sa2, sb2, G, F);
    NC_DMA_STEP_F8(kt + 2, sa2, sb2, sa3, sb3, F, G);
    NC_DMA_STEP_F8(kt + 3, sa3, sb3, sa4, sb4, G, F);
    NC_DMA_STEP_F8(kt + 4, sa4, sb4, sa0, sb0, F, G);
    NC_DMA_STEP_F8(kt + 5, sa0, sb0, sa1, sb1, G, F);
    NC_DMA_STEP_F8(kt + 6, sa1, sb1, sa2, sb2, F, G);
    NC_DMA_STEP_F8(kt + 7, sa2, sb2, sa3, sb3, G, F);
    NC_DMA_STEP_F8(kt + 8, sa3, sb3, sa4, sb4, F, G);
    NC_DMA_STEP_F8(kt + 9, sa4, sb4, sa0, sb0, G, F);
  }
  // kt is a multiple of 10: tile kt sits in stage 0 with its fragments in F
  if (kt < nk) NC_DMA_STEP_F8(kt, sa0, sb0, sa1, sb1, F, G);
  if (kt + 1 < nk) NC_DMA_STEP_F8(kt + 1, sa1, sb1, sa2, sb2, G, F);
  if (kt + 2 < nk) NC_DMA_STEP_F8(kt + 2, sa2, sb2, sa3, sb3, F, G);
  if (kt + 3 < nk) NC_DMA_STEP_F8(kt + 3, sa3, sb3, sa4, sb4, G, F);
  if (kt + 4 < nk) NC_DMA_STEP_F8(kt + 4, sa4, sb4, sa0, sb0, F, G);
  if (kt + 5 < nk) NC_DMA_STEP_F8(kt + 5, sa0, sb0, sa1, sb1, G, F);
  if (kt + 6 < nk) NC_DMA_STEP_F8(kt + 6, sa1, sb1, sa2, sb2, F, G);
  if (kt + 7 < nk) NC_DMA_STEP_F8(kt + 7, sa2, sb2, sa3, sb3, G, F);
  if (kt + 8 < nk) NC_DMA_STEP_F8(kt + 8, sa3, sb3, sa4, sb4, F, G);
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8) | (0 << 14));
}
#undef NC_DMA_STEP_F8

template <int LA, int LB, typename Epi, bool F8 = false>
__global__ void __launch_bounds__(256, 1) gemm_dma_kernel(GemmShape s, Epi epi) {
  constexpr int BM = 256, BN = 256, BK = kDmaBK;
  using Tile = DmaTile<LA, LB>;
  constexpr int E = Tile::OpA::ELEMS;
  __shared__ __align__(1024) bf16 sa0[E], sa1[E], sa2[E], sa3[E], sa4[E];
  __shared__ __align__(1024) bf16 sb0[E], sb1[E], sb2[E], sb3[E], sb4[E];

  const int tid = threadIdx.x;
  // the wave index through readfirstlane: uniform, so every LDS destination
  // of the direct-to-LDS loads (M0) is formed in scalar registers
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_m = (s.M + BM - 1) / BM, tiles_n = (s.N + BN - 1) / BN;
  int tm, tn, z;
  gemm_tile_coords(tiles_m, tiles_n, tm, tn, z);
  const int bi = z / s.n_split;  // batched problem, then K split
  z -= bi * s.n_split;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = z * s.k_split;
  const int kend = min(s.K, kbeg + s.k_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  TileAcc<bf16> acc;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.f;
  const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (BN / 2);

  typename Tile::OpA opa;
  typename Tile::OpB opb;
  opa.init(static_cast<const bf16*>(s.A) + bi * s.a_batch, s.lda, m0, s.M, wave, lane, s.a_panel);
  opb.init(static_cast<const bf16*>(s.B) + bi * s.b_batch, s.ldb, n0, s.N, wave, lane, 0);
  if constexpr (F8)
    dma_ring_f8<Tile>(acc, opa, opb, sa0, sa1, sa2, sa3, sa4, sb0, sb1, sb2, sb3, sb4, nk, kbeg, kend, wave, wm, wn,
                      lane);
  else
    dma_ring<Tile>(acc, opa, opb, sa0, sa1, sa2, sa3, sa4, sb0, sb1, sb2, sb3, sb4, nk, kbeg, kend, wave, wm, wn,
                   lane);
  __syncthreads();
  // the A stages become the waves' 32 x 128 float32 slabs, B stage 0 the row-sum scratch
  static_assert(E * sizeof(bf16) == 32 * 128 * sizeof(float), "one A stage holds one slab");
  bf16* slab = wave == 0 ? sa0 : wave == 1 ? sa1 : wave == 2 ? sa2 : sa3;
  const EpiCtx x{m0, n0, wm, wn, z, lane, wave, reinterpret_cast<float*>(sb0), bi, epi_scale(epi)};
  staged_epilogue<4, 4, Epi, F8>(acc.c, epi, x, reinterpret_cast<float*>(slab));
  epi.finish(x);
}


// ---------------------------------------------------------------- launcher

template <typename T, int LA, int LB, typename Epi>
nc_status launch_gemm(const GemmShape& s, const Epi& epi, hipStream_t stream) {
  using Cfg = GemmTile<T>;
  int tiles_m = (s.M + Cfg::BM - 1) / Cfg::BM, tiles_n = (s.N + Cfg::BN - 1) / Cfg::BN;
  long blocks = (long)tiles_m * tiles_n * s.n_split * s.batch;
  if (blocks <= 0) return NC_OK;
  // a packed store phase writes 8 columns at a time
  if (EpiPacked<Epi>::value && epi.N % 8 != 0) return NC_ERR_UNSUPPORTED;
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((gemm_dma_kernel<LA, LB, Epi>), dim3((unsigned)blocks), dim3(256), 0, stream, s,
                       epi);
  else
    hipLaunchKernelGGL((gemm_kernel<T, LA, LB, Epi>), dim3((unsigned)blocks), dim3(256), 0, stream, s,
                       epi);
  NC_LAUNCH_CHECK("gemm");
  return NC_OK;
}

// FP8 E4M3 operands, both K-contiguous, each stored as 16-bit pairs: s.K,
// s.lda, s.ldb count pairs.
template <typename Epi>
nc_status launch_gemm_f8(const GemmShape& s, const Epi& epi, hipStream_t stream) {
  int tiles_m = (s.M + 255) / 256, tiles_n = (s.N + 255) / 256;
  long blocks = (long)tiles_m * tiles_n * s.n_split * s.batch;
  if (blocks <= 0) return NC_OK;
  if (EpiPacked<Epi>::value && epi.N % 8 != 0) return NC_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((gemm_dma_kernel<kKc, kKc, Epi, true>), dim3((unsigned)blocks), dim3(256), 0, stream, s, epi);
  NC_LAUNCH_CHECK("gemm_f8");
  return NC_OK;
}

}  // namespace nc
