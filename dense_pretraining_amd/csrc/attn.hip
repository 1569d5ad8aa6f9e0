// Causal multi-query attention on gfx950, forward and backward.
//
// The architecture list on vpshk.cn (Q&A section) gives multi-query attention;
// next-token training (imeisheng.com, section "预训练") makes it causal. Per
// batch row and query head h (KV head g = h*G/H):
//   S = q k^T / sqrt(D), masked to key <= query position, P = softmax(S), o = P v.
//
// MI355X design:
//  * All n_rep = H/G query heads of one KV head are flattened into one row
//    space r = t * n_rep + (h - g*n_rep), t = r / n_rep. A 128-row block then
//    spans ~128/n_rep positions of every head, so one LDS-staged K/V tile is
//    shared by all heads and the causal diagonal is only ~13 positions wide
//    at H = 10 instead of 128.
//  * 32x32x16 bf16 MFMA. The score tile is computed transposed, S^T = K Q^T,
//    so each lane owns one query (lane % 32) and 16 of the 32 keys: the row
//    sum is lane-local, and the probabilities are already laid out as the
//    B operand of O^T += V^T P^T (the keys a lane holds are paired with the
//    matching V^T entries when V^T is read from LDS). No P round trip via LDS.
//  * QK norm bounds every score: |q|, |k| <= sqrt(D) after the per-head
//    RMSNorm, so |s| <= sqrt(D). exp(s - sqrt(D)) lies in [e^{-2 sqrt(D)}, 1],
//    so a fixed shift replaces the running maximum of online softmax.
//  * Backward without atomics: a dQ pass over query blocks (which also forms
//    Delta = rowsum(dO * O)), then a dK/dV pass over key blocks that sums all
//    heads' contributions in registers.
// Float storage (check mode) runs the same code with 32x32x2 f32 MFMAs.
#include "common.h"
#include "frag.h"
#include "kernels.h"

namespace nc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 2^x with the bare hardware instruction. Every argument here lies in
// [-2 sqrt(D) log2(e) - log2(T), 1], far from the range where the library
// exp2f needs its denormal rescaling.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A buffer descriptor from an address the caller knows to be the same in
// every lane. A descriptor the compiler cannot prove uniform sits in vector
// registers, and every buffer instruction using it is wrapped in a loop over
// the distinct values (readfirstlane, compare, exec mask); taking the address
// through readfirstlane keeps it in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_rsrc_uniform(const void* base) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return dma_rsrc(reinterpret_cast<const void*>(((unsigned long long)hi << 32) | lo));
}

// r / n for 0 <= r < 2^24 without an integer division.
struct DivN {
  int n;
  float inv;
  __device__ __forceinline__ int q(int r) const {
    int x = (int)((float)r * inv);
    x -= (x * n > r) ? 1 : 0;
    x += ((x + 1) * n <= r) ? 1 : 0;
    return x;
  }
};

// Swizzled [rows][D] tile: 16-byte chunk c of row r sits at chunk c ^ f(r).
// D = 128 bf16 (16 chunks a row): f(r) = 4 (r % 4) + (r / 4) % 4. Sixteen
// consecutive rows read at one chunk hit 16 distinct chunk slots, and the
// transposing read (rows k..k+3 x 4 chunks) covers all 64 banks once.
// D = 64 bf16 (8 chunks, two rows per 256-byte bank line): f(r) = 4 ((r/2) % 2)
// + (r / 4) % 4 does the same with the row parity selecting the half line.
template <typename T, int D>
struct Swz {
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int NC = D / VE;
  __device__ __forceinline__ static int f(int r) {
    if constexpr (NC >= 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  __device__ __forceinline__ static int at(int r, int col) { return (r * NC + ((col / VE) ^ f(r))) * VE + col % VE; }
};

// Fragment X[row][c0 .. c0+7] (c0 a multiple of 8).
template <typename T, int D>
__device__ __forceinline__ F8<T> swz_row8(const T* t, int row, int c0) {
  if constexpr (sizeof(T) == 2) {
    return ld_row8<T>(t + Swz<T, D>::at(row, c0));
  } else {
    return ld_split8<T>(t + Swz<T, D>::at(row, c0), t + Swz<T, D>::at(row, c0 + 4));
  }
}
// Fragment X[ka .. ka+3 | kb .. kb+3][c0 + lane % 16] (tile rows as k).
template <typename T, int D>
__device__ __forceinline__ F8<T> swz_tr8(const T* t, int ka, int kb, int c0, int lane) {
  F8<T> f;
  if constexpr (sizeof(T) == 2) {
    const int j = lane & 15;
    const int col = c0 + 4 * (j & 3);
    v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)const_cast<T*>(t + Swz<T, D>::at(ka + (j >> 2), col)));
    v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)const_cast<T*>(t + Swz<T, D>::at(kb + (j >> 2), col)));
    uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
    f.v = __builtin_bit_cast(bf16x8, make_uint4(ua.x, ua.y, ub.x, ub.y));
  } else {
    const int col = c0 + (lane & 15);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f.v[s] = t[Swz<T, D>::at(ka + s, col)];
      f.v[4 + s] = t[Swz<T, D>::at(kb + s, col)];
    }
  }
  return f;
}

// A bf16 tile read only through the transposing read (V in the forward and
// decode): 16-byte chunk c of row r sits at chunk slot
// 4 NC (r/4) + 16 (c/4) + 4 (r%4) + c%4. The 4 rows x 4 chunks one transposing
// read covers per 32 lanes then fill one 256-byte bank line, and the lane's
// fragments for different rows and column groups differ by constant offsets
// (one address register instead of one per fragment).
template <int D>
struct SwzT {
  static constexpr int NC = D / 8;
  static_assert(NC % 4 == 0, "whole 4-chunk groups");
  // inverse of the slot map: the row and chunk stored at slot u
  __device__ __forceinline__ static int row(int u) { return 4 * (u / (4 * NC)) + ((u >> 2) & 3); }
  __device__ __forceinline__ static int chunk(int u) { return 4 * ((u % (4 * NC)) >> 4) + (u & 3); }
};
// Fragment X[ka .. ka+3 | kb .. kb+3][32 dt + 16 ((lane/16)%2) + lane % 16]
// of a tile in the SwzT layout (ka, kb multiples of 4); float tiles keep the
// Swz layout.
template <typename T, int D>
__device__ __forceinline__ F8<T> vtr8(const T* t, int ka, int kb, int dt, int lane) {
  if constexpr (sizeof(T) == 2) {
    const int j = lane & 15;
    const int lp = 32 * (j >> 2) + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
    v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)const_cast<T*>(t + D * ka + 128 * dt + lp));
    v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)const_cast<T*>(t + D * kb + 128 * dt + lp));
    uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
    F8<T> f;
    f.v = __builtin_bit_cast(bf16x8, make_uint4(ua.x, ua.y, ub.x, ub.y));
    return f;
  } else {
    return swz_tr8<T, D>(t, ka, kb, 32 * dt + 16 * ((lane >> 4) & 1), lane);
  }
}

// ------------------------------------------------------------ tile staging
// Row-major tile [ROWS][D] -> LDS in the swizzled layout above, staged
// through registers; the row addresses come from a function (nullptr = zero row).
template <typename T, int ROWS, int D>
struct RowTile {
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int ELEMS = ROWS * D;
  static constexpr int N = ROWS * D / VE;
  static constexpr int PER = (N + 255) / 256;
  uint4 r[PER];
  template <typename AddrF>
  __device__ __forceinline__ void load(AddrF addr, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int u = tid + 256 * i;
      r[i] = make_uint4(0, 0, 0, 0);
      if (u < N) {
        int row = u / (D / VE), c = u % (D / VE);
        const T* p = addr(row);
        if (p) r[i] = *reinterpret_cast<const uint4*>(p + c * VE);
      }
    }
  }
  __device__ __forceinline__ void store(T* s, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int u = tid + 256 * i;
      if (u < N) {
        int row = u / (D / VE), c = u % (D / VE);
        *reinterpret_cast<uint4*>(s + Swz<T, D>::at(row, c * VE)) = r[i];
      }
    }
  }
};

// K and V tiles of 64 keys streamed straight into LDS (buffer_load ... lds),
// in the swizzled layout, through a 2-stage ring: tile t+1 loads while tile
// t is used, and no registers hold data in flight. Keys at or past T read as
// zeros. NW waves share the loads of a tile. With VT, a bf16 V tile lands in
// the SwzT layout (for kernels that read V only through the transposing read).
template <typename T, int D, int NW = 4, bool VT = false>
struct KvDma {
  static constexpr int BKV = 64;
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int TILE = BKV * D;        // elements of one K or V tile
  static constexpr int NI = TILE / VE / 64;   // 1 KB loads per tile
  static constexpr int NPW = 2 * NI / NW;     // per wave, K and V together
  static_assert((2 * NI) % NW == 0, "tile loads split evenly over the waves");
  const T* kbase;
  const T* vbase;
  long ldk, ldv;
  int T_;
  unsigned off[NPW];
  int row[NPW], blk[NPW];
  bool isv[NPW];

  __device__ __forceinline__ void init(const T* kb, long ldk_, const T* vb, long ldv_, int Tn, int wave, int lane) {
    kbase = kb;
    vbase = vb;
    ldk = ldk_;
    ldv = ldv_;
    T_ = Tn;
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int ins = wave * NPW + i;  // K instructions first, then V
      isv[i] = ins >= NI;
      blk[i] = ins % NI;
      const int u = 64 * blk[i] + lane;  // chunk slot inside the tile
      int col;
      if (VT && sizeof(T) == 2 && isv[i]) {
        row[i] = SwzT<D>::row(u);
        col = SwzT<D>::chunk(u) * VE;
      } else {
        row[i] = u / Swz<T, D>::NC;
        col = ((u % Swz<T, D>::NC) ^ Swz<T, D>::f(row[i])) * VE;
      }
      off[i] = (unsigned)(((long)row[i] * (isv[i] ? ldv : ldk) + col) * (long)sizeof(T));
    }
  }
  __device__ __forceinline__ void issue(int kt, T* __restrict__ sk, T* __restrict__ sv) const {
    const long key0 = (long)kt * BKV;
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const unsigned o = key0 + row[i] < T_ ? off[i] : kDmaOOB;
      // K or V by the wave's instruction index: the same in every lane
      __amdgpu_buffer_rsrc_t rs = dma_rsrc_uniform(isv[i] ? vbase + key0 * ldv : kbase + key0 * ldk);
      T* dst = (isv[i] ? sv : sk) + blk[i] * 64 * VE;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, o, 0, 0, 0);
    }
  }
};

// Runs body(kt, k tile, v tile) for kt = 0 .. nkt-1 over the ring. The stages
// are separate LDS arrays passed as __restrict__ parameters of this inlined
// function, so the compiler can tell one stage's loads from the other
// stage's reads.
template <typename T, int D, int NW, bool VT, typename Body>
__device__ __forceinline__ void kv_ring(const KvDma<T, D, NW, VT>& dma, int nkt, T* __restrict__ k0, T* __restrict__ v0,
                                        T* __restrict__ k1, T* __restrict__ v1, Body&& body) {
  dma.issue(0, k0, v0);
  int kt = 0;
  for (; kt + 2 <= nkt; kt += 2) {
    ring_barrier<0>();
    dma.issue(kt + 1, k1, v1);
    body(kt, k0, v0);
    ring_barrier<0>();
    dma.issue(kt + 2, k0, v0);
    body(kt + 1, k1, v1);
  }
  if (kt < nkt) {
    ring_barrier<0>();
    dma.issue(kt + 1, k1, v1);
    body(kt, k0, v0);
  }
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8) | (0 << 14));  // the loads past the end
}

// Key index held in accumulator slot v by lane half lh (C layout of a 32x32
// MFMA: rows 8*(v/4) + 4*lh + v%4).
__device__ __forceinline__ int crow(int v, int lh) { return 8 * (v >> 2) + 4 * lh + (v & 3); }

struct AttnGeom {
  int B, T, H, G, D, n_rep;
  long ld_qk, ld_v, ld_o, ld_dq;
  int q_off_k;  // column of K head 0 inside the qk rows (H*D)
  float inv_rep;
};

// Scheduling pattern for NM matrix products, each with RD of their LDS
// operand reads, spread over the vector work of the same block: two reads
// ahead, then one product, its reads and six vector instructions at a time.
template <int NM, int RD>
__device__ __forceinline__ void fwd_overlap() {
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * RD, 0);  // LDS reads ahead
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if (i + 2 < NM) __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
  }
}

// ============================================================ forward
// With AMAX, the largest stored |o| goes into the striped maximum at amax (the
// per-tensor scale of the FP8 output projection's operand).
template <typename T, int D, bool AMAX>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(AttnGeom g, const T* __restrict__ qk,
                                                          const T* __restrict__ vsrc, T* __restrict__ o,
                                                          float* __restrict__ lse, uint32_t* amax) {
  using Kv = KvDma<T, D, 4, true>;
  constexpr int BKV = Kv::BKV;
  __shared__ __align__(16) T ks0[Kv::TILE], vs0[Kv::TILE], ks1[Kv::TILE], vs1[Kv::TILE];

  const int tid = threadIdx.x, lane = tid & 63, lh = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nrows = g.T * g.n_rep;
  const int nqb = (nrows + 127) / 128;
  const int per = g.G * g.B;
  const int qb = nqb - 1 - (int)(blockIdx.x / per);  // longest query blocks first
  const int kvh = blockIdx.x % per % g.G, b = blockIdx.x % per / g.G;
  const int R0 = qb * 128;
  const long tok0 = (long)b * g.T;
  const DivN dv{g.n_rep, g.inv_rep};

  const int rq = R0 + 32 * wave + l32;
  const bool qok = rq < nrows;
  const int tq = qok ? dv.q(rq) : 0;
  const int hq = kvh * g.n_rep + (qok ? rq - tq * g.n_rep : 0);
  const int w_last = min(nrows - 1, R0 + 32 * wave + 31);
  const int t_wmax = dv.q(w_last);
  const int t_wmin = dv.q(min(nrows - 1, R0 + 32 * wave));
  const bool wfull = R0 + 32 * wave + 31 < nrows;
  const int t_bmax = dv.q(min(nrows - 1, R0 + 127));
  const int nkt = t_bmax / BKV + 1;

  // Q as the B operand of S^T = K Q^T: lane holds d = 16*s + 8*lh + (0..7) of its query.
  F8<T> qf[D / 16];
  const T* qrow = qk + (tok0 + tq) * g.ld_qk + (long)hq * D;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qf[s] = gld8<T>(qrow + 16 * s + 8 * lh, qok);

  Kv dma;
  dma.init(qk + tok0 * g.ld_qk + g.q_off_k + (long)kvh * D, g.ld_qk, vsrc + tok0 * g.ld_v + (long)kvh * D, g.ld_v,
           g.T, wave, lane);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  float lsum = 0.f;
  const float c1 = kLog2e / sqrtf((float)D);
  const float m0 = sqrtf((float)D) * kLog2e;  // fixed shift: |s| <= sqrt(D)

  kv_ring<T, D>(dma, nkt, ks0, vs0, ks1, vs1, [&](int kt, const T* sk, const T* sv) {
    if (wfull && kt * BKV + BKV - 1 <= t_wmin) {
      // Whole tile below the diagonal for every row of the wave: a straight
      // block in which the second sub-tile's score products run on the matrix
      // cores while the first sub-tile's exponentials run on the vector unit,
      // then the first sub-tile's P V products while the second's run.
      f32x16 sa, sb;
#pragma unroll
      for (int v = 0; v < 16; ++v) sa[v] = sb[v] = 0.f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) mma32(sa, swz_row8<T, D>(sk, l32, 16 * s + 8 * lh), qf[s]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < D / 16; ++s) mma32(sb, swz_row8<T, D>(sk, 32 + l32, 16 * s + 8 * lh), qf[s]);
      float pa[16], pb[16];
      float la = 0.f, lb = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        pa[v] = fast_exp2(sa[v] * c1 - m0);
        la += pa[v];
      }
      F8<T> pfa[2] = {pack8<T>(pa), pack8<T>(pa + 8)};
      fwd_overlap<D / 16, 1>();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int k0 = 16 * kk + 4 * lh;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          mma32(oacc[dt], vtr8<T, D>(sv, k0, k0 + 8, dt, lane), pfa[kk]);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        pb[v] = fast_exp2(sb[v] * c1 - m0);
        lb += pb[v];
      }
      F8<T> pfb[2] = {pack8<T>(pb), pack8<T>(pb + 8)};
      fwd_overlap<D / 16, 2>();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int k0 = 32 + 16 * kk + 4 * lh;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          mma32(oacc[dt], vtr8<T, D>(sv, k0, k0 + 8, dt, lane), pfb[kk]);
      }
      lsum += la + lb;
      return;
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kb = kt * BKV + 32 * sub;
      if (kb > t_wmax) continue;
      f32x16 sacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        F8<T> kf = swz_row8<T, D>(sk, 32 * sub + l32, 16 * s + 8 * lh);
        mma32(sacc, kf, qf[s]);
      }
      float p[16];
      if (wfull && kb + 31 <= t_wmin) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          p[v] = fast_exp2(sacc[v] * c1 - m0);
          lsum += p[v];
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          int key = kb + crow(v, lh);
          float e = fast_exp2(sacc[v] * c1 - m0);
          p[v] = (qok && key <= tq) ? e : 0.f;
          lsum += p[v];
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        F8<T> pf = pack8<T>(p + 8 * kk);
        const int k0 = 32 * sub + 16 * kk + 4 * lh;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          mma32(oacc[dt], vtr8<T, D>(sv, k0, k0 + 8, dt, lane), pf);
        }
      }
    }
  });

  lsum += __shfl_xor(lsum, 32, 64);
  float om = 0.f;  // AMAX: largest stored |o| of the lane
  if (qok) {
    const float inv = 1.f / lsum;
    T* orow = o + (tok0 + tq) * g.ld_o + (long)hq * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        T* dst = orow + 32 * dt + 8 * j + 4 * lh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ov = oacc[dt][4 * j + i] * inv;
          if constexpr (AMAX) om = fmaxf(om, fabsf(ov));
          dst[i] = from_f32<T>(ov);
        }
      }
    if (lh == 0) lse[(tok0 + tq) * g.H + hq] = (m0 + log2f(lsum)) / kLog2e;
  }
  // an FP8 operand's per-tensor scale: the wave's largest stored magnitude
  if constexpr (AMAX) amax_publish_wave(to_f32(from_f32<T>(om)), amax);
}

// ============================================================ decode: one query row per head
// One new position per sequence against the key/value cache. The n_rep query
// heads that share KV head g form the 32 columns of the score tile (unused
// columns carry zero queries), so the forward's S^T = K Q^T and O^T = V^T P^T
// products apply unchanged. Block (c, g, b) takes keys [c*kch, c*kch + kch)
// through 64-key tiles; wave w takes keys 32w .. 32w+31 of each tile. With the
// fixed shift the chunks' unnormalised sums merge by plain addition.
template <typename T, int D, int NST>
__global__ void __launch_bounds__(128) attn_decode_kernel(const T* __restrict__ q, long ldq, const T* __restrict__ ck,
                                                          const T* __restrict__ cv, int H, int G, int n, int cap,
                                                          int kch, float* __restrict__ po, float* __restrict__ pl) {
  using Kv = KvDma<T, D, 2, true>;
  constexpr int BKV = Kv::BKV;
  __shared__ __align__(16) T ks0[Kv::TILE], vs0[Kv::TILE];
  __shared__ __align__(16) T ks1[NST > 1 ? Kv::TILE : 8], vs1[NST > 1 ? Kv::TILE : 8];

  const int lane = threadIdx.x & 63, lh = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nrep = H / G;
  const int k_begin = c * kch;
  const int nk = min(n, k_begin + kch) - k_begin;
  const int nkt = (nk + BKV - 1) / BKV;
  const bool hok = l32 < nrep;
  const long GD = (long)G * D;

  F8<T> qf[D / 16];
  const T* qrow = q + (long)b * ldq + (long)(g * nrep + (hok ? l32 : 0)) * D;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qf[s] = gld8<T>(qrow + 16 * s + 8 * lh, hok);

  Kv dma;
  const long row0 = (long)b * cap + k_begin;
  dma.init(ck + row0 * GD + (long)g * D, GD, cv + row0 * GD + (long)g * D, GD, nk, wave, lane);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  float lsum = 0.f;
  const float c1 = kLog2e / sqrtf((float)D);
  const float m0 = sqrtf((float)D) * kLog2e;

  auto body = [&](int kt, const T* sk, const T* sv) {
    const int kb = kt * BKV + 32 * wave;
    if (kb >= nk) return;
    f32x16 sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) mma32(sacc, swz_row8<T, D>(sk, 32 * wave + l32, 16 * s + 8 * lh), qf[s]);
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float e = fast_exp2(sacc[v] * c1 - m0);
      p[v] = kb + crow(v, lh) < nk ? e : 0.f;
      lsum += p[v];
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const F8<T> pf = pack8<T>(p + 8 * kk);
      const int k0 = 32 * wave + 16 * kk + 4 * lh;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) mma32(oacc[dt], vtr8<T, D>(sv, k0, k0 + 8, dt, lane), pf);
    }
  };

  if constexpr (NST > 1) {
    kv_ring<T, D>(dma, nkt, ks0, vs0, ks1, vs1, body);
  } else {
    for (int kt = 0; kt < nkt; ++kt) {
      if (kt) __syncthreads();  // both waves are done with the previous tile
      dma.issue(kt, ks0, vs0);
      ring_barrier<0>();
      body(kt, ks0, vs0);
    }
  }
  lsum += __shfl_xor(lsum, 32, 64);

  // wave 1 hands its sums to wave 0 through the (now idle) K stage
  __syncthreads();
  float* red = reinterpret_cast<float*>(ks0);
  static_assert(Kv::TILE * sizeof(T) >= (D / 32) * 16 * 64 * sizeof(float), "reduction fits in one K stage");
  if (wave == 1) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[(dt * 16 + v) * 64 + lane] = oacc[dt][v];
    reinterpret_cast<float*>(vs0)[lane] = lsum;
  }
  __syncthreads();
  if (wave == 0 && hok) {
    const long prow = ((long)b * gridDim.x + c) * H + (long)g * nrep + l32;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float4 o4;
        o4.x = oacc[dt][4 * j + 0] + red[(dt * 16 + 4 * j + 0) * 64 + lane];
        o4.y = oacc[dt][4 * j + 1] + red[(dt * 16 + 4 * j + 1) * 64 + lane];
        o4.z = oacc[dt][4 * j + 2] + red[(dt * 16 + 4 * j + 2) * 64 + lane];
        o4.w = oacc[dt][4 * j + 3] + red[(dt * 16 + 4 * j + 3) * 64 + lane];
        *reinterpret_cast<float4*>(po + prow * D + 32 * dt + 8 * j + 4 * lh) = o4;
      }
    if (lh == 0) pl[prow] = lsum + reinterpret_cast<const float*>(vs0)[lane];
  }
}

// o[b][h][:] = sum_c po[b][c][h][:] / sum_c pl[b][c][h], chunks in order.
template <typename T>
__global__ void attn_decode_merge_kernel(const float* __restrict__ po, const float* __restrict__ pl, int H, int D,
                                         int nchunk, T* __restrict__ o, long ldo) {
  constexpr int U = 8;  // chunks whose loads are issued together
  const int h = blockIdx.x, b = blockIdx.y, dd = threadIdx.x;  // blockDim.x == D
  float l = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < nchunk; c0 += U) {
    float lv[U], ov[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u < nchunk) {
        const long r = ((long)b * nchunk + c0 + u) * H + h;
        lv[u] = pl[r];
        ov[u] = po[r * D + dd];
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u < nchunk) {
        l += lv[u];
        acc += ov[u];
      }
  }
  o[(long)b * ldo + (long)h * D + dd] = from_f32<T>(acc / l);
}

// ============================================================ backward: dQ pass (+ Delta)
template <typename T, int D>
__global__ void __launch_bounds__(256, 2) attn_bwd_dq_kernel(AttnGeom g, const T* __restrict__ qk,
                                                             const T* __restrict__ vsrc, const T* __restrict__ o,
                                                             const T* __restrict__ dO, const float* __restrict__ lse,
                                                             float2* __restrict__ rowstat, T* __restrict__ dq) {
  using Kv = KvDma<T, D>;
  constexpr int BKV = Kv::BKV;
  __shared__ __align__(16) T ks0[Kv::TILE], vs0[Kv::TILE], ks1[Kv::TILE], vs1[Kv::TILE];

  const int tid = threadIdx.x, lane = tid & 63, lh = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = (lane >> 4) & 1;
  const int nrows = g.T * g.n_rep;
  const int nqb = (nrows + 127) / 128;
  const int per = g.G * g.B;
  const int qb = nqb - 1 - (int)(blockIdx.x / per);
  const int kvh = blockIdx.x % per % g.G, b = blockIdx.x % per / g.G;
  const int R0 = qb * 128;
  const long tok0 = (long)b * g.T;
  const DivN dv{g.n_rep, g.inv_rep};

  const int rq = R0 + 32 * wave + l32;
  const bool qok = rq < nrows;
  const int tq = qok ? dv.q(rq) : 0;
  const int hq = kvh * g.n_rep + (qok ? rq - tq * g.n_rep : 0);
  const int t_wmax = dv.q(min(nrows - 1, R0 + 32 * wave + 31));
  const int t_wmin = dv.q(min(nrows - 1, R0 + 32 * wave));
  const bool wfull = R0 + 32 * wave + 31 < nrows;
  const int t_bmax = dv.q(min(nrows - 1, R0 + 127));
  const int nkt = t_bmax / BKV + 1;

  const long qi = (tok0 + tq) * g.H + hq;
  F8<T> qf[D / 16], df[D / 16];
  const T* qrow = qk + (tok0 + tq) * g.ld_qk + (long)hq * D;
  const T* drow = dO + (tok0 + tq) * g.ld_o + (long)hq * D;
  const T* orow = o + (tok0 + tq) * g.ld_o + (long)hq * D;
  float dsum = 0.f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = gld8<T>(qrow + 16 * s + 8 * lh, qok);
    df[s] = gld8<T>(drow + 16 * s + 8 * lh, qok);
    F8<T> of = gld8<T>(orow + 16 * s + 8 * lh, qok);
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum += to_f32(df[s].v[e]) * to_f32(of.v[e]);
  }
  dsum += __shfl_xor(dsum, 32, 64);
  const float dlt = dsum;
  const float lse2 = qok ? lse[qi] * kLog2e : 0.f;
  // (lse log2 e, -Delta) of each flattened row, in row order, for the dK/dV
  // pass (which starts its dP accumulators at -Delta)
  if (qok && lh == 0) rowstat[((long)b * g.G + kvh) * nrows + rq] = make_float2(lse2, -dlt);
  const float c1 = kLog2e / sqrtf((float)D);

  Kv dma;
  dma.init(qk + tok0 * g.ld_qk + g.q_off_k + (long)kvh * D, g.ld_qk, vsrc + tok0 * g.ld_v + (long)kvh * D, g.ld_v,
           g.T, wave, lane);

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) dqacc[i][v] = 0.f;

  kv_ring<T, D>(dma, nkt, ks0, vs0, ks1, vs1, [&](int kt, const T* sk, const T* sv) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kb = kt * BKV + 32 * sub;
      if (kb > t_wmax) continue;
      f32x16 sacc, pacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) { sacc[v] = 0.f; pacc[v] = 0.f; }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        F8<T> kf = swz_row8<T, D>(sk, 32 * sub + l32, 16 * s + 8 * lh);
        mma32(sacc, kf, qf[s]);
        F8<T> vf = swz_row8<T, D>(sv, 32 * sub + l32, 16 * s + 8 * lh);
        mma32(pacc, vf, df[s]);
      }
      float ds[16];
      if (wfull && kb + 31 <= t_wmin) {
#pragma unroll
        for (int v = 0; v < 16; ++v) ds[v] = fast_exp2(sacc[v] * c1 - lse2) * (pacc[v] - dlt);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          // a 0/1 factor, not a select: the compiler would put the exponential
          // under a branch per element (every score is bounded, so the
          // masked products are finite)
          const int key = kb + crow(v, lh);
          const float p = fast_exp2(sacc[v] * c1 - lse2);
          ds[v] = p * (pacc[v] - dlt) * (float)(qok && key <= tq);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        F8<T> sf = pack8<T>(ds + 8 * kk);
        const int k0 = 32 * sub + 16 * kk + 4 * lh;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          F8<T> kf = swz_tr8<T, D>(sk, k0, k0 + 8, 32 * dt + 16 * g16, lane);
          mma32(dqacc[dt], kf, sf);
        }
      }
    }
  });

  if (qok) {
    const float sc = 1.f / sqrtf((float)D);
    T* out = dq + (tok0 + tq) * g.ld_dq + (long)hq * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[32 * dt + 8 * j + 4 * lh + i] = from_f32<T>(dqacc[dt][4 * j + i] * sc);
  }
}

// ============================================================ backward: dK/dV pass
// Block: 128 keys, 8 waves. Waves w and w+4 share the 32 keys 32*(w%4) ..:
//   wave w   (P side)  holds K, forms S = Q K^T and P = exp(S - lse), passes P
//                      to its partner through LDS and accumulates dV += P^T dO;
//   wave w+4 (dS side) holds V, forms dP = dO V^T, takes P one tile later,
//                      dS = P (dP - Delta) and accumulates dK += dS^T Q.
// So each wave keeps one 32-key operand and one accumulator set (half of what
// one wave doing both needs), two waves share a SIMD, and no MFMA is repeated.
// The flattened query rows of all heads sharing the KV head stream through a
// 3-stage LDS ring of Q and dO tiles filled by direct-to-LDS loads
// (XOR-swizzled 16-byte chunks: conflict-free for the row reads of S and dP
// and for the transposing reads of dV and dK), each wave also staging its
// own copy of the tiles' (lse log2 e, -Delta) pairs. Tiles run from the last
// query row down, so that all key blocks of a sequence start on the same rows
// and share them in L2.

// A ring step covers NSUB sub-tiles of 32 query rows, one after the other
// between two barriers: with bf16 two (64 rows, 3 stages of 32 KB; 1-2 %
// faster than 32-row steps through 4 stages, which had twice the barriers);
// float tiles are twice the size and keep one.
template <typename T, int D>
struct DkdvShape {
  static constexpr int NSUB = sizeof(T) == 2 ? 2 : 1;
  static constexpr int BQ = 32 * NSUB;               // query rows per tile (ring step)
  static constexpr int WAVES = 8;
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int TILE = BQ * D;                // elements of one Q or dO tile
  static constexpr int NQI = TILE / VE / 64;         // 16-byte load instructions per tile
  static constexpr int NPW = 2 * NQI / WAVES;        // per wave, Q and dO together
  static constexpr int NI = NPW + NSUB;              // + the row statistics, 32 rows per load
  static constexpr int STAGES = 3;
  static constexpr int AHEAD = STAGES - 2;           // tiles in flight beyond the one waited for
  static constexpr int WAIT = (AHEAD - 1) * NI;
  static_assert((2 * NQI) % WAVES == 0, "tile loads split evenly over the waves");
};

// UP: the query tiles run from the key block's diagonal upwards, else from
// the last row down.
template <typename T, int D, bool UP = false>
struct DkdvCtx {
  using Sh = DkdvShape<T, D>;
  int nrows, r_start, ntiles, T_, kw0, lane, wave, kw;
  bool kok;
  DivN dvn;
  int n_rep, hbase;  // first query head of the KV head
  long ld_qk, ld_o;
  __amdgpu_buffer_rsrc_t rq, rd, rs;
  // per load instruction of this wave: tile row, chunk column offset, operand
  int lrow[Sh::NPW], lcol[Sh::NPW], lblk[Sh::NPW];
  bool ldo[Sh::NPW];
  // and, for the tile the next issue() loads: the row, its head index within
  // the KV group (h in [0, n_rep)) and its byte offset. Tiles are issued in
  // order, each BQ rows below the last, so these advance by a subtraction and
  // a borrow instead of a division per load.
  int nr[Sh::NPW], nh[Sh::NPW], noff[Sh::NPW];
  int dr, dstep[Sh::NPW], wrap[Sh::NPW];

  __device__ __forceinline__ int row0(int s) const { return r_start + Sh::BQ * (UP ? s : ntiles - 1 - s); }

  // The state for step 0, once (n_rep, hbase, lrow, lcol, ldo, ld_* set).
  __device__ __forceinline__ void init_rows() {
    const int dq = Sh::BQ / n_rep;
    dr = Sh::BQ - dq * n_rep;
#pragma unroll
    for (int i = 0; i < Sh::NPW; ++i) {
      const long ld = ldo[i] ? ld_o : ld_qk;
      const int r = row0(0) + lrow[i];
      const int t = dvn.q(r);  // rows up to nrows + BQ: inside the divider's range
      nr[i] = r;
      nh[i] = r - t * n_rep;
      noff[i] = (int)((t * ld + (long)(hbase + nh[i]) * D + lcol[i]) * (long)sizeof(T));
      dstep[i] = (int)(((long)dq * ld + (long)dr * D) * (long)sizeof(T));
      wrap[i] = (int)(((long)n_rep * D - ld) * (long)sizeof(T));
    }
  }

  // Loads of the tile processed at step s into one ring stage; steps are
  // issued in order 0, 1, 2, ...
  __device__ __forceinline__ void issue(int s, T* __restrict__ sq, T* __restrict__ sd, float* __restrict__ ss) {
    const int rq0 = row0(s);
    const bool live = s < ntiles;
#pragma unroll
    for (int i = 0; i < Sh::NPW; ++i) {
      const unsigned off = (live && nr[i] < nrows) ? (unsigned)noff[i] : kDmaOOB;
      // the same load of the next tile, BQ rows = dq positions and dr heads away:
      // down with a borrow, or up with a carry
      if constexpr (UP) {
        nr[i] += Sh::BQ;
        nh[i] += dr;
        noff[i] += dstep[i];
        const bool carry = nh[i] >= n_rep;
        nh[i] -= carry ? n_rep : 0;
        noff[i] -= carry ? wrap[i] : 0;
      } else {
        nr[i] -= Sh::BQ;
        nh[i] -= dr;
        noff[i] -= dstep[i];
        const bool borrow = nh[i] < 0;
        nh[i] += borrow ? n_rep : 0;
        noff[i] += borrow ? wrap[i] : 0;
      }
      T* dst = (ldo[i] ? sd : sq) + lblk[i] * 64 * Sh::VE;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ldo[i] ? rd : rq, (lds_void*)dst, 16, off, 0, 0, 0);
    }
    // per 32-row sub-tile: lanes 0-31 take the rows' lse2, lanes 32-63 their
    // -Delta, so each lands as 32 consecutive floats
#pragma unroll
    for (int u = 0; u < Sh::NSUB; ++u) {
      const int row = rq0 + 32 * u + (lane & 31);
      const unsigned soff = (live && row < nrows) ? (unsigned)(2 * row + (lane >> 5)) * 4u : kDmaOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(ss + 64 * (Sh::NSUB * wave + u)), 4, soff, 0, 0, 0);
    }
  }

  // Sub-tile u of step s has no unmasked pair for this wave's keys.
  __device__ __forceinline__ bool skip(int s, int u) const {
    if (s < 0 || s >= ntiles) return true;
    const int rq0 = row0(s) + 32 * u;
    return rq0 >= nrows || dvn.q(min(nrows - 1, rq0 + 31)) < kw0;
  }
  __device__ __forceinline__ bool full(int s, int u) const {
    const int rq0 = row0(s) + 32 * u;
    return kw0 + 32 <= T_ && rq0 + 32 <= nrows && dvn.q(rq0) >= kw0 + 31;
  }
};

// P side of sub-tile u (32 rows) of step s: S = Q K^T, P, hand P over, dV += P^T dO.
// Row rq0 + q is unmasked for this lane's key iff key <= (rq0 + q) / n_rep,
// i.e. q >= key n_rep - rq0, and rq0 + q < nrows: one unsigned range test per
// element after the exponentials, on every sub-tile. (A select before the
// exponentials became a branch around each of them; the test under a branch
// taken only on the diagonal was turned into selects on every sub-tile
// anyway, and an unmasked copy of the body as a block of its own pushed the
// kernel past its registers.)
template <typename T, int D, typename Ctx>
__device__ __forceinline__ void dkdv_tile_p_body(const Ctx& c, int s, int u, const T* __restrict__ sq,
                                                 const T* __restrict__ sdo, const float* __restrict__ st, F8<T>* pb,
                                                 f32x16* acc, const F8<T>* kf, float c1) {
  using Sh = DkdvShape<T, D>;
  sq += 32 * D * u;  // rows 32 u .. of the tile: the same swizzle (it repeats every 16 rows)
  sdo += 32 * D * u;
  pb += 512 * u;
  const int lane = c.lane, lh = lane >> 5, l32 = lane & 31, g16 = (lane >> 4) & 1;
  f32x16 sacc;
#pragma unroll
  for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
  for (int k = 0; k < D / 16; ++k) mma32(sacc, swz_row8<T, D>(sq, l32, 16 * k + 8 * lh), kf[k]);
  const float* sw = st + 64 * (Sh::NSUB * c.wave + u);
  float p[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 a = *reinterpret_cast<const float4*>(sw + 8 * j + 4 * lh);  // lse2 of the rows
    const float la[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) p[4 * j + i] = fast_exp2(sacc[4 * j + i] * c1 - la[i]);
  }
  {
    const int rq0 = c.row0(s) + 32 * u, key = c.kw0 + l32;
    const int lo = c.kok ? key * c.n_rep - rq0 : 0x3fffffff;  // q >= lo and q < nrows - rq0
    const unsigned span = (unsigned)max(0, c.nrows - rq0 - lo);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = 8 * j + 4 * lh + i;
        p[4 * j + i] = (unsigned)(q - lo) < span ? p[4 * j + i] : 0.f;
      }
  }
  const F8<T> pf0 = pack8<T>(p), pf1 = pack8<T>(p + 8);
  pb[(2 * c.kw) * 64 + lane] = pf0;
  pb[(2 * c.kw + 1) * 64 + lane] = pf1;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int k0 = 16 * kk + 4 * lh;
#pragma unroll
    for (int dti = 0; dti < D / 32; ++dti)
      mma32(acc[dti], swz_tr8<T, D>(sdo, k0, k0 + 8, 32 * dti + 16 * g16, lane), kk ? pf1 : pf0);
  }
}

template <typename T, int D, typename Ctx>
__device__ __forceinline__ void dkdv_tile_p(const Ctx& c, int s, int u, const T* __restrict__ sq,
                                            const T* __restrict__ sdo, const float* __restrict__ st, F8<T>* pb,
                                            f32x16* acc, const F8<T>* kf, float c1) {
  if (c.skip(s, u)) return;
  dkdv_tile_p_body<T, D>(c, s, u, sq, sdo, st, pb, acc, kf, c1);
}

// dS side of sub-tile u of step s: dP = dO V^T, dS = P (dP - Delta), dK += dS^T Q.
template <typename T, int D, typename Ctx>
__device__ __forceinline__ void dkdv_tile_ds(const Ctx& c, int s, int u, const T* __restrict__ sq,
                                             const T* __restrict__ sdo, const float* __restrict__ st,
                                             const F8<T>* pb, f32x16* acc, const F8<T>* vf) {
  if (c.skip(s, u)) return;
  using Sh = DkdvShape<T, D>;
  sq += 32 * D * u;
  sdo += 32 * D * u;
  pb += 512 * u;
  const int lane = c.lane, lh = lane >> 5, l32 = lane & 31, g16 = (lane >> 4) & 1;
  // dP - Delta: the accumulators start at the rows' -Delta
  const float* sw = st + 64 * (Sh::NSUB * c.wave + u);
  f32x16 pacc;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 a = *reinterpret_cast<const float4*>(sw + 32 + 8 * j + 4 * lh);
    pacc[4 * j] = a.x;
    pacc[4 * j + 1] = a.y;
    pacc[4 * j + 2] = a.z;
    pacc[4 * j + 3] = a.w;
  }
#pragma unroll
  for (int k = 0; k < D / 16; ++k) mma32(pacc, swz_row8<T, D>(sdo, l32, 16 * k + 8 * lh), vf[k]);
  const F8<T> pf0 = pb[(2 * c.kw) * 64 + lane], pf1 = pb[(2 * c.kw + 1) * 64 + lane];
  float ds[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) ds[v] = to_f32((v < 8 ? pf0 : pf1).v[v & 7]) * pacc[v];
  const F8<T> sf0 = pack8<T>(ds), sf1 = pack8<T>(ds + 8);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int k0 = 16 * kk + 4 * lh;
#pragma unroll
    for (int dti = 0; dti < D / 32; ++dti)
      mma32(acc[dti], swz_tr8<T, D>(sq, k0, k0 + 8, 32 * dti + 16 * g16, lane), kk ? sf1 : sf0);
  }
}

// One ring step s: wait for the tile of step s, refill the stage two tiles
// ahead, then the P side works on tile s and the dS side on tile s - 1 (whose
// P was handed over before this step's barrier).
#define NC_DKDV_STEP(S_, CUR, PRV, NXT)                                                                    \
  {                                                                                                        \
    const int s_ = (S_);                                                                                   \
    ring_barrier<Sh::WAIT>();                                                                              \
    c.issue(s_ + Sh::AHEAD, q##NXT, d##NXT, t##NXT);                                                      \
    _Pragma("unroll") for (int u_ = 0; u_ < Sh::NSUB; ++u_) {                                             \
      if constexpr (ROLE == 0)                                                                             \
        dkdv_tile_p<T, D>(c, s_, u_, q##CUR, d##CUR, t##CUR, pb + (s_ & 1) * 512 * Sh::NSUB, acc, kv, c1); \
      else                                                                                                 \
        dkdv_tile_ds<T, D>(c, s_ - 1, u_, q##PRV, d##PRV, t##PRV, pb + ((s_ - 1) & 1) * 512 * Sh::NSUB,    \
                           acc, kv);                                                                       \
    }                                                                                                      \
  }

template <int ROLE, typename T, int D, typename Ctx>
__device__ __forceinline__ void dkdv_ring(Ctx& c, f32x16* acc, const F8<T>* kv, F8<T>* pb,
                                          float c1, T* __restrict__ q0, T* __restrict__ q1, T* __restrict__ q2,
                                          T* __restrict__ q3, T* __restrict__ d0, T* __restrict__ d1,
                                          T* __restrict__ d2, T* __restrict__ d3, float* __restrict__ t0,
                                          float* __restrict__ t1, float* __restrict__ t2, float* __restrict__ t3) {
  using Sh = DkdvShape<T, D>;
  const int nsteps = c.ntiles + 1;  // the dS side trails by one tile
  c.issue(0, q0, d0, t0);
  if constexpr (Sh::STAGES == 4) {
    c.issue(1, q1, d1, t1);
    int s = 0;
    for (; s + 4 <= nsteps; s += 4) {
      NC_DKDV_STEP(s, 0, 3, 2);
      NC_DKDV_STEP(s + 1, 1, 0, 3);
      NC_DKDV_STEP(s + 2, 2, 1, 0);
      NC_DKDV_STEP(s + 3, 3, 2, 1);
    }
    if (s < nsteps) NC_DKDV_STEP(s, 0, 3, 2);
    if (s + 1 < nsteps) NC_DKDV_STEP(s + 1, 1, 0, 3);
    if (s + 2 < nsteps) NC_DKDV_STEP(s + 2, 2, 1, 0);
  } else {
    int s = 0;
    for (; s + 3 <= nsteps; s += 3) {
      NC_DKDV_STEP(s, 0, 2, 1);
      NC_DKDV_STEP(s + 1, 1, 0, 2);
      NC_DKDV_STEP(s + 2, 2, 1, 0);
    }
    if (s < nsteps) NC_DKDV_STEP(s, 0, 2, 1);
    if (s + 1 < nsteps) NC_DKDV_STEP(s + 1, 1, 0, 2);
  }
  // the last refills target tiles past the end; let them land before exit
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8) | (0 << 14));
}
#undef NC_DKDV_STEP

// One key block of the dK/dV pass (kblk), its query tiles walked down or up.
template <typename T, int D, bool UP>
__device__ __forceinline__ void dkdv_part(const AttnGeom& g, const T* __restrict__ qk, const T* __restrict__ vsrc,
                                          const T* __restrict__ dO, const float2* __restrict__ rowstat,
                                          T* __restrict__ dk, T* __restrict__ dv, long ld_dkv, int kblk, int kvh, int b,
                                          long tok0, int role, int lane, int lh, int l32, int wave, float c1,
                                          T* __restrict__ q0, T* __restrict__ q1, T* __restrict__ q2,
                                          T* __restrict__ q3, T* __restrict__ d0, T* __restrict__ d1,
                                          T* __restrict__ d2, T* __restrict__ d3, float* __restrict__ t0,
                                          float* __restrict__ t1, float* __restrict__ t2, float* __restrict__ t3,
                                          F8<T>* pb) {
  using Sh = DkdvShape<T, D>;
  const int kb0 = kblk * 128;

  DkdvCtx<T, D, UP> c;
  c.lane = lane;
  c.wave = wave;
  c.kw = wave & 3;
  c.kw0 = kb0 + 32 * c.kw;
  c.T_ = g.T;
  c.kok = c.kw0 + l32 < g.T;
  c.dvn = DivN{g.n_rep, g.inv_rep};
  c.n_rep = g.n_rep;
  c.hbase = kvh * g.n_rep;
  c.nrows = g.T * g.n_rep;
  c.r_start = (kb0 * g.n_rep) / Sh::BQ * Sh::BQ;
  c.ntiles = c.r_start < c.nrows ? (c.nrows - c.r_start + Sh::BQ - 1) / Sh::BQ : 0;
  c.ld_qk = g.ld_qk;
  c.ld_o = g.ld_o;
  c.rq = dma_rsrc(qk + tok0 * g.ld_qk);
  c.rd = dma_rsrc(dO + tok0 * g.ld_o);
  c.rs = dma_rsrc(rowstat + ((long)b * g.G + kvh) * c.nrows);
#pragma unroll
  for (int i = 0; i < Sh::NPW; ++i) {
    const int ins = wave * Sh::NPW + i;  // Q tile instructions first, then dO
    const int blk = ins % Sh::NQI;
    const int u = 64 * blk + lane;       // chunk slot inside the tile
    const int row = u / Swz<T, D>::NC, pc = u % Swz<T, D>::NC;
    c.ldo[i] = ins >= Sh::NQI;
    c.lblk[i] = blk;
    c.lrow[i] = row;
    c.lcol[i] = (pc ^ Swz<T, D>::f(row)) * Sh::VE;
  }
  c.init_rows();

  // own 32 keys: K (P side) or V (dS side) as B operands, 8 consecutive d per lane
  const int key = c.kw0 + l32;
  F8<T> kv[D / 16];
  const T* src = role == 0 ? qk + (tok0 + (c.kok ? key : 0)) * g.ld_qk + g.q_off_k + (long)kvh * D
                           : vsrc + (tok0 + (c.kok ? key : 0)) * g.ld_v + (long)kvh * D;
#pragma unroll
  for (int k = 0; k < D / 16; ++k) kv[k] = gld8<T>(src + 16 * k + 8 * lh, c.kok);
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

  if (role == 0) dkdv_ring<0, T, D>(c, acc, kv, pb, c1, q0, q1, q2, q3, d0, d1, d2, d3, t0, t1, t2, t3);
  else dkdv_ring<1, T, D>(c, acc, kv, pb, c1, q0, q1, q2, q3, d0, d1, d2, d3, t0, t1, t2, t3);

  if (c.kok) {
    const float sc = role == 0 ? 1.f : 1.f / sqrtf((float)D);
    T* out = (role == 0 ? dv : dk) + (tok0 + key) * ld_dkv + (long)kvh * D;
#pragma unroll
    for (int dti = 0; dti < D / 32; ++dti)
#pragma unroll
      for (int v = 0; v < 16; ++v) out[32 * dti + crow(v, lh)] = from_f32<T>(acc[dti][v] * sc);
  }
  // every wave is done with the ring and the hand-over buffers before the
  // next key block's loads overwrite them
  __syncthreads();
}

// Block p of a (sequence, KV head) takes two key blocks, p and nkb - 1 - p:
// their causal work adds up to the same for every p, so the grid of
// ceil(nkb / 2) blocks per sequence has no tail. The first key block walks
// the query tiles from the last row down, the second from its diagonal up.
// All first parts of a sequence start together on the last row; the second
// parts start at different times but one key block (20 tiles at 10 heads)
// lower for every tile they start earlier, so they too reach every row
// together. Either way a tile of Q and dO is fetched once and read from L2
// by every key block of its sequence (the blocks of one sequence share an
// XCD: workgroups go round-robin over the 8 XCDs and the sequence index is
// the block index modulo the (sequence, head) count).
template <typename T, int D>
__global__ void __launch_bounds__(512, 1) attn_bwd_dkdv_kernel(AttnGeom g, const T* __restrict__ qk,
                                                               const T* __restrict__ vsrc, const T* __restrict__ dO,
                                                               const float2* __restrict__ rowstat,
                                                               T* __restrict__ dk, T* __restrict__ dv, long ld_dkv) {
  using Sh = DkdvShape<T, D>;
  __shared__ __align__(16) T q0[Sh::TILE], q1[Sh::TILE], q2[Sh::TILE], q3[Sh::STAGES == 4 ? Sh::TILE : 1];
  __shared__ __align__(16) T d0[Sh::TILE], d1[Sh::TILE], d2[Sh::TILE], d3[Sh::STAGES == 4 ? Sh::TILE : 1];
  __shared__ __align__(16) float t0[64 * Sh::NSUB * Sh::WAVES], t1[64 * Sh::NSUB * Sh::WAVES],
      t2[64 * Sh::NSUB * Sh::WAVES], t3[Sh::STAGES == 4 ? 64 * Sh::NSUB * Sh::WAVES : 1];
  // P hand-over: [parity][sub-tile][key group][half][lane]
  __shared__ __align__(16) F8<T> pb[2 * 512 * Sh::NSUB];

  const int tid = threadIdx.x, lane = tid & 63, lh = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets and buffer resources
  const int per = g.G * g.B;
  const int nkb = (g.T + 127) / 128;
  const int pair = (int)(blockIdx.x / per);
  const int kvh = blockIdx.x % per % g.G, b = blockIdx.x % per / g.G;
  const long tok0 = (long)b * g.T;
  const int role = wave >> 2;
  const float c1 = kLog2e / sqrtf((float)D);

  dkdv_part<T, D, false>(g, qk, vsrc, dO, rowstat, dk, dv, ld_dkv, pair, kvh, b, tok0, role, lane, lh, l32, wave, c1,
                         q0, q1, q2, q3, d0, d1, d2, d3, t0, t1, t2, t3, pb);
  if (nkb - 1 - pair != pair)  // the middle key block of an odd count: one part
    dkdv_part<T, D, true>(g, qk, vsrc, dO, rowstat, dk, dv, ld_dkv, nkb - 1 - pair, kvh, b, tok0, role, lane, lh, l32,
                          wave, c1, q0, q1, q2, q3, d0, d1, d2, d3, t0, t1, t2, t3, pb);
}

// Unmasked (query, key) pairs of causal attention over all heads and rows.
double causal_pairs(const AttnGeom& g) { return (double)g.B * g.H * g.T * (g.T + 1.0) / 2.0; }

template <typename T, int D>
nc_status attn_fwd_impl(const AttnGeom& g, const T* qk, const T* v, T* o, float* lse, hipStream_t st,
                        uint32_t* amax) {
  int nqb = (g.T * g.n_rep + 127) / 128;
  const double tok = (double)g.B * g.T, es = sizeof(T);
  // S = Q K^T and O = P V: 4 D flops per pair
  ProfScope prof(NC_NAME(T, "attn_fwd"), 4.0 * D * causal_pairs(g),
                 es * tok * D * (2.0 * g.H + 2.0 * g.G) + 4.0 * tok * g.H, st);
  if (amax)
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, true>), dim3(nqb * g.G * g.B), dim3(256), 0, st, g, qk, v, o, lse,
                       amax);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, false>), dim3(nqb * g.G * g.B), dim3(256), 0, st, g, qk, v, o, lse,
                       amax);
  NC_LAUNCH_CHECK("attn_fwd");
  return NC_OK;
}

template <typename T, int D>
nc_status attn_bwd_impl(const AttnGeom& g, const T* qk, const T* v, const T* o, const T* dO, const float* lse,
                        float* rowstat, T* dq, T* dk, T* dv, long ld_dkv, hipStream_t st) {
  // the dK/dV ring addresses one sequence of Q and dO through 32-bit offsets
  if ((double)g.T * (double)(g.ld_qk > g.ld_o ? g.ld_qk : g.ld_o) * sizeof(T) >= (double)kDmaOOB)
    return NC_ERR_UNSUPPORTED;
  int nqb = (g.T * g.n_rep + 127) / 128;
  const double tok = (double)g.B * g.T, es = sizeof(T);
  float2* rs = reinterpret_cast<float2*>(rowstat);
  {
    // recompute S, then dP = dO V^T and dQ = dS K: 6 D flops per pair
    ProfScope prof(NC_NAME(T, "attn_bwd_dq"), 6.0 * D * causal_pairs(g),
                   es * tok * D * (4.0 * g.H + 2.0 * g.G) + 12.0 * tok * g.H, st);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D>), dim3(nqb * g.G * g.B), dim3(256), 0, st, g, qk, v, o, dO, lse,
                       rs, dq);
    NC_LAUNCH_CHECK("attn_bwd_dq");
  }
  int nkb = (g.T + 127) / 128;
  // recompute S and dP, then dV = P^T dO and dK = dS^T Q: 8 D flops per pair
  ProfScope prof(NC_NAME(T, "attn_bwd_dkdv"), 8.0 * D * causal_pairs(g),
                 es * tok * D * (2.0 * g.H + 4.0 * g.G) + 8.0 * tok * g.H, st);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D>), dim3((nkb + 1) / 2 * g.G * g.B), dim3(512), 0, st, g, qk, v, dO,
                     rs, dk, dv, ld_dkv);
  NC_LAUNCH_CHECK("attn_bwd_dkdv");
  return NC_OK;
}

// Keys per decode block: one 64-key tile while the grid stays within about
// two 2-wave blocks per CU, more tiles per block (through the 2-stage ring)
// for longer caches. (A target of five blocks per CU, one tile each at the
// benchmark's cache lengths, was 14 % slower: more blocks, each waiting on
// one load, and more chunk partials to merge.)
int decode_chunk_keys(int n, int BG) {
  const long work = (long)BG * ((n + 63) / 64);
  const long nt = (work + 511) / 512;
  return 64 * (int)(nt < 1 ? 1 : nt);
}

template <typename T, int D>
nc_status attn_decode_impl(const T* q, long ldq, const T* ck, const T* cv, int B, int H, int G, int n, int cap, T* o,
                           long ldo, float* po, float* pl, hipStream_t st) {
  const int kch = decode_chunk_keys(n, B * G);
  const int nchunk = (n + kch - 1) / kch;
  // reads every cached key and value once, plus the queries, writes the outputs
  ProfScope prof(NC_NAME(T, "attn_decode"), 4.0 * D * (double)B * H * n,
                 sizeof(T) * ((double)B * n * G * D * 2.0 + 2.0 * B * H * D), st);
  dim3 grid(nchunk, G, B);
  if (kch == 64)
    hipLaunchKernelGGL((attn_decode_kernel<T, D, 1>), grid, dim3(128), 0, st, q, ldq, ck, cv, H, G, n, cap, kch, po,
                       pl);
  else
    hipLaunchKernelGGL((attn_decode_kernel<T, D, 2>), grid, dim3(128), 0, st, q, ldq, ck, cv, H, G, n, cap, kch, po,
                       pl);
  NC_LAUNCH_CHECK("attn_decode");
  hipLaunchKernelGGL((attn_decode_merge_kernel<T>), dim3(H, B), dim3(D), 0, st, po, pl, H, D, nchunk, o, ldo);
  NC_LAUNCH_CHECK("attn_decode_merge");
  return NC_OK;
}

AttnGeom make_geom(const AttnArgs& a) {
  AttnGeom g;
  g.B = a.B; g.T = a.T; g.H = a.H; g.G = a.G; g.D = a.D; g.n_rep = a.H / a.G;
  g.ld_qk = a.ld_qk; g.ld_v = a.ld_v; g.ld_o = a.ld_o; g.ld_dq = a.ld_dq;
  g.q_off_k = a.H * a.D;
  g.inv_rep = 1.0f / (float)g.n_rep;
  return g;
}

}  // namespace

template <typename T>
nc_status attn_fwd(const AttnArgs& a, const T* qk, const T* v, T* o, float* lse, hipStream_t st, uint32_t* amax) {
  AttnGeom g = make_geom(a);
  if (a.D == 128) return attn_fwd_impl<T, 128>(g, qk, v, o, lse, st, amax);
  if (a.D == 64) return attn_fwd_impl<T, 64>(g, qk, v, o, lse, st, amax);
  return NC_ERR_UNSUPPORTED;
}

template <typename T>
nc_status attn_bwd(const AttnArgs& a, const T* qk, const T* v, const T* o, const T* dO, const float* lse,
                   float* rowstat, T* dq, T* dk, T* dv, long ld_dkv, hipStream_t st) {
  AttnGeom g = make_geom(a);
  if (a.D == 128) return attn_bwd_impl<T, 128>(g, qk, v, o, dO, lse, rowstat, dq, dk, dv, ld_dkv, st);
  if (a.D == 64) return attn_bwd_impl<T, 64>(g, qk, v, o, dO, lse, rowstat, dq, dk, dv, ld_dkv, st);
  return NC_ERR_UNSUPPORTED;
}

int attn_decode_chunks(int cap) { return (cap + 63) / 64; }

template <typename T>
nc_status attn_decode(const T* q, long ldq, const T* ck, const T* cv, int B, int H, int G, int D, int n, int cap,
                      T* o, long ldo, float* po, float* pl, hipStream_t st) {
  if (G < 1 || H % G != 0 || H / G > 32 || n < 1 || n > cap) return NC_ERR_UNSUPPORTED;
  // the DMA tiles address 64 cache rows through 32-bit offsets
  if (64.0 * G * D * sizeof(T) >= (double)kDmaOOB) return NC_ERR_UNSUPPORTED;
  if (D == 128) return attn_decode_impl<T, 128>(q, ldq, ck, cv, B, H, G, n, cap, o, ldo, po, pl, st);
  if (D == 64) return attn_decode_impl<T, 64>(q, ldq, ck, cv, B, H, G, n, cap, o, ldo, po, pl, st);
  return NC_ERR_UNSUPPORTED;
}
template nc_status attn_decode<bf16>(const bf16*, long, const bf16*, const bf16*, int, int, int, int, int, int, bf16*,
                                     long, float*, float*, hipStream_t);
template nc_status attn_decode<float>(const float*, long, const float*, const float*, int, int, int, int, int, int,
                                      float*, long, float*, float*, hipStream_t);

template nc_status attn_fwd<bf16>(const AttnArgs&, const bf16*, const bf16*, bf16*, float*, hipStream_t, uint32_t*);
template nc_status attn_fwd<float>(const AttnArgs&, const float*, const float*, float*, float*, hipStream_t,
                                   uint32_t*);
template nc_status attn_bwd<bf16>(const AttnArgs&, const bf16*, const bf16*, const bf16*, const bf16*, const float*,
                                  float*, bf16*, bf16*, bf16*, long, hipStream_t);
template nc_status attn_bwd<float>(const AttnArgs&, const float*, const float*, const float*, const float*,
                                   const float*, float*, float*, float*, float*, long, hipStream_t);

}  // namespace nc
