// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include "common.h"

namespace nc {

// Times one launch with HIP events while profiling is on (prof.hip); `name`
// must be a string literal. flops/bytes: the launch's algorithmic work.
class ProfScope {
 public:
  ProfScope(const char* name, double flops, double bytes, hipStream_t st);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  int slot_;
  hipStream_t st_;
};

template <typename T> constexpr bool is_bf16() { return sizeof(T) == 2; }
#define NC_NAME(T, base) (is_bf16<T>() ? base "_bf16" : base "_f32")

// ------------------------------------------------------------ GEMM (gemm.hip)
// y[M,N] = act(x[M,K] W[N,K]^T) (+ res[M,N]); relu_sq_out makes act the
// ReLU^2 activation max(.,0)^2, else the identity.
template <typename T>
nc_status gemm_xwt(const T* x, const T* w, T* y, const T* res, int M, int N, int K, bool relu_sq_out,
                   hipStream_t st);
// dx[M,K] = dy[M,N] W[N,K]; with act = max(u,0)^2 given, dx = (dy W) * 2 sqrt(act),
// the input gradient of the ReLU^2 activation.
// dy_panel: dy stored in column panels (stride dy_panel elements), else 0.
template <typename T>
nc_status gemm_dyw(const T* dy, const T* w, T* dx, const T* act, int M, int N, int K, hipStream_t st,
                   long dy_panel = 0);
// dW[N,K] (+)= dy[M,N]^T x[M,K] (float32), split over M when that helps fill
// the GPU (partials in `partial`, summed in a fixed order).
template <typename T>
nc_status gemm_dw(const T* dy, const T* x, float* dw, int M, int N, int K, int accumulate, float* partial,
                  size_t partial_elems, hipStream_t st, long dy_panel = 0);
size_t gemm_dw_partial_elems(int M, int N, int K);
// Unembedding with the softcap epilogue: z = c tanh((x W^T)/c) stored [M,N] in column panels;
// part[M, lmhead_tiles(N)] = per-tile sums of exp(z); zt[m] = z[m][targets[m]].
template <typename T>
nc_status gemm_lmhead(const T* x, const T* w, T* z, int M, int N, int K, float cap, const int32_t* targets,
                      float* part, float* zt, hipStream_t st);
int lmhead_tiles(int N, bool bf16_storage);
// y = act(x[M,K] W[N,K]^T) (+ res) for a few rows (M up to a tile): the
// reduction is split so that enough workgroups stream W, the float32 partials
// are summed in a fixed order; y in the storage type or float32.
template <typename T>
nc_status gemm_xwt_small(const T* x, const T* w, void* y, bool y_f32, const T* res, bool relu_sq, int M, int N, int K,
                         float* partial, size_t partial_elems, hipStream_t st);
size_t gemm_small_partial_elems(int M, int N, int K);

// ------------------------------------------------------------ rows (rows.hip)
nc_status fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t st);
nc_status fill_f32(float* p, float v, size_t n, hipStream_t st);
// y = x / sqrt(mean(x^2)+eps) per row, r = the scale; with idx, row m reads x[idx[m]].
template <typename T>
nc_status rmsnorm_fwd(const T* x, const int32_t* idx, int V, T* y, float* r, int M, int d, float eps,
                      uint32_t* status, hipStream_t st);
// dx = (res) + r (dy - y mean(dy y)); output T or float.
template <typename T, typename TO>
nc_status rmsnorm_bwd(const T* dy, const T* y, const float* r, const T* res, TO* dx, int M, int d, hipStream_t st);
// cos/sin [T, D/2] of t * base^(-2i/D), evaluated in double.
nc_status rope_table(float* cs, float* sn, int T, int D, float base, hipStream_t st);
// Per token and head (H+G heads): N_D then rotate; qkv [M, ld_in] -> qk [M, ld_out].
// Row m is at position pos0 + m % T_.
template <typename T>
nc_status qknorm_rope_fwd(const T* qkv, long ld_in, T* qk, long ld_out, const float* cs, const float* sn, int M,
                          int T_, int nheads, int D, float eps, hipStream_t st, int pos0 = 0);
// In place on g [M, ld_g] (first nheads*D columns): g <- N_D_bwd(R^T g) with
// the forward recomputed from the raw qkv.
template <typename T>
nc_status qknorm_rope_bwd(const T* qkv, long ld_in, T* g, long ld_g, const float* cs, const float* sn, int M, int T_,
                          int nheads, int D, float eps, hipStream_t st);
// Cross-entropy: lse[m] = log(sum of part[m][:]); loss = mean over valid
// targets of lse - zt; nv = count of valid targets; writes loss and status.
nc_status xent_loss(const float* part, int ntiles, const float* zt, const int32_t* targets, int M, int V, float* lse,
                    float* row_loss, float* block_sums, int* block_counts, float* loss, int* nv, uint32_t* status,
                    hipStream_t st);
size_t xent_loss_blocks(int M);
// In place: z <- (exp(z - lse) - onehot) * dloss/nv * (1 - (z/c)^2) on valid rows, 0 elsewhere.
template <typename T>
nc_status xent_dz(T* z, int M, int V, const float* lse, const int32_t* targets, const int* nv, float dloss, float cap,
                  hipStream_t st);
// out (+)= sum_z partial[z] (fixed order) for float arrays of n elements.
nc_status splitk_reduce(const float* partial, int nsplit, size_t n, float* out, int accumulate, hipStream_t st);

// ------------------------------------------------------------ inference (infer.hip)
// cache[b][pos0 + t] <- rows b * Tsrc + t of k and v (G*D columns each).
template <typename T>
nc_status kv_store(const T* k, long ldk, const T* v, long ldv, T* ck, T* cv, int B, int Tsrc, int pos0, int cap,
                   int GD, hipStream_t st);
// o [B, H*D] = attention of one query per head (q [B, ld_q], heads in order)
// over keys 0..n-1 of the cache (attn.hip; H/G <= 32); po/pl: float scratch
// of B * attn_decode_chunks(cap) * H * (D + 1) elements.
template <typename T>
nc_status attn_decode(const T* q, long ldq, const T* ck, const T* cv, int B, int H, int G, int D, int n, int cap,
                      T* o, long ldo, float* po, float* pl, hipStream_t st);
int attn_decode_chunks(int cap);
// out[b] = lowest index of the largest c tanh(z[b][v]/c).
nc_status argmax_softcap(const float* z, long ldz, int B, int V, float cap, int32_t* out, hipStream_t st);
template <typename T>
nc_status splitk_act(const float* part, int nsplit, int M, int N, void* y, bool y_f32, const T* res, bool relu_sq,
                     hipStream_t st);
nc_status iota_i32(int32_t* out, int n, int start, int step, hipStream_t st);

// ------------------------------------------------------------ attention (attn.hip)
struct AttnArgs {
  int B, T, H, G, D;
  long ld_qk;  // row stride of qk (q heads then k heads)
  long ld_v;   // row stride of the v source
  long ld_o;   // row stride of o and dO
  long ld_dq;  // row stride of dq
};
template <typename T>
nc_status attn_fwd(const AttnArgs& a, const T* qk, const T* v, T* o, float* lse, hipStream_t st);
template <typename T>
// rowstat: scratch of 2 * B * T * H floats, the per-row (lse log2 e, Delta)
// pairs the dQ pass hands to the dK/dV pass.
nc_status attn_bwd(const AttnArgs& a, const T* qk, const T* v, const T* o, const T* dO, const float* lse,
                   float* rowstat, T* dq, T* dk, T* dv, long ld_dkv, hipStream_t st);

// ------------------------------------------------------------ embedding grad (embed_bwd.hip)
struct EmbedSortBufs {
  int* hist;      // [n_chunks * V]
  int* seg;       // [V + 1] segment starts (exclusive scan of counts)
  int* perm;      // [M] token positions sorted by (id, position)
  int* sid;       // [M] ids in sorted order
  float* spill;   // [n_windows * 2 * d]
};
size_t embed_sort_bytes(int M, int V, int d);
EmbedSortBufs embed_sort_carve(void* base, int M, int V, int d);
// dwte[v] (+)= sum over m with idx[m] = v of de[m]; de float [M,d].
nc_status embed_scatter(const int32_t* idx, const float* de, float* dwte, int M, int V, int d, int accumulate,
                        const EmbedSortBufs& b, hipStream_t st);

}  // namespace nc
