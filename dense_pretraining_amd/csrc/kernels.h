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
// y[M,N] = alpha * x[M,K] w[N,K]^T + beta * res (res optional, [M,N], the
// layout of y). batch independent products: problem b at x + b x_batch,
// w + b w_batch and y, res + b y_batch.
template <typename T>
nc_status gemm_xwt_axpby(const T* x, const T* w, T* y, const T* res, int M, int N, int K, float alpha, float beta,
                         hipStream_t st, int batch = 1, long x_batch = 0, long w_batch = 0, long y_batch = 0);
// a[C,C] = x^T x for x [R,C] (the Gram matrix, in the storage type); batched as above.
template <typename T>
nc_status gemm_gram(const T* x, T* a, int R, int C, hipStream_t st, int batch = 1, long x_batch = 0, long a_batch = 0);
template <typename T>
nc_status gemm_dyw(const T* dy, const T* w, T* dx, const T* act, int M, int N, int K, hipStream_t st,
                   long dy_panel = 0);
// dx[M,K] = diag(q) dy[M,N] W[N,K]: the unembedding's input gradient, q one factor per row.
template <typename T>
nc_status gemm_dyw_scaled(const T* dy, const T* w, T* dx, const float* q, int M, int N, int K, hipStream_t st,
                          long dy_panel = 0);
// dW[N,K] (+)= dy[M,N]^T x[M,K] (float32), split over M when that helps fill
// the GPU (partials in `partial`, summed in a fixed order).
template <typename T>
nc_status gemm_dw(const T* dy, const T* x, float* dw, int M, int N, int K, int accumulate, float* partial,
                  size_t partial_elems, hipStream_t st, long dy_panel = 0);
size_t gemm_dw_partial_elems(int M, int N, int K);
// Unembedding with the softcap epilogue: z = c tanh((x W^T)/c) stored [M,N] in column panels;
// part[M, lmhead_tiles(N)] = per-tile sums of exp(z). With grad: u = exp(z - c) (1 - (z/c)^2) / 4
// is stored instead and the sums are of exp(z - c).
template <typename T>
nc_status gemm_lmhead(const T* x, const T* w, T* z, int M, int N, int K, float cap, float* part, hipStream_t st,
                      bool grad = false);
int lmhead_tiles(int N, bool bf16_storage);

// ------------------------------------------------------------ few-row products (skinny.hip)
// y = epi(diag(s) x[M,K] W[N,K]^T) (+ res), s[m] = 1/rms(x[m]) when norm, else 1.
// epi: kSkinnyStore, kSkinnyReluSq, or kSkinnyArgmax (cand[m][t] = the largest
// c tanh(.. / c) of row m over column tile t and its column; y unused).
// K % 64 == 0, N % 8 == 0. part: float scratch of skinny_part_elems(M, N, K)
// for the partial sums of a K split (none needed when that is 0).
// kSkinnyPartial: only the float32 partial sums (and sums of squares) are
// written to part, even unsplit, for a caller-supplied finishing kernel.
enum { kSkinnyStore = 0, kSkinnyReluSq = 1, kSkinnyArgmax = 2, kSkinnyPartial = 3 };
struct SkinnyPlan {
  int mt, nmt, ntn, nsplit, kper;
};
SkinnyPlan skinny_plan(int M, int N, int K);
size_t skinny_part_elems(int M, int N, int K);  // at least M * (N + 1) for kSkinnyPartial
int skinny_col_tiles(int N);
template <typename T>
nc_status gemm_skinny(const T* x, long ldx, const T* w, int M, int N, int K, bool norm, float eps, int epi, T* y,
                      long ldy, const T* res, long ldres, float cap, float2* cand, float* part, size_t part_elems,
                      hipStream_t st);
// out[m] = the column of the largest of cand[m][0 .. ntn) (ties: lowest column).
nc_status argmax_cand(const float2* cand, int M, int ntn, int32_t* out, hipStream_t st);

// ------------------------------------------------------------ rows (rows.hip)
nc_status fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t st);
nc_status fill_f32(float* p, float v, size_t n, hipStream_t st);
// y = x / sqrt(mean(x^2)+eps) per row, r = the scale; with idx, row m reads x[idx[m]].
// With amax (not with idx): the stored |y| into the striped maximum at amax
// (kAmaxWords words, cleared by the caller).
template <typename T>
nc_status rmsnorm_fwd(const T* x, const int32_t* idx, int V, T* y, float* r, int M, int d, float eps,
                      uint32_t* status, hipStream_t st, uint32_t* amax = nullptr);
// dx = (res) + r (dy - y mean(dy y)); output T or float.
template <typename T, typename TO>
nc_status rmsnorm_bwd(const T* dy, const T* y, const float* r, const T* res, TO* dx, int M, int d, hipStream_t st);
// cos/sin [T, D/2] of t * base^(-2i/D), evaluated in double.
// Rows t0 .. t0+T-1 of the rotation table, written to rows 0 .. T-1.
nc_status rope_table(float* cs, float* sn, int T, int D, float base, hipStream_t st, int t0 = 0);
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
// Cross-entropy: lse[m] = shift + log(sum of part[m][:]) (the sums taken of
// exp(z - shift)); loss = mean over valid targets of lse - z_t, with the
// target's logit z_t = c tanh(x[m] . w[t] / c) recomputed from the
// unembedding's input x [M, d] and weight w [V, d] (also written to zt[m]
// when zt is given); nv = count of valid targets; writes loss and status.
template <typename T>
nc_status xent_loss(const float* part, int ntiles, const T* x, const T* w, int d, float cap, const int32_t* targets,
                    int M, int V, float* lse, float* block_sums, int* block_counts, float* loss, int* nv,
                    uint32_t* status, hipStream_t st, float shift = 0.f, float* zt = nullptr);
size_t xent_loss_blocks(int M);
// The backward's pass over the rows (not the logits) when the head stored
// u = exp(z - c) (1 - (z/c)^2) / 4: u[m][t] -= S (1 - (zt/c)^2) / 4 at each
// row's target, S = exp(lse - c); q[m] = 4 dloss / nv / S on rows with a
// target, 0 elsewhere; xs = diag(q) xf. Then dz = diag(q) u.
template <typename T>
nc_status xent_grad_prep(T* u, int M, int V, const float* lse, const float* zt, const int32_t* targets, const int* nv,
                         float dloss, float cap, const T* xf, int d, T* xs, float* q, hipStream_t st);
// out (+)= sum_z partial[z] (fixed order) for float arrays of n elements.
nc_status splitk_reduce(const float* partial, int nsplit, size_t n, float* out, int accumulate, hipStream_t st);

// ------------------------------------------------------------ inference (infer.hip)
// One decode step (nc_decode_step's kernels) on a caller buffer holding only
// the step's own scratch (api.hip); *need receives the bytes it takes, and
// nothing is launched when buf_bytes is smaller (NC_ERR_WORKSPACE).
nc_status decode_step_on(const nc_config* cfg, const void* params, const int32_t* tok, int pos, void* cache,
                         int32_t* next_tok, uint32_t* status, void* buf, size_t buf_bytes, size_t* need,
                         hipStream_t st);
// cache[b][pos0 + t] <- rows b * Tsrc + t of k and v (G*D columns each).
template <typename T>
nc_status kv_store(const T* k, long ldk, const T* v, long ldv, T* ck, T* cv, int B, int Tsrc, int pos0, int cap,
                   int GD, hipStream_t st);
// Decode step's attention inputs from the split-K partials of x W_qkv^T
// (gemm_skinny with kSkinnyPartial, nsplit splits): sum, input RMSNorm scale,
// QK norm and rotation (cs/sn: the table row of position pos); q heads to
// q [B, ldq], the new key and value to position pos of the cache.
template <typename T>
nc_status qkv_finish(const float* part, int nsplit, int B, int d, int H, int G, int D, float eps, const float* cs,
                     const float* sn, T* q, long ldq, T* ck, T* cv, int pos, int cap, hipStream_t st);
// o [B, H*D] = attention of one query per head (q [B, ld_q], heads in order)
// over keys 0..n-1 of the cache (attn.hip; H/G <= 32); po/pl: float scratch
// of B * attn_decode_chunks(cap) * H * (D + 1) elements.
template <typename T>
nc_status attn_decode(const T* q, long ldq, const T* ck, const T* cv, int B, int H, int G, int D, int n, int cap,
                      T* o, long ldo, float* po, float* pl, hipStream_t st);
int attn_decode_chunks(int cap);

// ------------------------------------------------------------ attention (attn.hip)
struct AttnArgs {
  int B, T, H, G, D;
  long ld_qk;  // row stride of qk (q heads then k heads)
  long ld_v;   // row stride of the v source
  long ld_o;   // row stride of o and dO
  long ld_dq;  // row stride of dq
};
// o = causal softmax(q k^T / sqrt(D)) v per query head, lse per (row, head).
// With amax: the stored |o| into the striped maximum at amax.
template <typename T>
nc_status attn_fwd(const AttnArgs& a, const T* qk, const T* v, T* o, float* lse, hipStream_t st,
                   uint32_t* amax = nullptr);
template <typename T>
// rowstat: scratch of 2 * B * T * H floats, the per-row (lse log2 e, -Delta)
// pairs the dQ pass hands to the dK/dV pass.
nc_status attn_bwd(const AttnArgs& a, const T* qk, const T* v, const T* o, const T* dO, const float* lse,
                   float* rowstat, T* dq, T* dk, T* dv, long ld_dkv, hipStream_t st);

// ------------------------------------------------------------ FP8 forward products (fp8.hip, gemm.hip)
// Up to kFp8TabMax tensors handled by one launch: x[k] holds 8 * n8[k]
// elements, q[k] receives their E4M3 codes.
constexpr int kFp8TabMax = 4;
template <typename T>
struct Fp8Tab {
  const T* x[kFp8TabMax];
  long n8[kFp8TabMax];
  uint8_t* q[kFp8TabMax];
};
// Tensor k's maximum |x[k]| into amax + k * kAmaxWords (striped float bits,
// see common.h; the caller clears the words).
template <typename T>
nc_status fp8_amax(const Fp8Tab<T>& t, int count, uint32_t* amax, hipStream_t st);
// q[k] = E4M3(clip(x[k] * 448 / a, +-448)), scale[k] = a / 448 with a the maximum
// held at amax + k * kAmaxWords
// (1 and 1 when a = 0): one read of x, one write of the codes.
template <typename T>
nc_status fp8_quantize(const Fp8Tab<T>& t, int count, const uint32_t* amax, float* scale, hipStream_t st);

// Per-tensor words of one block's FP8 products, in this order.
enum Fp8Slot { kF8H1, kF8O, kF8H2, kF8Act, kF8Wqkv, kF8Wo, kF8W1, kF8W2, kF8Slots };
// Scratch of the FP8 forward products: the current activation operand's codes
// (xq: M * largest K bytes), the block's four weight matrices' codes packed
// in slot order (wq), kF8Slots scales, and kF8Slots striped maxima of
// kAmaxWords words each.
struct Fp8Buf {
  uint8_t *xq, *wq;
  float* scale;
  uint32_t* amax;
};
// y[M,N] = act((xq wq^T) * sx * sw) (+ res) from E4M3 codes (xq [M,K], wq [N,K]),
// bf16 storage; K % 16 == 0. With amax_out: the stored |y| into the striped
// maximum at amax_out.
nc_status gemm_fp8(const uint8_t* xq, const uint8_t* wq, const float* sx, const float* sw, bf16* y, const bf16* res,
                   int M, int N, int K, bool relu_sq_out, uint32_t* amax_out, hipStream_t st);

// ------------------------------------------------------------ optimizer (opt.hip)
// master = widen(params), s1 = 0 (n elements), s2 = 0 (n2 elements).
template <typename T>
nc_status opt_init(const T* params, float* master, float* s1, size_t n, float* s2, size_t n2, hipStream_t st);
// AdamW over n elements (n % 4 == 0): m, v, w updated in place, p = w in the storage type.
template <typename T>
nc_status adamw_step(const float* g, float* w, float* m, float* v, T* p, size_t n, float lr, float beta1,
                     float beta2, float eps, float wd, int step, hipStream_t st);
// One kind of block matrix for a Muon step: L matrices w [R, C] (float32
// master, p its stored copy) with gradients g and momenta mom, matrix l at
// + l * ls elements of each.
template <typename T>
struct MuonKind {
  const float* g;
  float* mom;
  float* w;
  T* p;
  int R, C;
};
// One Muon step of nk kinds whose tall forms (rows >= columns) have the same
// shape: their Newton-Schulz products run as one batch of nk * L matrices;
// work: muon_work_bytes(R, C, nk * L, bf16) bytes.
template <typename T>
nc_status muon_step(const MuonKind<T>* kinds, int nk, int L, long ls, float lr, float mu, int nesterov, float wd,
                    void* work, size_t work_bytes, hipStream_t st);
size_t muon_work_bytes(int R, int C, int L, bool bf16_storage);

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
// dwte[v] (+)= sum over m with idx[m] = v of de[m], de = N_bwd(dx0) the
// backward of x0 = N(Wte[idx]) (x0 and r0 as the forward stored them), formed
// on the fly. d <= 256 * 16 / sizeof(T).
template <typename T>
nc_status embed_bwd(const int32_t* idx, const T* x0, const float* r0, const T* dx0, float* dwte, int M, int V, int d,
                    int accumulate, const EmbedSortBufs& b, hipStream_t st);

}  // namespace nc
