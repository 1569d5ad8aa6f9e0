// C ABI of the library: argument checks, buffer carving and the order of
// kernel launches for each entry point. Every launch goes to the caller's
// stream; nothing here allocates device memory or synchronises (except
// nc_read_status).
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace nc {

static thread_local std::string g_last_error;

nc_status record_hip_error(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return NC_ERR_HIP;
}

namespace {

constexpr size_t kStatusBytes = 256;

struct Dims {
  long M;
  int B, T, d, H, G, D, F, V, L, QKV, HD, QK;
  float eps, cap, base;
  int dtype;
  size_t es;  // bytes per stored element
  bool fp8;   // forward block products in FP8 E4M3 (bf16 storage)
};

nc_status make_dims(const nc_config* c, Dims* o, bool need_depth) {
  if (!c) return NC_ERR_INVALID_ARG;
  if (c->dtype != NC_BF16 && c->dtype != NC_F32 && c->dtype != NC_BF16_FP8) return NC_ERR_UNSUPPORTED;
  if (c->d_model <= 0 || c->n_head <= 0 || c->head_dim <= 0 || c->n_kv_head <= 0 || c->d_ff <= 0 || c->vocab <= 0 ||
      c->batch <= 0 || c->seq_len <= 0 || (need_depth && c->depth <= 0) || c->depth < 0)
    return NC_ERR_SHAPE;
  if (c->n_head % c->n_kv_head != 0) return NC_ERR_SHAPE;
  if (!(c->softcap > 0.f) || !(c->rope_base > 0.f) || !(c->norm_eps >= 0.f)) return NC_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return NC_ERR_UNSUPPORTED;
  if (c->d_model % 64 != 0 || c->d_model > 2048 || c->d_ff % 64 != 0 || c->vocab % 8 != 0) return NC_ERR_UNSUPPORTED;
  long M = (long)c->batch * c->seq_len;
  if (M > 0x7fffffffL || c->batch > 65535 || c->n_kv_head > 65535) return NC_ERR_UNSUPPORTED;
  long qkv = (long)(c->n_head + 2 * c->n_kv_head) * c->head_dim;
  if (qkv * c->d_model > 0x7fffffffL || (long)c->d_ff * c->d_model > 0x7fffffffL ||
      (long)c->vocab * c->d_model > 0x7fffffffL || M * c->d_ff > 0x7fffffffL || M * qkv > 0x7fffffffL)
    return NC_ERR_UNSUPPORTED;
  // a weight-gradient tile of the unembedding spans 8 logit panels of M * kPanel
  // elements, addressed with 32-bit byte offsets; the unembedding epilogue
  // multiplies the panel stride in 24 bits
  if (M * kPanel * 8 * 2 > 0x7fffffffL || M * kPanel >= (1L << 24)) return NC_ERR_UNSUPPORTED;
  o->M = M;
  o->B = c->batch;
  o->T = c->seq_len;
  o->d = c->d_model;
  o->H = c->n_head;
  o->G = c->n_kv_head;
  o->D = c->head_dim;
  o->F = c->d_ff;
  o->V = c->vocab;
  o->L = c->depth;
  o->QKV = (int)qkv;
  o->HD = c->n_head * c->head_dim;
  o->QK = (c->n_head + c->n_kv_head) * c->head_dim;
  o->eps = c->norm_eps;
  o->cap = c->softcap;
  o->base = c->rope_base;
  o->dtype = c->dtype;
  o->es = c->dtype == NC_F32 ? 4 : 2;
  o->fp8 = c->dtype == NC_BF16_FP8;
  return NC_OK;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Sequential carving of a caller buffer into 256-byte aligned pieces.
struct Carver {
  char* p;
  size_t used = 0;
  explicit Carver(void* base) : p(static_cast<char*>(base)) {}
  template <typename U>
  U* take(size_t n) {
    U* r = reinterpret_cast<U*>(p ? p + used : nullptr);
    used += align_up(n * sizeof(U), 256);
    return r;
  }
};

template <typename T>
struct BlockSaved {
  float *r1, *lse, *r2, *cs, *sn;
  T *h1, *qkv, *qk, *o, *x1, *h2, *act;  // act = max(h2 W1^T, 0)^2
};
template <typename T>
BlockSaved<T> carve_block_saved(Carver& c, const Dims& m, bool table) {
  BlockSaved<T> s;
  s.r1 = c.take<float>(m.M);
  s.h1 = c.take<T>(m.M * m.d);
  s.qkv = c.take<T>(m.M * m.QKV);
  s.qk = c.take<T>(m.M * m.QK);
  s.o = c.take<T>(m.M * m.HD);
  s.lse = c.take<float>(m.M * m.H);
  s.x1 = c.take<T>(m.M * m.d);
  s.r2 = c.take<float>(m.M);
  s.h2 = c.take<T>(m.M * m.d);
  s.act = c.take<T>(m.M * m.F);
  s.cs = table ? c.take<float>((size_t)m.T * m.D / 2) : nullptr;
  s.sn = table ? c.take<float>((size_t)m.T * m.D / 2) : nullptr;
  return s;
}

template <typename T>
struct BlockScratch {
  T *du, *dh, *dx1, *dy, *dqkv;
  float *rowstat, *partial;
  size_t partial_elems;
};
size_t block_partial_elems(const Dims& m) {
  size_t a = gemm_dw_partial_elems((int)m.M, m.d, m.F);
  size_t b = gemm_dw_partial_elems((int)m.M, m.F, m.d);
  size_t c = gemm_dw_partial_elems((int)m.M, m.d, m.HD);
  size_t e = gemm_dw_partial_elems((int)m.M, m.QKV, m.d);
  size_t r = a;
  if (b > r) r = b;
  if (c > r) r = c;
  if (e > r) r = e;
  return r;
}
template <typename T>
BlockScratch<T> carve_block_scratch(Carver& c, const Dims& m) {
  BlockScratch<T> s;
  s.du = c.take<T>(m.M * m.F);
  s.dh = c.take<T>(m.M * m.d);
  s.dx1 = c.take<T>(m.M * m.d);
  s.dy = c.take<T>(m.M * m.HD);
  s.dqkv = c.take<T>(m.M * m.QKV);
  s.rowstat = c.take<float>(2 * m.M * m.H);
  s.partial_elems = block_partial_elems(m);
  s.partial = c.take<float>(s.partial_elems ? s.partial_elems : 1);
  return s;
}

template <typename T>
struct HeadSaved {
  T *xf, *z;  // z: what the softcap epilogue stores per logit (see head_fwd_t)
  float *rf, *lse, *zt;
  int* nv;
};
template <typename T>
HeadSaved<T> carve_head_saved(Carver& c, const Dims& m) {
  HeadSaved<T> s;
  s.xf = c.take<T>(m.M * m.d);
  s.rf = c.take<float>(m.M);
  s.z = c.take<T>(logit_elems(m.M, m.V));  // column panels of kPanel
  s.lse = c.take<float>(m.M);
  s.zt = c.take<float>(m.M);
  s.nv = c.take<int>(1);
  return s;
}

template <typename T>
struct HeadScratch {
  float *part, *block_sums, *partial, *q;
  int* block_counts;
  T *dxf, *xs;
  size_t partial_elems;
};
template <typename T>
HeadScratch<T> carve_head_scratch(Carver& c, const Dims& m) {
  HeadScratch<T> s;
  s.part = c.take<float>(m.M * lmhead_tiles(m.V, m.es == 2));
  s.block_sums = c.take<float>(xent_loss_blocks((int)m.M));
  s.block_counts = c.take<int>(xent_loss_blocks((int)m.M));
  s.q = c.take<float>(m.M);
  s.dxf = c.take<T>(m.M * m.d);
  s.xs = c.take<T>(m.M * m.d);
  s.partial_elems = gemm_dw_partial_elems((int)m.M, m.V, m.d);
  s.partial = c.take<float>(s.partial_elems ? s.partial_elems : 1);
  return s;
}

struct EmbedScratch {
  void* sort;
};
EmbedScratch carve_embed_scratch(Carver& c, const Dims& m) {
  EmbedScratch s;
  s.sort = c.take<char>(embed_sort_bytes((int)m.M, m.V, m.d));
  return s;
}

// Elements of a block's four weight matrices, in FP8 slot order.
void fp8_weight_sizes(const Dims& m, size_t* n) {
  n[0] = (size_t)m.QKV * m.d;
  n[1] = (size_t)m.d * m.HD;
  n[2] = (size_t)m.F * m.d;
  n[3] = (size_t)m.d * m.F;
}

// The codes of the largest activation operand (act [M, F] at most), the
// block's four weight matrices' codes, and the per-tensor scales and maxima.
Fp8Buf carve_fp8(Carver& c, const Dims& m) {
  Fp8Buf b;
  long kmax = m.d > m.HD ? m.d : m.HD;
  kmax = kmax > m.F ? kmax : m.F;
  size_t n[4];
  fp8_weight_sizes(m, n);
  b.xq = c.take<uint8_t>((size_t)m.M * kmax);
  b.wq = c.take<uint8_t>(n[0] + n[1] + n[2] + n[3]);
  b.scale = c.take<float>(kF8Slots);
  b.amax = c.take<uint32_t>((size_t)kF8Slots * kAmaxWords);
  return b;
}

size_t block_saved_bytes(const Dims& m, bool table) {
  Carver c(nullptr);
  if (m.es == 2) carve_block_saved<bf16>(c, m, table);
  else carve_block_saved<float>(c, m, table);
  return c.used;
}
size_t head_saved_bytes(const Dims& m) {
  Carver c(nullptr);
  if (m.es == 2) carve_head_saved<bf16>(c, m);
  else carve_head_saved<float>(c, m);
  return c.used;
}
// Scratch after the status word: the largest of the entry points' needs.
size_t scratch_body_bytes(const Dims& m) {
  Carver a(nullptr), b(nullptr), e(nullptr);
  if (m.es == 2) {
    carve_block_scratch<bf16>(a, m);
    carve_head_scratch<bf16>(b, m);
  } else {
    carve_block_scratch<float>(a, m);
    carve_head_scratch<float>(b, m);
  }
  carve_embed_scratch(e, m);
  size_t r = a.used;
  if (b.used > r) r = b.used;
  if (e.used > r) r = e.used;
  if (m.fp8) {
    Carver f(nullptr);
    carve_fp8(f, m);
    if (f.used > r) r = f.used;
  }
  return r;
}

size_t param_offsets(const Dims& m, size_t* off) {
  size_t o = 0;
  off[0] = o;
  o += (size_t)m.V * m.d;
  for (int l = 0; l < m.L; ++l) {
    off[1 + 4 * l] = o;
    o += (size_t)m.QKV * m.d;
    off[2 + 4 * l] = o;
    o += (size_t)m.d * m.HD;
    off[3 + 4 * l] = o;
    o += (size_t)m.F * m.d;
    off[4 + 4 * l] = o;
    o += (size_t)m.d * m.F;
  }
  off[1 + 4 * m.L] = o;
  o += (size_t)m.V * m.d;
  return o;
}

size_t model_workspace_bytes(const Dims& m) {
  size_t b = kStatusBytes;
  b += 2 * align_up((size_t)m.T * m.D / 2 * sizeof(float), 256);
  b += (size_t)(m.L + 1) * align_up((size_t)m.M * m.d * m.es, 256);
  b += align_up((size_t)m.M * sizeof(float), 256);
  b += (size_t)m.L * block_saved_bytes(m, false);
  b += head_saved_bytes(m);
  b += align_up((size_t)m.M * m.d * m.es, 256);
  b += scratch_body_bytes(m);
  return b;
}

// ------------------------------------------------------------ typed steps

template <typename T>
struct BlockW {
  const T *wqkv, *wo, *w1, *w2;
};

// The block forward with the four projections as FP8 products (bf16 storage).
// Each activation's maximum comes from the kernel that writes it; the
// weights are quantised first, all four in one pass.
nc_status block_fwd_fp8(const Dims& m, const BlockW<bf16>& w, const bf16* x, bf16* x_out, const BlockSaved<bf16>& s,
                        const float* cs, const float* sn, const Fp8Buf& f, hipStream_t st) {
  const int M = (int)m.M;
  if (m.d % 16 || m.HD % 16 || m.F % 16) return NC_ERR_UNSUPPORTED;
  size_t n[4];
  fp8_weight_sizes(m, n);
  Fp8Tab<bf16> wt{{w.wqkv, w.wo, w.w1, w.w2},
                  {(long)n[0] / 8, (long)n[1] / 8, (long)n[2] / 8, (long)n[3] / 8},
                  {f.wq, f.wq + n[0], f.wq + n[0] + n[1], f.wq + n[0] + n[1] + n[2]}};
  auto amax = [&](int slot) { return f.amax + (size_t)slot * kAmaxWords; };
  NC_TRY(fill_u32(f.amax, 0u, (size_t)kF8Slots * kAmaxWords, st));
  NC_TRY(fp8_amax(wt, 4, amax(kF8Wqkv), st));
  NC_TRY(fp8_quantize(wt, 4, amax(kF8Wqkv), f.scale + kF8Wqkv, st));
  // one activation operand: its codes into xq (its maximum is already in amax(slot))
  auto quant = [&](const bf16* a, long elems, int slot) -> nc_status {
    Fp8Tab<bf16> t{{a}, {elems / 8}, {f.xq}};
    return fp8_quantize(t, 1, amax(slot), f.scale + slot, st);
  };
  const float* sc = f.scale;
  NC_TRY(rmsnorm_fwd<bf16>(x, nullptr, 0, s.h1, s.r1, M, m.d, m.eps, nullptr, st, amax(kF8H1)));
  NC_TRY(quant(s.h1, m.M * m.d, kF8H1));
  NC_TRY(gemm_fp8(f.xq, wt.q[0], sc + kF8H1, sc + kF8Wqkv, s.qkv, nullptr, M, m.QKV, m.d, false, nullptr, st));
  NC_TRY(qknorm_rope_fwd<bf16>(s.qkv, m.QKV, s.qk, m.QK, cs, sn, M, m.T, m.H + m.G, m.D, m.eps, st));
  AttnArgs a{m.B, m.T, m.H, m.G, m.D, m.QK, m.QKV, m.HD, m.QKV};
  NC_TRY(attn_fwd<bf16>(a, s.qk, s.qkv + (size_t)(m.H + m.G) * m.D, s.o, s.lse, st, amax(kF8O)));
  NC_TRY(quant(s.o, m.M * m.HD, kF8O));
  NC_TRY(gemm_fp8(f.xq, wt.q[1], sc + kF8O, sc + kF8Wo, s.x1, x, M, m.d, m.HD, false, nullptr, st));
  NC_TRY(rmsnorm_fwd<bf16>(s.x1, nullptr, 0, s.h2, s.r2, M, m.d, m.eps, nullptr, st, amax(kF8H2)));
  NC_TRY(quant(s.h2, m.M * m.d, kF8H2));
  NC_TRY(gemm_fp8(f.xq, wt.q[2], sc + kF8H2, sc + kF8W1, s.act, nullptr, M, m.F, m.d, true, amax(kF8Act), st));
  NC_TRY(quant(s.act, m.M * m.F, kF8Act));
  NC_TRY(gemm_fp8(f.xq, wt.q[3], sc + kF8Act, sc + kF8W2, x_out, s.x1, M, m.d, m.F, false, nullptr, st));
  return NC_OK;
}

template <typename T>
nc_status block_fwd_t(const Dims& m, const BlockW<T>& w, const T* x, T* x_out, const BlockSaved<T>& s,
                      const float* cs, const float* sn, hipStream_t st, const Fp8Buf* f8 = nullptr) {
  if constexpr (sizeof(T) == 2) {
    if (m.fp8) return f8 ? block_fwd_fp8(m, w, x, x_out, s, cs, sn, *f8, st) : NC_ERR_INVALID_ARG;
  }
  const int M = (int)m.M;
  NC_TRY(rmsnorm_fwd<T>(x, nullptr, 0, s.h1, s.r1, M, m.d, m.eps, nullptr, st));
  NC_TRY(gemm_xwt<T>(s.h1, w.wqkv, s.qkv, nullptr, M, m.QKV, m.d, false, st));
  NC_TRY(qknorm_rope_fwd<T>(s.qkv, m.QKV, s.qk, m.QK, cs, sn, M, m.T, m.H + m.G, m.D, m.eps, st));
  AttnArgs a{m.B, m.T, m.H, m.G, m.D, m.QK, m.QKV, m.HD, m.QKV};
  NC_TRY(attn_fwd<T>(a, s.qk, s.qkv + (size_t)(m.H + m.G) * m.D, s.o, s.lse, st));
  NC_TRY(gemm_xwt<T>(s.o, w.wo, s.x1, x, M, m.d, m.HD, false, st));
  NC_TRY(rmsnorm_fwd<T>(s.x1, nullptr, 0, s.h2, s.r2, M, m.d, m.eps, nullptr, st));
  NC_TRY(gemm_xwt<T>(s.h2, w.w1, s.act, nullptr, M, m.F, m.d, true, st));
  NC_TRY(gemm_xwt<T>(s.act, w.w2, x_out, s.x1, M, m.d, m.F, false, st));
  return NC_OK;
}

template <typename T>
nc_status block_bwd_t(const Dims& m, const BlockW<T>& w, const T* x, const BlockSaved<T>& s, const float* cs,
                      const float* sn, const T* dx_out, T* dx_in, const nc_block_grads& g, int acc,
                      const BlockScratch<T>& c, hipStream_t st) {
  (void)x;
  const int M = (int)m.M;
  // MLP: x_out = x1 + act W2^T, act = max(h2 W1^T, 0)^2
  NC_TRY(gemm_dw<T>(dx_out, s.act, g.w2, M, m.d, m.F, acc, c.partial, c.partial_elems, st));
  NC_TRY(gemm_dyw<T>(dx_out, w.w2, c.du, s.act, M, m.d, m.F, st));
  NC_TRY(gemm_dw<T>(c.du, s.h2, g.w1, M, m.F, m.d, acc, c.partial, c.partial_elems, st));
  NC_TRY(gemm_dyw<T>(c.du, w.w1, c.dh, nullptr, M, m.F, m.d, st));
  NC_TRY(rmsnorm_bwd<T, T>(c.dh, s.h2, s.r2, dx_out, c.dx1, M, m.d, st));
  // attention output projection: x1 = x + o Wo^T
  NC_TRY(gemm_dw<T>(c.dx1, s.o, g.wo, M, m.d, m.HD, acc, c.partial, c.partial_elems, st));
  NC_TRY(gemm_dyw<T>(c.dx1, w.wo, c.dy, nullptr, M, m.d, m.HD, st));
  // attention, then rotation + QK norm
  AttnArgs a{m.B, m.T, m.H, m.G, m.D, m.QK, m.QKV, m.HD, m.QKV};
  NC_TRY(attn_bwd<T>(a, s.qk, s.qkv + (size_t)(m.H + m.G) * m.D, s.o, c.dy, s.lse, c.rowstat, c.dqkv,
                     c.dqkv + (size_t)m.H * m.D, c.dqkv + (size_t)(m.H + m.G) * m.D, m.QKV, st));
  NC_TRY(qknorm_rope_bwd<T>(s.qkv, m.QKV, c.dqkv, m.QKV, cs, sn, M, m.T, m.H + m.G, m.D, m.eps, st));
  // QKV projection and the pre-attention norm
  NC_TRY(gemm_dw<T>(c.dqkv, s.h1, g.wqkv, M, m.QKV, m.d, acc, c.partial, c.partial_elems, st));
  NC_TRY(gemm_dyw<T>(c.dqkv, w.wqkv, c.dh, nullptr, M, m.QKV, m.d, st));
  NC_TRY(rmsnorm_bwd<T, T>(c.dh, s.h1, s.r1, c.dx1, dx_in, M, m.d, st));
  return NC_OK;
}

template <typename T>
nc_status head_fwd_t(const Dims& m, const T* x, const T* wlm, const int32_t* tg, float* loss, const HeadSaved<T>& s,
                     const HeadScratch<T>& c, uint32_t* status, hipStream_t st) {
  const int M = (int)m.M;
  NC_TRY(rmsnorm_fwd<T>(x, nullptr, 0, s.xf, s.rf, M, m.d, m.eps, nullptr, st));
  // the logits are not stored: per logit, u = exp(z' - c) (1 - (z'/c)^2), and
  // per row the sums of exp(z' - c), so lse = c + log(sum)
  NC_TRY(gemm_lmhead<T>(s.xf, wlm, s.z, M, m.V, m.d, m.cap, c.part, st, true));
  NC_TRY(xent_loss<T>(c.part, lmhead_tiles(m.V, m.es == 2), s.xf, wlm, m.d, m.cap, tg, M, m.V, s.lse, c.block_sums,
                      c.block_counts, loss, s.nv, status, st, m.cap, s.zt));
  return NC_OK;
}

template <typename T>
nc_status head_bwd_t(const Dims& m, const T* wlm, const int32_t* tg, const HeadSaved<T>& s, float dloss, T* dx,
                     float* dwlm, int acc, const HeadScratch<T>& c, hipStream_t st) {
  const int M = (int)m.M;
  // dz = diag(q) u' (u' = u with each row's target element corrected): the
  // row factor q goes into the input-grad product's epilogue and, as xs =
  // diag(q) xf, into the weight-grad product's operand
  NC_TRY(xent_grad_prep<T>(s.z, M, m.V, s.lse, s.zt, tg, s.nv, dloss, m.cap, s.xf, m.d, c.xs, c.q, st));
  NC_TRY(gemm_dyw_scaled<T>(s.z, wlm, c.dxf, c.q, M, m.V, m.d, st, (long)M * kPanel));
  NC_TRY(gemm_dw<T>(s.z, c.xs, dwlm, M, m.V, m.d, acc, c.partial, c.partial_elems, st, (long)M * kPanel));
  NC_TRY(rmsnorm_bwd<T, T>(c.dxf, s.xf, s.rf, nullptr, dx, M, m.d, st));
  return NC_OK;
}

template <typename T>
nc_status embed_bwd_t(const Dims& m, const int32_t* idx, const T* x0, const float* r0, const T* dx0, float* dwte,
                      int acc, const EmbedScratch& c, hipStream_t st) {
  const int M = (int)m.M;
  return embed_bwd<T>(idx, x0, r0, dx0, dwte, M, m.V, m.d, acc, embed_sort_carve(c.sort, M, m.V, m.d), st);
}

template <typename T>
nc_status model_t(const Dims& m, const T* params, const int32_t* idx, const int32_t* tg, float* loss, float* grads,
                  float dloss, int acc, void* ws, hipStream_t st) {
  std::vector<size_t> off(2 + 4 * (size_t)m.L);
  param_offsets(m, off.data());
  uint32_t* status = static_cast<uint32_t*>(ws);
  Carver c(static_cast<char*>(ws) + kStatusBytes);
  float* cs = c.take<float>((size_t)m.T * m.D / 2);
  float* sn = c.take<float>((size_t)m.T * m.D / 2);
  std::vector<T*> xs(m.L + 1);
  for (int l = 0; l <= m.L; ++l) xs[l] = c.take<T>(m.M * m.d);
  float* r0 = c.take<float>(m.M);
  std::vector<BlockSaved<T>> sv(m.L);
  for (int l = 0; l < m.L; ++l) sv[l] = carve_block_saved<T>(c, m, false);
  HeadSaved<T> hs = carve_head_saved<T>(c, m);
  T* gx = c.take<T>(m.M * m.d);
  size_t body = c.used;
  Carver c1(static_cast<char*>(ws) + kStatusBytes + body);
  BlockScratch<T> bsc = carve_block_scratch<T>(c1, m);
  Carver c2(static_cast<char*>(ws) + kStatusBytes + body);
  HeadScratch<T> hsc = carve_head_scratch<T>(c2, m);
  Carver c3(static_cast<char*>(ws) + kStatusBytes + body);
  EmbedScratch esc = carve_embed_scratch(c3, m);
  Carver c4(static_cast<char*>(ws) + kStatusBytes + body);  // the forward only (before the head uses the area)
  const Fp8Buf f8 = carve_fp8(c4, m);

  auto bw = [&](int l) {
    BlockW<T> w;
    w.wqkv = params + off[1 + 4 * l];
    w.wo = params + off[2 + 4 * l];
    w.w1 = params + off[3 + 4 * l];
    w.w2 = params + off[4 + 4 * l];
    return w;
  };
  auto bg = [&](int l) {
    nc_block_grads g;
    g.wqkv = grads + off[1 + 4 * l];
    g.wo = grads + off[2 + 4 * l];
    g.w1 = grads + off[3 + 4 * l];
    g.w2 = grads + off[4 + 4 * l];
    return g;
  };

  NC_TRY(rope_table(cs, sn, m.T, m.D, m.base, st));
  NC_TRY(rmsnorm_fwd<T>(params + off[0], idx, m.V, xs[0], r0, (int)m.M, m.d, m.eps, status, st));
  for (int l = 0; l < m.L; ++l) NC_TRY(block_fwd_t<T>(m, bw(l), xs[l], xs[l + 1], sv[l], cs, sn, st, &f8));
  const T* wlm = params + off[1 + 4 * m.L];
  NC_TRY(head_fwd_t<T>(m, xs[m.L], wlm, tg, loss, hs, hsc, status, st));
  NC_TRY(head_bwd_t<T>(m, wlm, tg, hs, dloss, gx, grads + off[1 + 4 * m.L], acc, hsc, st));
  for (int l = m.L - 1; l >= 0; --l) NC_TRY(block_bwd_t<T>(m, bw(l), xs[l], sv[l], cs, sn, gx, gx, bg(l), acc, bsc, st));
  NC_TRY(embed_bwd_t<T>(m, idx, xs[0], r0, gx, grads + off[0], acc, esc, st));
  return NC_OK;
}

// ------------------------------------------------------------ inference
// Workspace of nc_prefill / nc_decode_step: status word, RoPE tables for the
// cache capacity, then the prefill buffers and the decode buffers (the same
// bytes: one call uses one set), then what both use (final norm, logits,
// split partials).
template <typename T>
struct InferBufs {
  float *cs, *sn;
  T *px0, *px1;  // [B*cap, d] residual streams of the prompt pass
  BlockSaved<T> ps;
  T *x, *qk, *o, *x1, *act;  // one row per sequence
  float *r, *po, *pl;
  float* part;  // split-K partials of the few-row products
  size_t part_elems;
  float2* cand;  // [B][column tiles of V] logit maxima
  size_t bytes;
};

Dims prompt_dims(const Dims& m, int n_prompt) {
  Dims p = m;
  p.T = n_prompt;
  p.M = (long)m.B * n_prompt;
  return p;
}

template <typename T>
InferBufs<T> carve_infer(void* ws, const Dims& m) {
  InferBufs<T> b;
  char* base = static_cast<char*>(ws);
  Carver c(base ? base + kStatusBytes : nullptr);
  b.cs = c.take<float>((size_t)m.T * m.D / 2);
  b.sn = c.take<float>((size_t)m.T * m.D / 2);
  const size_t head = c.used;
  char* u = base ? base + kStatusBytes + head : nullptr;
  Carver cp(u);  // prompt pass (capacity-sized)
  b.px0 = cp.take<T>(m.M * m.d);
  b.px1 = cp.take<T>(m.M * m.d);
  b.ps = carve_block_saved<T>(cp, m, false);
  Carver cd(u);  // decode step
  const long B = m.B;
  b.x = cd.take<T>(B * m.d);
  b.qk = cd.take<T>(B * m.QK);
  b.o = cd.take<T>(B * m.HD);
  b.x1 = cd.take<T>(B * m.d);
  b.act = cd.take<T>(B * m.F);
  b.r = cd.take<float>(B);
  const int nch = attn_decode_chunks(m.T);
  b.po = cd.take<float>((size_t)B * nch * m.H * m.D);
  b.pl = cd.take<float>((size_t)B * nch * m.H);
  const size_t uni = cp.used > cd.used ? cp.used : cd.used;
  Carver cs(base ? base + kStatusBytes + head + uni : nullptr);
  size_t pe = 0;
  const int shapes[5][2] = {{m.QKV, m.d}, {m.d, m.HD}, {m.F, m.d}, {m.d, m.F}, {m.V, m.d}};
  for (auto& nk : shapes) {
    const size_t e = skinny_part_elems((int)B, nk[0], nk[1]);
    pe = e > pe ? e : pe;
  }
  b.part = cs.take<float>(pe ? pe : 1);
  b.part_elems = pe;
  b.cand = cs.take<float2>((size_t)B * skinny_col_tiles(m.V));
  b.bytes = kStatusBytes + head + uni + cs.used;
  return b;
}

// The decode step's buffers alone, carved from base with nothing before them:
// the rotation row of the step's position, one row per sequence of each
// activation, the attention partials, the few-row products' split partials
// and the logit maxima (the decode part of carve_infer, without the status
// word and the prompt pass).
template <typename T>
InferBufs<T> carve_decode(void* base, const Dims& m) {
  InferBufs<T> b{};
  Carver cd(base);
  const long B = m.B;
  b.cs = cd.take<float>((size_t)m.D / 2);
  b.sn = cd.take<float>((size_t)m.D / 2);
  b.x = cd.take<T>(B * m.d);
  b.qk = cd.take<T>(B * m.QK);
  b.o = cd.take<T>(B * m.HD);
  b.x1 = cd.take<T>(B * m.d);
  b.act = cd.take<T>(B * m.F);
  b.r = cd.take<float>(B);
  const int nch = attn_decode_chunks(m.T);
  b.po = cd.take<float>((size_t)B * nch * m.H * m.D);
  b.pl = cd.take<float>((size_t)B * nch * m.H);
  // split partials: the QKV product always writes them (qkv_finish sums them),
  // the others only when their reduction is split
  size_t pe = skinny_part_elems((int)B, m.QKV, m.d);
  const int shapes[4][2] = {{m.d, m.HD}, {m.F, m.d}, {m.d, m.F}, {m.V, m.d}};
  for (auto& nk : shapes) {
    const size_t e = skinny_plan((int)B, nk[0], nk[1]).nsplit > 1 ? skinny_part_elems((int)B, nk[0], nk[1]) : 0;
    pe = e > pe ? e : pe;
  }
  b.part = cd.take<float>(pe);
  b.part_elems = pe;
  b.cand = cd.take<float2>((size_t)B * skinny_col_tiles(m.V));
  b.bytes = cd.used;
  return b;
}

nc_status infer_dims(const nc_config* cfg, Dims* m) {
  NC_TRY(make_dims(cfg, m, true));
  if (m->fp8) return NC_ERR_UNSUPPORTED;
  if (m->H / m->G > 32) return NC_ERR_UNSUPPORTED;
  return NC_OK;
}

size_t infer_cache_bytes(const Dims& m) { return (size_t)m.L * 2 * m.B * m.T * m.G * m.D * m.es; }

template <typename T>
T* cache_at(void* cache, const Dims& m, int l, int kv) {
  return static_cast<T*>(cache) + ((size_t)l * 2 + kv) * m.B * m.T * m.G * m.D;
}

// Final norm of one row per sequence (row b at x + b * ldx), softcapped
// logits, greedy choice.
template <typename T>
nc_status infer_head(const Dims& m, const T* wlm, const T* x, long ldx, const InferBufs<T>& b, int32_t* next_tok,
                     hipStream_t st) {
  NC_TRY(gemm_skinny<T>(x, ldx, wlm, m.B, m.V, m.d, true, m.eps, kSkinnyArgmax, nullptr, 0, nullptr, 0, m.cap, b.cand,
                        b.part, b.part_elems, st));
  return argmax_cand(b.cand, m.B, skinny_col_tiles(m.V), next_tok, st);
}

// x W^T for the decode step's rows, with the optional input norm, ReLU^2 and residual.
template <typename T>
nc_status decode_mm(const Dims& m, const InferBufs<T>& b, const T* x, long ldx, const T* w, int N, int K, bool norm,
                    bool relu_sq, T* y, long ldy, const T* res, hipStream_t st) {
  return gemm_skinny<T>(x, ldx, w, m.B, N, K, norm, m.eps, relu_sq ? kSkinnyReluSq : kSkinnyStore, y, ldy, res, ldy,
                        0.f, nullptr, b.part, b.part_elems, st);
}

template <typename T>
nc_status prefill_t(const Dims& m, const T* params, const int32_t* idx, int n_prompt, void* cache, int32_t* next_tok,
                    void* ws, hipStream_t st) {
  std::vector<size_t> off(2 + 4 * (size_t)m.L);
  param_offsets(m, off.data());
  uint32_t* status = static_cast<uint32_t*>(ws);
  const InferBufs<T> b = carve_infer<T>(ws, m);
  const Dims p = prompt_dims(m, n_prompt);
  NC_TRY(rope_table(b.cs, b.sn, n_prompt, m.D, m.base, st));
  NC_TRY(rmsnorm_fwd<T>(params + off[0], idx, m.V, b.px0, b.ps.r1, (int)p.M, m.d, m.eps, status, st));
  T* x = b.px0;
  T* y = b.px1;
  for (int l = 0; l < m.L; ++l) {
    BlockW<T> w{params + off[1 + 4 * l], params + off[2 + 4 * l], params + off[3 + 4 * l], params + off[4 + 4 * l]};
    NC_TRY(block_fwd_t<T>(p, w, x, y, b.ps, b.cs, b.sn, st));
    NC_TRY(kv_store<T>(b.ps.qk + (size_t)m.H * m.D, m.QK, b.ps.qkv + (size_t)(m.H + m.G) * m.D, m.QKV,
                       cache_at<T>(cache, m, l, 0), cache_at<T>(cache, m, l, 1), m.B, n_prompt, 0, m.T, m.G * m.D,
                       st));
    T* t = x;
    x = y;
    y = t;
  }
  return infer_head<T>(m, params + off[1 + 4 * m.L], x + (size_t)(n_prompt - 1) * m.d, (long)n_prompt * m.d, b,
                       next_tok, st);
}

// One decode step on the buffers b (carve_infer or carve_decode); bad token
// ids set bits of *status when status is not null.
template <typename T>
nc_status decode_t(const Dims& m, const T* params, const int32_t* tok, int pos, void* cache, int32_t* next_tok,
                   const InferBufs<T>& b, uint32_t* status, hipStream_t st) {
  std::vector<size_t> off(2 + 4 * (size_t)m.L);
  param_offsets(m, off.data());
  const int B = m.B;
  NC_TRY(rope_table(b.cs, b.sn, 1, m.D, m.base, st, pos));  // the one row of position pos
  const int qkv_split = skinny_plan(B, m.QKV, m.d).nsplit;
  NC_TRY(rmsnorm_fwd<T>(params + off[0], tok, m.V, b.x, b.r, B, m.d, m.eps, status, st));
  for (int l = 0; l < m.L; ++l) {
    const T* wqkv = params + off[1 + 4 * l];
    const T* wo = params + off[2 + 4 * l];
    const T* w1 = params + off[3 + 4 * l];
    const T* w2 = params + off[4 + 4 * l];
    T* ck = cache_at<T>(cache, m, l, 0);
    T* cv = cache_at<T>(cache, m, l, 1);
    NC_TRY(gemm_skinny<T>(b.x, m.d, wqkv, B, m.QKV, m.d, true, m.eps, kSkinnyPartial, nullptr, 0, nullptr, 0, 0.f,
                          nullptr, b.part, b.part_elems, st));
    NC_TRY(qkv_finish<T>(b.part, qkv_split, B, m.d, m.H, m.G, m.D, m.eps, b.cs, b.sn, b.qk, m.QK, ck, cv, pos, m.T,
                         st));
    NC_TRY(attn_decode<T>(b.qk, m.QK, ck, cv, B, m.H, m.G, m.D, pos + 1, m.T, b.o, m.HD, b.po, b.pl, st));
    NC_TRY(decode_mm<T>(m, b, b.o, m.HD, wo, m.d, m.HD, false, false, b.x1, m.d, b.x, st));
    NC_TRY(decode_mm<T>(m, b, b.x1, m.d, w1, m.F, m.d, true, true, b.act, m.F, nullptr, st));
    NC_TRY(decode_mm<T>(m, b, b.act, m.F, w2, m.d, m.F, false, false, b.x, m.d, b.x1, st));
  }
  return infer_head<T>(m, params + off[1 + 4 * m.L], b.x, m.d, b, next_tok, st);
}

// ---------------------------------------------------------------- optimizer
// The block matrices of layer l as (offset, rows, cols) in the parameter
// layout: Wq, Wk, Wv (row blocks of the packed projection), Wo, W1, W2.
struct MatSpec {
  size_t off;
  int R, C;
};
void layer_matrices(const Dims& m, const size_t* off, int l, MatSpec* out) {
  const size_t q = off[1 + 4 * l];
  out[0] = {q, m.H * m.D, m.d};
  out[1] = {q + (size_t)m.H * m.D * m.d, m.G * m.D, m.d};
  out[2] = {q + (size_t)(m.H + m.G) * m.D * m.d, m.G * m.D, m.d};
  out[3] = {off[2 + 4 * l], m.d, m.HD};
  out[4] = {off[3 + 4 * l], m.F, m.d};
  out[5] = {off[4 + 4 * l], m.d, m.F};
}

// The six kinds grouped by the shape of their tall form (rows >= columns):
// a group's Newton-Schulz products run as one batch. group[k] is kind k's
// group (the index of the group's first kind).
void muon_groups(const MatSpec* ms, int* group) {
  for (int k = 0; k < 6; ++k) {
    group[k] = k;
    const int rk = ms[k].R > ms[k].C ? ms[k].R : ms[k].C, ck = ms[k].R > ms[k].C ? ms[k].C : ms[k].R;
    for (int j = 0; j < k; ++j) {
      const int rj = ms[j].R > ms[j].C ? ms[j].R : ms[j].C, cj = ms[j].R > ms[j].C ? ms[j].C : ms[j].R;
      if (rj == rk && cj == ck) {
        group[k] = group[j];
        break;
      }
    }
  }
}

size_t opt_workspace_bytes(const Dims& m) {
  std::vector<size_t> off(2 + 4 * (size_t)m.L);
  param_offsets(m, off.data());
  MatSpec ms[6];
  layer_matrices(m, off.data(), 0, ms);
  int group[6];
  muon_groups(ms, group);
  size_t w = 0;
  for (int k = 0; k < 6; ++k) {
    if (group[k] != k) continue;
    int nk = 0;
    for (int j = 0; j < 6; ++j) nk += group[j] == k;
    const size_t b = muon_work_bytes(ms[k].R, ms[k].C, nk * m.L, m.es == 2);
    w = b > w ? b : w;
  }
  return w;
}

bool hparams_ok(const nc_opt_hparams* h) {
  auto fin = [](float v) { return v == v && v < 3.0e38f && v > -3.0e38f; };
  return h && fin(h->lr_matrix) && fin(h->lr_embed) && fin(h->lr_unembed) && h->lr_matrix >= 0.f &&
         h->lr_embed >= 0.f && h->lr_unembed >= 0.f && h->momentum >= 0.f && h->momentum < 1.f &&
         h->beta1 >= 0.f && h->beta1 < 1.f && h->beta2 >= 0.f && h->beta2 < 1.f && h->eps > 0.f && fin(h->eps) &&
         h->wd_matrix >= 0.f && h->wd_adam >= 0.f && fin(h->wd_matrix) && fin(h->wd_adam) && h->step >= 1 &&
         (h->nesterov == 0 || h->nesterov == 1);
}

template <typename T>
nc_status opt_step_t(const Dims& m, const nc_opt_hparams& h, T* params, const float* grads, float* state, void* ws,
                     size_t ws_bytes, hipStream_t st) {
  std::vector<size_t> off(2 + 4 * (size_t)m.L);
  const size_t n = param_offsets(m, off.data());
  float* master = state;
  float* s1 = state + n;
  float* s2 = s1 + n;
  const size_t vd = (size_t)m.V * m.d;
  const size_t lm = off[1 + 4 * m.L];
  NC_TRY(adamw_step<T>(grads, master, s1, s2, params, vd, h.lr_embed, h.beta1, h.beta2, h.eps, h.wd_adam, h.step,
                       st));
  NC_TRY(adamw_step<T>(grads + lm, master + lm, s1 + lm, s2 + vd, params + lm, vd, h.lr_unembed, h.beta1, h.beta2,
                       h.eps, h.wd_adam, h.step, st));
  // each kind of block matrix, all layers at once: layer l's copy lies l * ls elements after layer 0's
  const long ls = m.L > 1 ? (long)(off[5] - off[1]) : 0;
  MatSpec ms[6];
  layer_matrices(m, off.data(), 0, ms);
  int group[6];
  muon_groups(ms, group);
  for (int k = 0; k < 6; ++k) {
    if (group[k] != k) continue;
    MuonKind<T> kinds[6];
    int nk = 0;
    for (int j = 0; j < 6; ++j)
      if (group[j] == k)
        kinds[nk++] = MuonKind<T>{grads + ms[j].off, s1 + ms[j].off, master + ms[j].off, params + ms[j].off, ms[j].R,
                                  ms[j].C};
    NC_TRY(muon_step<T>(kinds, nk, m.L, ls, h.lr_matrix, h.momentum, h.nesterov, h.wd_matrix, ws, ws_bytes, st));
  }
  return NC_OK;
}

}  // namespace

// The decode step on one caller-supplied buffer holding only its own scratch
// (carve_decode), for the allocation-free entry point: checks the arguments
// like nc_decode_step and reports the bytes needed in *need. With buf NULL it
// stops there (a query: nothing touches the device); otherwise it launches
// only when buf holds that many bytes.
nc_status decode_step_on(const nc_config* cfg, const void* params, const int32_t* tok, int pos, void* cache,
                         int32_t* next_tok, uint32_t* status, void* buf, size_t buf_bytes, size_t* need,
                         hipStream_t st) {
  Dims m;
  NC_TRY(infer_dims(cfg, &m));
  if (!params || !tok || !cache || !next_tok || !need) return NC_ERR_INVALID_ARG;
  if (pos < 1 || pos >= m.T) return NC_ERR_SHAPE;
  if (!aligned(params) || !aligned(tok) || !aligned(cache) || !aligned(next_tok) || !aligned(buf) ||
      (status && (reinterpret_cast<uintptr_t>(status) & 3u)))
    return NC_ERR_ALIGN;
  *need = m.es == 2 ? carve_decode<bf16>(nullptr, m).bytes : carve_decode<float>(nullptr, m).bytes;
  if (!buf) return NC_OK;
  if (buf_bytes < *need) return NC_ERR_WORKSPACE;
  if (m.es == 2)
    return decode_t<bf16>(m, static_cast<const bf16*>(params), tok, pos, cache, next_tok, carve_decode<bf16>(buf, m),
                          status, st);
  return decode_t<float>(m, static_cast<const float*>(params), tok, pos, cache, next_tok, carve_decode<float>(buf, m),
                         status, st);
}

}  // namespace nc

using namespace nc;

extern "C" {

int nc_abi_version(void) { return NC_ABI_VERSION; }

const char* nc_status_str(int s) {
  switch (s) {
    case NC_OK: return "ok";
    case NC_ERR_INVALID_ARG: return "invalid argument";
    case NC_ERR_SHAPE: return "bad shape";
    case NC_ERR_ALIGN: return "misaligned buffer";
    case NC_ERR_WORKSPACE: return "workspace too small";
    case NC_ERR_UNSUPPORTED: return "unsupported configuration";
    case NC_ERR_HIP: return "HIP error";
    case NC_ERR_DEVICE_DATA: return "device data error";
    default: return "unknown status";
  }
}

const char* nc_last_hip_error(void) { return g_last_error.c_str(); }

nc_status nc_validate(const nc_config* cfg) {
  Dims m;
  return make_dims(cfg, &m, true);
}

nc_status nc_param_layout(const nc_config* cfg, size_t* offsets, size_t n_offsets, size_t* n_params) {
  Dims m;
  NC_TRY(make_dims(cfg, &m, true));
  if (!offsets || !n_params || n_offsets < (size_t)(2 + 4 * m.L)) return NC_ERR_INVALID_ARG;
  *n_params = param_offsets(m, offsets);
  return NC_OK;
}

nc_status nc_query_sizes(const nc_config* cfg, nc_sizes* s) {
  Dims m;
  NC_TRY(make_dims(cfg, &m, false));
  if (!s) return NC_ERR_INVALID_ARG;
  s->block_saved = block_saved_bytes(m, true);
  s->lmhead_saved = head_saved_bytes(m);
  s->scratch = kStatusBytes + scratch_body_bytes(m);
  if (m.L > 0) {
    std::vector<size_t> off(2 + 4 * (size_t)m.L);
    s->n_params = param_offsets(m, off.data());
    s->model_workspace = model_workspace_bytes(m);
  } else {
    s->n_params = 0;
    s->model_workspace = 0;
  }
  return NC_OK;
}

nc_status nc_workspace_size(const nc_config* cfg, size_t* model_bytes, size_t* block_saved_bytes,
                            size_t* scratch_bytes) {
  nc_sizes s;
  NC_TRY(nc_query_sizes(cfg, &s));
  if (model_bytes) *model_bytes = s.model_workspace;
  if (block_saved_bytes) *block_saved_bytes = s.block_saved;
  if (scratch_bytes) *scratch_bytes = s.scratch;
  return NC_OK;
}

nc_status nc_read_status(const void* scratch, uint32_t* flags, void* stream) {
  if (!scratch || !flags) return NC_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, scratch, sizeof(v), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return record_hip_error(e, "nc_read_status copy");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return record_hip_error(e, "nc_read_status sync");
  *flags = v;
  return v ? NC_ERR_DEVICE_DATA : NC_OK;
}

nc_status nc_clear_status(void* scratch, void* stream) {
  if (!scratch) return NC_ERR_INVALID_ARG;
  if (!aligned(scratch)) return NC_ERR_ALIGN;
  return fill_u32(static_cast<uint32_t*>(scratch), 0u, 1, static_cast<hipStream_t>(stream));
}

nc_status nc_embed_fwd(const nc_config* cfg, const int32_t* idx, const void* wte, void* x0, float* r0, void* scratch,
                       void* stream) {
  Dims m;
  NC_TRY(make_dims(cfg, &m, false));
  if (!idx || !wte || !x0 || !r0 || !scratch) return NC_ERR_INVALID_ARG;
  if (!aligned(idx) || !aligned(wte) || !aligned(x0) || !aligned(r0) || !aligned(scratch)) return NC_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t* status = static_cast<uint32_t*>(scratch);
  if (m.es == 2)
    return rmsnorm_fwd<bf16>(static_cast<const bf16*>(wte), idx, m.V, static_cast<bf16*>(x0), r0, (int)m.M, m.d, m.eps,
                             status, st);
  return rmsnorm_fwd<float>(static_cast<const float*>(wte), idx, m.V, static_cast<float*>(x0), r0, (int)m.M, m.d, m.eps,
                            status, st);
}

nc_status nc_embed_bwd(const nc_config* cfg, const int32_t* idx, const void* x0, const float* r0, const void* dx0,
                       float* dwte, int accumulate, void* scratch, void* stream) {
  Dims m;
  NC_TRY(make_dims(cfg, &m, false));
  if (!idx || !x0 || !r0 || !dx0 || !dwte || !scratch) return NC_ERR_INVALID_ARG;
  if (!aligned(idx) || !aligned(x0) || !aligned(r0) || !aligned(dx0) || !aligned(dwte) || !aligned(scratch))
    return NC_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carver c(static_cast<char*>(scratch) + kStatusBytes);
  EmbedScratch e = carve_embed_scratch(c, m);
  if (m.es == 2)
    return embed_bwd_t<bf16>(m, idx, static_cast<const bf16*>(x0), r0, static_cast<const bf16*>(dx0), dwte,
                             accumulate, e, st);
  return embed_bwd_t<float>(m, idx, static_cast<const float*>(x0), r0, static_cast<const float*>(dx0), dwte,
                            accumulate, e, st);
}

nc_status nc_block_fwd(const nc_config* cfg, const nc_block_params* w, const void* x_in, void* x_out, void* saved,
                       void* scratch, void* stream) {
  Dims m;
  NC_TRY(make_dims(cfg, &m, false));
  if (!w || !w->wqkv || !w->wo || !w->w1 || !w->w2 || !x_in || !x_out || !saved || !scratch)
    return NC_ERR_INVALID_ARG;
  if (!aligned(w->wqkv) || !aligned(w->wo) || !aligned(w->w1) || !aligned(w->w2) || !aligned(x_in) ||
      !aligned(x_out) || !aligned(saved) || !aligned(scratch))
    return NC_ERR_ALIGN;
  if (x_in == x_out) return NC_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carver c(saved);
  if (m.es == 2) {
    BlockSaved<bf16> s = carve_block_saved<bf16>(c, m, true);
    NC_TRY(rope_table(s.cs, s.sn, m.T, m.D, m.base, st));
    BlockW<bf16> bw{static_cast<const bf16*>(w->wqkv), static_cast<const bf16*>(w->wo),
                    static_cast<const bf16*>(w->w1), static_cast<const bf16*>(w->w2)};
    Carver cf(static_cast<char*>(scratch) + kStatusBytes);
    const Fp8Buf f8 = carve_fp8(cf, m);
    return block_fwd_t<bf16>(m, bw, static_cast<const bf16*>(x_in), static_cast<bf16*>(x_out), s, s.cs, s.sn, st,
                             &f8);
  }
  BlockSaved<float> s = carve_block_saved<float>(c, m, true);
  NC_TRY(rope_table(s.cs, s.sn, m.T, m.D, m.base, st));
  BlockW<float> bw{static_cast<const float*>(w->wqkv), static_cast<const float*>(w->wo),
                   static_cast<const float*>(w->w1), static_cast<const float*>(w->w2)};
  return block_fwd_t<float>(m, bw, static_cast<const float*>(x_in), static_cast<float*>(x_out), s, s.cs, s.sn, st);
}

nc_status nc_block_bwd(const nc_config* cfg, const nc_block_params* w, const void* x_in, const void* saved,
                       const void* dx_out, void* dx_in, const nc_block_grads* grads, int accumulate, void* scratch,
                       void* stream) {
  Dims m;
  NC_TRY(make_dims(cfg, &m, false));
  if (!w || !w->wqkv || !w->wo || !w->w1 || !w->w2 || !x_in || !saved || !dx_out || !dx_in || !grads ||
      !grads->wqkv || !grads->wo || !grads->w1 || !grads->w2 || !scratch)
    return NC_ERR_INVALID_ARG;
  if (!aligned(w->wqkv) || !aligned(w->wo) || !aligned(w->w1) || !aligned(w->w2) || !aligned(x_in) ||
      !aligned(saved) || !aligned(dx_out) || !aligned(dx_in) || !aligned(grads->wqkv) || !aligned(grads->wo) ||
      !aligned(grads->w1) || !aligned(grads->w2) || !aligned(scratch))
    return NC_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carver c(const_cast<void*>(saved));
  Carver cs(static_cast<char*>(scratch) + kStatusBytes);
  if (m.es == 2) {
    BlockSaved<bf16> s = carve_block_saved<bf16>(c, m, true);
    BlockScratch<bf16> sc = carve_block_scratch<bf16>(cs, m);
    BlockW<bf16> bw{static_cast<const bf16*>(w->wqkv), static_cast<const bf16*>(w->wo),
                    static_cast<const bf16*>(w->w1), static_cast<const bf16*>(w->w2)};
    return block_bwd_t<bf16>(m, bw, static_cast<const bf16*>(x_in), s, s.cs, s.sn, static_cast<const bf16*>(dx_out),
                             static_cast<bf16*>(dx_in), *grads, accumulate, sc, st);
  }
  BlockSaved<float> s = carve_block_saved<float>(c, m, true);
  BlockScratch<float> sc = carve_block_scratch<float>(cs, m);
  BlockW<float> bw{static_cast<const float*>(w->wqkv), static_cast<const float*>(w->wo),
                   static_cast<const float*>(w->w1), static_cast<const float*>(w->w2)};
  return block_bwd_t<float>(m, bw, static_cast<const float*>(x_in), s, s.cs, s.sn, static_cast<const float*>(dx_out),
                            static_cast<float*>(dx_in), *grads, accumulate, sc, st);
}

nc_status nc_lmhead_softcap_xent_fwd(const nc_config* cfg, const void* x, const void* wlm, const int32_t* targets,
                                     float* loss, void* saved, void* scratch, void* stream) {
  Dims m;
  NC_TRY(make_dims(cfg, &m, false));
  if (!x || !wlm || !targets || !loss || !saved || !scratch) return NC_ERR_INVALID_ARG;
  if (!aligned(x) || !aligned(wlm) || !aligned(targets) || !aligned(saved) || !aligned(scratch)) return NC_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t* status = static_cast<uint32_t*>(scratch);
  Carver c(saved);
  Carver cs(static_cast<char*>(scratch) + kStatusBytes);
  if (m.es == 2) {
    HeadSaved<bf16> s = carve_head_saved<bf16>(c, m);
    HeadScratch<bf16> sc = carve_head_scratch<bf16>(cs, m);
    return head_fwd_t<bf16>(m, static_cast<const bf16*>(x), static_cast<const bf16*>(wlm), targets, loss, s, sc,
                            status, st);
  }
  HeadSaved<float> s = carve_head_saved<float>(c, m);
  HeadScratch<float> sc = carve_head_scratch<float>(cs, m);
  return head_fwd_t<float>(m, static_cast<const float*>(x), static_cast<const float*>(wlm), targets, loss, s, sc,
                           status, st);
}

nc_status nc_lmhead_softcap_xent_bwd(const nc_config* cfg, const void* x, const void* wlm, const int32_t* targets,
                                     void* saved, float dloss, void* dx, float* dwlm, int accumulate, void* scratch,
                                     void* stream) {
  Dims m;
  NC_TRY(make_dims(cfg, &m, false));
  if (!x || !wlm || !targets || !saved || !dx || !dwlm || !scratch) return NC_ERR_INVALID_ARG;
  if (!aligned(x) || !aligned(wlm) || !aligned(targets) || !aligned(saved) || !aligned(dx) || !aligned(dwlm) ||
      !aligned(scratch))
    return NC_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carver c(saved);
  Carver cs(static_cast<char*>(scratch) + kStatusBytes);
  if (m.es == 2) {
    HeadSaved<bf16> s = carve_head_saved<bf16>(c, m);
    HeadScratch<bf16> sc = carve_head_scratch<bf16>(cs, m);
    return head_bwd_t<bf16>(m, static_cast<const bf16*>(wlm), targets, s, dloss, static_cast<bf16*>(dx), dwlm,
                            accumulate, sc, st);
  }
  HeadSaved<float> s = carve_head_saved<float>(c, m);
  HeadScratch<float> sc = carve_head_scratch<float>(cs, m);
  return head_bwd_t<float>(m, static_cast<const float*>(wlm), targets, s, dloss, static_cast<float*>(dx), dwlm,
                           accumulate, sc, st);
}

nc_status nc_infer_query_sizes(const nc_config* cfg, nc_infer_sizes* out) {
  Dims m;
  NC_TRY(infer_dims(cfg, &m));
  if (!out) return NC_ERR_INVALID_ARG;
  out->cache = infer_cache_bytes(m);
  out->workspace = m.es == 2 ? carve_infer<bf16>(nullptr, m).bytes : carve_infer<float>(nullptr, m).bytes;
  return NC_OK;
}

nc_status nc_prefill(const nc_config* cfg, const void* params, const int32_t* idx, int n_prompt, void* cache,
                     int32_t* next_tok, void* workspace, size_t workspace_bytes, void* stream) {
  Dims m;
  NC_TRY(infer_dims(cfg, &m));
  if (!params || !idx || !cache || !next_tok || !workspace) return NC_ERR_INVALID_ARG;
  if (n_prompt < 1 || n_prompt > m.T) return NC_ERR_SHAPE;
  if (!aligned(params) || !aligned(idx) || !aligned(cache) || !aligned(next_tok) || !aligned(workspace))
    return NC_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (m.es == 2) {
    if (workspace_bytes < carve_infer<bf16>(nullptr, m).bytes) return NC_ERR_WORKSPACE;
    return prefill_t<bf16>(m, static_cast<const bf16*>(params), idx, n_prompt, cache, next_tok, workspace, st);
  }
  if (workspace_bytes < carve_infer<float>(nullptr, m).bytes) return NC_ERR_WORKSPACE;
  return prefill_t<float>(m, static_cast<const float*>(params), idx, n_prompt, cache, next_tok, workspace, st);
}

nc_status nc_decode_step(const nc_config* cfg, const void* params, const int32_t* tok, int pos, void* cache,
                         int32_t* next_tok, void* workspace, size_t workspace_bytes, void* stream) {
  Dims m;
  NC_TRY(infer_dims(cfg, &m));
  if (!params || !tok || !cache || !next_tok || !workspace) return NC_ERR_INVALID_ARG;
  if (pos < 1 || pos >= m.T) return NC_ERR_SHAPE;
  if (!aligned(params) || !aligned(tok) || !aligned(cache) || !aligned(next_tok) || !aligned(workspace))
    return NC_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (m.es == 2) {
    if (workspace_bytes < carve_infer<bf16>(nullptr, m).bytes) return NC_ERR_WORKSPACE;
    return decode_t<bf16>(m, static_cast<const bf16*>(params), tok, pos, cache, next_tok,
                          carve_infer<bf16>(workspace, m), static_cast<uint32_t*>(workspace), st);
  }
  if (workspace_bytes < carve_infer<float>(nullptr, m).bytes) return NC_ERR_WORKSPACE;
  return decode_t<float>(m, static_cast<const float*>(params), tok, pos, cache, next_tok,
                         carve_infer<float>(workspace, m), static_cast<uint32_t*>(workspace), st);
}

nc_status nc_opt_query_sizes(const nc_config* cfg, nc_opt_sizes* out) {
  Dims m;
  NC_TRY(make_dims(cfg, &m, true));
  if (!out) return NC_ERR_INVALID_ARG;
  std::vector<size_t> off(2 + 4 * (size_t)m.L);
  const size_t n = param_offsets(m, off.data());
  out->state = 4 * (2 * n + 2 * (size_t)m.V * m.d);
  out->workspace = opt_workspace_bytes(m);
  return NC_OK;
}

nc_status nc_opt_init(const nc_config* cfg, const void* params, void* state, void* stream) {
  Dims m;
  NC_TRY(make_dims(cfg, &m, true));
  if (!params || !state) return NC_ERR_INVALID_ARG;
  if (!aligned(params) || !aligned(state)) return NC_ERR_ALIGN;
  std::vector<size_t> off(2 + 4 * (size_t)m.L);
  const size_t n = param_offsets(m, off.data());
  float* sp = static_cast<float*>(state);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t n2 = 2 * (size_t)m.V * m.d;
  if (m.es == 2) return opt_init<bf16>(static_cast<const bf16*>(params), sp, sp + n, n, sp + 2 * n, n2, st);
  return opt_init<float>(static_cast<const float*>(params), sp, sp + n, n, sp + 2 * n, n2, st);
}

nc_status nc_opt_step(const nc_config* cfg, const nc_opt_hparams* hp, void* params, const float* grads, void* state,
                      void* workspace, size_t workspace_bytes, void* stream) {
  Dims m;
  NC_TRY(make_dims(cfg, &m, true));
  if (!hparams_ok(hp) || !params || !grads || !state || !workspace) return NC_ERR_INVALID_ARG;
  if (!aligned(params) || !aligned(grads) || !aligned(state) || !aligned(workspace)) return NC_ERR_ALIGN;
  if (workspace_bytes < opt_workspace_bytes(m)) return NC_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (m.es == 2)
    return opt_step_t<bf16>(m, *hp, static_cast<bf16*>(params), grads, static_cast<float*>(state), workspace,
                            workspace_bytes, st);
  return opt_step_t<float>(m, *hp, static_cast<float*>(params), grads, static_cast<float*>(state), workspace,
                           workspace_bytes, st);
}

nc_status nc_model_loss_and_grad(const nc_config* cfg, const void* params, const int32_t* idx, const int32_t* targets,
                                 float* loss, float* grads, float dloss, int accumulate, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  Dims m;
  NC_TRY(make_dims(cfg, &m, true));
  if (!params || !idx || !targets || !loss || !grads || !workspace) return NC_ERR_INVALID_ARG;
  if (!aligned(params) || !aligned(idx) || !aligned(targets) || !aligned(grads) || !aligned(workspace))
    return NC_ERR_ALIGN;
  if (workspace_bytes < model_workspace_bytes(m)) return NC_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (m.es == 2)
    return model_t<bf16>(m, static_cast<const bf16*>(params), idx, targets, loss, grads, dloss, accumulate, workspace,
                         st);
  return model_t<float>(m, static_cast<const float*>(params), idx, targets, loss, grads, dloss, accumulate, workspace,
                        st);
}

}  // extern "C"
