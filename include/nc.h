/* nc.h - C ABI of the MI355X (gfx950) nanochat pretraining step.
 *
 * One GPU's forward + backward through the decoder described by the
 * architecture list of the page "安德烈·卡帕西推出nanochat：极简全栈AI训练项目"
 * (vpshk.cn, Q&A section "卡帕西亲自揭秘背后技术"): a dense Transformer with
 * rotary embeddings (no position table), QK norm, untied embedding and
 * unembedding, a norm right after the token embedding, a ReLU^2 MLP,
 * parameter-free RMSNorm, bias-free linears, multi-query attention and a
 * logit softcap; trained by next-token cross-entropy (page "100美元成本、
 * 8000行代码纯手搓克隆ChatGPT!" on imeisheng.com, section "预训练", which also
 * fixes the per-GPU batch of 32 rows x 2048 tokens and the depth-20 shape of
 * 1280 channels and 10 heads of 128).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named in the argument lists are DEVICE pointers unless marked
 *    "host". `stream` is a hipStream_t passed as void* (NULL = null stream).
 *  - The caller owns all memory. The library never allocates or frees device
 *    memory and never synchronises the stream, except nc_read_status. It keeps
 *    no pointer after returning, beyond the kernels already queued.
 *  - Storage type: cfg->dtype = NC_BF16 stores weights, activations and
 *    activation gradients as bfloat16 (round to nearest even); NC_F32 stores
 *    them as float (the check mode). Statistics, GEMM accumulation, softmax,
 *    loss and all weight gradients are float32 in both modes. NC_BF16_FP8
 *    stores as NC_BF16 and runs the four forward projections of every block
 *    (QKV, O, W1, W2) as FP8 E4M3 products: each operand is rounded to E4M3
 *    under one scale per tensor (its largest magnitude maps to 448), the
 *    products accumulate in float32, and the result is scaled back. The page
 *    on pomoai.com says nanochat's newest version trains with FP8 and gives no
 *    recipe; this per-tensor, forward-only form is the plainest reading. The
 *    backward is the NC_BF16 one on the same bf16 activations (the rounding
 *    is treated as the identity). Inference (nc_prefill, nc_decode_step)
 *    returns NC_ERR_UNSUPPORTED for it.
 *  - Layouts are row-major. Weights use the [out, in] layout of a linear
 *    layer. M = batch * seq_len tokens; token m is row b = m / seq_len,
 *    position t = m % seq_len. d = d_model, H = n_head, G = n_kv_head,
 *    D = head_dim, F = d_ff, V = vocab, QKV = (H + 2G) * D.
 *  - Wqkv is [QKV, d] = rows of Wq [H*D, d], then Wk [G*D, d], then Wv [G*D, d].
 *  - idx and targets are int32 [M]. A target of -1 is ignored by the loss.
 *  - Every function returns nc_status; nothing throws across the ABI. Argument
 *    checks run before anything is queued: on error nothing was launched.
 *    NC_ERR_HIP means a launch failed (text via nc_last_hip_error).
 *  - Data errors found on the device (a token id outside [0,V), a target
 *    outside [-1,V), every target ignored, a non-finite loss) set bits of a
 *    sticky 32-bit status word kept in the first bytes of `scratch` (or of the
 *    model `workspace`); kernels then treat a bad id as a zero row and a bad
 *    target as ignored, with no out-of-bounds access. Read the word with
 *    nc_read_status, clear it with nc_clear_status (clear it once after
 *    allocating a scratch buffer).
 *  - All buffers must be 16-byte aligned (NC_ERR_ALIGN otherwise).
 *  - Results are deterministic: no floating-point atomics are used.
 *  - Calls that share a scratch buffer must not run concurrently.
 */
#ifndef NC_H_
#define NC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NC_ABI_VERSION 1

typedef enum nc_status {
  NC_OK = 0,
  NC_ERR_INVALID_ARG = 1, /* null pointer or bad flag */
  NC_ERR_SHAPE = 2,       /* inconsistent or non-positive shape */
  NC_ERR_ALIGN = 3,       /* a buffer is not 16-byte aligned */
  NC_ERR_WORKSPACE = 4,   /* workspace smaller than nc_query_sizes says */
  NC_ERR_UNSUPPORTED = 5, /* shape the kernels do not implement (see nc_validate) */
  NC_ERR_HIP = 6,         /* a HIP launch or runtime call failed */
  NC_ERR_DEVICE_DATA = 7  /* nc_read_status found a set device status bit */
} nc_status;

typedef enum nc_dtype { NC_BF16 = 0, NC_F32 = 1, NC_BF16_FP8 = 2 } nc_dtype;

/* Device status bits (see nc_read_status). */
#define NC_STATUS_BAD_TOKEN 0x1u
#define NC_STATUS_BAD_TARGET 0x2u
#define NC_STATUS_NONFINITE_LOSS 0x4u
#define NC_STATUS_NO_TARGETS 0x8u

/* Model and batch shape (host struct). softcap c: logits become c*tanh(z/c);
 * rope_base theta: pair i of a head rotates by t * theta^(-2i/D);
 * norm_eps: epsilon of every RMSNorm, the per-head QK norm included. */
typedef struct nc_config {
  int32_t depth, d_model, n_head, head_dim, n_kv_head, d_ff, vocab, batch, seq_len;
  float softcap, rope_base, norm_eps;
  int32_t dtype; /* nc_dtype */
} nc_config;

/* One block's weights, storage dtype: wqkv [QKV,d], wo [d,H*D], w1 [F,d], w2 [d,F]. */
typedef struct nc_block_params {
  const void *wqkv, *wo, *w1, *w2;
} nc_block_params;

/* One block's weight gradients, float32, same shapes as nc_block_params. */
typedef struct nc_block_grads {
  float *wqkv, *wo, *w1, *w2;
} nc_block_grads;

/* Buffer sizes in bytes for a configuration (see nc_query_sizes). */
typedef struct nc_sizes {
  size_t block_saved;     /* `saved` of nc_block_fwd/bwd (one block) */
  size_t lmhead_saved;    /* `saved` of nc_lmhead_softcap_xent_fwd/bwd */
  size_t scratch;         /* `scratch` of every per-function entry point */
  size_t model_workspace; /* `workspace` of nc_model_loss_and_grad */
  size_t n_params;        /* elements of the flat parameter buffer */
} nc_sizes;

/* ---------------------------------------------------------------- queries */

int nc_abi_version(void);
const char* nc_status_str(int status);
/* Text of the last HIP error seen by this thread ("" if none). */
const char* nc_last_hip_error(void);

/* Checks a configuration. NC_ERR_SHAPE: a non-positive size, H % G != 0,
 * d/H/F/V not matching. NC_ERR_UNSUPPORTED: head_dim not 64 or 128, d_model
 * or d_ff not a multiple of 64, vocab not a multiple of 8, more than
 * 2^31 - 1 elements in any tensor, 2^19 or more tokens (batch * seq_len),
 * dtype unknown. */
nc_status nc_validate(const nc_config* cfg);

/* Host outputs. offsets[0] = Wte [V,d]; for layer l (0-based)
 * offsets[1+4l .. 4+4l] = Wqkv, Wo, W1, W2; offsets[1+4L] = Wlm [V,d].
 * Offsets count elements of the flat parameter buffer, in which the
 * tensors are stored back to back in this order. n_offsets must be >= 2+4L. */
nc_status nc_param_layout(const nc_config* cfg, size_t* offsets, size_t n_offsets, size_t* n_params);

nc_status nc_query_sizes(const nc_config* cfg, nc_sizes* sizes /* host */);

/* The same sizes in three host outputs, any of which may be NULL:
 * model_bytes = the `workspace` of nc_model_loss_and_grad, block_saved_bytes
 * = one block's `saved`, scratch_bytes = the `scratch` of the per-function
 * entry points. Errors as nc_validate. */
nc_status nc_workspace_size(const nc_config* cfg, size_t* model_bytes, size_t* block_saved_bytes,
                            size_t* scratch_bytes);

/* Copies the status word from the start of `scratch` (or a model workspace)
 * to *flags (host) after synchronising `stream`. Returns NC_OK when no bit is
 * set, NC_ERR_DEVICE_DATA otherwise. */
nc_status nc_read_status(const void* scratch, uint32_t* flags, void* stream);
/* Queues a kernel that zeroes the status word. */
nc_status nc_clear_status(void* scratch, void* stream);

/* ------------------------------------------------------------- embedding */

/* Token embedding followed by the parameter-free norm the architecture list
 * places right after it: x0[m] = N(Wte[idx[m]]), N(v) = v / sqrt(mean(v^2) + eps).
 * idx int32 [M]; wte [V,d]; x0 [M,d] (out); r0 float [M] (out) =
 * 1/sqrt(mean(Wte[idx[m]]^2) + eps), kept for the backward. */
nc_status nc_embed_fwd(const nc_config* cfg, const int32_t* idx, const void* wte, void* x0,
                       float* r0, void* scratch, void* stream);

/* Backward of nc_embed_fwd: de = N_bwd(dx0) = r0 * (dx0 - x0 * mean(dx0 * x0)),
 * dWte[v] = sum over m with idx[m] = v of de[m], in a fixed order: the
 * positions sorted by (id, m) are cut into windows of 64; inside a window a
 * run of equal ids is summed in increasing m, and an id whose run crosses
 * windows adds its per-window partial sums in window order. The result is
 * bitwise deterministic for fixed inputs. dwte float [V,d]: overwritten, or
 * added to when accumulate != 0 (rows of ids absent from idx are then left
 * unchanged). */
nc_status nc_embed_bwd(const nc_config* cfg, const int32_t* idx, const void* x0, const float* r0,
                       const void* dx0, float* dwte, int accumulate, void* scratch, void* stream);

/* ----------------------------------------------------------------- block */

/* One pre-norm block: h = N(x); [q|k|v] = h Wqkv^T; q, k <- RoPE(N_D(.)) per
 * head; o = causal multi-query attention (head h uses KV head h*G/H, scale
 * 1/sqrt(D)); x1 = x + o Wo^T; u = N(x1) W1^T; x_out = x1 + max(u,0)^2 W2^T.
 * x_in, x_out [M,d] (must not alias). saved [block_saved bytes] receives the
 * activations nc_block_bwd needs; it stays borrowed until that call. */
nc_status nc_block_fwd(const nc_config* cfg, const nc_block_params* w, const void* x_in,
                       void* x_out, void* saved, void* scratch, void* stream);

/* Backward of nc_block_fwd given dx_out = dLoss/dx_out [M,d]; writes
 * dx_in [M,d] (may alias dx_out) and the weight gradients (float32; written,
 * or added to when accumulate != 0). x_in and saved as passed to the forward. */
nc_status nc_block_bwd(const nc_config* cfg, const nc_block_params* w, const void* x_in,
                       const void* saved, const void* dx_out, void* dx_in,
                       const nc_block_grads* grads, int accumulate, void* scratch, void* stream);

/* ------------------------------------------------------------ LM head + loss */

/* Final norm, untied unembedding, logit softcap and next-token cross-entropy:
 * xf = N(x); z = xf Wlm^T; z' = c tanh(z/c);
 * loss = mean over m with targets[m] != -1 of logsumexp(z'[m]) - z'[m][targets[m]].
 * x [M,d]; wlm [V,d]; loss: one float (device, out). saved [lmhead_saved bytes]
 * keeps xf, per logit u = exp(z' - c) (1 - (z'/c)^2) / 4 (storage dtype, [M,V]; the
 * logits themselves are not kept), the row log-sum-exps and the targets'
 * softcapped logits. */
nc_status nc_lmhead_softcap_xent_fwd(const nc_config* cfg, const void* x, const void* wlm,
                                     const int32_t* targets, float* loss, void* saved,
                                     void* scratch, void* stream);

/* Backward of the above scaled by dloss: dz = (softmax(z') - onehot(target))
 * * dloss / Nv * (1 - (z'/c)^2) on valid rows (0 on ignored rows);
 * dWlm = dz^T xf; dx = N_bwd(dz Wlm). dz is never formed: with S the row's
 * sum of exp(z' - c), dz = dloss / Nv / S (u - onehot(target) S (1 - (z'_t/c)^2)),
 * the target's element of u in `saved` is corrected in place (call it once
 * per forward) and the row factor goes into both products. dx [M,d] (out);
 * dwlm float [V,d] (written, or added to when accumulate != 0). */
nc_status nc_lmhead_softcap_xent_bwd(const nc_config* cfg, const void* x, const void* wlm,
                                     const int32_t* targets, void* saved, float dloss, void* dx,
                                     float* dwlm, int accumulate, void* scratch, void* stream);

/* ---------------------------------------------------------------- model */

/* The whole step: embedding, depth blocks, LM head + loss, then the backward
 * of all of them. params: flat buffer in the storage dtype laid out as
 * nc_param_layout says; grads: float32, same layout (written, or added to
 * when accumulate != 0); loss: one float (device, out); dloss scales every
 * gradient (1 for a plain step, 1/n to average n micro-steps).
 * workspace [workspace_bytes >= model_workspace] holds every activation of
 * the step plus scratch; its first bytes are the device status word. */
nc_status nc_model_loss_and_grad(const nc_config* cfg, const void* params, const int32_t* idx,
                                 const int32_t* targets, float* loss, float* grads, float dloss,
                                 int accumulate, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* ---------------------------------------------------------------- products */

/* One linear-layer product of the step, run by the same kernel and epilogue
 * that nc_block_*, nc_lmhead_* and nc_opt_step launch for it (the bias-free
 * linears and the untied unembedding with its logit softcap of the
 * architecture list on vpshk.cn; the Newton-Schulz steps of the optimizer
 * below). It lets a caller run, time or check one product in isolation.
 * Operands are row-major in the storage dtype (NC_BF16 or NC_F32), float32
 * accumulation; bf16 outputs are rounded to nearest even once. */
typedef enum nc_gemm_kind {
  NC_GEMM_XWT = 0,         /* y[M,N] = a[M,K] b[N,K]^T, plus aux[M,N] when aux != NULL (the QKV,
                              O and W2 forward products; aux is the residual stream) */
  NC_GEMM_XWT_RELUSQ = 1,  /* y[M,N] = max(a b^T, 0)^2 (the MLP's first product and its ReLU^2) */
  NC_GEMM_DYW = 2,         /* y[M,K] = a[M,N] b[N,K] (an input gradient: dy times the weight) */
  NC_GEMM_DYW_DRELUSQ = 3, /* y[M,K] = (a b) * 2 sqrt(aux[M,K]) with aux = max(u,0)^2 as the MLP
                              forward stored it: the gradient through ReLU^2 */
  NC_GEMM_DW = 4,          /* yf[N,K] = a[M,N]^T b[M,K] in float32, or yf += when accumulate != 0
                              (a weight gradient, the reduction over the M tokens; split over M
                              when that fills the GPU, partials in scratch, summed in a fixed order) */
  NC_GEMM_SOFTCAP = 5,     /* z = a b^T, y = c tanh(z / c) with c = softcap, stored in column
                              panels of 32: element (m, n) at (n/32)*32M + 32m + n%32 (y holds
                              M * ceil(N/32)*32 elements); yf[M, ceil(N/256)] (bf16) or
                              [M, ceil(N/128)] (f32) receives, per row and 256- (128-) column
                              tile, the float32 sum of exp(y) before rounding */
  NC_GEMM_AXPBY = 6,       /* y[M,N] = alpha a b^T, plus beta aux[M,N] when aux != NULL */
  NC_GEMM_GRAM = 7         /* y[K,K] = a[M,K]^T a (b and N unused) */
} nc_gemm_kind;

typedef struct nc_gemm_args {
  int32_t kind;       /* nc_gemm_kind */
  int32_t dtype;      /* NC_BF16 or NC_F32: storage type of a, b, aux and y */
  int32_t M, N, K;    /* M >= 1 (any), N and K multiples of 8 */
  const void* a;      /* device */
  const void* b;      /* device */
  const void* aux;    /* device, see the kinds; NULL otherwise */
  void* y;            /* device output in the storage type (not NC_GEMM_DW) */
  float* yf;          /* device float32 output (NC_GEMM_DW, NC_GEMM_SOFTCAP) */
  int32_t a_panels;   /* NC_GEMM_DYW / NC_GEMM_DW: a [M,N] is stored in the column panels
                         NC_GEMM_SOFTCAP writes (as the head's backward reads its dz) */
  int32_t accumulate; /* NC_GEMM_DW */
  float alpha, beta;  /* NC_GEMM_AXPBY */
  float softcap;      /* NC_GEMM_SOFTCAP, > 0 */
} nc_gemm_args;

/* Scratch bytes nc_gemm needs for args (0 unless a split NC_GEMM_DW). */
nc_status nc_gemm_scratch_size(const nc_gemm_args* args /* host */, size_t* bytes /* host */);

/* Runs the product on `stream`. Checks (before any launch): NC_ERR_INVALID_ARG
 * for an unknown kind or a missing pointer, NC_ERR_SHAPE for a non-positive
 * size, NC_ERR_UNSUPPORTED for N or K not a multiple of 8 or a tensor over
 * 2^31 - 1 elements, NC_ERR_ALIGN for a pointer not 16-byte aligned,
 * NC_ERR_WORKSPACE when scratch is smaller than nc_gemm_scratch_size. Outputs
 * must not alias inputs. */
nc_status nc_gemm(const nc_gemm_args* args /* host */, void* scratch, size_t scratch_bytes, void* stream);

/* ---------------------------------------------------------------- inference */

/* Greedy generation with a key/value cache: a prefill pass over the prompts,
 * then one decode step per new token (the inference engine the pages describe:
 * imeisheng.com, feature list and the end of section "预训练"; geoz.com.cn,
 * sections "推理与部署" and "高效推理引擎与交互界面"). cfg->batch is the number
 * of sequences and cfg->seq_len the cache capacity in positions. Greedy
 * decoding is a reading: the next token is the lowest id whose softcapped
 * logit c*tanh(z/c) is largest. */

/* Buffer sizes in bytes for inference (see nc_infer_query_sizes). */
typedef struct nc_infer_sizes {
  size_t cache;     /* K/V cache: [depth][2][batch][seq_len][n_kv_head*head_dim], storage dtype */
  size_t workspace; /* `workspace` of nc_prefill and nc_decode_step */
} nc_infer_sizes;

/* Sizes for cfg (NC_ERR_UNSUPPORTED when n_head / n_kv_head > 32). */
nc_status nc_infer_query_sizes(const nc_config* cfg, nc_infer_sizes* out);

/* Prompt pass. idx [batch, n_prompt] token ids (device), 1 <= n_prompt <=
 * seq_len. Fills cache positions 0 .. n_prompt-1 of every layer: K after QK
 * norm and rotation at [l][0][b][t][:], V at [l][1][b][t][:]. next_tok
 * [batch] (device, out): the greedy token after each prompt. params as for
 * nc_model_loss_and_grad. workspace [workspace bytes], its first bytes the
 * device status word (bad token ids set NC_STATUS_BAD_TOKEN and read as row 0
 * of the embedding). */
nc_status nc_prefill(const nc_config* cfg, const void* params, const int32_t* idx, int n_prompt, void* cache,
                     int32_t* next_tok, void* workspace, size_t workspace_bytes, void* stream);

/* One decode step for every sequence: tok [batch] (device) sits at position
 * pos (0 < pos < seq_len; positions 0 .. pos-1 are already in the cache).
 * Appends its K and V at pos and writes next_tok [batch] (device, out), the
 * greedy token that follows. Steps of one stream are ordered; the caller feeds
 * next_tok back as tok with pos + 1. */
nc_status nc_decode_step(const nc_config* cfg, const void* params, const int32_t* tok, int pos, void* cache,
                         int32_t* next_tok, void* workspace, size_t workspace_bytes, void* stream);

/* The decode step for callers that cannot allocate device memory or hand
 * over a workspace (code under graph capture, tight serving loops): the same
 * kernels as nc_decode_step, with their scratch in a static device array of
 * NC_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds from the
 * library's load to the end of the process. It calls no allocating routine.
 * The scratch holds one row per sequence of every activation, the attention
 * partials (batch * ceil(seq_len / 64) * n_head * (head_dim + 1) floats) and
 * the logit maxima: about 10 MB at 64 sequences of the depth-20 shape with a
 * 1280-position cache. Arguments as nc_decode_step; status (device, may be
 * NULL) receives NC_STATUS_BAD_TOKEN (OR-ed in) for a token id outside
 * [0, vocab). NC_ERR_WORKSPACE (before any launch) when the configuration
 * needs more scratch than the array holds. Every call on one GPU shares that
 * GPU's array and leaves its contents behind: calls that overlap on one GPU
 * (two streams, two threads) race and must be serialised by the caller. */
#define NC_NOALLOC_SCRATCH_BYTES (32u << 20)
nc_status nc_decode_step_noalloc(const nc_config* cfg, const void* params, const int32_t* tok, int pos, void* cache,
                                 int32_t* next_tok, uint32_t* status, void* stream);

/* ---------------------------------------------------------------- optimizer
 * The optimizer step (the page on vpshk.cn, Q&A section "卡帕西亲自揭秘背后技术",
 * names Muon + AdamW; imeisheng.com, section "预训练": Muon for the matrices,
 * AdamW for the embedding and the unembedding, no other trainable parameters,
 * the learning rate scaled by 1/sqrt(d_model) and its multiplier falling
 * linearly to 0 at the end of training). Muon is not defined on the pages;
 * its published definition is used (K. Jordan, 2024): Nesterov momentum, then
 * five steps of the quintic Newton-Schulz iteration with coefficients
 * (3.4445, -4.7750, 2.0315) on the update scaled to unit Frobenius norm, the
 * step scaled by max(1, rows/cols)^(1/2). Wq, Wk and Wv are three matrices to
 * Muon although the parameter buffer packs them. The learning rates passed in
 * already carry the schedule; the library holds no step counter. */

typedef struct nc_opt_hparams {
  float lr_matrix;  /* Muon, every block matrix */
  float lr_embed;   /* AdamW, Wte */
  float lr_unembed; /* AdamW, Wlm */
  float momentum;   /* Muon momentum, in [0, 1) */
  int32_t nesterov; /* 1: the Nesterov look-ahead g + momentum * buffer; 0: the buffer */
  float beta1, beta2, eps; /* AdamW; betas in [0, 1), eps > 0 */
  float wd_matrix, wd_adam; /* decoupled weight decay: w *= 1 - lr * wd before the update */
  int32_t step;     /* 1-based step count, for AdamW's bias correction */
} nc_opt_hparams;

typedef struct nc_opt_sizes {
  size_t state;     /* float32: master weights [n_params], s1 [n_params], s2 [2 vocab d_model] */
  size_t workspace; /* scratch of nc_opt_step */
} nc_opt_sizes;

/* Sizes for cfg (depth >= 1). */
nc_status nc_opt_query_sizes(const nc_config* cfg, nc_opt_sizes* out);

/* state (device, state bytes): master = params widened to float32, moments 0.
 * params as for nc_model_loss_and_grad. */
nc_status nc_opt_init(const nc_config* cfg, const void* params, void* state, void* stream);

/* One step: updates state from grads (device, float32, parameter layout, as
 * written by nc_model_loss_and_grad) and writes params (device, storage dtype)
 * = the new master weights rounded. State layout: master [n_params]; s1
 * [n_params] holds AdamW's first moment in the Wte and Wlm ranges and Muon's
 * momentum elsewhere; s2 [2 vocab d_model] holds AdamW's second moment of Wte
 * then of Wlm. Hyperparameters are checked before any launch (NC_ERR_INVALID_ARG).
 * workspace: nc_opt_sizes.workspace bytes. */
nc_status nc_opt_step(const nc_config* cfg, const nc_opt_hparams* hp, void* params, const float* grads, void* state,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- tracing */

/* Kernel timing. While enabled, every kernel launch of the library is
 * bracketed by two HIP events on the launch's stream and recorded with its
 * algorithmic work (model FLOPs, and the bytes the kernel must at least read
 * and write). on != 0 clears the record and starts recording; on == 0 stops.
 * Events are created by the HIP runtime when first needed and reused; no
 * device buffer is allocated. Recording costs two event records per launch. */
nc_status nc_profile_enable(int on);

/* Restricts the recording to the launches of one kernel class, named as in the
 * summary below (a host string, copied); NULL or "" records every launch
 * again. Timing one kernel costs two event records per launch of that kernel
 * only, so a timed run of the whole step can carry it. Takes effect for
 * launches issued after the call. */
nc_status nc_profile_only(const char* kernel_class);

/* Waits for the recorded events and writes, into buf (host, buf_len bytes), a
 * JSON object {"kernel": {"launches": n, "ms": t, "flops": f, "bytes": b}, ...}
 * summed per kernel. *written (host) receives the bytes needed including the
 * terminating NUL; NC_ERR_INVALID_ARG if buf is NULL or too small. */
nc_status nc_profile_summary(char* buf, size_t buf_len, size_t* written);

#ifdef __cplusplus
}
#endif

#endif /* NC_H_ */
