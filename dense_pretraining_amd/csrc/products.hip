// nc_gemm: one linear-layer product of the step at a time, through the same
// kernels and epilogues the block, head and optimizer entry points launch
// (bias-free linears and an untied, softcapped unembedding: the architecture
// list on vpshk.cn). Argument checks, then one launcher call.
#include "common.h"
#include "kernels.h"

namespace nc {
namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape and pointer checks shared by nc_gemm and nc_gemm_scratch_size.
nc_status gemm_args_ok(const nc_gemm_args* a) {
  if (!a) return NC_ERR_INVALID_ARG;
  if (a->dtype != NC_BF16 && a->dtype != NC_F32) return NC_ERR_UNSUPPORTED;
  if (a->kind < NC_GEMM_XWT || a->kind > NC_GEMM_GRAM) return NC_ERR_INVALID_ARG;
  if (a->M <= 0 || a->K <= 0 || (a->kind != NC_GEMM_GRAM && a->N <= 0)) return NC_ERR_SHAPE;
  // 16-byte operand chunks: every row length and every K-outer row count a multiple of 8
  if (a->K % 8 != 0 || (a->kind != NC_GEMM_GRAM && a->N % 8 != 0)) return NC_ERR_UNSUPPORTED;
  const long M = a->M, N = a->kind == NC_GEMM_GRAM ? a->K : a->N, K = a->K;
  // the [M, N] logits of the softcap product and a panelled a (the logit
  // gradient) are addressed per 32-column panel, as the unembedding does
  const bool panel_mn = a->kind == NC_GEMM_SOFTCAP || a->a_panels;
  if ((!panel_mn && M * N > 0x7fffffffL) || M * K > 0x7fffffffL || N * K > 0x7fffffffL) return NC_ERR_UNSUPPORTED;
  if (a->kind == NC_GEMM_SOFTCAP && (M * kPanel * 8 * 2 > 0x7fffffffL || M * kPanel >= (1L << 24)))
    return NC_ERR_UNSUPPORTED;
  if (a->a_panels && a->kind != NC_GEMM_DYW && a->kind != NC_GEMM_DW) return NC_ERR_INVALID_ARG;
  if (a->a_panels && (M * kPanel * 8 * 4 > 0x7fffffffL || M * kPanel >= (1L << 24))) return NC_ERR_UNSUPPORTED;
  const bool want_y = a->kind != NC_GEMM_DW;
  const bool want_yf = a->kind == NC_GEMM_DW || a->kind == NC_GEMM_SOFTCAP;
  const bool want_aux = a->kind == NC_GEMM_DYW_DRELUSQ;
  if (!a->a || (a->kind != NC_GEMM_GRAM && !a->b) || (want_y && !a->y) || (want_yf && !a->yf) ||
      (want_aux && !a->aux))
    return NC_ERR_INVALID_ARG;
  if (a->aux && a->kind != NC_GEMM_XWT && a->kind != NC_GEMM_DYW_DRELUSQ && a->kind != NC_GEMM_AXPBY)
    return NC_ERR_INVALID_ARG;
  if (!aligned16(a->a) || !aligned16(a->b) || !aligned16(a->aux) || !aligned16(a->y) || !aligned16(a->yf))
    return NC_ERR_ALIGN;
  if (a->kind == NC_GEMM_SOFTCAP && !(a->softcap > 0.f)) return NC_ERR_INVALID_ARG;
  return NC_OK;
}

size_t gemm_scratch_bytes(const nc_gemm_args* a) {
  if (a->kind != NC_GEMM_DW) return 0;
  return gemm_dw_partial_elems(a->M, a->N, a->K) * sizeof(float);
}

template <typename T>
nc_status run_gemm(const nc_gemm_args* a, float* partial, size_t partial_elems, hipStream_t st) {
  const T* A = static_cast<const T*>(a->a);
  const T* B = static_cast<const T*>(a->b);
  const T* X = static_cast<const T*>(a->aux);
  T* Y = static_cast<T*>(a->y);
  const int M = a->M, N = a->N, K = a->K;
  const long panel = a->a_panels ? (long)M * kPanel : 0;
  switch (a->kind) {
    case NC_GEMM_XWT: return gemm_xwt<T>(A, B, Y, X, M, N, K, false, st);
    case NC_GEMM_XWT_RELUSQ: return gemm_xwt<T>(A, B, Y, nullptr, M, N, K, true, st);
    case NC_GEMM_DYW: return gemm_dyw<T>(A, B, Y, nullptr, M, N, K, st, panel);
    case NC_GEMM_DYW_DRELUSQ: return gemm_dyw<T>(A, B, Y, X, M, N, K, st, panel);
    case NC_GEMM_DW: return gemm_dw<T>(A, B, a->yf, M, N, K, a->accumulate, partial, partial_elems, st, panel);
    case NC_GEMM_SOFTCAP: return gemm_lmhead<T>(A, B, Y, M, N, K, a->softcap, a->yf, st);
    case NC_GEMM_AXPBY: return gemm_xwt_axpby<T>(A, B, Y, X, M, N, K, a->alpha, a->beta, st);
    case NC_GEMM_GRAM: return gemm_gram<T>(A, Y, M, K, st);
    default: return NC_ERR_INVALID_ARG;
  }
}

}  // namespace
}  // namespace nc

using namespace nc;

extern "C" {

nc_status nc_gemm_scratch_size(const nc_gemm_args* args, size_t* bytes) {
  NC_TRY(gemm_args_ok(args));
  if (!bytes) return NC_ERR_INVALID_ARG;
  *bytes = gemm_scratch_bytes(args);
  return NC_OK;
}

nc_status nc_gemm(const nc_gemm_args* args, void* scratch, size_t scratch_bytes, void* stream) {
  NC_TRY(gemm_args_ok(args));
  const size_t need = gemm_scratch_bytes(args);
  if (need > 0 && (!scratch || scratch_bytes < need)) return NC_ERR_WORKSPACE;
  if (need > 0 && !aligned16(scratch)) return NC_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(scratch);
  const size_t pe = scratch_bytes / sizeof(float);
  if (args->dtype == NC_BF16) return run_gemm<bf16>(args, part, pe, st);
  return run_gemm<float>(args, part, pe, st);
}

}  // extern "C"
