// q4_gemm_s64: S=64 chunked-prefill product on MFMA (placeholder until the
// MFMA kernel lands; returns Q4DEC_ERR_UNSUPPORTED after validation).
#include "q4dec_internal.h"

extern "C" int q4_gemm_s64(const void* packed, int64_t n, int64_t k, const uint16_t* x, int64_t n_tok, float* y,
                           void* stream) {
  using namespace q4dec;
  (void)stream;
  if (!packed) return fail(Q4DEC_ERR_NULL, "q4_gemm_s64: packed is NULL");
  if (!x) return fail(Q4DEC_ERR_NULL, "q4_gemm_s64: x is NULL");
  if (!y) return fail(Q4DEC_ERR_NULL, "q4_gemm_s64: y is NULL");
  if (n <= 0 || n >= (int64_t(1) << 31)) return fail(Q4DEC_ERR_SHAPE, "q4_gemm_s64: n out of range");
  if (k <= 0 || k % 32) return fail(Q4DEC_ERR_SHAPE, "q4_gemm_s64: k must be a positive multiple of 32");
  if (n_tok < 1 || n_tok > 64) return fail(Q4DEC_ERR_SHAPE, "q4_gemm_s64: n_tok must be in [1, 64]");
  return fail(Q4DEC_ERR_UNSUPPORTED, "q4_gemm_s64: not built yet");
}
