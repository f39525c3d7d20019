// Per-Layer-Embedding gather: out[t, j] = RN_fp32(q[id_t, j] * s[id_t] * mult)
// ("visible-cx/gemma-4-E2B-CoreAI", PLE gather-table sidecar section: int8
// table, fp32 per-row scale, embed_scale_pl 16.0).
//
// The int8 * fp32 product is exact in fp64; its product with the fp32
// multiplier is split into a rounded fp64 head and an exact fma tail, and the
// fp32 rounding of the head is corrected when the head sits exactly on a
// rounding midpoint. The result is the exact product rounded once to fp32 for
// any multiplier (for 16.0 the plain fp32 product would already be exact).
#include <math.h>

#include "q4dec_internal.h"

namespace q4dec {

__device__ __forceinline__ float round_product(int q, float s, double m) {
  const double p = double(q) * double(s);  // exact: 8 + 24 significant bits
  const double hi = p * m;
  const double lo = fma(p, m, -hi);        // exact remainder
  float f = float(hi);
  if (lo != 0.0) {
    const double back = double(f);
    if (back != hi) {
      const float other = back < hi ? nextafterf(f, INFINITY) : nextafterf(f, -INFINITY);
      // hi exactly halfway between f and other: the sign of lo decides
      if (2.0 * hi == back + double(other)) {
        const bool want_up = lo > 0.0;
        if ((other > f) == want_up) f = other;
      }
    }
  }
  return f;
}

// One thread handles 16 consecutive elements of one output row.
__global__ __launch_bounds__(256) void ple_gather_kernel(const int8_t* __restrict__ table,
                                                         const float* __restrict__ row_scale, int vocab, int dim,
                                                         const int32_t* __restrict__ ids, double mult,
                                                         float* __restrict__ out, int32_t* __restrict__ err,
                                                         int vec_ok) {
  const int t = blockIdx.y;
  const int j0 = (blockIdx.x * 256 + threadIdx.x) * 16;
  if (j0 >= dim) return;
  const int id = ids[t];
  float* o = out + size_t(t) * size_t(dim) + j0;
  const int cnt = min(16, dim - j0);
  if (id < 0 || id >= vocab) {
    if (err && j0 == 0) *err = 1;
    for (int i = 0; i < cnt; ++i) o[i] = 0.0f;
    return;
  }
  const float s = row_scale[id];
  const int8_t* src = table + size_t(id) * size_t(dim) + j0;
  if (vec_ok && cnt == 16) {
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = round_product(int(int8_t(w[i >> 2] >> (8 * (i & 3)))), s, mult);
    float4* o4 = reinterpret_cast<float4*>(o);
#pragma unroll
    for (int i = 0; i < 4; ++i) o4[i] = make_float4(r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]);
  } else {
    for (int i = 0; i < cnt; ++i) o[i] = round_product(int(src[i]), s, mult);
  }
}

}  // namespace q4dec

extern "C" int ple_gather(const int8_t* table, const float* row_scale, int64_t vocab, int64_t dim,
                          const int32_t* ids, int64_t n_ids, float mult, float* out, int32_t* err_flag,
                          void* stream) {
  using namespace q4dec;
  if (!table) return fail(Q4DEC_ERR_NULL, "ple_gather: table is NULL");
  if (!row_scale) return fail(Q4DEC_ERR_NULL, "ple_gather: row_scale is NULL");
  if (!ids) return fail(Q4DEC_ERR_NULL, "ple_gather: ids is NULL");
  if (!out) return fail(Q4DEC_ERR_NULL, "ple_gather: out is NULL");
  if (vocab <= 0 || vocab >= (int64_t(1) << 31))
    return fail(Q4DEC_ERR_SHAPE, "ple_gather: vocab must be in [1, 2^31) (got %lld)", (long long)vocab);
  if (dim <= 0 || dim >= (int64_t(1) << 31))
    return fail(Q4DEC_ERR_SHAPE, "ple_gather: dim must be in [1, 2^31) (got %lld)", (long long)dim);
  if (n_ids < 0 || n_ids > 65535)
    return fail(Q4DEC_ERR_SHAPE, "ple_gather: n_ids must be in [0, 65535] (got %lld)", (long long)n_ids);
  if (!aligned(row_scale, 4) || !aligned(ids, 4) || !aligned(out, 4))
    return fail(Q4DEC_ERR_ALIGN, "ple_gather: row_scale, ids and out must be 4-byte aligned");
  if (n_ids == 0) return Q4DEC_OK;
  const int vec_ok = (dim % 16 == 0) && aligned(table, 16) && aligned(out, 16);
  const int64_t per_row_threads = (dim + 15) / 16;
  dim3 grid(unsigned((per_row_threads + 255) / 256), unsigned(n_ids));
  hipLaunchKernelGGL(ple_gather_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), table, row_scale,
                     int(vocab), int(dim), ids, double(mult), out, err_flag, vec_ok);
  return launch_status("ple_gather");
}
