// Row gathers.
//
// ple_gather: out[t, j] = RN_fp32(q[id_t, j] * s[id_t] * mult)
// ("visible-cx/gemma-4-E2B-CoreAI", PLE gather-table sidecar section: int8
// table, fp32 per-row scale, embed_scale_pl 16.0).
//
// rowq_gather: the same on the dense per-row INT2 / INT4 packing with one
// scale per group of columns ("Gemma-4 E2B mobile mixed-bit QAT weights":
// the INT2 input embedding [262144, 1536] with a per-row scale, and the INT4
// PLE table of 35 layer-major 128-byte blocks per row with one scale per row
// and layer).
//
// The int8 * fp32 product is exact in fp64; its product with the fp32
// multiplier is split into a rounded fp64 head and an exact fma tail, and the
// fp32 rounding of the head is corrected when the head sits exactly on a
// rounding midpoint. The result is the exact product rounded once to fp32 for
// any multiplier (for 16.0 the plain fp32 product would already be exact).
#include <math.h>

#include "q4dec_internal.h"

namespace q4dec {
Q4DEC_DEBUG_READER(ple_gather)

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
  Q4_DCHECK(int64_t(gridDim.x) * 256 * 16 >= dim, kDbgGatherGrid);
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

// One thread handles one 4-byte word of packed codes (16 INT2 or 8 INT4
// values of one output row), which lies inside one scale group; small words
// keep the per-thread chain short, since one id is the common call. An INT2
// code is 0, +-1 or -2, so its product with an fp32 scale below 2^126 is
// exact in fp32 and one fp32 multiply by mult rounds the exact product once;
// INT4 codes (and INT2 with larger scales) take the exact fp64 path.
template <int BITS>
__global__ __launch_bounds__(256) void rowq_gather_kernel(const uint32_t* __restrict__ w,
                                                          const float* __restrict__ scales, int vocab, int dim,
                                                          int group, const int32_t* __restrict__ ids, float mult,
                                                          float* __restrict__ out, int32_t* __restrict__ err) {
  constexpr int kPer = 32 / BITS;  // values per word
  const int words = dim / kPer;
  Q4_DCHECK(int64_t(gridDim.x) * 256 >= words, kDbgGatherGrid);
  const int t = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= words) return;
  const int id = ids[t];
  float4* o4 = reinterpret_cast<float4*>(out + size_t(t) * size_t(dim) + size_t(c) * kPer);
  if (id < 0 || id >= vocab) {
    if (err && c == 0) *err = 1;
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) o4[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    return;
  }
  const uint32_t wd = w[size_t(id) * size_t(words) + c];
  const float s = scales[size_t(id) * size_t(dim / group) + (c * kPer) / group];
  const bool fast = BITS == 2 && fabsf(s) < 0x1p126f;
  float r[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t u = (wd >> (BITS * i)) & ((1u << BITS) - 1u);
    const int code = int(u) - (u >> (BITS - 1) ? (1 << BITS) : 0);  // two's complement
    r[i] = fast ? (float(code) * s) * mult : round_product(code, s, double(mult));
  }
#pragma unroll
  for (int i = 0; i < kPer / 4; ++i) o4[i] = make_float4(r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]);
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

extern "C" int rowq_gather(const void* w, const float* scales, int64_t vocab, int64_t dim, int32_t bits,
                           int64_t group, const int32_t* ids, int64_t n_ids, float mult, float* out,
                           int32_t* err_flag, void* stream) {
  using namespace q4dec;
  const char* name = "rowq_gather";
  if (!w) return fail(Q4DEC_ERR_NULL, "%s: w is NULL", name);
  if (!scales) return fail(Q4DEC_ERR_NULL, "%s: scales is NULL", name);
  if (!ids) return fail(Q4DEC_ERR_NULL, "%s: ids is NULL", name);
  if (!out) return fail(Q4DEC_ERR_NULL, "%s: out is NULL", name);
  if (bits != 2 && bits != 4) return fail(Q4DEC_ERR_SHAPE, "%s: bits must be 2 or 4 (got %d)", name, int(bits));
  if (vocab <= 0 || vocab >= (int64_t(1) << 31))
    return fail(Q4DEC_ERR_SHAPE, "%s: vocab must be in [1, 2^31) (got %lld)", name, (long long)vocab);
  const int64_t per = 128 / bits;  // values per 16-byte chunk
  if (dim <= 0 || dim >= (int64_t(1) << 31) || dim % per)
    return fail(Q4DEC_ERR_SHAPE, "%s: dim must be a positive multiple of %lld for %d-bit codes (got %lld)", name,
                (long long)per, int(bits), (long long)dim);
  if (group <= 0 || group % per || dim % group)
    return fail(Q4DEC_ERR_SHAPE, "%s: group must divide dim and be a multiple of %lld (got %lld)", name,
                (long long)per, (long long)group);
  if (n_ids < 0 || n_ids > 65535)
    return fail(Q4DEC_ERR_SHAPE, "%s: n_ids must be in [0, 65535] (got %lld)", name, (long long)n_ids);
  if (!aligned(w, 16)) return fail(Q4DEC_ERR_ALIGN, "%s: w must be 16-byte aligned", name);
  if (!aligned(out, 16)) return fail(Q4DEC_ERR_ALIGN, "%s: out must be 16-byte aligned", name);
  if (!aligned(scales, 4) || !aligned(ids, 4))
    return fail(Q4DEC_ERR_ALIGN, "%s: scales and ids must be 4-byte aligned", name);
  if (n_ids == 0) return Q4DEC_OK;
  const int64_t words = dim * bits / 32;
  const dim3 grid(unsigned((words + 255) / 256), unsigned(n_ids));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint32_t* w32 = static_cast<const uint32_t*>(w);
  if (bits == 2)
    hipLaunchKernelGGL(rowq_gather_kernel<2>, grid, dim3(256), 0, st, w32, scales, int(vocab), int(dim), int(group),
                       ids, mult, out, err_flag);
  else
    hipLaunchKernelGGL(rowq_gather_kernel<4>, grid, dim3(256), 0, st, w32, scales, int(vocab), int(dim), int(group),
                       ids, mult, out, err_flag);
  return launch_status(name);
}
