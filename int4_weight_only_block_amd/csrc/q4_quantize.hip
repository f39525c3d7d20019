// q4_quantize: bf16 weights -> q4_0 codes and fp16 block scales, the export
// step in front of q4_pack ("Gemma 4 E2B (text decoder) - Core AI", QAT
// weights section: q4_0 is per-block-32 absmax symmetric int4 on the ggml
// q4_0 grid; "visible-cx/gemma-4-E2B-CoreAI", Provenance: the int4 rounding
// happens at export). One thread quantises one 32-wide block; every step is
// fp32 and each code is rint of the correctly rounded quotient, the same
// integer a host evaluating the same steps gets.
#include "q4dec_internal.h"

namespace q4dec {
Q4DEC_DEBUG_READER(q4_quantize)

__global__ __launch_bounds__(256) void q4_quantize_kernel(const uint16_t* __restrict__ x, int64_t n_blocks, int rule,
                                                          int8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                          int32_t* __restrict__ err) {
  Q4_DCHECK(int64_t(gridDim.x) * blockDim.x >= n_blocks, kDbgQuantGrid);
  const int64_t blk = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + blk * 32);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
  float v[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
  }
  // value of largest magnitude, lowest index on ties; NaNs never win (a
  // block of NaNs keeps its first value)
  float m = v[0], am = -1.0f;
  bool has_nan = false;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const bool nan = v[j] != v[j];
    has_nan |= nan;
    const float a = nan ? -1.0f : fabsf(v[j]);
    if (a > am) {
      am = a;
      m = v[j];
    }
  }
  const float d = rule == 0 ? m * -0.125f : __fdiv_rn(fabsf(m), 7.0f);  // m / -8 is exact
  uint16_t dbits = __builtin_bit_cast(uint16_t, (_Float16)d);             // round to nearest even
  if ((dbits & 0x7FFFu) == 0) dbits = 0;                                   // +0, not -0
  const float d32 = float(__builtin_bit_cast(_Float16, dbits));
  const bool usable = d32 == d32 && fabsf(d32) <= 65504.0f && d32 != 0.0f;
  const float lo = rule == 0 ? -8.0f : -7.0f;
  // The code is rint of the correctly rounded quotient. |x / d16| <= 8.004
  // on both grids, so t = x * RN(1 / d16) lies within 1.5e-6 of RN(x / d16)
  // (two roundings of 2^-24 relative each) and has the same rint unless its
  // fraction is within 4e-6 of one half; only then is the division done.
  const float rcp = usable ? __fdiv_rn(1.0f, d32) : 0.0f;
  uint32_t packed[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float xv = v[4 * i + b];
      float t = xv * rcp;
      const bool near_half = fabsf(t - floorf(t) - 0.5f) < 4e-6f;
      // wave-uniform test, so the division runs only in the rare waves
      // that need it (a per-lane branch is turned into computing both)
      if (__builtin_amdgcn_ballot_w64(near_half) != 0) {
        asm volatile("" ::: "memory");  // keeps the division inside the branch
        if (near_half) t = __fdiv_rn(xv, d32);
      }
      float q = usable ? rintf(t) : 0.0f;
      q = q != q ? 0.0f : fminf(fmaxf(q, lo), 7.0f);
      word |= (uint32_t(int32_t(q)) & 0xFFu) << (8 * b);
    }
    packed[i] = word;
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + blk * 32);
  dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  scales[blk] = dbits;
  if (err && (has_nan || !(fabsf(d32) <= 65504.0f))) *err = 1;
}

}  // namespace q4dec

extern "C" int q4_quantize(const uint16_t* x, int64_t n, int64_t k, int32_t rule, int8_t* codes, uint16_t* scales,
                           int32_t* err_flag, void* stream) {
  using namespace q4dec;
  if (!x) return fail(Q4DEC_ERR_NULL, "q4_quantize: x is NULL");
  if (!codes) return fail(Q4DEC_ERR_NULL, "q4_quantize: codes is NULL");
  if (!scales) return fail(Q4DEC_ERR_NULL, "q4_quantize: scales is NULL");
  if (n <= 0) return fail(Q4DEC_ERR_SHAPE, "q4_quantize: n must be > 0 (got %lld)", (long long)n);
  if (k <= 0 || k % 32)
    return fail(Q4DEC_ERR_SHAPE, "q4_quantize: k must be a positive multiple of 32 (got %lld)", (long long)k);
  if (rule != Q4DEC_QUANT_Q4_0 && rule != Q4DEC_QUANT_ABSMAX7)
    return fail(Q4DEC_ERR_SHAPE, "q4_quantize: rule must be Q4DEC_QUANT_Q4_0 or Q4DEC_QUANT_ABSMAX7 (got %d)",
                int(rule));
  if (!aligned(x, 16)) return fail(Q4DEC_ERR_ALIGN, "q4_quantize: x must be 16-byte aligned");
  if (!aligned(codes, 16)) return fail(Q4DEC_ERR_ALIGN, "q4_quantize: codes must be 16-byte aligned");
  if (!aligned(scales, 2)) return fail(Q4DEC_ERR_ALIGN, "q4_quantize: scales must be 2-byte aligned");
  const int64_t n_blocks = n * (k / 32);
  const int64_t grid = (n_blocks + 255) / 256;
  if (grid > 0x7FFFFFFF) return fail(Q4DEC_ERR_SHAPE, "q4_quantize: matrix too large");
  hipLaunchKernelGGL(q4_quantize_kernel, dim3(unsigned(grid)), dim3(256), 0, static_cast<hipStream_t>(stream), x,
                     n_blocks, int(rule), codes, scales, err_flag);
  return launch_status("q4_quantize");
}
