// q4_gemm_s64: S<=64 chunked-prefill product Y[s, r] = sum_k X[s, k] * w[r, k]
// on the matrix cores ("visible-cx/gemma-4-E2B-CoreAI": the prefill entry
// point has a static query width of 64 and reads the weights once per 64
// tokens).
//
// Numerics. A bf16 or fp16 copy of c * d would round the 15-bit product, so
// the weights enter the MFMA as exact fp16 integer codes (the nibble trick of
// the GEMV) and each 32-wide block's fp16 scale is applied in fp32 after the
// block's v_mfma_f32_16x16x32_f16: acc += T_b * d[r, b]. Activations are
// converted once per call into fp16 scaled by a per-token power of two (the
// largest magnitude of the token lands in [2^14, 2^15)), which is undone on
// the output. Products are exact; only fp32 sums round.
//
// Work split. A workgroup (4 waves) owns 64 output rows (16 per wave) for all
// 64 token slots and one K slice; the activation chunk of 4 blocks is staged
// in LDS and shared by the 4 waves. Small-N matrices split K over several
// workgroups; their partial sums go to the workspace and a second kernel adds
// them in a fixed order, so results are deterministic.
#include <math.h>

#include <algorithm>

#include "q4dec_internal.h"

namespace q4dec {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kTok = 64;    // token slots
constexpr int kTileN = 64;  // weight rows per workgroup
constexpr int kChunk = 4;   // 32-wide blocks per LDS chunk

struct GemmPlan {
  int slices;        // K slices
  int bps;           // blocks per slice
  size_t xh_off, xf_off, part_off, total;
};

static GemmPlan gemm_plan(int64_t n, int64_t k) {
  GemmPlan p{};
  const int B = int(k / 32);
  const int64_t tiles = (n + kTileN - 1) / kTileN;
  // enough workgroups to cover the chip, slices of at least 8 blocks
  int s = 1;
  while (tiles * s < 512 && B / (2 * s) >= 8) s *= 2;
  p.slices = s;
  p.bps = (B + s - 1) / s;
  p.slices = (B + p.bps - 1) / p.bps;
  p.xh_off = 0;
  p.xf_off = align256(size_t(kTok) * size_t(k) * 2);
  p.part_off = p.xf_off + 256;
  p.total = p.part_off + (p.slices > 1 ? align256(size_t(p.slices) * kTok * size_t(n) * 4) : 0);
  return p;
}

// One workgroup per token slot: find the token's largest exponent, convert
// its row to scaled fp16, store 2^E. Slots >= n_tok are zero-filled.
__global__ __launch_bounds__(256) void gemm_x_prep_kernel(const uint16_t* __restrict__ x, int k, int n_tok,
                                                          _Float16* __restrict__ xh, float* __restrict__ xf) {
  const int s = blockIdx.x;
  _Float16* dst = xh + size_t(s) * size_t(k);
  if (s >= n_tok) {
    for (int i = threadIdx.x; i < k; i += 256) dst[i] = (_Float16)0.0f;
    if (threadIdx.x == 0) xf[s] = 0.0f;
    return;
  }
  const uint16_t* src = x + size_t(s) * size_t(k);
  uint32_t emax = 1;
  for (int i = threadIdx.x; i < k; i += 256) emax = max(emax, (uint32_t(src[i]) >> 7) & 0xFFu);
  for (int off = 32; off >= 1; off >>= 1) emax = max(emax, uint32_t(__shfl_xor(int(emax), off)));
  __shared__ uint32_t wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = emax;
  __syncthreads();
  emax = max(max(wm[0], wm[1]), max(wm[2], wm[3]));
  const int e = int(emax) - 127 - 14;
  for (int i = threadIdx.x; i < k; i += 256) dst[i] = (_Float16)ldexpf(bf16_to_f32(src[i]), -e);
  if (threadIdx.x == 0) xf[s] = ldexpf(1.0f, e);
}

__device__ __forceinline__ half8_t codes_f16x8(uint32_t w, uint32_t m_lo, uint32_t m_hi, uint32_t magic) {
  const CodePairs cp = unpack_dword(w, m_lo, m_hi, magic);
  half8_t r;
  r[0] = cp.p[0][0]; r[1] = cp.p[0][1]; r[2] = cp.p[1][0]; r[3] = cp.p[1][1];
  r[4] = cp.p[2][0]; r[5] = cp.p[2][1]; r[6] = cp.p[3][0]; r[7] = cp.p[3][1];
  return r;
}

template <bool PARTIAL>
__global__ __launch_bounds__(256) void q4_gemm_kernel(const uint8_t* __restrict__ nib, const uint16_t* __restrict__ scl,
                                                      const _Float16* __restrict__ xh, const float* __restrict__ xf,
                                                      int n, int k, int n_tok, int bps, float* __restrict__ out) {
  __shared__ uint4 xs[kChunk][kTok][4];  // [block][token][k quarter], 16 KB
  const int B = k >> 5;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4;        // k group of this lane in a block: k = 8q .. 8q+7
  const int col = lane & 15;      // output row within the wave's 16
  const int r_lane = blockIdx.x * kTileN + wave * 16 + col;
  const bool r_ok = r_lane < n;
  const int r_c = r_ok ? r_lane : n - 1;
  const int b_begin = blockIdx.y * bps;
  const int b_end = min(B, b_begin + bps);
  const uint8_t* wrow = nib + size_t(r_c) * size_t(k >> 1);
  const uint16_t* srow = scl + size_t(r_c) * size_t(B);

  uint32_t m_lo, m_hi, magic;
  asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(m_lo));
  asm volatile("v_mov_b32 %0, 0x00F000F0" : "=v"(m_hi));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

  float4_t acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int b0 = b_begin; b0 < b_end; b0 += kChunk) {
    const int nb = min(kChunk, b_end - b0);
    // weights of this chunk: dword q of each block of row r_c
    uint32_t wq[kChunk];
    uint32_t sd[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      if (c < nb) {
        wq[c] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(wrow + size_t(b0 + c) * 16) + q);
        sd[c] = __builtin_nontemporal_load(srow + b0 + c);
      } else {
        wq[c] = 0u;
        sd[c] = 0u;
      }
    }
    // stage the activation chunk: kChunk blocks x 64 tokens x 64 bytes
#pragma unroll
    for (int i = 0; i < (kChunk * kTok * 4) / 256; ++i) {
      const int idx = threadIdx.x + 256 * i;
      const int c = idx / (kTok * 4);
      const int rem = idx % (kTok * 4);
      const int s = rem >> 2, qq = rem & 3;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (c < nb) v = *reinterpret_cast<const uint4*>(xh + size_t(s) * size_t(k) + size_t(b0 + c) * 32 + qq * 8);
      xs[c][s][qq] = v;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      if (c < nb) {
        const half8_t bw = codes_f16x8(wq[c], m_lo, m_hi, magic);
        const float d = float(__builtin_bit_cast(_Float16, uint16_t(sd[c])));
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint4 av = xs[c][16 * m + col][q];
          const half8_t a = __builtin_bit_cast(half8_t, av);
          const float4_t t =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bw, float4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][i] = fmaf(t[i], d, acc[m][i]);
        }
      }
    }
    __syncthreads();
  }

  // lane holds tokens s = 16m + 4q + i of output row r_lane
  if (!r_ok) return;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 16 * m + 4 * q + i;
      if (PARTIAL) {
        out[(size_t(blockIdx.y) * kTok + s) * size_t(n) + r_lane] = acc[m][i] * xf[s];
      } else if (s < n_tok) {
        out[size_t(s) * size_t(n) + r_lane] = acc[m][i] * xf[s];
      }
    }
  }
}

// y[s, r] = sum over slices, in slice order.
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part, int slices, int n,
                                                          int n_tok, float* __restrict__ y) {
  const size_t total = size_t(n_tok) * size_t(n);
  const size_t stride = size_t(kTok) * size_t(n);
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += size_t(gridDim.x) * 256) {
    float v = part[i];
    for (int sl = 1; sl < slices; ++sl) v += part[size_t(sl) * stride + i];
    y[i] = v;
  }
}

}  // namespace q4dec

extern "C" size_t q4_gemm_workspace_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0 || k % 32 || k > Q4DEC_MAX_K) return 0;
  return q4dec::gemm_plan(n, k).total;
}

extern "C" int q4_gemm_s64(const void* packed, int64_t n, int64_t k, const uint16_t* x, int64_t n_tok, float* y,
                           void* ws, size_t ws_bytes, void* stream) {
  using namespace q4dec;
  if (!packed) return fail(Q4DEC_ERR_NULL, "q4_gemm_s64: packed is NULL");
  if (!x) return fail(Q4DEC_ERR_NULL, "q4_gemm_s64: x is NULL");
  if (!y) return fail(Q4DEC_ERR_NULL, "q4_gemm_s64: y is NULL");
  if (!ws) return fail(Q4DEC_ERR_NULL, "q4_gemm_s64: ws is NULL");
  if (n <= 0 || n >= (int64_t(1) << 31))
    return fail(Q4DEC_ERR_SHAPE, "q4_gemm_s64: n must be in [1, 2^31) (got %lld)", (long long)n);
  if (k <= 0 || k % 32)
    return fail(Q4DEC_ERR_SHAPE, "q4_gemm_s64: k must be a positive multiple of 32 (got %lld)", (long long)k);
  if (k > Q4DEC_MAX_K)
    return fail(Q4DEC_ERR_UNSUPPORTED, "q4_gemm_s64: k must be <= %d (got %lld)", Q4DEC_MAX_K, (long long)k);
  if (n_tok < 1 || n_tok > 64)
    return fail(Q4DEC_ERR_SHAPE, "q4_gemm_s64: n_tok must be in [1, 64] (got %lld)", (long long)n_tok);
  if (!aligned(packed, 16)) return fail(Q4DEC_ERR_ALIGN, "q4_gemm_s64: packed must be 16-byte aligned");
  if (!aligned(x, 2)) return fail(Q4DEC_ERR_ALIGN, "q4_gemm_s64: x must be 2-byte aligned");
  if (!aligned(y, 4)) return fail(Q4DEC_ERR_ALIGN, "q4_gemm_s64: y must be 4-byte aligned");
  if (!aligned(ws, 256)) return fail(Q4DEC_ERR_ALIGN, "q4_gemm_s64: ws must be 256-byte aligned");
  const GemmPlan p = gemm_plan(n, k);
  if (ws_bytes < p.total)
    return fail(Q4DEC_ERR_WORKSPACE, "q4_gemm_s64: ws_bytes %zu < required %zu", ws_bytes, p.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  _Float16* xh = reinterpret_cast<_Float16*>(w8 + p.xh_off);
  float* xf = reinterpret_cast<float*>(w8 + p.xf_off);
  float* part = reinterpret_cast<float*>(w8 + p.part_off);
  const uint8_t* nib = static_cast<const uint8_t*>(packed);
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(nib + nib_plane_bytes(n, k));
  hipLaunchKernelGGL(gemm_x_prep_kernel, dim3(kTok), dim3(256), 0, st, x, int(k), int(n_tok), xh, xf);
  const dim3 grid(unsigned((n + kTileN - 1) / kTileN), unsigned(p.slices));
  if (p.slices == 1) {
    hipLaunchKernelGGL(q4_gemm_kernel<false>, grid, dim3(256), 0, st, nib, scl, xh, xf, int(n), int(k), int(n_tok),
                       p.bps, y);
  } else {
    hipLaunchKernelGGL(q4_gemm_kernel<true>, grid, dim3(256), 0, st, nib, scl, xh, xf, int(n), int(k), int(n_tok),
                       p.bps, part);
    const size_t total = size_t(n_tok) * size_t(n);
    const unsigned rgrid = unsigned(std::min<size_t>((total + 255) / 256, 4096));
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3(rgrid), dim3(256), 0, st, part, p.slices, int(n), int(n_tok), y);
  }
  return launch_status("q4_gemm_s64");
}
