// S=1 q4_0 dequant-GEMV and the LM head with softcap + argmax.
//
// Weight stream: each lane owns a fixed set of 32-wide k-blocks of its row
// group (block b = j * LPR + t for j < BPL, t = lane % LPR), keeps the matching
// activations in registers for the whole kernel, and walks down the rows. One
// 16-byte non-temporal load per lane per block; LPR lanes of a row read
// LPR * 16 contiguous bytes, so every load instruction is fully coalesced in
// the row-major nibble plane. Codes are unpacked to exact fp16 integers in
// registers and reduced with v_dot2c_f32_f16 against activations converted
// once per workgroup into block-scaled fp16 (LDS), then each block partial is
// scaled by its fp16 weight scale and the block's power of two in fp32. The
// LPR partials of a row are summed with DPP.
//
// Decode is weight-bandwidth-bound ("Gemma 4 E2B (text decoder) - Core AI",
// "What it took": the device is bandwidth-bound; E4B card: about 2.1 GB of
// int4 weights read per token), so everything here serves the weight stream.
#include <math.h>
#include <limits.h>

#include "q4dec_internal.h"

namespace q4dec {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int LPR, int BPL, bool HEAD>
__global__ __launch_bounds__(kThreads) void q4_rows_kernel(const uint8_t* __restrict__ nib,
                                                           const uint16_t* __restrict__ scl,
                                                           const uint16_t* __restrict__ x, int n, int k, int ipw,
                                                           float* __restrict__ y, uint2* __restrict__ partials) {
  constexpr int RPW = 64 / LPR;  // rows per wave per iteration
  constexpr int MAXB = LPR * BPL;
  __shared__ uint32_t xs[MAXB * 16];
  __shared__ float xf[MAXB];
  const int B = k >> 5;

  // Stage the activations once per workgroup as block-scaled fp16 pairs.
  for (int b = threadIdx.x; b < B; b += kThreads) xf[b] = convert_x_block(x + 32 * b, xs + 16 * b);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = lane % LPR;
  const int r = lane / LPR;

  uint32_t xr[BPL][16];
  float fr[BPL];
#pragma unroll
  for (int j = 0; j < BPL; ++j) {
    const int b = j * LPR + t;
    if (b < B) {
      const uint4* s4 = reinterpret_cast<const uint4*>(xs + 16 * b);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint4 v = s4[i];
        xr[j][4 * i + 0] = v.x; xr[j][4 * i + 1] = v.y; xr[j][4 * i + 2] = v.z; xr[j][4 * i + 3] = v.w;
      }
      fr[j] = xf[b];
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) xr[j][i] = 0u;
      fr[j] = 0.0f;
    }
  }

  uint32_t m_lo, m_hi, magic;
  asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(m_lo));
  asm volatile("v_mov_b32 %0, 0x00F000F0" : "=v"(m_hi));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

  const int RG = (n + RPW - 1) / RPW;
  const int rg_base = blockIdx.x * kWaves * ipw + wave;
  const size_t row_bytes = size_t(k) >> 1;
  float best = -INFINITY;
  int bidx = INT_MAX;

  for (int i = 0; i < ipw; ++i) {
    const int rg = rg_base + i * kWaves;
    if (rg >= RG) break;
    const int row = rg * RPW + r;
    const bool rv = row < n;
    const int rowc = rv ? row : n - 1;
    const u32x4* np = reinterpret_cast<const u32x4*>(nib + size_t(rowc) * row_bytes);
    const uint16_t* sp = scl + size_t(rowc) * size_t(B);
    uint4 q[BPL];
    uint32_t s[BPL];
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int b = j * LPR + t;
      if (b < B) {
        const u32x4 v = __builtin_nontemporal_load(np + b);
        q[j] = make_uint4(v.x, v.y, v.z, v.w);
        s[j] = __builtin_nontemporal_load(sp + b);
      } else {
        q[j] = make_uint4(0u, 0u, 0u, 0u);
        s[j] = 0u;
      }
    }
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int b = j * LPR + t;
      if (b < B) {
        const float p = block_dot(q[j], xr[j], m_lo, m_hi, magic);
        const float d = float(__builtin_bit_cast(_Float16, uint16_t(s[j])));
        acc = fmaf(d * p, fr[j], acc);
      }
    }
    acc = group_sum<LPR>(acc);
    if constexpr (!HEAD) {
      if (t == 0 && rv) y[row] = acc;
    } else {
      if (rv && better(acc, row, best, bidx)) {
        best = acc;
        bidx = row;
      }
    }
  }

  if constexpr (HEAD) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(best, off);
      const int oi = __shfl_xor(bidx, off);
      if (better(ov, oi, best, bidx)) {
        best = ov;
        bidx = oi;
      }
    }
    __shared__ float sv[kWaves];
    __shared__ int si[kWaves];
    if (lane == 0) {
      sv[wave] = best;
      si[wave] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < kWaves; ++w)
        if (better(sv[w], si[w], best, bidx)) {
          best = sv[w];
          bidx = si[w];
        }
      partials[blockIdx.x] = make_uint2(__builtin_bit_cast(uint32_t, best), uint32_t(bidx));
    }
  }
}

__global__ __launch_bounds__(256) void lmhead_reduce_kernel(const uint2* __restrict__ partials, int g, float cap,
                                                            int32_t* __restrict__ idx_out,
                                                            float* __restrict__ val_out) {
  float best = -INFINITY;
  int bidx = INT_MAX;
  for (int i = threadIdx.x; i < g; i += 256) {
    const uint2 p = partials[i];
    const float v = __builtin_bit_cast(float, p.x);
    const int ix = int(p.y);
    if (better(v, ix, best, bidx)) {
      best = v;
      bidx = ix;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(best, off);
    const int oi = __shfl_xor(bidx, off);
    if (better(ov, oi, best, bidx)) {
      best = ov;
      bidx = oi;
    }
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bidx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], best, bidx)) {
        best = sv[w];
        bidx = si[w];
      }
    if (bidx == INT_MAX) {
      *idx_out = -1;
      *val_out = __builtin_nanf("");
    } else {
      *idx_out = bidx;
      *val_out = cap > 0.0f ? cap * tanhf(best / cap) : best;
    }
  }
}

// ---------------------------------------------------------------- dispatch
struct Plan {
  int lpr, bpl, rpw, rg, ipw, grid;
};

static Plan make_plan(int64_t n, int64_t k) {
  const int B = int(k / 32);
  Plan p{};
  if ((B + 15) / 16 <= 5) {
    p.lpr = 16;
  } else if ((B + 31) / 32 <= 5) {
    p.lpr = 32;
  } else {
    p.lpr = 64;
  }
  p.bpl = (B + p.lpr - 1) / p.lpr;
  p.rpw = 64 / p.lpr;
  p.rg = int((n + p.rpw - 1) / p.rpw);
  const int waves_max = device_cu_count() * 16;
  p.ipw = (p.rg + waves_max - 1) / waves_max;
  const int waves = (p.rg + p.ipw - 1) / p.ipw;
  p.grid = (waves + kWaves - 1) / kWaves;
  return p;
}

template <bool HEAD>
static int launch_rows(const Plan& p, const uint8_t* nib, const uint16_t* scl, const uint16_t* x, int n, int k,
                       float* y, uint2* partials, hipStream_t st) {
#define Q4_CASE(L, BP)                                                                                     \
  if (p.lpr == L && p.bpl == BP) {                                                                         \
    hipLaunchKernelGGL((q4_rows_kernel<L, BP, HEAD>), dim3(p.grid), dim3(kThreads), 0, st, nib, scl, x, n, \
                       k, p.ipw, y, partials);                                                             \
    return Q4DEC_OK;                                                                                       \
  }
  Q4_CASE(16, 1) Q4_CASE(16, 2) Q4_CASE(16, 3) Q4_CASE(16, 4) Q4_CASE(16, 5)
  Q4_CASE(32, 3) Q4_CASE(32, 4) Q4_CASE(32, 5)
  Q4_CASE(64, 3) Q4_CASE(64, 4) Q4_CASE(64, 5) Q4_CASE(64, 6) Q4_CASE(64, 7) Q4_CASE(64, 8)
#undef Q4_CASE
  return fail(Q4DEC_ERR_UNSUPPORTED, "no kernel for k=%d (lpr=%d, bpl=%d)", k, p.lpr, p.bpl);
}

static int check_common(const char* fn, const void* packed, int64_t n, const char* nname, int64_t k,
                        const uint16_t* x) {
  if (!packed) return fail(Q4DEC_ERR_NULL, "%s: packed is NULL", fn);
  if (!x) return fail(Q4DEC_ERR_NULL, "%s: x is NULL", fn);
  if (n <= 0 || n >= (int64_t(1) << 31)) return fail(Q4DEC_ERR_SHAPE, "%s: %s must be in [1, 2^31) (got %lld)", fn, nname, (long long)n);
  if (k <= 0 || k % 32) return fail(Q4DEC_ERR_SHAPE, "%s: k must be a positive multiple of 32 (got %lld)", fn, (long long)k);
  if (k > Q4DEC_MAX_K) return fail(Q4DEC_ERR_UNSUPPORTED, "%s: k must be <= %d (got %lld)", fn, Q4DEC_MAX_K, (long long)k);
  if (!aligned(packed, 16)) return fail(Q4DEC_ERR_ALIGN, "%s: packed must be 16-byte aligned", fn);
  if (!aligned(x, 16)) return fail(Q4DEC_ERR_ALIGN, "%s: x must be 16-byte aligned", fn);
  return Q4DEC_OK;
}

static constexpr int kMaxPartials = 8192;

}  // namespace q4dec

extern "C" int q4_gemv(const void* packed, int64_t n, int64_t k, const uint16_t* x, float* y, void* stream) {
  using namespace q4dec;
  int rc = check_common("q4_gemv", packed, n, "n", k, x);
  if (rc) return rc;
  if (!y) return fail(Q4DEC_ERR_NULL, "q4_gemv: y is NULL");
  if (!aligned(y, 4)) return fail(Q4DEC_ERR_ALIGN, "q4_gemv: y must be 4-byte aligned");
  const Plan p = make_plan(n, k);
  const uint8_t* nib = static_cast<const uint8_t*>(packed);
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(nib + nib_plane_bytes(n, k));
  rc = launch_rows<false>(p, nib, scl, x, int(n), int(k), y, nullptr, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  return launch_status("q4_gemv");
}

extern "C" size_t lmhead_workspace_bytes(int64_t vocab, int64_t k) {
  (void)vocab;
  (void)k;
  return size_t(q4dec::kMaxPartials) * sizeof(uint2);
}

extern "C" int lmhead_softcap_argmax(const void* packed, int64_t vocab, int64_t k, const uint16_t* x, float cap,
                                     void* ws, size_t ws_bytes, int32_t* idx_out, float* val_out, void* stream) {
  using namespace q4dec;
  int rc = check_common("lmhead_softcap_argmax", packed, vocab, "vocab", k, x);
  if (rc) return rc;
  if (!ws) return fail(Q4DEC_ERR_NULL, "lmhead_softcap_argmax: ws is NULL");
  if (!idx_out) return fail(Q4DEC_ERR_NULL, "lmhead_softcap_argmax: idx_out is NULL");
  if (!val_out) return fail(Q4DEC_ERR_NULL, "lmhead_softcap_argmax: val_out is NULL");
  if (!aligned(ws, 8)) return fail(Q4DEC_ERR_ALIGN, "lmhead_softcap_argmax: ws must be 8-byte aligned");
  if (!aligned(idx_out, 4) || !aligned(val_out, 4))
    return fail(Q4DEC_ERR_ALIGN, "lmhead_softcap_argmax: idx_out and val_out must be 4-byte aligned");
  const size_t need = lmhead_workspace_bytes(vocab, k);
  if (ws_bytes < need)
    return fail(Q4DEC_ERR_WORKSPACE, "lmhead_softcap_argmax: ws_bytes %zu < required %zu", ws_bytes, need);
  const Plan p = make_plan(vocab, k);
  if (p.grid > kMaxPartials) return fail(Q4DEC_ERR_UNSUPPORTED, "lmhead_softcap_argmax: too many workgroups");
  const uint8_t* nib = static_cast<const uint8_t*>(packed);
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(nib + nib_plane_bytes(vocab, k));
  uint2* partials = static_cast<uint2*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = launch_rows<true>(p, nib, scl, x, int(vocab), int(k), nullptr, partials, st);
  if (rc) return rc;
  hipLaunchKernelGGL(lmhead_reduce_kernel, dim3(1), dim3(256), 0, st, partials, p.grid, cap, idx_out, val_out);
  return launch_status("lmhead_softcap_argmax");
}
