// Internal helpers shared by the libq4dec translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "q4dec.h"

namespace q4dec {

// ---------------------------------------------------------------- host side
// Thread-local error text; returns `code` so call sites can `return fail(...)`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
// Compute units of the current device (cached per device id).
int device_cu_count();

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Planes of a packed [n, k] matrix, in order: nibbles, then fp16 scales.
inline size_t nib_plane_bytes(int64_t n, int64_t k) { return align256(size_t(n) * size_t(k) / 2); }
inline size_t scale_plane_bytes(int64_t n, int64_t k) { return align256(size_t(n) * size_t(k / 32) * 2); }

// Multi-vector GEMV on the matrix cores (q4_multi.hip), for 2 <= m <= 8:
// dynamic LDS it needs, and the launch (arguments already validated).
size_t multi_mfma_lds_bytes(int m, int64_t k);
int multi_mfma_launch(const uint8_t* nib, const uint16_t* scl, int64_t n, int64_t k, const uint16_t* x, int m,
                      float* y, hipStream_t stream);

inline int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(Q4DEC_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return Q4DEC_OK;
}

// ------------------------------------------------ launch-contract checks
// Built with -DQ4DEC_DEBUG=1, each kernel first checks, uniformly across its
// workgroup, that the launch fits what its code assumes: the activation
// staging holds every block, a plan marked full has no ragged lane, the grid
// covers every row, tile and K slice. A failed check sets its bit in the
// translation unit's debug word and the workgroup returns before it touches
// memory; q4dec_debug_status() collects and clears the words of every unit.
// Release builds compile the checks away.
#ifndef Q4DEC_DEBUG
#define Q4DEC_DEBUG 0
#endif

// One bit per check; each translation unit owns its own bits.
enum DebugBit : int {
  kDbgGemvStaging = 0,   // q4_rows_kernel: B > staged blocks
  kDbgGemvFull = 1,      // q4_rows_kernel: full plan with ragged lanes
  kDbgGemvRows = 2,      // q4_rows_kernel: grid * waves * ipw < row groups
  kDbgRowqStaging = 3,   // rowq_rows_kernel: blocks or chunks beyond the lanes
  kDbgRowqFull = 4,      // rowq_rows_kernel: full plan with ragged lanes
  kDbgRowqRows = 5,      // rowq_rows_kernel: grid does not cover the rows
  kDbgMultiStaging = 6,  // q4_multi_kernel: lane segments do not cover k
  kDbgMultiRows = 7,     // q4_multi_kernel: grid does not cover the rows
  kDbgGemmChunks = 9,    // q4_gemm_chunk_kernel: k or the slice not whole chunks
  kDbgGemmSlices = 10,   // q4_gemm kernels: slices miss or overrun K
  kDbgGemmTiles = 11,    // q4_gemm kernels: tiles do not cover the rows
  kDbgGatherGrid = 15,   // ple / rowq gather: grid does not cover the ids
  kDbgPackGrid = 17,     // q4_pack_kernel: grid does not cover the blocks
  kDbgQuantGrid = 18,    // q4_quantize_kernel: grid does not cover the blocks
  kDbgSelfTest = 31,     // q4dec_debug_selftest: always fails
};

namespace {
// this translation unit's debug word (device memory, zero at load)
__device__ uint32_t g_debug_word;
// reads and clears this unit's word (host; synchronous)
inline uint32_t debug_take_local() {
  uint32_t w = 0;
  const uint32_t z = 0;
  if (hipMemcpyFromSymbol(&w, HIP_SYMBOL(g_debug_word), sizeof(w), 0, hipMemcpyDeviceToHost) != hipSuccess) return 0;
  (void)hipMemcpyToSymbol(HIP_SYMBOL(g_debug_word), &z, sizeof(z), 0, hipMemcpyHostToDevice);
  return w;
}
}  // namespace

// every unit's reader (defined by Q4DEC_DEBUG_READER in each .hip file)
uint32_t debug_take_q4_gemv();
uint32_t debug_take_q4_multi();
uint32_t debug_take_q4_chain();
uint32_t debug_take_q4_gemm();
uint32_t debug_take_rowq_gemv();
uint32_t debug_take_ple_gather();
uint32_t debug_take_q4_pack();
uint32_t debug_take_q4_quantize();
uint32_t debug_take_api();
#define Q4DEC_DEBUG_READER(unit) \
  uint32_t debug_take_##unit() { return debug_take_local(); }

// In a kernel, before any barrier or memory access: a uniform condition.
#define Q4_DCHECK(cond, bit)                                                            \
  do {                                                                                  \
    if (Q4DEC_DEBUG && !(cond)) {                                                       \
      if (threadIdx.x == 0) atomicOr(&::q4dec::g_debug_word, 1u << int(::q4dec::bit)); \
      return;                                                                           \
    }                                                                                   \
  } while (0)

// ------------------------------------------------------------- device side
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Packed layout of one 32-weight block (16 bytes, four dwords). Dword q holds
// the codes of k = 8q .. 8q+7 as unsigned nibbles n = c + 8:
//   byte0 = n[8q+0] | n[8q+2] << 4      byte1 = n[8q+4] | n[8q+6] << 4
//   byte2 = n[8q+1] | n[8q+3] << 4      byte3 = n[8q+5] | n[8q+7] << 4
// so masking a dword with 0x000F000F yields the pair (k=8q, 8q+1) in the low
// nibble of each 16-bit half, 0x00F000F0 the pair (8q+2, 8q+3), and the same
// two masks on dword >> 8 the pairs (8q+4, 8q+5) and (8q+6, 8q+7).
__device__ __forceinline__ uint32_t pack_dword(const int8_t* c8) {
  auto nb = [&](int i) -> uint32_t { return uint32_t(c8[i] + 8) & 15u; };
  uint32_t b0 = nb(0) | (nb(2) << 4);
  uint32_t b1 = nb(4) | (nb(6) << 4);
  uint32_t b2 = nb(1) | (nb(3) << 4);
  uint32_t b3 = nb(5) | (nb(7) << 4);
  return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t orv) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(mask), "v"(orv));
  return r;
}

// Exact fp16 code pairs of one dword. 0x6400 is fp16 1024 with unit spacing,
// so OR-ing a nibble n into bits 0-3 gives 1024 + n and into bits 4-7 gives
// 1024 + 16 n; subtracting 1032, or scaling by 1/16 and subtracting 72,
// leaves c = n - 8 exactly.
struct CodePairs { half2_t p[4]; };
__device__ __forceinline__ CodePairs unpack_dword(uint32_t w, uint32_t m_lo, uint32_t m_hi, uint32_t magic) {
  const half2_t off_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2_t sc_hi = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
  uint32_t w8 = w >> 8;
  CodePairs r;
  r.p[0] = __builtin_bit_cast(half2_t, and_or(w, m_lo, magic)) + off_lo;
  r.p[1] = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(w, m_hi, magic)), sc_hi, off_hi);
  r.p[2] = __builtin_bit_cast(half2_t, and_or(w8, m_lo, magic)) + off_lo;
  r.p[3] = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(w8, m_hi, magic)), sc_hi, off_hi);
  return r;
}

// sum_{j<32} c_j * x'_j for one block, with x' as 16 fp16 pairs (k order).
__device__ __forceinline__ float block_dot(uint4 q, const uint32_t* xh, uint32_t m_lo, uint32_t m_hi, uint32_t magic) {
  float acc = 0.0f;
  const uint32_t ws[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    CodePairs cp = unpack_dword(ws[i], m_lo, m_hi, magic);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_fdot2(cp.p[j], __builtin_bit_cast(half2_t, xh[4 * i + j]), acc, false);
  }
  return acc;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) {
  return __builtin_bit_cast(float, h16 << 16);
}

// Activation staging scales a group of bf16 values (a block, a vector or a
// token) by the power of two that puts the group's largest exponent at 2^14
// and stores fp16. A nonzero value with exponent field E keeps all its bits
// only if emax - E <= kMaxSpan (its last significand bit, 2^(E - emax + 7)
// after scaling, must not fall below fp16's smallest step 2^-24). A group
// with a wider span is computed on the exact path instead.
constexpr int kMaxSpan = 31;

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Exponent range of 2N bf16 values (N words): emax = largest exponent field
// (at least 1), emin = smallest exponent field among the nonzero values
// (subnormals count as 1, whose last significand bit they share; 255 when
// all are zero, so a zero never lowers the minimum). Computed on the
// magnitude bits (exponent above mantissa, so they order like the values'
// magnitudes) with packed 16-bit integer ops: the largest magnitude has the
// largest exponent, and subtracting 1 with wrap-around sends a zero
// magnitude to 0xFFFF, out of the minimum.
template <int N>
__device__ __forceinline__ void block_exp_range(const uint32_t (&w)[N], uint32_t& emax, uint32_t& emin) {
  u16x2 mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
  const u16x2 one = {1, 1};
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const u16x2 z = __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu);
    mx = __builtin_elementwise_max(mx, z);
    mn = __builtin_elementwise_min(mn, u16x2(z - one));
  }
  const uint32_t big = max(uint32_t(mx[0]), uint32_t(mx[1]));
  const uint32_t small = min(uint32_t(mn[0]), uint32_t(mn[1]));  // 0xFFFF: no nonzero value
  emax = max(big >> 7, 1u);
  emin = small == 0xFFFFu ? 255u : max((small + 1u) >> 7, 1u);
}

// sum_{j<32} c_j * x_j for one block with x as stored (bf16 [32], 16-byte
// aligned), in fp32: every product is exact, only the sum rounds.
__device__ __forceinline__ float block_dot_exact(uint4 q, const uint4* __restrict__ xb, uint32_t m_lo,
                                                 uint32_t m_hi, uint32_t magic) {
  float acc = 0.0f;
  const uint32_t ws[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 xv = xb[i];  // bf16 k = 8i .. 8i+7, two per word
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    const CodePairs cp = unpack_dword(ws[i], m_lo, m_hi, magic);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf(float(cp.p[j][0]), bf16_to_f32(xw[j] & 0xFFFFu), acc);
      acc = fmaf(float(cp.p[j][1]), bf16_to_f32(xw[j] >> 16), acc);
    }
  }
  return acc;
}

// ---- cross-lane sums ------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum over aligned groups of L lanes (L in 4..64); every lane of the group
// receives the total.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (L >= 8) v += dpp_f<0x141>(v);   // row_half_mirror
  if constexpr (L >= 16) v += dpp_f<0x140>(v);  // row_mirror
  if constexpr (L >= 32) v += __shfl_xor(v, 16);
  if constexpr (L >= 64) v += __shfl_xor(v, 32);
  return v;
}

// (value desc, index asc) comparator for the argmax; NaN never wins.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Best (value, row) of the wave into every lane.
__device__ __forceinline__ void wave_best(float& best, int& bidx) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(best, off);
    const int oi = __shfl_xor(bidx, off);
    if (better(ov, oi, best, bidx)) {
      best = ov;
      bidx = oi;
    }
  }
}

// tanh-form GELU in fp32: 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))).
__device__ __forceinline__ float gelu_tanh(float g) {
  const float k0 = 0.7978845608028654f, k1 = 0.044715f;
  return 0.5f * g * (1.0f + tanhf(k0 * (g + k1 * g * g * g)));
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Stage x (bf16 [32 B]) into LDS as block-scaled fp16 pairs (block b at
// xs[16 b], quarter i in slot i ^ (b & 3), 2^E in xf[b]); E puts the block's
// largest magnitude in [2^14, 2^15), so every bf16 value keeps its 8-bit
// significand unless it lies below 2^-31 times that maximum. Four lanes share a
// 32-wide block, one 16-byte quarter each, and agree on the block's largest
// exponent with two xor shuffles. The loads are issued first (stage_x_load,
// NXL quarters per thread) and converted later (stage_x_store): vector memory
// counters retire in order, so loads issued before the weight loads can be
// waited for while the weights are still in flight.
template <int NT, int NXL>
__device__ __forceinline__ void stage_x_load(const uint16_t* __restrict__ x, int B, uint4 (&v)[NXL]) {
  const uint4* src = reinterpret_cast<const uint4*>(x);
  // unconditional (a clamped index past the end), so the wait for these
  // loads can be counted past the weight loads that follow
#pragma unroll
  for (int u = 0; u < NXL; ++u) v[u] = src[min(int(threadIdx.x) + u * NT, 4 * B - 1)];
}

// Returns true if one of this thread's blocks is "wide": a nonzero value lies
// more than 31 binades below the block's largest exponent, so its scaled fp16
// copy would lose significand bits (or flush to zero). The kernel then reads
// x as stored instead (exact path).
template <int NT, int NXL>
__device__ __forceinline__ bool stage_x_store(const uint4 (&v)[NXL], int B, uint32_t* __restrict__ xs,
                                              float* __restrict__ xf) {
  bool wide = false;
  // every lane converts (a clamped duplicate past the end, not stored): a
  // conditional use would let the compiler sink the load past the weights
#pragma unroll
  for (int u = 0; u < NXL; ++u) {
    const int qi = int(threadIdx.x) + u * NT;
    {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      uint32_t emax, emin;
      block_exp_range(w, emax, emin);
      emax = max(emax, uint32_t(__shfl_xor(int(emax), 1)));
      emax = max(emax, uint32_t(__shfl_xor(int(emax), 2)));
      emin = min(emin, uint32_t(__shfl_xor(int(emin), 1)));
      emin = min(emin, uint32_t(__shfl_xor(int(emin), 2)));
      // the span test right here (pinned by the empty asm), so the exponent
      // fields die before the conversion
      int w_u = int(emax) - int(emin) > kMaxSpan;
      asm volatile("" : "+v"(w_u));
      wide |= w_u != 0;
      const int e = int(emax) - 127 - 14;
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half2_t h = {(_Float16)ldexpf(bf16_to_f32(w[i] & 0xFFFFu), -e),
                           (_Float16)ldexpf(bf16_to_f32(w[i] >> 16), -e)};
        o[i] = __builtin_bit_cast(uint32_t, h);
      }
      const int b = qi >> 2, q = qi & 3;
      if (qi < 4 * B) {
        reinterpret_cast<uint4*>(xs + 16 * b)[q ^ (b & 3)] = make_uint4(o[0], o[1], o[2], o[3]);
        if (q == 0) xf[b] = ldexpf(1.0f, e);
      }
    }
  }
  return wide;
}

// Per-vector argmax over per-workgroup (value bits, row) partials: vector v's
// entries sit at partials[w * stride + v] for w < g. One workgroup per
// vector writes idx_out[v] and cap * tanh(best / cap) (the raw best for
// cap <= 0) to val_out[v]; idx -1 and NaN when no value compares.
void reduce_argmax_partials(const uint2* partials, int g, int stride, int nvec, float cap, int32_t* idx_out,
                            float* val_out, hipStream_t st);


}  // namespace q4dec
