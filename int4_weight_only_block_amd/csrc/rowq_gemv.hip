// rowq_gemv: per-row symmetric INT8 / INT4 / INT2 matvec on the dense packing
// of the mixed-bit recipe ("Gemma-4 E2B mobile mixed-bit QAT weights" knowledge page:
// decode recipe with per-channel symmetric linear weights, all zero points 0,
// bytes = elements * bits / 8; packing convention: INT2 holds 4 codes per byte
// with the first code in bits [1:0], two's complement, INT4 likewise with
// nibbles, low nibble first; the INT8 PLE gate / projection matrices are
// signed bytes; receiving-end design: the integer-weighted sum is scaled by
// the row's scale once).
//
// The weight stream follows q4_gemv: lane t of a row group owns chunks t,
// t + LPR, ... of its row (16 bytes: 64 INT2 or 32 INT4 codes; 32 bytes: 32
// INT8 codes, so every chunk holds whole 32-wide blocks) and walks down
// the rows with one row group of loads in flight. Because a lane meets the
// same chunks on every row, its share of x lives in registers: the workgroup
// converts x once into LDS, each lane copies its blocks out, and the row loop
// touches no LDS.
//
// Codes are not converted to fp16 on their own. Each field is read at bit
// offset s of an fp16 whose exponent is that of 1024 (OR with 0x6400), so the
// half holds 1024 + 2^s * u exactly, u = code + 2 (INT2), code + 8 (INT4) or
// code + 128 (INT8, s = 0) after an XOR of the packed word. Subtracting the
// exact fp16 constant 1024 + 2^s * offset in the same packed add leaves
// 2^s * code exactly (dotc below), and the matching activation is stored
// pre-multiplied by 2^-s, so each product in the dot is code * x exactly and
// only the fp32 accumulation rounds.
//
// Staging scales each 32-wide block by one power of two. A block whose
// nonzero values span more binades than that copy holds exactly (31 minus
// the largest field offset) is "wide": it is staged as stored (bf16) and
// enters the packed fp16 dot as zeros, and the lanes that hold it add its
// sum separately, each code decoded as a signed integer and multiplied by x
// in fp32, where every product is exact. A row step whose lanes hold no wide
// block skips that branch.
#include <limits.h>
#include <math.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "q4dec_internal.h"

namespace q4dec {
Q4DEC_DEBUG_READER(rowq_gemv)
namespace {

constexpr int kRWaves = 4;
constexpr int kRThreads = 64 * kRWaves;

// field isolation in plain C: the compiler forms v_and_or_b32 / v_bitop3_b32
// itself and so knows the hazards between it and the dot product
__device__ __forceinline__ uint32_t field(uint32_t a, uint32_t mask, uint32_t magic) { return (a & mask) | magic; }

// Codes enter the dot product exactly: a field read at bit offset S of each
// half is the fp16 value 1024 + 2^S * u with u = code + OFF, so subtracting
// the exact constant 1024 + OFF * 2^S leaves 2^S * code (|2^S code| <= 1024,
// exact); the activation was staged pre-multiplied by 2^-S. (Leaving the
// constant in and removing its sum per block saves this add, but then the
// error grows with sum |x| instead of sum |code * x|, which breaks the GEMV
// bound on rows whose codes are mostly zero.)
template <int S, int OFF>
__device__ __forceinline__ float dotc(uint32_t fld, uint32_t b, float c) {
  constexpr _Float16 k = _Float16(-(1024 + (OFF << S)));
  const half2_t kk = {k, k};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, fld) + kk, __builtin_bit_cast(half2_t, b), c, false);
}

// One dword of codes against its activation pairs. Pair f of dword d of a
// 32-code block holds block elements elem(d, f) and elem(d, f) + kSecond,
// matching the low-half and high-half field that one AND-OR isolates.
template <int BITS>
struct Fields;

template <>
struct Fields<2> {
  static constexpr int kPairs = 8;   // pairs per dword
  static constexpr int kDwords = 2;  // dwords per block
  static constexpr int kSecond = 8;
  static constexpr int kOffset = 2;  // u = code + 2
  __device__ static constexpr int elem(int d, int f) { return 16 * d + f; }
  // bit offset (within each half) at which field f is read: fields 0-2 from
  // w << 4, fields 3-4 from w, fields 5-7 from w >> 6, so every field lands
  // at bits 4-9 and two shifts serve all eight
  __device__ static constexpr int shift(int f) { return f == 0 || f == 5 ? 4 : (f == 1 || f == 3 || f == 6) ? 6 : 8; }
  __device__ __forceinline__ static float dot(uint32_t w, const uint32_t* xp, float p, uint32_t magic) {
    w ^= 0xAAAAAAAAu;
    const uint32_t a = w << 4, c = w >> 6;
    p = dotc<4, kOffset>(field(a, 0x00300030u, magic), xp[0], p);
    p = dotc<6, kOffset>(field(a, 0x00C000C0u, magic), xp[1], p);
    p = dotc<8, kOffset>(field(a, 0x03000300u, magic), xp[2], p);
    p = dotc<6, kOffset>(field(w, 0x00C000C0u, magic), xp[3], p);
    p = dotc<8, kOffset>(field(w, 0x03000300u, magic), xp[4], p);
    p = dotc<4, kOffset>(field(c, 0x00300030u, magic), xp[5], p);
    p = dotc<6, kOffset>(field(c, 0x00C000C0u, magic), xp[6], p);
    p = dotc<8, kOffset>(field(c, 0x03000300u, magic), xp[7], p);
    return p;
  }
};

template <>
struct Fields<4> {
  static constexpr int kPairs = 4;
  static constexpr int kDwords = 4;
  static constexpr int kSecond = 4;
  static constexpr int kOffset = 8;  // u = code + 8
  __device__ static constexpr int elem(int d, int f) { return 8 * d + f; }
  // every nibble is moved to bits 4-7 of each half
  __device__ static constexpr int shift(int) { return 4; }
  __device__ __forceinline__ static float dot(uint32_t w, const uint32_t* xp, float p, uint32_t magic) {
    w ^= 0x88888888u;
    const uint32_t s[4] = {w << 4, w, w >> 4, w >> 8};  // nibbles 0 1 2 3
#pragma unroll
    for (int f = 0; f < 4; ++f) p = dotc<4, kOffset>(field(s[f], 0x00F000F0u, magic), xp[f], p);
    return p;
  }
};

template <>
struct Fields<8> {
  static constexpr int kPairs = 2;
  static constexpr int kDwords = 8;
  static constexpr int kSecond = 2;
  static constexpr int kOffset = 128;  // u = code + 128
  __device__ static constexpr int elem(int d, int f) { return 4 * d + f; }
  // bytes 0 and 2 of a word are read in place, bytes 1 and 3 after w >> 8
  __device__ static constexpr int shift(int) { return 0; }
  __device__ __forceinline__ static float dot(uint32_t w, const uint32_t* xp, float p, uint32_t magic) {
    w ^= 0x80808080u;
    p = dotc<0, kOffset>(field(w, 0x00FF00FFu, magic), xp[0], p);
    p = dotc<0, kOffset>(field(w >> 8, 0x00FF00FFu, magic), xp[1], p);
    return p;
  }
};

// 16-byte loads per chunk: one for INT2 / INT4, two for INT8
template <int BITS>
constexpr int kChunkLoads = BITS == 8 ? 2 : 1;

// Stage block b of x: its 16 activation pairs, element e scaled by 2^-(E + s)
// where 2^E brings the block's largest bf16 exponent to 2^14 (as in q4_gemv)
// and s is the shift of the field the element meets; quarter i of the 64
// bytes goes to slot i ^ (sw & 3); xe receives 2^E. The codes met in the dot
// product are exact fp16 values 2^s * code, so each product is exact and
// only the fp32 accumulation rounds.
// Largest field shift s of a format: the staged values carry an extra 2^-s,
// which narrows the span of binades a block can hold exactly.
template <int BITS>
constexpr int kMaxShift = BITS == 2 ? 8 : BITS == 4 ? 4 : 0;

// A block is "wide" when a nonzero value lies more than kMaxSpan - kMaxShift
// binades below its largest exponent, so its scaled fp16 copy would lose
// bits. A wide block is stored as it came (bf16 pairs in element order) and
// xe receives -1, which marks it.
template <int BITS>
__device__ __forceinline__ void stage_block(const uint4 (&src)[4], uint32_t* __restrict__ dst, int sw,
                                            float* __restrict__ xe, bool store) {
  using F = Fields<BITS>;
  uint32_t raw[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    raw[4 * i] = v.x; raw[4 * i + 1] = v.y; raw[4 * i + 2] = v.z; raw[4 * i + 3] = v.w;
  }
  auto elem = [&](int e) -> float {
    const uint32_t v = raw[e >> 1];
    return __builtin_bit_cast(float, (e & 1) ? (v & 0xFFFF0000u) : (v << 16));
  };
  uint32_t emax, emin;
  block_exp_range(raw, emax, emin);
  // the span test right here (pinned by the empty asm), so the 32 exponent
  // fields die before the conversion instead of living across it
  int wide = int(emax) - int(emin) > kMaxSpan - kMaxShift<BITS>;
  asm volatile("" : "+v"(wide));
  const int e = int(emax) - 127 - 14;
  uint32_t out[16];
#pragma unroll
  for (int d = 0; d < F::kDwords; ++d) {
#pragma unroll
    for (int f = 0; f < F::kPairs; ++f) {
      const int e0 = F::elem(d, f), s = F::shift(f);
      const half2_t h = {(_Float16)ldexpf(elem(e0), -e - s), (_Float16)ldexpf(elem(e0 + F::kSecond), -e - s)};
      out[d * F::kPairs + f] = __builtin_bit_cast(uint32_t, h);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i] = wide ? raw[i] : out[i];
  if (store) {
    uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
    for (int i = 0; i < 4; ++i) d4[i ^ (sw & 3)] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    *xe = wide ? -1.0f : ldexpf(1.0f, e);
  }
}

enum RowqMode { kRowqGemv = 0, kRowqGelu = 1, kRowqHead = 2 };

// Most workgroups (partials) of one head launch.
constexpr int kRowqMaxPartials = 8192;

// Best (value, row) of the wave into every lane.
__device__ __forceinline__ void rq_wave_best(float& best, int& bidx) {
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

// fused [gate; up] epilogue: tanh-form GELU in fp32 and the bf16 rounding of
// the product (same definitions as the q4_0 fused kernel)
__device__ __forceinline__ float rq_gelu_tanh(float g) {
  const float k0 = 0.7978845608028654f, k1 = 0.044715f;
  return 0.5f * g * (1.0f + tanhf(k0 * (g + k1 * g * g * g)));
}
__device__ __forceinline__ uint16_t rq_bf16_rne(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// DEPTH row groups of loads in flight per wave (1 or 2). MODE kRowqGemv
// writes y[row] (fp32); kRowqGelu reads the n rows as [gate; up] and writes
// bf16(gelu(g_j) * u_j) for j < n / 2: lane groups r < RPW / 2 take gate
// rows, the others the up rows of the same outputs, so each pair of sums is
// 32 lanes apart after the row reduction; kRowqHead keeps the best (scaled
// sum, row) of the workgroup's rows and writes it to out[blockIdx.x].
template <int BITS, int LPR, int CPL, int DEPTH, int MODE, bool FULL>
__global__ __launch_bounds__(kRThreads) void rowq_rows_kernel(const uint8_t* __restrict__ w,
                                                              const float* __restrict__ row_scale,
                                                              const uint16_t* __restrict__ x, int n, int k, int ipw,
                                                              void* __restrict__ out) {
  using F = Fields<BITS>;
  constexpr int CH = kChunkLoads<BITS>;
  constexpr int RPW = 64 / LPR;
  static_assert(MODE != kRowqGelu || RPW >= 2, "the gate/up pairing needs two rows per wave step");
  constexpr int UPW = MODE == kRowqGelu ? RPW / 2 : RPW;  // outputs per wave step
  constexpr int BPC = BITS == 2 ? 2 : 1;  // activation blocks per 16-byte chunk
  constexpr int NB = CPL * BPC;           // blocks held by one lane
  constexpr int MAXB = LPR * NB;
  __shared__ uint32_t xs[MAXB * 16];
  __shared__ float xc[MAXB];
  const int U = (k * BITS) / (128 * CH);  // chunks per row
  const int B = k >> 5;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane % LPR;
  const int r = lane / LPR;
  const int units = MODE == kRowqGelu ? n / 2 : n;
  const int RG = (units + UPW - 1) / UPW;
  const int rg_base = blockIdx.x * kRWaves * ipw + wave;
  const size_t row_bytes = size_t(U) * 16 * CH;
  const int iters = rg_base < RG ? min(ipw, (RG - rg_base + kRWaves - 1) / kRWaves) : 0;
  Q4_DCHECK(B <= MAXB && U <= LPR * CPL, kDbgRowqStaging);
  Q4_DCHECK(!FULL || U == LPR * CPL, kDbgRowqFull);
  Q4_DCHECK(int64_t(gridDim.x) * kRWaves * ipw >= RG, kDbgRowqRows);
  auto row_of = [&](int i) {
    if constexpr (MODE == kRowqGelu) {
      const int v = (rg_base + i * kRWaves) * UPW + (r % UPW);
      return (v < units ? v : units - 1) + (r / UPW) * units;
    } else {
      const int row = (rg_base + i * kRWaves) * RPW + r;
      return row < n ? row : n - 1;
    }
  };

  // a row group's weights and its per-row scale are loaded together; the
  // scale is then at hand when the sum is ready, instead of a load issued
  // behind the next group's weights and waited for with them
  uint4 qa[CPL][CH], qb[CPL][CH];
  float sa = 0.0f, sb = 0.0f;
  auto load = [&](uint4(&q)[CPL][CH], float& sc, int row) {
    const u32x4* p = reinterpret_cast<const u32x4*>(w + size_t(row) * row_bytes);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = j * LPR + t;
      if (FULL || c < U) {
#pragma unroll
        for (int h = 0; h < CH; ++h) {
          const u32x4 v = __builtin_nontemporal_load(p + c * CH + h);
          q[j][h] = make_uint4(v.x, v.y, v.z, v.w);
        }
      }
    }
    sc = row_scale[row];
  };
  // Activation loads first (vector memory counters retire in order, so the
  // staging below waits only for these), then the first row groups' weights.
  // Loads and conversions are unconditional, on clamped indices, and only the
  // stores are guarded, so the compiler cannot sink a load past the weights;
  // a wave with no rows loads the clamped last row and never uses it.
  constexpr int NXB = (MAXB + kRThreads - 1) / kRThreads;  // x blocks per thread
  u32x4 xr[NXB][4];
#pragma unroll
  for (int u = 0; u < NXB; ++u) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x) + 4 * min(int(threadIdx.x) + u * kRThreads, B - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[u][i] = src[i];
  }
  load(qa, sa, row_of(0));
  if (DEPTH == 2) load(qb, sb, row_of(1));
  // an unconditional use of the activation registers here keeps their loads
  // ahead of the weight loads (the conversion feeds only guarded stores, which
  // would otherwise let the compiler move the loads into the guarded block)
#pragma unroll
  for (int u = 0; u < NXB; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(xr[u][i]));

#pragma unroll
  for (int u = 0; u < NXB; ++u) {
    const int b = int(threadIdx.x) + u * kRThreads, bc = min(b, B - 1);
    const uint4 v4[4] = {make_uint4(xr[u][0].x, xr[u][0].y, xr[u][0].z, xr[u][0].w),
                         make_uint4(xr[u][1].x, xr[u][1].y, xr[u][1].z, xr[u][1].w),
                         make_uint4(xr[u][2].x, xr[u][2].y, xr[u][2].z, xr[u][2].w),
                         make_uint4(xr[u][3].x, xr[u][3].y, xr[u][3].z, xr[u][3].w)};
    stage_block<BITS>(v4, xs + 16 * bc, bc / BPC, xc + bc, b < B);
  }
  // LDS writes done and visible; the weight loads above stay in flight
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // The lane's activation blocks, copied out of LDS into registers. A wide
  // block l sets bit l of wbits: its packed dot (bf16 bits read as fp16
  // pairs, meaningless) is dropped, and dot_wide adds its sum from the bf16
  // copy in LDS instead.
  uint32_t xp[NB][16];
  float xf[NB];
  uint32_t wbits = 0;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = j * LPR + t;
    if (FULL || c < U) {
#pragma unroll
      for (int bb = 0; bb < BPC; ++bb) {
        const int b = c * BPC + bb, l = j * BPC + bb;
        const uint4* s4 = reinterpret_cast<const uint4*>(xs + 16 * b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 q4 = s4[i ^ (c & 3)];
          xp[l][4 * i] = q4.x; xp[l][4 * i + 1] = q4.y; xp[l][4 * i + 2] = q4.z; xp[l][4 * i + 3] = q4.w;
        }
        xf[l] = xc[b];
        wbits |= uint32_t(xf[l] < 0.0f) << l;
      }
    }
  }

  uint32_t magic;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

  // sum_e code_e * x_e over wide block j * BPC + bb of the lane: kDwords
  // dwords of codes (first code in the lowest bits, two's complement) against
  // x as stored (bf16 pairs in element order, read back from LDS); each code
  // is sign-extended by a left and an arithmetic right shift (the sbfe
  // builtin's result was converted to float as if unsigned), every product
  // is exact in fp32 and only the sum rounds.
  auto dot_wide = [&](const uint32_t* wd, int j, int bb) __attribute__((always_inline)) -> float {
    constexpr int PER = 32 / BITS;  // codes per dword
    // the LDS addresses are formed here from the lane index: hoisted out of
    // the row loop as invariants, the four per block would each hold a
    // register
    int tt = t;
    asm volatile("" : "+v"(tt));
    const int sw = j * LPR + tt, b = sw * BPC + bb;
    const uint4* s4 = reinterpret_cast<const uint4*>(xs + 16 * b);
    float p = 0.0f;
    // one 16-byte quarter (8 elements) at a time, so few registers are live
    // beside the row loop's own
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = s4[i ^ (sw & 3)];
      const uint32_t xw[4] = {v.x, v.y, v.z, v.w};
      // the quarter's code words, tied by an empty asm to its x load: left
      // free, the compiler decodes all 32 codes ahead of the first load and
      // holds them at once
      constexpr int NW = (8 + PER - 1) / PER;  // code words per quarter
      uint32_t cw[NW];
#pragma unroll
      for (int m = 0; m < NW; ++m) {
        cw[m] = wd[(8 * i) / PER + m];
        asm volatile("" : "+v"(cw[m]) : "v"(v.x));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = 8 * i + u;
        const int code = int(cw[u / PER] << (32 - BITS - (e % PER) * BITS)) >> (32 - BITS);
        const uint32_t xv = xw[u >> 1];
        p = fmaf(float(code), __builtin_bit_cast(float, (u & 1) ? (xv & 0xFFFF0000u) : (xv << 16)), p);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return p;
  };

  auto dot = [&](uint4(&q)[CPL][CH], float& sc, bool refill, int row_next) -> float {
    const u32x4* pn = reinterpret_cast<const u32x4*>(w + size_t(row_next) * row_bytes);
    if (refill) sc = row_scale[row_next];
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = j * LPR + t;
      if (FULL || c < U) {
        uint32_t wd[4 * CH];
#pragma unroll
        for (int h = 0; h < CH; ++h) {
          wd[4 * h] = q[j][h].x; wd[4 * h + 1] = q[j][h].y; wd[4 * h + 2] = q[j][h].z; wd[4 * h + 3] = q[j][h].w;
        }
#pragma unroll
        for (int bb = 0; bb < BPC; ++bb) {
          const int l = j * BPC + bb;
          float p = 0.0f;
#pragma unroll
          for (int d = 0; d < F::kDwords; ++d) p = F::dot(wd[bb * F::kDwords + d], &xp[l][d * F::kPairs], p, magic);
          const float a2 = fmaf(p, xf[l], acc);
          acc = (wbits >> l) & 1u ? acc : a2;
        }
        // the chunk's wide blocks (lane-divergent, skipped by every wave
        // whose lanes hold none; marked unlikely, so the code sits outside
        // the loop)
        if (__builtin_expect(((wbits >> (j * BPC)) & ((1u << BPC) - 1u)) != 0, 0)) {
#pragma unroll
          for (int bb = 0; bb < BPC; ++bb)
            if ((wbits >> (j * BPC + bb)) & 1u) acc += dot_wide(&wd[bb * F::kDwords], j, bb);
        }
        // keep one chunk's work together so its temporaries die before the
        // next chunk's begin
        asm volatile("" : "+v"(acc));
        __builtin_amdgcn_sched_barrier(0);
        if (refill) {
#pragma unroll
          for (int h = 0; h < CH; ++h) {
            const u32x4 v = __builtin_nontemporal_load(pn + c * CH + h);
            q[j][h] = make_uint4(v.x, v.y, v.z, v.w);
          }
        }
      }
    }
    return acc;
  };
  float best = -INFINITY;
  int bidx = INT_MAX;
  auto emit = [&](int i, float acc, float sc) {
    acc = group_sum<LPR>(acc);
    if constexpr (MODE == kRowqHead) {
      const int row = (rg_base + i * kRWaves) * RPW + r;
      if (row < n) {
        const float v = acc * sc;
        if (better(v, row, best, bidx)) {
          best = v;
          bidx = row;
        }
      }
    } else if constexpr (MODE == kRowqGelu) {
      const float v = acc * sc;
      const float up = __shfl_xor(v, 32);  // the up row's scaled sum
      const int j = (rg_base + i * kRWaves) * UPW + r;
      if (t == 0 && r < UPW && j < units) static_cast<uint16_t*>(out)[j] = rq_bf16_rne(rq_gelu_tanh(v) * up);
    } else {
      const int row = (rg_base + i * kRWaves) * RPW + r;
      if (t == 0 && row < n) static_cast<float*>(out)[row] = acc * sc;
    }
  };
  // row group i: its scale is read before dot() may refill it for a later group
  auto step = [&](int i, uint4(&q)[CPL][CH], float& sc, bool refill, int row_next) {
    const float s_i = sc;
    const float acc = dot(q, sc, refill, row_next);
    emit(i, acc, s_i);
  };
  if constexpr (DEPTH == 1) {
    for (int i = 0; i + 1 < iters; ++i) step(i, qa, sa, true, row_of(i + 1));
    if (iters > 0) step(iters - 1, qa, sa, false, 0);
  } else {
    // qa holds row group i, qb row group i + 1; each refills two ahead
    int i = 0;
    for (; i + 3 < iters; i += 2) {
      step(i, qa, sa, true, row_of(i + 2));
      step(i + 1, qb, sb, true, row_of(i + 3));
    }
    if (i + 2 < iters) {  // three left
      step(i, qa, sa, true, row_of(i + 2));
      step(i + 1, qb, sb, false, 0);
      step(i + 2, qa, sa, false, 0);
    } else {
      if (i < iters) step(i, qa, sa, false, 0);
      if (i + 1 < iters) step(i + 1, qb, sb, false, 0);
    }
  }
  if constexpr (MODE == kRowqHead) {
    rq_wave_best(best, bidx);
    __shared__ float sv[kRWaves];
    __shared__ int si[kRWaves];
    if (lane == 0) {
      sv[wave] = best;
      si[wave] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int v = 1; v < kRWaves; ++v)
        if (better(sv[v], si[v], best, bidx)) {
          best = sv[v];
          bidx = si[v];
        }
      static_cast<uint2*>(out)[blockIdx.x] = make_uint2(__builtin_bit_cast(uint32_t, best), uint32_t(bidx));
    }
  }
}

struct RPlan {
  int lpr, cpl, rpw, rg, ipw, grid;
  const void* fn;
};

// (lanes per row, chunks per lane) pairs the plan below can ask for; the
// GELU mode needs two rows per wave step, so at most 32 lanes per row
template <int BITS, int MODE, bool FULL>
const void* pick_rowq(int lpr, int cpl) {
#define RQ_CASE(L, C)                                                                                  \
  if (lpr == L && cpl == C) {                                                                          \
    if constexpr (MODE != kRowqGelu || L <= 32)                                                        \
      return reinterpret_cast<const void*>(&rowq_rows_kernel<BITS, L, C, 1, MODE, FULL>);              \
    else                                                                                               \
      return nullptr;                                                                                  \
  }
  if constexpr (BITS == 2) {
    RQ_CASE(8, 1) RQ_CASE(8, 2) RQ_CASE(8, 3)
    RQ_CASE(16, 1) RQ_CASE(16, 2) RQ_CASE(16, 3)
    RQ_CASE(32, 1) RQ_CASE(32, 2) RQ_CASE(32, 3)
    RQ_CASE(64, 1) RQ_CASE(64, 2) RQ_CASE(64, 3) RQ_CASE(64, 4)
  } else {  // INT4 and INT8: one 32-wide block per chunk
    RQ_CASE(8, 1) RQ_CASE(8, 2) RQ_CASE(8, 3) RQ_CASE(8, 4) RQ_CASE(8, 5) RQ_CASE(8, 6)
    RQ_CASE(16, 1) RQ_CASE(16, 2) RQ_CASE(16, 3) RQ_CASE(16, 4) RQ_CASE(16, 5) RQ_CASE(16, 6)
    RQ_CASE(32, 1) RQ_CASE(32, 2) RQ_CASE(32, 3) RQ_CASE(32, 4) RQ_CASE(32, 5) RQ_CASE(32, 6)
    RQ_CASE(64, 1) RQ_CASE(64, 2) RQ_CASE(64, 3) RQ_CASE(64, 4) RQ_CASE(64, 5) RQ_CASE(64, 6) RQ_CASE(64, 7)
    RQ_CASE(64, 8)
  }
#undef RQ_CASE
  return nullptr;
}

int rowq_blocks_per_cu(const void* fn) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(fn, dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kRThreads, 0) != hipSuccess || nb <= 0) nb = 1;
  cache[key] = nb;
  return nb;
}

// The plan for U chunks per row at a given split: chunks per lane, kernel,
// row groups, row walk and grid.
template <int BITS, int MODE>
RPlan rowq_plan_at(int64_t n, int U, int lpr) {
  RPlan p{};
  p.lpr = lpr;
  p.cpl = (U + p.lpr - 1) / p.lpr;
  const bool full = U == p.lpr * p.cpl;
  p.fn = full ? pick_rowq<BITS, MODE, true>(p.lpr, p.cpl) : pick_rowq<BITS, MODE, false>(p.lpr, p.cpl);
  p.rpw = 64 / p.lpr;
  if (!p.fn) return p;
  const int64_t units = MODE == kRowqGelu ? n / 2 : n;
  const int upw = MODE == kRowqGelu ? p.rpw / 2 : p.rpw;
  p.rg = int((units + upw - 1) / upw);
  const int cus = device_cu_count();
  const int waves_max = cus * rowq_blocks_per_cu(p.fn) * kRWaves;
  p.ipw = (p.rg + waves_max - 1) / waves_max;
  // one-row waves: every workgroup stages all of x for 4 rows per step, so
  // walk rows until the grid is about one workgroup per CU (INT2 [1536,
  // 12288]: 6.2 -> 5.3 us; INT4 [2560, 10240]: 7.4 -> 6.6 us)
  if (p.rpw == 1) p.ipw = std::max(p.ipw, (p.rg + cus * kRWaves - 1) / (cus * kRWaves));
  const int waves = (p.rg + p.ipw - 1) / p.ipw;
  p.grid = (waves + kRWaves - 1) / kRWaves;
  return p;
}

template <int BITS, int MODE>
RPlan rowq_plan(int64_t n, int64_t k) {
  constexpr int BPC = BITS == 2 ? 2 : 1;
  const int U = int((k * BITS) / (128 * kChunkLoads<BITS>));
  // smallest split of at least 8 lanes (128 contiguous bytes per row and
  // instruction) whose lanes hold at most 6 activation blocks (108 VGPRs);
  // rows too wide for that take 64 lanes and up to 8 blocks
  int lpr = 64;
  for (int l = 8; l <= 64; l *= 2)
    if ((U + l - 1) / l * BPC <= 6) {
      lpr = l;
      break;
    }
  RPlan p = rowq_plan_at<BITS, MODE>(n, U, lpr);
  // a matrix too small to give every CU a workgroup spreads each row over
  // more lanes: more, shorter waves (INT8 [256, 1536]: 4.0 -> 2.7 us; INT4
  // [2048, 1536]: 3.5 -> 3.0 us)
  const int cus = device_cu_count();
  while (p.fn && p.grid < cus && p.lpr < 64) {
    const RPlan q = rowq_plan_at<BITS, MODE>(n, U, 2 * p.lpr);
    if (!q.fn || q.grid <= p.grid) break;
    p = q;
  }
  return p;
}

// argument checks shared by both entry points; returns 0 or an error code
int rowq_check(const char* name, const void* w, const float* row_scale, int64_t n, int64_t k, int32_t bits,
               const uint16_t* x, const void* out, const char* out_name, int64_t max_k) {
  if (!w) return fail(Q4DEC_ERR_NULL, "%s: w is NULL", name);
  if (!row_scale) return fail(Q4DEC_ERR_NULL, "%s: row_scale is NULL", name);
  if (!x) return fail(Q4DEC_ERR_NULL, "%s: x is NULL", name);
  if (!out) return fail(Q4DEC_ERR_NULL, "%s: %s is NULL", name, out_name);
  if (bits != 2 && bits != 4 && bits != 8)
    return fail(Q4DEC_ERR_SHAPE, "%s: bits must be 2, 4 or 8 (got %d)", name, int(bits));
  if (n <= 0 || n >= (int64_t(1) << 31))
    return fail(Q4DEC_ERR_SHAPE, "%s: n must be in [1, 2^31) (got %lld)", name, (long long)n);
  const int64_t kq = bits == 2 ? 64 : 32;  // one chunk of codes
  if (k <= 0 || k % kq)
    return fail(Q4DEC_ERR_SHAPE, "%s: k must be a positive multiple of %lld for %d-bit codes (got %lld)", name,
                (long long)kq, int(bits), (long long)k);
  if (k > max_k)
    return fail(Q4DEC_ERR_UNSUPPORTED, "%s: k must be <= %lld (got %lld)", name, (long long)max_k, (long long)k);
  if (!aligned(w, 16)) return fail(Q4DEC_ERR_ALIGN, "%s: w must be 16-byte aligned", name);
  if (!aligned(x, 16)) return fail(Q4DEC_ERR_ALIGN, "%s: x must be 16-byte aligned", name);
  if (!aligned(row_scale, 4)) return fail(Q4DEC_ERR_ALIGN, "%s: row_scale must be 4-byte aligned", name);
  return 0;
}

template <int MODE>
int rowq_launch(const char* name, const void* w, const float* row_scale, int64_t n, int64_t k, int32_t bits,
                const uint16_t* x, void* out, void* stream) {
  const RPlan p = bits == 2 ? rowq_plan<2, MODE>(n, k) : bits == 4 ? rowq_plan<4, MODE>(n, k) : rowq_plan<8, MODE>(n, k);
  if (!p.fn) return fail(Q4DEC_ERR_UNSUPPORTED, "%s: no kernel for k=%lld", name, (long long)k);
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  int ni = int(n), ki = int(k), ipw = p.ipw;
  void* args[] = {&wp, &row_scale, &x, &ni, &ki, &ipw, &out};
  hipError_t e = hipLaunchKernel(p.fn, dim3(p.grid), dim3(kRThreads), args, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(Q4DEC_ERR_HIP, "%s: kernel launch failed: %s", name, hipGetErrorString(e));
  return launch_status(name);
}

}  // namespace
}  // namespace q4dec

extern "C" int rowq_gemv(const void* w, const float* row_scale, int64_t n, int64_t k, int32_t bits,
                         const uint16_t* x, float* y, void* stream) {
  using namespace q4dec;
  if (int rc = rowq_check("rowq_gemv", w, row_scale, n, k, bits, x, y, "y", Q4DEC_MAX_K)) return rc;
  if (!aligned(y, 4)) return fail(Q4DEC_ERR_ALIGN, "rowq_gemv: y must be 4-byte aligned");
  return rowq_launch<kRowqGemv>("rowq_gemv", w, row_scale, n, k, bits, x, y, stream);
}

extern "C" int rowq_gemv_gelu_mul(const void* w, const float* row_scale, int64_t n, int64_t k, int32_t bits,
                                  const uint16_t* x, uint16_t* a, void* stream) {
  using namespace q4dec;
  if (int rc = rowq_check("rowq_gemv_gelu_mul", w, row_scale, n, k, bits, x, a, "a", Q4DEC_GELU_MAX_K)) return rc;
  if (n % 2) return fail(Q4DEC_ERR_SHAPE, "rowq_gemv_gelu_mul: n must be even ([gate; up] rows, got %lld)",
                         (long long)n);
  if (!aligned(a, 2)) return fail(Q4DEC_ERR_ALIGN, "rowq_gemv_gelu_mul: a must be 2-byte aligned");
  return rowq_launch<kRowqGelu>("rowq_gemv_gelu_mul", w, row_scale, n, k, bits, x, a, stream);
}

extern "C" size_t rowq_head_workspace_bytes(int64_t vocab, int64_t k, int32_t bits) {
  (void)vocab;
  (void)k;
  (void)bits;
  return size_t(q4dec::kRowqMaxPartials) * sizeof(uint2);
}

extern "C" int rowq_softcap_argmax(const void* w, const float* row_scale, int64_t vocab, int64_t k, int32_t bits,
                                   const uint16_t* x, float cap, void* ws, size_t ws_bytes, int32_t* idx_out,
                                   float* val_out, void* stream) {
  using namespace q4dec;
  const char* name = "rowq_softcap_argmax";
  if (int rc = rowq_check(name, w, row_scale, vocab, k, bits, x, ws, "ws", Q4DEC_MAX_K)) return rc;
  if (!idx_out) return fail(Q4DEC_ERR_NULL, "%s: idx_out is NULL", name);
  if (!val_out) return fail(Q4DEC_ERR_NULL, "%s: val_out is NULL", name);
  if (!aligned(ws, 8)) return fail(Q4DEC_ERR_ALIGN, "%s: ws must be 8-byte aligned", name);
  if (!aligned(idx_out, 4) || !aligned(val_out, 4))
    return fail(Q4DEC_ERR_ALIGN, "%s: idx_out and val_out must be 4-byte aligned", name);
  const size_t need = rowq_head_workspace_bytes(vocab, k, bits);
  if (ws_bytes < need) return fail(Q4DEC_ERR_WORKSPACE, "%s: ws_bytes %zu < required %zu", name, ws_bytes, need);
  const RPlan p = bits == 2   ? rowq_plan<2, kRowqHead>(vocab, k)
                  : bits == 4 ? rowq_plan<4, kRowqHead>(vocab, k)
                              : rowq_plan<8, kRowqHead>(vocab, k);
  if (!p.fn) return fail(Q4DEC_ERR_UNSUPPORTED, "%s: no kernel for k=%lld", name, (long long)k);
  if (p.grid > kRowqMaxPartials) return fail(Q4DEC_ERR_UNSUPPORTED, "%s: too many workgroups", name);
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  int ni = int(vocab), ki = int(k), ipw = p.ipw;
  void* part = ws;
  void* args[] = {&wp, &row_scale, &x, &ni, &ki, &ipw, &part};
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipLaunchKernel(p.fn, dim3(p.grid), dim3(kRThreads), args, 0, st);
  if (e != hipSuccess) return fail(Q4DEC_ERR_HIP, "%s: kernel launch failed: %s", name, hipGetErrorString(e));
  reduce_argmax_partials(static_cast<const uint2*>(ws), p.grid, 1, 1, cap, idx_out, val_out, st);
  return launch_status(name);
}
