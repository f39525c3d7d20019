// S=1 q4_0 dequant-GEMV and the LM head with softcap + argmax.
//
// Weight stream: each lane owns a fixed set of 32-wide k-blocks of its row
// group (block b = j * LPR + t for j < BPL, t = lane % LPR), reads the matching
// activations from LDS (broadcast across the row groups of a wave), and walks
// down the rows. One
// 16-byte non-temporal load per lane per block; LPR lanes of a row read
// LPR * 16 contiguous bytes, so every load instruction is fully coalesced in
// the row-major nibble plane. The 2-byte scale loads of one instruction cover
// only part of a cache line, so they go through the cache (a streaming load
// would let the line be dropped and fetched again for the next block). Codes are unpacked to exact fp16 integers in
// registers and reduced with v_dot2c_f32_f16 against activations converted
// once per workgroup into block-scaled fp16 in LDS, then each block partial is
// scaled by its fp16 weight scale and the block's power of two in fp32. The
// LPR partials of a row are summed with DPP.
//
// Decode is weight-bandwidth-bound ("Gemma 4 E2B (text decoder) - Core AI",
// "What it took": the device is bandwidth-bound; E4B card: about 2.1 GB of
// int4 weights read per token), so everything here serves the weight stream.
#include <math.h>
#include <limits.h>

#include <map>
#include <tuple>
#include <mutex>
#include <utility>

#include <algorithm>

#include "q4dec_internal.h"

namespace q4dec {
Q4DEC_DEBUG_READER(q4_gemv)

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Per-lane state of the weight stream: this lane's blocks of the current row
// group in flight and the power-of-two factors of its activation blocks.
template <int LPR, int BPL, bool FULL>
struct Lane {
  uint4 q[BPL];
  uint32_t s[BPL];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ nib, const uint16_t* __restrict__ scl, int row,
                                       int t, int B, size_t row_bytes) {
    const u32x4* np = reinterpret_cast<const u32x4*>(nib + size_t(row) * row_bytes);
    const uint16_t* sp = scl + size_t(row) * size_t(B);
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int b = j * LPR + t;
      if (FULL || b < B) {
        const u32x4 v = __builtin_nontemporal_load(np + b);
        q[j] = make_uint4(v.x, v.y, v.z, v.w);
        s[j] = sp[b];
      }
    }
  }

  // Dot product of the row group held in q/s against the activations in LDS;
  // with REFILL, block j's registers are reloaded from `row_next` right after
  // their last use, so a row group of loads stays in flight per wave.
  template <bool REFILL>
  __device__ __forceinline__ float dot(const uint8_t* __restrict__ nib, const uint16_t* __restrict__ scl,
                                       const uint32_t* __restrict__ xs, const float* fr, int row_next, int t,
                                       int B, size_t row_bytes, uint32_t m_lo, uint32_t m_hi, uint32_t magic) {
    const u32x4* np = reinterpret_cast<const u32x4*>(nib + size_t(row_next) * row_bytes);
    const uint16_t* sp = scl + size_t(row_next) * size_t(B);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int b = j * LPR + t;
      if (FULL || b < B) {
        uint32_t xh[16];
        const uint4* s4 = reinterpret_cast<const uint4*>(xs + 16 * b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = s4[i ^ (b & 3)];  // quarter i sits in slot i ^ (b & 3)
          xh[4 * i + 0] = v.x; xh[4 * i + 1] = v.y; xh[4 * i + 2] = v.z; xh[4 * i + 3] = v.w;
        }
        const float p = block_dot(q[j], xh, m_lo, m_hi, magic);
        const float d = float(__builtin_bit_cast(_Float16, uint16_t(s[j])));
        acc = fmaf(d * p, fr[j], acc);
        if constexpr (REFILL) {
          __builtin_amdgcn_sched_barrier(0);
          const u32x4 v = __builtin_nontemporal_load(np + b);
          q[j] = make_uint4(v.x, v.y, v.z, v.w);
          s[j] = sp[b];
        }
      }
    }
    return acc;
  }

  // The same row sum with the activations read as stored (bf16 from x,
  // converted to fp32 exactly) and each block loaded on its own: the path
  // for an x whose blocks span too many binades for the scaled fp16 copy.
  // One block at a time (no unrolling), so it needs fewer registers than
  // the streaming path beside it.
  __device__ __forceinline__ float dot_exact(const uint8_t* __restrict__ nib, const uint16_t* __restrict__ scl,
                                             const uint16_t* __restrict__ x, int row, int t, int B,
                                             size_t row_bytes, uint32_t m_lo, uint32_t m_hi, uint32_t magic) {
    const u32x4* np = reinterpret_cast<const u32x4*>(nib + size_t(row) * row_bytes);
    const uint16_t* sp = scl + size_t(row) * size_t(B);
    float acc = 0.0f;
#pragma unroll 1
    for (int j = 0; j < BPL; ++j) {
      const int b = j * LPR + t;
      if (FULL || b < B) {
        const u32x4 v = np[b];
        const float p = block_dot_exact(make_uint4(v.x, v.y, v.z, v.w), reinterpret_cast<const uint4*>(x + 32 * b),
                                        m_lo, m_hi, magic);
        acc = fmaf(float(__builtin_bit_cast(_Float16, sp[b])), p, acc);
      }
    }
    return acc;
  }
};

// Most activation vectors one multi-vector GEMV launch takes.
constexpr int kMaxVecs = 8;

// Upper bound on head workgroups (one (value, row) partial each), and the
// partials each thread of the head's last workgroup loads at once.
constexpr int kMaxPartials = 8192;
constexpr int kReduceBatch = 16;

// What a row kernel does with its row sums.
enum RowMode : int {
  kGemv = 0,  // y[row] = sum (fp32)
  kHead = 1,  // per-workgroup (max, lowest row) partial
  kGelu = 2,  // fused [gate; up] rows: a[j] = bf16(gelu_tanh(gate_j) * up_j)
};

// Where the head's last workgroup leaves its result: an arrival counter
// (zero between calls), the capped maximum and its row.
struct HeadOut {
  uint32_t* counter;
  int32_t* idx;
  float* val;
  float cap;
};

template <int LPR, int BPL, int MODE, bool FULL>
__global__ __launch_bounds__(kThreads) void q4_rows_kernel(const uint8_t* __restrict__ nib,
                                                           const uint16_t* __restrict__ scl,
                                                           const uint16_t* __restrict__ x, int n, int k, int ipw,
                                                           void* __restrict__ out, uint2* __restrict__ partials,
                                                           HeadOut ho) {
  constexpr int RPW = 64 / LPR;  // rows per wave per iteration
  // GELU mode: lane groups r < RPW/2 take gate rows, the others the up rows
  // of the same outputs (n/2 apart), so each output's pair ends up 32 lanes
  // apart after the row reduction
  static_assert(MODE != kGelu || RPW >= 2, "the gate/up pairing needs two rows per wave step");
  constexpr int UPW = MODE == kGelu ? RPW / 2 : RPW;  // outputs per wave step
  constexpr int MAXB = LPR * BPL;
  // activations as block-scaled fp16 pairs: block b at xs[16 b], its four
  // 16-byte quarters swizzled (quarter i in slot i ^ (b & 3)) so the 16
  // distinct blocks of one ds_read_b128 hit distinct banks
  __shared__ uint32_t xs[MAXB * 16];
  __shared__ float xf[MAXB];
  const int B = k >> 5;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane % LPR;
  const int r = lane / LPR;
  const int units = MODE == kGelu ? n / 2 : n;  // outputs (row pairs in GELU mode)
  const int RG = (units + UPW - 1) / UPW;
  const int rg_base = blockIdx.x * kWaves * ipw + wave;
  const size_t row_bytes = size_t(k) >> 1;
  // row groups this wave walks: rg_base, rg_base + kWaves, ... (uniform)
  const int iters = rg_base < RG ? min(ipw, (RG - rg_base + kWaves - 1) / kWaves) : 0;
  Q4_DCHECK(B <= MAXB, kDbgGemvStaging);
  Q4_DCHECK(!FULL || B == MAXB, kDbgGemvFull);
  Q4_DCHECK(int64_t(gridDim.x) * kWaves * ipw >= RG, kDbgGemvRows);
  auto row_of = [&](int i) {
    if constexpr (MODE == kGelu) {
      const int v = (rg_base + i * kWaves) * UPW + (r % UPW);
      return (v < units ? v : units - 1) + (r / UPW) * units;
    } else {
      const int row = (rg_base + i * kWaves) * RPW + r;
      return row < n ? row : n - 1;
    }
  };

  // Activation loads first, then the first row group's weights; the
  // activations are converted while the weights are in flight.
  constexpr int NXL = (4 * MAXB + kThreads - 1) / kThreads;  // x quarters per thread
  uint4 xv[NXL];
  stage_x_load<kThreads, NXL>(x, B, xv);
  Lane<LPR, BPL, FULL> L;
  // (a wave with no rows loads the clamped last row and never uses it)
  L.load(nib, scl, row_of(0), t, B, row_bytes);
  // a wide block anywhere in x puts every workgroup (all stage the same x)
  // on the exact path
  __shared__ int wide_w[kWaves];
  const bool wide_t = stage_x_store<kThreads, NXL>(xv, B, xs, xf);
  const bool wide_wave = __ballot(wide_t) != 0;
  if (lane == 0) wide_w[wave] = wide_wave;
  __syncthreads();
  // uniform by construction; readfirstlane lets the compiler branch on it
  // as a scalar, so the two paths do not hold registers at the same time
  const bool exact = __builtin_amdgcn_readfirstlane(wide_w[0] | wide_w[1] | wide_w[2] | wide_w[3]) != 0;

  float fr[BPL];
#pragma unroll
  for (int j = 0; j < BPL; ++j) {
    const int b = j * LPR + t;
    fr[j] = (FULL || b < B) ? xf[b] : 0.0f;
  }

  uint32_t m_lo, m_hi, magic;
  asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(m_lo));
  asm volatile("v_mov_b32 %0, 0x00F000F0" : "=v"(m_hi));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

  float best = -INFINITY;
  int bidx = INT_MAX;
  auto emit = [&](int i, float acc) {
    acc = group_sum<LPR>(acc);
    if constexpr (MODE == kGemv) {
      const int row = (rg_base + i * kWaves) * RPW + r;
      if (t == 0 && row < n) static_cast<float*>(out)[row] = acc;
    } else if constexpr (MODE == kHead) {
      const int row = (rg_base + i * kWaves) * RPW + r;
      if (row < n && better(acc, row, best, bidx)) {
        best = acc;
        bidx = row;
      }
    } else {
      const float up = __shfl_xor(acc, 32);  // the up row's sum
      const int v = (rg_base + i * kWaves) * UPW + r;
      if (t == 0 && r < UPW && v < units)
        static_cast<uint16_t*>(out)[v] = f32_to_bf16_rne(gelu_tanh(acc) * up);
    }
  };
  if (exact) {
    for (int i = 0; i < iters; ++i)
      emit(i, L.dot_exact(nib, scl, x, row_of(i), t, B, row_bytes, m_lo, m_hi, magic));
  } else {
    for (int i = 0; i + 1 < iters; ++i) {
      const float acc = L.template dot<true>(nib, scl, xs, fr, row_of(i + 1), t, B, row_bytes, m_lo, m_hi, magic);
      emit(i, acc);
    }
    if (iters > 0) {
      const float acc = L.template dot<false>(nib, scl, xs, fr, 0, t, B, row_bytes, m_lo, m_hi, magic);
      emit(iters - 1, acc);
    }
  }

  if constexpr (MODE == kHead) {
    // pass 1: this workgroup's best (value, row) into its partial slot
    wave_best(best, bidx);
    __shared__ float sv[kWaves];
    __shared__ int si[kWaves];
    if (lane == 0) {
      sv[wave] = best;
      si[wave] = bidx;
    }
    __syncthreads();
    __shared__ int s_last;
    if (threadIdx.x == 0) {
      for (int w = 1; w < kWaves; ++w)
        if (better(sv[w], si[w], best, bidx)) {
          best = sv[w];
          bidx = si[w];
        }
      // publish the partial at the coherence point, then count this
      // workgroup in; the last one to arrive has every partial
      const uint64_t pv = uint64_t(__builtin_bit_cast(uint32_t, best)) | (uint64_t(uint32_t(bidx)) << 32);
      __hip_atomic_store(reinterpret_cast<uint64_t*>(partials) + blockIdx.x, pv, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      const uint32_t old = __hip_atomic_fetch_add(ho.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = old + 1u == gridDim.x;
    }
    __syncthreads();
    if (!s_last) return;
    // pass 2 in the last workgroup: every thread loads its partials (up to
    // kReduceBatch at once) before comparing; the comparator is a total order
    // on (value, row), so the result does not depend on the order
    best = -INFINITY;
    bidx = INT_MAX;
    const int g = gridDim.x;
    for (int base = 0; base < g; base += kThreads * kReduceBatch) {
      uint64_t pv[kReduceBatch];
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) {
        const int i = base + int(threadIdx.x) + j * kThreads;
        pv[j] = i < g ? __hip_atomic_load(reinterpret_cast<const uint64_t*>(partials) + i, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT)
                      : (uint64_t(uint32_t(INT_MAX)) << 32) | __builtin_bit_cast(uint32_t, -INFINITY);
      }
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) {
        const float v = __builtin_bit_cast(float, uint32_t(pv[j]));
        const int ix = int(uint32_t(pv[j] >> 32));
        if (better(v, ix, best, bidx)) {
          best = v;
          bidx = ix;
        }
      }
    }
    wave_best(best, bidx);
    __syncthreads();  // the pass-1 slots are read before they are reused
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
      if (bidx == INT_MAX) {
        *ho.idx = -1;
        *ho.val = __builtin_nanf("");
      } else {
        *ho.idx = bidx;
        // the cap is increasing: capping the winner alone gives the capped maximum
        *ho.val = ho.cap > 0.0f ? ho.cap * tanhf(best / ho.cap) : best;
      }
      __hip_atomic_store(ho.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------- dispatch
struct Plan {
  int lpr, bpl, rpw, rg, ipw, grid;
  bool full;
  const void* fn;
};

template <int L, int BP, int MODE, bool FULL>
static const void* kernel_ptr() {
  if constexpr (MODE == kGelu && L == 64) {
    return nullptr;  // one row per wave step: no gate/up pairing
  } else if constexpr (MODE != kHead && L == 8) {
    return nullptr;  // eight-lane rows: head only
  } else {
    return reinterpret_cast<const void*>(&q4_rows_kernel<L, BP, MODE, FULL>);
  }
}

template <int MODE, bool FULL>
static const void* pick_kernel(int lpr, int bpl) {
#define Q4_CASE(L, BP) \
  if (lpr == L && bpl == BP) return kernel_ptr<L, BP, MODE, FULL>();
  Q4_CASE(8, 1) Q4_CASE(8, 2) Q4_CASE(8, 3) Q4_CASE(8, 4) Q4_CASE(8, 5) Q4_CASE(8, 6)
  Q4_CASE(16, 1) Q4_CASE(16, 2) Q4_CASE(16, 3) Q4_CASE(16, 4) Q4_CASE(16, 5)
  Q4_CASE(32, 2) Q4_CASE(32, 3) Q4_CASE(32, 4) Q4_CASE(32, 5) Q4_CASE(32, 6)
  Q4_CASE(64, 1) Q4_CASE(64, 2) Q4_CASE(64, 3) Q4_CASE(64, 4) Q4_CASE(64, 5) Q4_CASE(64, 6) Q4_CASE(64, 7) Q4_CASE(64, 8)
#undef Q4_CASE
  return nullptr;
}

// Resident workgroups per CU of a kernel (cached per kernel and device).
static int blocks_per_cu(const void* fn, size_t dyn_lds = 0) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, size_t>, int> cache;
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_tuple(fn, dev, dyn_lds);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kThreads, dyn_lds) != hipSuccess || nb <= 0) nb = 1;
  cache[key] = nb;
  return nb;
}

// Largest LDS allocation one workgroup may make on the current device.
static size_t max_lds_per_block() {
  int dev = 0, v = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0) v = 65536;
  return size_t(v);
}

template <int MODE>
static Plan plan_for(int64_t n, int B, int lpr) {
  Plan p{};
  p.lpr = lpr;
  p.bpl = (B + lpr - 1) / lpr;
  p.full = (B == lpr * p.bpl);
  p.fn = p.full ? pick_kernel<MODE, true>(lpr, p.bpl) : pick_kernel<MODE, false>(lpr, p.bpl);
  p.rpw = 64 / lpr;
  if (!p.fn) return p;
  // outputs per wave step: rows, or gate/up row pairs in GELU mode (a GELU
  // kernel exists only for rpw >= 2)
  const int64_t units = MODE == kGelu ? n / 2 : n;
  const int upw = MODE == kGelu ? p.rpw / 2 : p.rpw;
  p.rg = int((units + upw - 1) / upw);
  // one resident round: every workgroup is live at once
  const int cus = device_cu_count();
  const int waves_max = cus * blocks_per_cu(p.fn) * kWaves;
  p.ipw = (p.rg + waves_max - 1) / waves_max;
  // With one row per wave, converting x into LDS costs a workgroup about as
  // much as its rows; let each wave walk up to three rows while the grid
  // still covers most of the CUs.
  if (p.rpw == 1 && p.ipw < 3) {
    for (int want = 3; want > p.ipw; --want) {
      const int64_t grid = ((p.rg + want - 1) / want + kWaves - 1) / kWaves;
      if (grid * 5 >= int64_t(cus) * 4) {
        p.ipw = want;
        break;
      }
    }
  }
  // Measured on the E4B fused gate/up [20480, 2560] (occupancy 4, so two
  // row groups per wave): walking three is faster (7.8 vs 8.4 us; 1, 3 and 5
  // row groups per wave all beat 2 and 4 there and on the plain GEMV)
  if (MODE == kGelu && p.ipw == 2) p.ipw = 3;
  // likewise a plain GEMV whose one round would put more than four
  // workgroups on every CU walks three row groups per wave (E4B gate+up
  // [20480, 2560]: 7.34 -> 7.19 us in two sweeps)
  if (MODE == kGemv && p.ipw == 1 && (p.rg + kWaves - 1) / kWaves > 4 * cus) p.ipw = 3;
  const int waves = (p.rg + p.ipw - 1) / p.ipw;
  p.grid = (waves + kWaves - 1) / kWaves;
  return p;
}

template <int MODE>
static Plan make_plan(int64_t n, int64_t k) {
  const int B = int(k / 32);
  int lpr = 64;
  if (MODE == kHead && (B + 7) / 8 <= 6) {
    // the head walks many rows per wave: eight lanes per row (still 128
    // contiguous bytes per row and instruction) keep up to six blocks per
    // lane in flight (E2B head [262144, 1536]: 39.3 -> 38.2 us)
    lpr = 8;
  } else if ((B + 15) / 16 <= 5) {
    lpr = 16;
  } else if ((B + 31) / 32 <= 6) {
    lpr = 32;
  }
  Plan p = plan_for<MODE>(n, B, lpr);
  if constexpr (MODE == kHead) {
    // About four workgroups per CU, each walking several row groups per
    // wave: a whole number of workgroups per CU balances the stream (E2B
    // head [262144, 1536]: 2 or 4 per CU 38.6-38.9 us, 2.7 or 3.2 per CU 41-46
    // us), and fewer workgroups stage x fewer times and leave fewer partials.
    if (p.fn) {
      const int64_t target = 4 * int64_t(device_cu_count()) * kWaves;
      p.ipw = int(std::max<int64_t>(1, (p.rg + target - 1) / target));
      const int waves = (p.rg + p.ipw - 1) / p.ipw;
      p.grid = (waves + kWaves - 1) / kWaves;
    }
    return p;
  }
  // A matrix that fits one resident round at this split takes the widest
  // split up to 32 lanes that still fills every lane: shorter block chains
  // per wave and more waves to cover the load latency. (64-lane rows with
  // few blocks per lane measured slower: E2B down [1536, 6144] 3.78 us at 64
  // lanes against 3.43 at 32, E4B O [2560, 2048] 2.91 against 2.70.)
  if (p.fn && p.ipw == 1) {
    for (int wide = 32; wide > lpr; wide /= 2) {
      if (B % wide || B / wide < 1) continue;
      const Plan q = plan_for<MODE>(n, B, wide);
      if (q.fn && q.ipw == 1) return q;
    }
  }
  return p;
}

static int launch_rows(const Plan& p, const uint8_t* nib, const uint16_t* scl, const uint16_t* x, int n, int k,
                       void* out, uint2* partials, hipStream_t st, HeadOut ho = HeadOut{}) {
  if (!p.fn) return fail(Q4DEC_ERR_UNSUPPORTED, "no kernel for k=%d (lpr=%d, bpl=%d)", k, p.lpr, p.bpl);
  int ipw = p.ipw;
  void* args[] = {&nib, &scl, &x, &n, &k, &ipw, &out, &partials, &ho};
  hipError_t e = hipLaunchKernel(p.fn, dim3(p.grid), dim3(kThreads), args, 0, st);
  if (e != hipSuccess) return fail(Q4DEC_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return Q4DEC_OK;
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


}  // namespace q4dec

extern "C" int q4_gemv(const void* packed, int64_t n, int64_t k, const uint16_t* x, float* y, void* stream) {
  using namespace q4dec;
  int rc = check_common("q4_gemv", packed, n, "n", k, x);
  if (rc) return rc;
  if (!y) return fail(Q4DEC_ERR_NULL, "q4_gemv: y is NULL");
  if (!aligned(y, 4)) return fail(Q4DEC_ERR_ALIGN, "q4_gemv: y must be 4-byte aligned");
  const Plan p = make_plan<kGemv>(n, k);
  const uint8_t* nib = static_cast<const uint8_t*>(packed);
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(nib + nib_plane_bytes(n, k));
  rc = launch_rows(p, nib, scl, x, int(n), int(k), y, nullptr, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  return launch_status("q4_gemv");
}

extern "C" size_t lmhead_workspace_bytes(int64_t vocab, int64_t k) {
  (void)vocab;
  (void)k;
  return size_t(q4dec::kMaxPartials) * sizeof(uint2) + 256;  // partials, then the arrival counter's line
}

namespace q4dec {

// Checks shared by the two head entry points (everything but the workspace).
static int head_check(const char* fn, const void* packed, int64_t vocab, int64_t k, const uint16_t* x,
                      const int32_t* idx_out, const float* val_out) {
  int rc = check_common(fn, packed, vocab, "vocab", k, x);
  if (rc) return rc;
  if (!idx_out) return fail(Q4DEC_ERR_NULL, "%s: idx_out is NULL", fn);
  if (!val_out) return fail(Q4DEC_ERR_NULL, "%s: val_out is NULL", fn);
  if (!aligned(idx_out, 4) || !aligned(val_out, 4))
    return fail(Q4DEC_ERR_ALIGN, "%s: idx_out and val_out must be 4-byte aligned", fn);
  return Q4DEC_OK;
}

// Both passes of the head in one launch, with the per-workgroup partials in
// `partials` (kMaxPartials entries; the plan never needs more) followed by
// the arrival counter (zero on entry, left zero).
static int head_run(const char* fn, const void* packed, int64_t vocab, int64_t k, const uint16_t* x, float cap,
                    uint2* partials, int32_t* idx_out, float* val_out, hipStream_t st) {
  const Plan p = make_plan<kHead>(vocab, k);
  if (p.grid > kMaxPartials)
    return fail(Q4DEC_ERR_UNSUPPORTED, "%s: the head needs %d workgroup partials, more than the %d it holds", fn,
                p.grid, kMaxPartials);
  const uint8_t* nib = static_cast<const uint8_t*>(packed);
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(nib + nib_plane_bytes(vocab, k));
  const HeadOut ho{reinterpret_cast<uint32_t*>(partials + kMaxPartials), idx_out, val_out, cap};
  int rc = launch_rows(p, nib, scl, x, int(vocab), int(k), nullptr, partials, st, ho);
  if (rc) return rc;
  return launch_status(fn);
}

// Partials of lmhead_softcap_argmax_noalloc: a file-scope device array in
// place of a caller workspace (kMaxPartials entries and the arrival
// counter's 256-byte line, 64.25 KiB on every GPU the library runs on, held
// until the process ends; zero when the code object is loaded, and every
// call leaves the counter at zero). In host code `scratch`
// names a host-side stand-in, not the device memory: kernels get the device
// address that hipGetSymbolAddress returns for the current device, looked
// up once per device and kept.
static __device__ __align__(256) uint2 scratch[kMaxPartials + 32];

static int scratch_partials(const char* fn, uint2** out) {
  static std::mutex mu;
  static uint2* ptr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(Q4DEC_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(Q4DEC_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(Q4DEC_ERR_HIP, "%s: scratch address lookup failed on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    ptr[dev] = static_cast<uint2*>(p);
  }
  *out = ptr[dev];
  return Q4DEC_OK;
}

}  // namespace q4dec

extern "C" int lmhead_softcap_argmax(const void* packed, int64_t vocab, int64_t k, const uint16_t* x, float cap,
                                     void* ws, size_t ws_bytes, int32_t* idx_out, float* val_out, void* stream) {
  using namespace q4dec;
  const char* fn = "lmhead_softcap_argmax";
  int rc = head_check(fn, packed, vocab, k, x, idx_out, val_out);
  if (rc) return rc;
  if (!ws) return fail(Q4DEC_ERR_NULL, "%s: ws is NULL", fn);
  if (!aligned(ws, 8)) return fail(Q4DEC_ERR_ALIGN, "%s: ws must be 8-byte aligned", fn);
  const size_t need = lmhead_workspace_bytes(vocab, k);
  if (ws_bytes < need) return fail(Q4DEC_ERR_WORKSPACE, "%s: ws_bytes %zu < required %zu", fn, ws_bytes, need);
  return head_run(fn, packed, vocab, k, x, cap, static_cast<uint2*>(ws), idx_out, val_out,
                  static_cast<hipStream_t>(stream));
}

extern "C" int lmhead_softcap_argmax_noalloc(const void* packed, int64_t vocab, int64_t k, const uint16_t* x,
                                             float cap, int32_t* idx_out, float* val_out, void* stream) {
  using namespace q4dec;
  const char* fn = "lmhead_softcap_argmax_noalloc";
  int rc = head_check(fn, packed, vocab, k, x, idx_out, val_out);
  if (rc) return rc;
  uint2* partials = nullptr;
  rc = scratch_partials(fn, &partials);
  if (rc) return rc;
  return head_run(fn, packed, vocab, k, x, cap, partials, idx_out, val_out, static_cast<hipStream_t>(stream));
}

extern "C" int q4_gemv_gelu_mul(const void* packed, int64_t n, int64_t k, const uint16_t* x, uint16_t* a,
                                void* stream) {
  using namespace q4dec;
  int rc = check_common("q4_gemv_gelu_mul", packed, n, "n", k, x);
  if (rc) return rc;
  if (n % 2) return fail(Q4DEC_ERR_SHAPE, "q4_gemv_gelu_mul: n must be even ([gate; up] rows), got %lld", (long long)n);
  if (!a) return fail(Q4DEC_ERR_NULL, "q4_gemv_gelu_mul: a is NULL");
  if (!aligned(a, 2)) return fail(Q4DEC_ERR_ALIGN, "q4_gemv_gelu_mul: a must be 2-byte aligned");
  const Plan p = make_plan<kGelu>(n, k);
  if (!p.fn)
    return fail(Q4DEC_ERR_UNSUPPORTED, "q4_gemv_gelu_mul: k must be <= %d (got %lld)", Q4DEC_GELU_MAX_K,
                (long long)k);
  const uint8_t* nib = static_cast<const uint8_t*>(packed);
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(nib + nib_plane_bytes(n, k));
  rc = launch_rows(p, nib, scl, x, int(n), int(k), a, nullptr, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  return launch_status("q4_gemv_gelu_mul");
}

extern "C" int q4_gemv_multi(const void* packed, int64_t n, int64_t k, const uint16_t* x, int64_t m, float* y,
                             void* stream) {
  using namespace q4dec;
  int rc = check_common("q4_gemv_multi", packed, n, "n", k, x);
  if (rc) return rc;
  if (m < 1 || m > kMaxVecs)
    return fail(Q4DEC_ERR_SHAPE, "q4_gemv_multi: m must be in [1, %d] (got %lld)", kMaxVecs, (long long)m);
  if (!y) return fail(Q4DEC_ERR_NULL, "q4_gemv_multi: y is NULL");
  if (!aligned(y, 4)) return fail(Q4DEC_ERR_ALIGN, "q4_gemv_multi: y must be 4-byte aligned");
  if (m == 1) return q4_gemv(packed, n, k, x, y, stream);
  const size_t lds = multi_mfma_lds_bytes(int(m), k);
  if (lds > max_lds_per_block())
    return fail(Q4DEC_ERR_UNSUPPORTED, "q4_gemv_multi: m * k too large (%zu bytes of LDS, device allows %zu)", lds,
                max_lds_per_block());
  const uint8_t* nib = static_cast<const uint8_t*>(packed);
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(nib + nib_plane_bytes(n, k));
  return multi_mfma_launch(nib, scl, n, k, x, int(m), y, static_cast<hipStream_t>(stream));
}
