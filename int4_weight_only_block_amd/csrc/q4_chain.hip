// q4_gemv_chain: one persistent launch over a chain of S=1 q4_0 GEMVs (and an
// optional LM head as the last link), in place of one launch per matrix.
//
// Why. Decode reads about 2.1 GB of int4 weights per token (E4B card,
// bandwidth cost-model paragraph: bytes per token over the device bandwidth
// plus a fixed per-step cost), spread over 168 layer matrices of 3-30 MB and
// the head. One launch per matrix pays a fixed dispatch cost each time and
// starts every matrix's weight stream only after the previous kernel has
// drained; the mixed-bit page's fused gate/up paragraph makes the same point
// for its device (fewer dispatches per layer, +8%). Here every workgroup
// walks all links in order: as soon as it has finished its rows of link i it
// issues the weight loads of its first row group of link i + 1, and only then
// waits for the other workgroups to finish link i (the next link's input may
// be this link's output), so the wait runs under the weight stream.
//
// Layout and arithmetic per link are those of the S=1 GEMV (q4_gemv.hip):
// lane t of a row group owns blocks t, t + LPR, ... of its row (one 16-byte
// non-temporal load each), activations are staged once per workgroup as
// block-scaled fp16 in LDS (exact path for blocks spanning more than 31
// binades), codes are unpacked exactly and reduced with v_dot2c_f32_f16, row
// sums with DPP. The split (lanes per row, blocks per lane) is chosen per
// link at build time and read at run time.
//
// Synchronisation. One workgroup of 16 waves per compute unit, so 256 arrive
// per barrier. A workgroup arrives on one of 16 counters (each on its own
// 256-byte line) with an agent-scope relaxed atomic add, after its outputs,
// stored with agent-scope relaxed atomic stores (written through to the
// device coherence point), have completed. A waiting workgroup's first wave
// polls the 16 counters with agent-scope atomic loads until each holds its
// target. Every wait is bounded by the real-time clock: on expiry the
// workgroup sets the error word and leaves; a later call finds the word set
// and does nothing until the caller zeroes the workspace. After the last
// link each workgroup counts itself out (two levels of counters with
// returned values); the last one out reduces the head's partials and resets
// every counter to zero, so the next launch finds them clear without a
// memset (which a captured graph must not contain). Later links read earlier
// outputs with ordinary loads: the host checks that no 256-byte line an
// output touches is read or written by any earlier link, so no cache can
// hold a stale copy of it when it is read.
#include <limits.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>
#include <vector>

#include "q4dec_internal.h"

namespace q4dec {
Q4DEC_DEBUG_READER(q4_chain)
namespace {

constexpr int kCWaves = 16;                // waves per workgroup
constexpr int kCThreads = 64 * kCWaves;    // 1024: one workgroup per compute unit
constexpr int kCPerCu = 16 / kCWaves;      // workgroups per compute unit (16 waves per CU)
constexpr int kCBpl = 5;                   // blocks per lane held in flight (k <= 64 * 5 * 32)
constexpr int kGroups = 16;                // arrival counters
constexpr int kLine = 256;                 // bytes per counter line
constexpr uint32_t kMagic = 0x48433451u;   // table tag
constexpr int kMaxChainPartials = 4096;    // workgroups of one chain launch (head partials)

// workspace layout (bytes)
constexpr size_t kWsErr = 0;                                    // uint32 error word
constexpr size_t kWsArrive = kLine;                             // kGroups lines
constexpr size_t kWsDone = kWsArrive + size_t(kGroups) * kLine; // kGroups + 1 lines
constexpr size_t kWsPartials = kWsDone + size_t(kGroups + 1) * kLine;
constexpr size_t kWsBytes = kWsPartials + size_t(kMaxChainPartials) * sizeof(uint2);

// error word bits
constexpr uint32_t kErrTimeout = 1u;
constexpr uint32_t kErrTable = 2u;

struct ChainHeader {  // 64 bytes; first entry of the device table
  uint32_t magic;
  int32_t n_links;
  int32_t grid;
  int32_t lds_bytes;
  uint64_t checksum;  // of the link entries
  float cap;
  int32_t max_b;
  int64_t spin_ticks;  // wait bound in real-time clock ticks (100 MHz)
  uint32_t pad[6];
};
static_assert(sizeof(ChainHeader) == 64, "header size");

struct ChainEntry {  // 64 bytes per link
  const uint8_t* nib;
  const uint16_t* scl;
  const uint16_t* x;
  void* out;
  int32_t n, k;
  int32_t rg;        // row groups (outputs per wave step, rounded up)
  int32_t arrivals;  // arrivals each workgroup has made after this link (targets of the next wait)
  int16_t lpr, bpl;
  int8_t mode, full, wait, pad0;
  int32_t pad1;
};
static_assert(sizeof(ChainEntry) == 64, "entry size");

uint64_t fnv1a(const void* p, size_t n, uint64_t h = 1469598103934665603ull) {
  const uint8_t* b = static_cast<const uint8_t*>(p);
  for (size_t i = 0; i < n; ++i) {
    h ^= b[i];
    h *= 1099511628211ull;
  }
  return h;
}

// Sum over the LPR lanes of a row (LPR in {16, 32, 64}, uniform).
__device__ __forceinline__ float row_sum(float v, int lpr) {
  v = group_sum<16>(v);
  if (lpr >= 32) v += __shfl_xor(v, 16);
  if (lpr >= 64) v += __shfl_xor(v, 32);
  return v;
}

// Pointers read from the link table are generic to the compiler, which then
// emits flat loads; those count against the LDS counter as well, so every
// wait for the activations in LDS would also wait for every weight load in
// flight. All of them point to device (global) memory: say so.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* glob(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kCThreads) void q4_chain_kernel(const uint8_t* __restrict__ table, int n_links,
                                                             uint64_t checksum, uint8_t* __restrict__ ws,
                                                             int32_t* __restrict__ idx_out,
                                                             float* __restrict__ val_out) {
  extern __shared__ uint32_t dyn[];
  const ChainHeader* hdr = reinterpret_cast<const ChainHeader*>(table);
  const ChainEntry* links = reinterpret_cast<const ChainEntry*>(table + sizeof(ChainHeader));
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + kWsErr);
  uint32_t* arrive = reinterpret_cast<uint32_t*>(ws + kWsArrive);  // group g at arrive[g * kLine / 4]
  uint32_t* done = reinterpret_cast<uint32_t*>(ws + kWsDone);
  uint2* partials = reinterpret_cast<uint2*>(ws + kWsPartials);
  constexpr int kStride = kLine / 4;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x;
  const int grp = blockIdx.x % kGroups;

  __shared__ int s_flag;
  __shared__ float s_bv[kCWaves];
  __shared__ int s_bi[kCWaves];
  __shared__ int s_wide[kCWaves];

  // The table must be the one the host validated, and no earlier call may
  // have failed (the counters would be inconsistent).
  if (threadIdx.x == 0) {
    const bool ok = hdr->magic == kMagic && hdr->n_links == n_links && hdr->checksum == checksum && hdr->grid == G;
    if (!ok && blockIdx.x == 0) __hip_atomic_fetch_or(err, kErrTable, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flag = ok && ld_agent(err) == 0u;
  }
  __syncthreads();
  if (!s_flag) return;
  const int64_t spin = hdr->spin_ticks;
  const int max_b = hdr->max_b;
  uint32_t* xs = dyn;                                        // [max_b * 16] fp16 pairs
  float* xf = reinterpret_cast<float*>(dyn + max_b * 16);    // [max_b] block factors

  uint32_t m_lo, m_hi, magic;
  asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(m_lo));
  asm volatile("v_mov_b32 %0, 0x00F000F0" : "=v"(m_hi));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

  // this lane's weight registers (one row group of one link)
  uint4 q[kCBpl];
  uint32_t sd[kCBpl];
  const int W = G * kCWaves;          // waves in the grid
  // wave slot: consecutive slots sit in consecutive workgroups (compute
  // units); slot s walks row groups s, s + W, s + 2W, ... of a link, so at
  // each step the grid reads one contiguous stretch of every matrix
  const int gw = wave * G + blockIdx.x;

  // row of row group (it) of link L for this lane (clamped into range)
  // lanes per row are 16, 32 or 64: shifts instead of divisions
  auto lg_of = [](int lpr) { return lpr == 16 ? 4 : lpr == 32 ? 5 : 6; };
  auto row_of = [&](const ChainEntry& L, int it) -> int {
    const int lg = lg_of(L.lpr);
    const int r = lane >> lg;
    const int rg = gw + it * W;
    if (L.mode == Q4DEC_LINK_GELU) {
      const int units = L.n >> 1, lu = 5 - lg;  // upw = 2^lu outputs per step (lpr <= 32)
      const int v = (rg << lu) + (r & ((1 << lu) - 1));
      return (v < units ? v : units - 1) + (r >> lu) * units;
    }
    const int row = (rg << (6 - lg)) + r;
    return row < L.n ? row : L.n - 1;
  };
  auto iters_of = [&](const ChainEntry& L) -> int { return gw < L.rg ? (L.rg - gw + W - 1) / W : 0; };
  // Every lane issues all kCBpl loads of a row group, on a clamped block
  // index: blocks past the row's end (or past the link's blocks per lane)
  // reload the row's last block, an address the other lanes of the
  // instruction already read, and their use is dropped by a select. With no
  // branch in the row loop the compiler can count the loads in flight and
  // wait for one row group without draining the next one's refills.
  auto load = [&](const ChainEntry& L, int row) {
    const int t = lane & (L.lpr - 1);
    const int B = L.k >> 5;
    auto np = glob(reinterpret_cast<const u32x4*>(L.nib + size_t(row) * size_t(L.k >> 1)));
    auto sp = glob(L.scl + size_t(row) * size_t(B));
#pragma unroll
    for (int j = 0; j < kCBpl; ++j) {
      const int b = min(j * L.lpr + t, B - 1);
      const u32x4 v = __builtin_nontemporal_load(np + b);
      q[j] = make_uint4(v.x, v.y, v.z, v.w);
      sd[j] = sp[b];
    }
  };

  // prefetch of link 0
  {
    const ChainEntry L0 = links[0];
    if (iters_of(L0) > 0) load(L0, row_of(L0, 0));
  }

  for (int i = 0; i < n_links; ++i) {
    const ChainEntry L = links[i];
    const int B = L.k >> 5;
    const int lpr = L.lpr;
    const int t = lane & (lpr - 1);
    const int rpw = 64 >> lg_of(lpr);
    const int r = lane >> lg_of(lpr);
    const int iters = iters_of(L);

    // ---- wait until every workgroup has finished the links before this one
    if (L.wait && i > 0) {
      const uint32_t arr = uint32_t(links[i - 1].arrivals);
      if (wave == 0) {
        const uint32_t m_g = lane < kGroups ? uint32_t((G - lane + kGroups - 1) / kGroups) : 0u;
        const uint32_t target = arr * m_g;
        const uint64_t t0 = wall_clock64();
        int timed_out = 0;
        while (true) {
          const uint32_t v = lane < kGroups ? ld_agent(arrive + lane * kStride) : 0xFFFFFFFFu;
          if (__all(v >= target)) break;
          if (int64_t(wall_clock64() - t0) > spin) {
            timed_out = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        if (lane == 0) {
          if (timed_out) __hip_atomic_fetch_or(err, kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          s_flag = timed_out;
        }
      }
      __syncthreads();
      if (s_flag) return;
    }

    // ---- stage x (block-scaled fp16 in LDS), exact path for wide blocks
    bool wide_t = false;
    {
      auto src = glob(reinterpret_cast<const u32x4*>(L.x));
      for (int qi = threadIdx.x; qi < 4 * B; qi += kCThreads) {
        const u32x4 v = src[qi];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t emax, emin;
        block_exp_range(w, emax, emin);
        // the four quarters of a block sit in lanes 4j .. 4j+3 of one wave
        // (qi and threadIdx.x agree modulo 4 and kCThreads is a multiple of 64)
        emax = max(emax, uint32_t(__shfl_xor(int(emax), 1)));
        emax = max(emax, uint32_t(__shfl_xor(int(emax), 2)));
        emin = min(emin, uint32_t(__shfl_xor(int(emin), 1)));
        emin = min(emin, uint32_t(__shfl_xor(int(emin), 2)));
        wide_t |= int(emax) - int(emin) > kMaxSpan;
        const int e = int(emax) - 127 - 14;
        uint32_t o[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const half2_t h = {(_Float16)ldexpf(bf16_to_f32(w[c] & 0xFFFFu), -e),
                             (_Float16)ldexpf(bf16_to_f32(w[c] >> 16), -e)};
          o[c] = __builtin_bit_cast(uint32_t, h);
        }
        const int b = qi >> 2, qq = qi & 3;
        reinterpret_cast<uint4*>(xs + 16 * b)[qq ^ (b & 3)] = make_uint4(o[0], o[1], o[2], o[3]);
        if (qq == 0) xf[b] = ldexpf(1.0f, e);
      }
    }
    {
      const bool wide_wave = __ballot(wide_t) != 0;
      if (lane == 0) s_wide[wave] = wide_wave;
    }
    __syncthreads();
    int wide_any = 0;
#pragma unroll
    for (int w = 0; w < kCWaves; ++w) wide_any |= s_wide[w];
    const bool exact = __builtin_amdgcn_readfirstlane(wide_any) != 0;

    float fr[kCBpl];
#pragma unroll
    for (int j = 0; j < kCBpl; ++j) fr[j] = xf[min(j * lpr + t, B - 1)];

    // ---- rows
    float best = -INFINITY;
    int bidx = INT_MAX;
    auto emit = [&](int it, float acc) {
      acc = row_sum(acc, lpr);
      const int rg = gw + it * W;
      if (L.mode == Q4DEC_LINK_GEMV) {
        const int row = rg * rpw + r;
        if (t == 0 && row < L.n)
          __hip_atomic_store(glob(static_cast<float*>(L.out)) + row, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else if (L.mode == Q4DEC_LINK_HEAD) {
        const int row = rg * rpw + r;
        if (row < L.n && better(acc, row, best, bidx)) {
          best = acc;
          bidx = row;
        }
      } else {
        const float up = __shfl_xor(acc, 32);  // the up row's sum
        const int upw = rpw >> 1;
        const int v = rg * upw + r;
        if (t == 0 && r < upw && v < (L.n >> 1))
          __hip_atomic_store(glob(static_cast<uint16_t*>(L.out)) + v, f32_to_bf16_rne(gelu_tanh(acc) * up),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    };
    if (exact) {
      for (int it = 0; it < iters; ++it) {
        const int row = row_of(L, it);
        auto np = glob(reinterpret_cast<const u32x4*>(L.nib + size_t(row) * size_t(L.k >> 1)));
        auto sp = glob(L.scl + size_t(row) * size_t(B));
        float acc = 0.0f;
#pragma unroll 1
        for (int j = 0; j < L.bpl; ++j) {
          const int b = j * lpr + t;
          if (b < B) {
            const u32x4 v = np[b];
            const float p = block_dot_exact(make_uint4(v.x, v.y, v.z, v.w),
                                            reinterpret_cast<const uint4*>(L.x + 32 * b), m_lo, m_hi, magic);
            acc = fmaf(float(__builtin_bit_cast(_Float16, sp[b])), p, acc);
          }
        }
        emit(it, acc);
      }
    } else {
      // One row group; with REFILL (compile time: the last row group is
      // peeled off) block j's registers are reloaded for the next row group
      // right after their last use, in place, so a row group of loads stays
      // in flight per wave.
      auto step = [&](int it, auto refill_tag) {
        constexpr bool REFILL = decltype(refill_tag)::value;
        const int row_next = REFILL ? row_of(L, it + 1) : 0;
        auto np = glob(reinterpret_cast<const u32x4*>(L.nib + size_t(row_next) * size_t(L.k >> 1)));
        auto sp = glob(L.scl + size_t(row_next) * size_t(B));
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < kCBpl; ++j) {
          const int bj = j * lpr + t;
          const int b = min(bj, B - 1);
          uint32_t xh[16];
          const uint4* s4 = reinterpret_cast<const uint4*>(xs + 16 * b);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint4 v = s4[c ^ (b & 3)];
            xh[4 * c + 0] = v.x; xh[4 * c + 1] = v.y; xh[4 * c + 2] = v.z; xh[4 * c + 3] = v.w;
          }
          const float p = block_dot(q[j], xh, m_lo, m_hi, magic);
          const float d = float(__builtin_bit_cast(_Float16, uint16_t(sd[j])));
          const float a2 = fmaf(d * p, fr[j], acc);
          acc = j < L.bpl && bj < B ? a2 : acc;  // a select: a dropped block cannot turn the sum NaN
          if constexpr (REFILL) {
            __builtin_amdgcn_sched_barrier(0);
            const u32x4 v = __builtin_nontemporal_load(np + b);
            q[j] = make_uint4(v.x, v.y, v.z, v.w);
            sd[j] = sp[b];
          }
        }
        emit(it, acc);
      };
      for (int it = 0; it + 1 < iters; ++it) step(it, std::true_type{});
      if (iters > 0) step(iters - 1, std::false_type{});
    }

    if (L.mode == Q4DEC_LINK_HEAD) {
      // this workgroup's best (value, row) of the link into its partial slot
      wave_best(best, bidx);
      if (lane == 0) {
        s_bv[wave] = best;
        s_bi[wave] = bidx;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        for (int w = 1; w < kCWaves; ++w)
          if (better(s_bv[w], s_bi[w], best, bidx)) {
            best = s_bv[w];
            bidx = s_bi[w];
          }
        const uint64_t pv = uint64_t(__builtin_bit_cast(uint32_t, best)) | (uint64_t(uint32_t(bidx)) << 32);
        __hip_atomic_store(reinterpret_cast<uint64_t*>(partials) + blockIdx.x, pv, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }

    // ---- arrive (when the next link waits), then prefetch the next link
    const bool next_waits = i + 1 < n_links && links[i + 1].wait;
    if (next_waits) {
      // every store of this link has reached the coherence point before the
      // workgroup's arrival is counted
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_fetch_add(arrive + grp * kStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      __syncthreads();  // LDS of this link fully consumed before the next staging
    }
    if (i + 1 < n_links) {
      const ChainEntry N = links[i + 1];
      if (iters_of(N) > 0) load(N, row_of(N, 0));
    }
  }

  // ---- count out; the last workgroup reduces the head and resets the counters
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t m_g = uint32_t((G - grp + kGroups - 1) / kGroups);
    const uint32_t old = __hip_atomic_fetch_add(done + grp * kStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int last = 0;
    if (old + 1u == m_g) {
      const uint32_t groups = uint32_t(G < kGroups ? G : kGroups);
      const uint32_t o2 = __hip_atomic_fetch_add(done + kGroups * kStride, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
      last = o2 + 1u == groups;
    }
    s_flag = last;
  }
  __syncthreads();
  if (!s_flag) return;
  // every other workgroup has finished all its links and waits
  const ChainEntry LL = links[n_links - 1];
  if (LL.mode == Q4DEC_LINK_HEAD) {
    float best = -INFINITY;
    int bidx = INT_MAX;
    for (int w = threadIdx.x; w < G; w += kCThreads) {
      const uint64_t pv = __hip_atomic_load(reinterpret_cast<const uint64_t*>(partials) + w, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
      const float v = __builtin_bit_cast(float, uint32_t(pv));
      const int ix = int(uint32_t(pv >> 32));
      if (better(v, ix, best, bidx)) {
        best = v;
        bidx = ix;
      }
    }
    wave_best(best, bidx);
    if (lane == 0) {
      s_bv[wave] = best;
      s_bi[wave] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < kCWaves; ++w)
        if (better(s_bv[w], s_bi[w], best, bidx)) {
          best = s_bv[w];
          bidx = s_bi[w];
        }
      const float cap = hdr->cap;
      if (bidx == INT_MAX) {
        *idx_out = -1;
        *val_out = __builtin_nanf("");
      } else {
        *idx_out = bidx;
        *val_out = cap > 0.0f ? cap * tanhf(best / cap) : best;
      }
    }
  }
  if (threadIdx.x < kGroups) {
    __hip_atomic_store(arrive + threadIdx.x * kStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(done + threadIdx.x * kStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x == kGroups)
    __hip_atomic_store(done + kGroups * kStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ host
int chain_blocks_per_cu(size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<size_t, int>, int> cache;
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(lds, dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(&q4_chain_kernel), kCThreads,
                                                   lds) != hipSuccess)
    nb = 0;
  cache[key] = nb;
  return nb;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi) rounded out to whole lines
};
Range lines_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a & ~uintptr_t(kLine - 1), (a + bytes + kLine - 1) & ~uintptr_t(kLine - 1)};
}
bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

}  // namespace
}  // namespace q4dec

extern "C" size_t q4_chain_table_bytes(int64_t n_links) {
  if (n_links <= 0 || n_links > Q4DEC_CHAIN_MAX_LINKS) return 0;
  return sizeof(q4dec::ChainHeader) + size_t(n_links) * sizeof(q4dec::ChainEntry);
}

extern "C" size_t q4_chain_workspace_bytes(void) { return q4dec::kWsBytes; }

extern "C" int q4_chain_build(const q4_chain_link* links, int64_t n_links, float cap, int64_t spin_us, void* table,
                              size_t table_bytes) {
  using namespace q4dec;
  const char* fn = "q4_chain_build";
  if (!links) return fail(Q4DEC_ERR_NULL, "%s: links is NULL", fn);
  if (!table) return fail(Q4DEC_ERR_NULL, "%s: table is NULL", fn);
  if (n_links <= 0 || n_links > Q4DEC_CHAIN_MAX_LINKS)
    return fail(Q4DEC_ERR_SHAPE, "%s: n_links must be in [1, %d] (got %lld)", fn, Q4DEC_CHAIN_MAX_LINKS,
                (long long)n_links);
  const size_t need = q4_chain_table_bytes(n_links);
  if (table_bytes < need) return fail(Q4DEC_ERR_WORKSPACE, "%s: table_bytes %zu < required %zu", fn, table_bytes, need);
  if (!aligned(table, 8)) return fail(Q4DEC_ERR_ALIGN, "%s: table must be 8-byte aligned", fn);
  if (spin_us < 0) return fail(Q4DEC_ERR_SHAPE, "%s: spin_us must be >= 0", fn);
  ChainHeader* hdr = static_cast<ChainHeader*>(table);
  ChainEntry* ent = reinterpret_cast<ChainEntry*>(static_cast<uint8_t*>(table) + sizeof(ChainHeader));
  memset(table, 0, need);
  int max_b = 0, arrivals = 0;
  std::vector<Range> outs(static_cast<size_t>(n_links)), ins(static_cast<size_t>(n_links));
  for (int64_t i = 0; i < n_links; ++i) {
    const q4_chain_link& l = links[i];
    const int64_t n = l.n, k = l.k;
    if (!l.packed) return fail(Q4DEC_ERR_NULL, "%s: link %lld: packed is NULL", fn, (long long)i);
    if (!l.x) return fail(Q4DEC_ERR_NULL, "%s: link %lld: x is NULL", fn, (long long)i);
    if (l.mode != Q4DEC_LINK_GEMV && l.mode != Q4DEC_LINK_GELU && l.mode != Q4DEC_LINK_HEAD)
      return fail(Q4DEC_ERR_SHAPE, "%s: link %lld: unknown mode %d", fn, (long long)i, int(l.mode));
    if (l.mode == Q4DEC_LINK_HEAD && i != n_links - 1)
      return fail(Q4DEC_ERR_SHAPE, "%s: link %lld: a head link must be the last link", fn, (long long)i);
    if (l.mode != Q4DEC_LINK_HEAD && !l.out)
      return fail(Q4DEC_ERR_NULL, "%s: link %lld: out is NULL", fn, (long long)i);
    if (n <= 0 || n >= (int64_t(1) << 31))
      return fail(Q4DEC_ERR_SHAPE, "%s: link %lld: n must be in [1, 2^31) (got %lld)", fn, (long long)i, (long long)n);
    if (k <= 0 || k % 32)
      return fail(Q4DEC_ERR_SHAPE, "%s: link %lld: k must be a positive multiple of 32 (got %lld)", fn, (long long)i,
                  (long long)k);
    if (k > Q4DEC_CHAIN_MAX_K)
      return fail(Q4DEC_ERR_UNSUPPORTED, "%s: link %lld: k must be <= %d (got %lld)", fn, (long long)i,
                  Q4DEC_CHAIN_MAX_K, (long long)k);
    if (l.mode == Q4DEC_LINK_GELU && (n % 2 || k > Q4DEC_CHAIN_GELU_MAX_K))
      return fail(Q4DEC_ERR_SHAPE, "%s: link %lld: a GELU link needs an even n and k <= %d", fn, (long long)i,
                  Q4DEC_CHAIN_GELU_MAX_K);
    if (!aligned(l.packed, 16) || !aligned(l.x, 16))
      return fail(Q4DEC_ERR_ALIGN, "%s: link %lld: packed and x must be 16-byte aligned", fn, (long long)i);
    if (l.out && !aligned(l.out, l.mode == Q4DEC_LINK_GEMV ? 4 : 2))
      return fail(Q4DEC_ERR_ALIGN, "%s: link %lld: out is misaligned", fn, (long long)i);
    const int B = int(k / 32);
    // the smallest split whose lanes hold at most kCBpl blocks (16 lanes
    // only up to 5, as the single-matrix GEMV)
    int lpr = 16;
    if ((B + 15) / 16 > 5) lpr = 32;
    if (lpr == 32 && (B + 31) / 32 > kCBpl) lpr = 64;
    if (l.mode == Q4DEC_LINK_GELU && lpr > 32)
      return fail(Q4DEC_ERR_SHAPE, "%s: link %lld: GELU k too large", fn, (long long)i);
    const int bpl = (B + lpr - 1) / lpr;
    const int rpw = 64 / lpr;
    const int64_t units = l.mode == Q4DEC_LINK_GELU ? n / 2 : n;
    const int upw = l.mode == Q4DEC_LINK_GELU ? rpw / 2 : rpw;
    ChainEntry& e = ent[i];
    e.nib = static_cast<const uint8_t*>(l.packed);
    e.scl = reinterpret_cast<const uint16_t*>(e.nib + nib_plane_bytes(n, k));
    e.x = l.x;
    e.out = l.out;
    e.n = int32_t(n);
    e.k = int32_t(k);
    e.rg = int32_t((units + upw - 1) / upw);
    e.lpr = int16_t(lpr);
    e.bpl = int16_t(bpl);
    e.mode = int8_t(l.mode);
    e.full = int8_t(B == lpr * bpl);
    e.wait = int8_t(l.wait != 0);
    max_b = std::max(max_b, B);
    ins[size_t(i)] = lines_of(l.x, size_t(k) * 2);
    const size_t out_bytes = l.mode == Q4DEC_LINK_GEMV ? size_t(n) * 4 : l.mode == Q4DEC_LINK_GELU ? size_t(n) : 0;
    outs[size_t(i)] = out_bytes ? lines_of(l.out, out_bytes) : Range{0, 0};
  }
  // arrivals: a workgroup arrives after link i when link i + 1 waits
  for (int64_t i = 0; i < n_links; ++i) {
    if (i + 1 < n_links && ent[i + 1].wait) ++arrivals;
    ent[i].arrivals = arrivals;
  }
  // Outputs: read by later links only after a wait, and never in a line an
  // earlier (or the same) link reads or another link writes.
  for (int64_t i = 0; i < n_links; ++i) {
    if (!outs[size_t(i)].hi) continue;
    for (int64_t h = 0; h <= i; ++h)
      if (overlap(outs[size_t(i)], ins[size_t(h)]))
        return fail(Q4DEC_ERR_SHAPE,
                    "%s: link %lld's output shares a %d-byte line with the input of link %lld, which runs no later",
                    fn, (long long)i, kLine, (long long)h);
    for (int64_t j = 0; j < n_links; ++j)
      if (j != i && outs[size_t(j)].hi && overlap(outs[size_t(i)], outs[size_t(j)]))
        return fail(Q4DEC_ERR_SHAPE, "%s: the outputs of links %lld and %lld share a %d-byte line", fn, (long long)i,
                    (long long)j, kLine);
    bool waited = false;
    for (int64_t j = i + 1; j < n_links; ++j) {
      waited |= ent[j].wait != 0;
      if (!waited && overlap(outs[size_t(i)], ins[size_t(j)]))
        return fail(Q4DEC_ERR_SHAPE, "%s: link %lld reads link %lld's output without a wait in between", fn,
                    (long long)j, (long long)i);
    }
  }
  const size_t lds = size_t(max_b) * 16 * 4 + size_t(max_b) * 4;
  const int nb = chain_blocks_per_cu(lds);
  if (nb < 1) return fail(Q4DEC_ERR_UNSUPPORTED, "%s: the chain kernel does not fit on a compute unit", fn);
  const int grid = device_cu_count() * std::min(kCPerCu, nb);
  if (grid > kMaxChainPartials) return fail(Q4DEC_ERR_UNSUPPORTED, "%s: too many compute units", fn);
  hdr->magic = kMagic;
  hdr->n_links = int32_t(n_links);
  hdr->grid = grid;
  hdr->lds_bytes = int32_t(lds);
  hdr->cap = cap;
  hdr->max_b = max_b;
  hdr->spin_ticks = (spin_us == 0 ? int64_t(500000) : spin_us) * 100;  // 100 MHz real-time clock
  hdr->checksum = fnv1a(ent, size_t(n_links) * sizeof(ChainEntry));
  return Q4DEC_OK;
}

extern "C" int q4_gemv_chain(const void* table_host, const void* table_dev, void* ws, size_t ws_bytes,
                             int32_t* idx_out, float* val_out, void* stream) {
  using namespace q4dec;
  const char* fn = "q4_gemv_chain";
  if (!table_host) return fail(Q4DEC_ERR_NULL, "%s: table_host is NULL", fn);
  if (!table_dev) return fail(Q4DEC_ERR_NULL, "%s: table_dev is NULL", fn);
  if (!ws) return fail(Q4DEC_ERR_NULL, "%s: ws is NULL", fn);
  if (!aligned(table_dev, 64)) return fail(Q4DEC_ERR_ALIGN, "%s: table_dev must be 64-byte aligned", fn);
  if (!aligned(ws, 256)) return fail(Q4DEC_ERR_ALIGN, "%s: ws must be 256-byte aligned", fn);
  if (ws_bytes < kWsBytes) return fail(Q4DEC_ERR_WORKSPACE, "%s: ws_bytes %zu < required %zu", fn, ws_bytes, kWsBytes);
  const ChainHeader* hdr = static_cast<const ChainHeader*>(table_host);
  if (hdr->magic != kMagic || hdr->n_links <= 0 || hdr->n_links > Q4DEC_CHAIN_MAX_LINKS)
    return fail(Q4DEC_ERR_SHAPE, "%s: table_host is not a table built by q4_chain_build", fn);
  const ChainEntry* ent =
      reinterpret_cast<const ChainEntry*>(static_cast<const uint8_t*>(table_host) + sizeof(ChainHeader));
  const uint64_t sum = fnv1a(ent, size_t(hdr->n_links) * sizeof(ChainEntry));
  if (sum != hdr->checksum) return fail(Q4DEC_ERR_SHAPE, "%s: table_host was modified after q4_chain_build", fn);
  if (hdr->grid % device_cu_count() != 0)
    return fail(Q4DEC_ERR_UNSUPPORTED, "%s: the table was built for another device", fn);
  if (ent[hdr->n_links - 1].mode == Q4DEC_LINK_HEAD) {
    if (!idx_out || !val_out) return fail(Q4DEC_ERR_NULL, "%s: a chain ending in a head needs idx_out and val_out", fn);
    if (!aligned(idx_out, 4) || !aligned(val_out, 4))
      return fail(Q4DEC_ERR_ALIGN, "%s: idx_out and val_out must be 4-byte aligned", fn);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* tab = static_cast<const uint8_t*>(table_dev);
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  int nl = hdr->n_links;
  uint64_t cs = hdr->checksum;
  void* args[] = {&tab, &nl, &cs, &w8, &idx_out, &val_out};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&q4_chain_kernel), dim3(unsigned(hdr->grid)),
                                 dim3(kCThreads), args, size_t(hdr->lds_bytes), st);
  if (e != hipSuccess) return fail(Q4DEC_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  return launch_status(fn);
}
