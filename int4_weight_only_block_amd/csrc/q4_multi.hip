// q4_multi: multi-vector q4_0 GEMV on the matrix cores, y[v, r] = W[r, :] .
// x[v, :] for 2 <= m <= 8 activation vectors ("Gemma-4 E2B mobile mixed-bit
// QAT weights", MTP speculative-decoding sections P5c/P5d: a verify pass reads
// the weights once for the few draft rows it checks).
//
// Mapping. v_mfma_f32_4x4x4_16b_bf16 runs 16 independent 4x4x4 products per
// wave; in 4-lane group g, lane 4g + i holds row i of A (four k values),
// lane 4g + i holds column i of B, and lane 4g + i receives column i of C.
// So lane 4g + j takes weight row j of the wave's 4-row group as its B
// column and activation vector j as its A row, and its C column holds the 4
// vectors' partial sums for its own row: the block scale of that row is
// folded in on the lane itself (acc += d * C), with no data from other lanes.
// The 16 lane groups of a wave own 16 different blocks of the same 4 rows (a
// row's lanes read 16 consecutive 16-byte blocks, 256 contiguous bytes), and
// each lane walks its blocks t * 16 + g down the row.
//
// Numerics. q4_pack's dword d of a block holds the codes of k = 8d .. 8d+7;
// they become 16 * c in bf16 (exact), so one MFMA takes 4 codes in k order
// and the matching 4 activations straight from LDS, where each vector is
// stored as given (bf16, no conversion). Every product is exact in fp32, the
// matrix cores add a block's products in fp32, the block scale is folded in
// fp32 and the factor 1/16 is applied once at the end (exact), as in the
// S=64 GEMM: there is no range limit on x beyond fp32's own.
#include <limits.h>
#include <math.h>

#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>

#include "q4_codes.h"
#include "q4dec_internal.h"

namespace q4dec {
Q4DEC_DEBUG_READER(q4_multi)
namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));  // 4 bf16, the 4x4x4 MFMA operand
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMWaves = 4;
constexpr int kMThreads = 64 * kMWaves;
constexpr int kMaxBpl = 6;  // blocks per lane per row segment

constexpr int kMultiVecs = 8;         // most vectors of one launch
constexpr int kMultiPartials = 8192;  // most workgroups of one head launch
constexpr int kMXLoads = 5;           // x pieces per thread loaded ahead of the weights

// halves per activation row in LDS: k plus 8 (16 bytes), so the 4 vectors a
// 4-lane group reads sit in different bank quads
__device__ __host__ inline int x_stride(int k) { return k + 8; }

// What the kernel does with its row sums.
enum MultiMode : int {
  kMultiGemv = 0,  // y[v, row] (fp32)
  kMultiHead = 1,  // per workgroup and vector: the largest sum and its lowest row
};

// Best (value, row) of the wave into every lane (the single-vector head's
// comparator: larger value, then lower row; NaN never wins).
__device__ __forceinline__ void multi_wave_best(float& best, int& bidx) {
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

// partials (head mode): entry blockIdx.x * kMultiVecs + v holds the
// workgroup's best (value bits, row) for vector v.
template <int BPL, int NG, int MODE, bool FULL>
__global__ __launch_bounds__(kMThreads) void q4_multi_kernel(const uint8_t* __restrict__ nib,
                                                             const uint16_t* __restrict__ scl,
                                                             const uint16_t* __restrict__ x, int n, int k, int m,
                                                             int nseg, int ipw, float* __restrict__ y,
                                                             uint2* __restrict__ partials) {
  extern __shared__ uint32_t dyn_lds[];
  const int B = k >> 5;
  const int xsn = x_stride(k);
  _Float16* xs = reinterpret_cast<_Float16*>(dyn_lds);  // [4 * NG][xsn]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 2;  // which of the 16 blocks of a step
  const int j = lane & 3;     // weight row of the 4-row group, and activation vector within a group of 4
  const int RG = (n + 3) / 4;
  const int rg_base = blockIdx.x * kMWaves * ipw + wave;
  const int iters = rg_base < RG ? min(ipw, (RG - rg_base + kMWaves - 1) / kMWaves) : 0;
  Q4_DCHECK(nseg * 16 * BPL >= B && (!FULL || nseg * 16 * BPL == B), kDbgMultiStaging);
  Q4_DCHECK(int64_t(gridDim.x) * kMWaves * ipw >= RG, kDbgMultiRows);
  const int units = iters * nseg;  // (row group, segment) steps this wave walks
  const size_t row_bytes = size_t(k) >> 1;
  auto row_of = [&](int u) {
    const int row = (rg_base + (u / nseg) * kMWaves) * 4 + j;
    return row < n ? row : n - 1;
  };
  auto block_of = [&](int u, int t) { return (u % nseg) * (16 * BPL) + t * 16 + grp; };

  uint4 q[BPL];
  uint16_t sd[BPL];  // 16-bit, so no zero-extension is redone on the refilled values
  auto load = [&](int u) {
    const int row = row_of(u);
    const u32x4* np = reinterpret_cast<const u32x4*>(nib + size_t(row) * row_bytes);
    const uint16_t* sp = scl + size_t(row) * size_t(B);
#pragma unroll
    for (int t = 0; t < BPL; ++t) {
      const int b = block_of(u, t);
      if (FULL || b < B) {
        const u32x4 v = __builtin_nontemporal_load(np + b);
        q[t] = make_uint4(v.x, v.y, v.z, v.w);
        sd[t] = sp[b];
      }
    }
  };
  // Stage x as stored: the m bf16 rows into LDS (row v at xs + v * xsn),
  // rows m .. 4 * NG - 1 zero, with no conversion, so every code-activation
  // product the matrix cores form is exact and x has no range limit beyond
  // fp32's own. The first kMXLoads 16-byte pieces of each thread are loaded
  // before the first weights (vector memory counters retire in order, so
  // their stores then wait for these loads only); the loads are
  // unconditional on a clamped index and an empty asm use after the weight
  // loads keeps the compiler from moving them behind the weights.
  const int k8 = k >> 3;
  const int have = m * k8;        // 16-byte pieces of x
  const int tot = 4 * NG * k8;    // 16-byte pieces of the LDS rows
  const uint4* xq = reinterpret_cast<const uint4*>(x);
  auto put = [&](int idx, const uint4& w) {
    const int v = idx / k8, i = idx - v * k8;
    *reinterpret_cast<uint4*>(xs + size_t(v) * xsn + 8 * i) = idx < have ? w : make_uint4(0u, 0u, 0u, 0u);
  };
  uint4 xr[kMXLoads];
#pragma unroll
  for (int u = 0; u < kMXLoads; ++u) xr[u] = xq[min(int(threadIdx.x) + u * kMThreads, have - 1)];
  // (a wave with no rows loads the clamped last row and never uses it)
  load(0);
#pragma unroll
  for (int u = 0; u < kMXLoads; ++u) asm volatile("" : "+v"(xr[u].x), "+v"(xr[u].y), "+v"(xr[u].z), "+v"(xr[u].w));
#pragma unroll
  for (int u = 0; u < kMXLoads; ++u) {
    const int idx = int(threadIdx.x) + u * kMThreads;
    if (idx < tot) put(idx, xr[u]);
  }
  // the rest (long rows, many vectors) in batches of eight loads in flight
  for (int base = int(threadIdx.x) + kMXLoads * kMThreads; base < tot; base += 8 * kMThreads) {
    uint4 r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) r[u] = xq[min(base + u * kMThreads, have - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (base + u * kMThreads < tot) put(base + u * kMThreads, r[u]);
  }
  // LDS writes done and visible; the weight loads above stay in flight
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  float acc[NG][4];
  float best[NG][4];  // head mode: best (sum, row) per vector over this lane's rows
  int bidx[NG][4];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[g][i] = 0.0f;
      best[g][i] = -INFINITY;
      bidx[g][i] = INT_MAX;
    }

  // After the last segment of a row group: sum the 16 lane groups (lanes
  // 4g + j for fixed j); lanes 0..3 hold the row group's results, vector
  // 4 * g + i of row j in acc[g][i].
  auto finish = [&](int u) {
    if (u % nseg == nseg - 1) {
      const int row = (rg_base + (u / nseg) * kMWaves) * 4 + j;
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = acc[g][i];
          s += __shfl_xor(s, 4);
          s += __shfl_xor(s, 8);
          s += __shfl_xor(s, 16);
          s += __shfl_xor(s, 32);
          const int v = 4 * g + i;
          if constexpr (MODE == kMultiGemv) {
            if (grp == 0 && row < n && v < m) y[size_t(v) * size_t(n) + row] = s * 0.0625f;
          } else {
            const float val = s * 0.0625f;
            if (row < n && v < m && better(val, row, best[g][i], bidx[g][i])) {
              best[g][i] = val;
              bidx[g][i] = row;
            }
          }
          acc[g][i] = 0.0f;
        }
    }
  };

  // One (row group, segment) step; with REFILL each block's registers are
  // reloaded for step u + 1 right after their last use. REFILL is a
  // compile-time flag (the last step is peeled off) so the refilled values
  // land in place instead of being copied, which would wait on their loads.
  auto step = [&](int u, auto refill_tag) {
    constexpr bool REFILL = decltype(refill_tag)::value;
    const int row_next = REFILL ? row_of(u + 1) : 0;
    const u32x4* np = reinterpret_cast<const u32x4*>(nib + size_t(row_next) * row_bytes);
    const uint16_t* sp = scl + size_t(row_next) * size_t(B);
#pragma unroll
    for (int t = 0; t < BPL; ++t) {
      const int b = block_of(u, t);
      if (FULL || b < B) {
        const uint32_t wd[4] = {q[t].x, q[t].y, q[t].z, q[t].w};
        const float d = float(__builtin_bit_cast(_Float16, sd[t]));
        f32x4_t c[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) c[g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
          // 16 * c for k = 8dd .. 8dd+7 in order, exact in bf16
          const u32x4 bw = codes16_bf16_pairs(wd[dd]);
          const short4_t b_lo = __builtin_bit_cast(short4_t, make_uint2(bw.x, bw.y));
          const short4_t b_hi = __builtin_bit_cast(short4_t, make_uint2(bw.z, bw.w));
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const uint4 xa = *reinterpret_cast<const uint4*>(xs + size_t(4 * g + j) * xsn + 32 * b + 8 * dd);
            const short4_t a_lo = __builtin_bit_cast(short4_t, make_uint2(xa.x, xa.y));
            const short4_t a_hi = __builtin_bit_cast(short4_t, make_uint2(xa.z, xa.w));
            c[g] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a_lo, b_lo, c[g], 0, 0, 0);
            c[g] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a_hi, b_hi, c[g], 0, 0, 0);
          }
        }
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[g][i] = fmaf(d, c[g][i], acc[g][i]);
        if constexpr (REFILL) {
          const int bn = block_of(u + 1, t);
          if (FULL || bn < B) {
            const u32x4 v = __builtin_nontemporal_load(np + bn);
            q[t] = make_uint4(v.x, v.y, v.z, v.w);
            sd[t] = sp[bn];
          }
        }
      }
    }
    finish(u);
  };
  for (int u = 0; u + 1 < units; ++u) step(u, std::true_type{});
  if (units > 0) step(units - 1, std::false_type{});

  if constexpr (MODE == kMultiHead) {
    // the workgroup's best (value, row) per vector into its partial slots
    __shared__ float sv[kMWaves][4 * NG];
    __shared__ int si[kMWaves][4 * NG];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float b = best[g][i];
        int bi = bidx[g][i];
        multi_wave_best(b, bi);
        if (lane == 0) {
          sv[wave][4 * g + i] = b;
          si[wave][4 * g + i] = bi;
        }
      }
    __syncthreads();
    if (int(threadIdx.x) < m) {
      const int v = threadIdx.x;
      float b = sv[0][v];
      int bi = si[0][v];
      for (int w = 1; w < kMWaves; ++w)
        if (better(sv[w][v], si[w][v], b, bi)) {
          b = sv[w][v];
          bi = si[w][v];
        }
      partials[size_t(blockIdx.x) * kMultiVecs + v] = make_uint2(__builtin_bit_cast(uint32_t, b), uint32_t(bi));
    }
  }
}

// Second launch of the multi-vector head and of the 64-token head:
// workgroup v reduces the partials of vector v (entries w * stride + v) and
// caps the winner (the cap is increasing, so capping the winner alone gives
// the capped maximum). Each thread issues its loads in batches of 16 before
// comparing; the comparator is a total order, so the order does not matter.
constexpr int kMRedBatch = 16;
__global__ __launch_bounds__(kMThreads) void argmax_partials_reduce_kernel(const uint2* __restrict__ partials,
                                                                           int g, int stride, float cap,
                                                                           int32_t* __restrict__ idx_out,
                                                                           float* __restrict__ val_out) {
  const int v = blockIdx.x;
  float best = -INFINITY;
  int bidx = INT_MAX;
  for (int base = 0; base < g; base += kMThreads * kMRedBatch) {
    uint2 p[kMRedBatch];
#pragma unroll
    for (int j = 0; j < kMRedBatch; ++j) {
      const int i = base + threadIdx.x + j * kMThreads;
      p[j] = i < g ? partials[size_t(i) * size_t(stride) + v]
                   : make_uint2(__builtin_bit_cast(uint32_t, -INFINITY), uint32_t(INT_MAX));
    }
#pragma unroll
    for (int j = 0; j < kMRedBatch; ++j) {
      const float pv = __builtin_bit_cast(float, p[j].x);
      const int pi = int(p[j].y);
      if (better(pv, pi, best, bidx)) {
        best = pv;
        bidx = pi;
      }
    }
  }
  multi_wave_best(best, bidx);
  __shared__ float sv[kMWaves];
  __shared__ int si[kMWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bidx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kMWaves; ++w)
      if (better(sv[w], si[w], best, bidx)) {
        best = sv[w];
        bidx = si[w];
      }
    if (bidx == INT_MAX) {
      idx_out[v] = -1;
      val_out[v] = __builtin_nanf("");
    } else {
      idx_out[v] = bidx;
      val_out[v] = cap > 0.0f ? cap * tanhf(best / cap) : best;
    }
  }
}

template <int NG, int MODE, bool FULL>
const void* pick_multi(int bpl) {
  switch (bpl) {
    case 1: return reinterpret_cast<const void*>(&q4_multi_kernel<1, NG, MODE, FULL>);
    case 2: return reinterpret_cast<const void*>(&q4_multi_kernel<2, NG, MODE, FULL>);
    case 3: return reinterpret_cast<const void*>(&q4_multi_kernel<3, NG, MODE, FULL>);
    case 4: return reinterpret_cast<const void*>(&q4_multi_kernel<4, NG, MODE, FULL>);
    case 5: return reinterpret_cast<const void*>(&q4_multi_kernel<5, NG, MODE, FULL>);
    case 6: return reinterpret_cast<const void*>(&q4_multi_kernel<6, NG, MODE, FULL>);
    default: return nullptr;
  }
}

int multi_blocks_per_cu(const void* fn, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, size_t, int>, int> cache;
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(fn, lds, dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kMThreads, lds) != hipSuccess || nb <= 0) nb = 1;
  cache[key] = nb;
  return nb;
}

// Largest LDS allocation one workgroup may make on the current device.
size_t max_lds_per_block_bytes() {
  int dev = 0, v = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0) v = 65536;
  return size_t(v);
}

struct MultiPlan {
  const void* fn;
  int nseg, ipw, grid;
  size_t lds;
};

template <int MODE>
MultiPlan multi_plan(int64_t n, int64_t k, int m) {
  MultiPlan p{};
  const int B = int(k / 32);
  p.nseg = (B + 16 * kMaxBpl - 1) / (16 * kMaxBpl);
  const int bpl = (B + 16 * p.nseg - 1) / (16 * p.nseg);
  const bool full = B == 16 * bpl * p.nseg;
  const int ng = (m + 3) / 4;
  p.fn = ng == 1 ? (full ? pick_multi<1, MODE, true>(bpl) : pick_multi<1, MODE, false>(bpl))
                 : (full ? pick_multi<2, MODE, true>(bpl) : pick_multi<2, MODE, false>(bpl));
  if (!p.fn) return p;
  p.lds = multi_mfma_lds_bytes(m, k);
  const int rg = int((n + 3) / 4);
  const int cus = device_cu_count();
  const int waves_max = cus * multi_blocks_per_cu(p.fn, p.lds) * kMWaves;
  p.ipw = (rg + waves_max - 1) / waves_max;
  const int waves = (rg + p.ipw - 1) / p.ipw;
  p.grid = (waves + kMWaves - 1) / kMWaves;
  return p;
}

int multi_run(const MultiPlan& p, const uint8_t* nib, const uint16_t* scl, int64_t n, int64_t k, const uint16_t* x,
              int m, float* y, uint2* partials, hipStream_t stream, const char* name) {
  int ni = int(n), ki = int(k), mi = m, ns = p.nseg, ip = p.ipw;
  void* args[] = {&nib, &scl, &x, &ni, &ki, &mi, &ns, &ip, &y, &partials};
  hipError_t e = hipLaunchKernel(p.fn, dim3(p.grid), dim3(kMThreads), args, p.lds, stream);
  if (e != hipSuccess) return fail(Q4DEC_ERR_HIP, "%s: kernel launch failed: %s", name, hipGetErrorString(e));
  return launch_status(name);
}

}  // namespace

void reduce_argmax_partials(const uint2* partials, int g, int stride, int nvec, float cap, int32_t* idx_out,
                            float* val_out, hipStream_t st) {
  hipLaunchKernelGGL(argmax_partials_reduce_kernel, dim3(unsigned(nvec)), dim3(kMThreads), 0, st, partials, g, stride,
                     cap, idx_out, val_out);
}

size_t multi_mfma_lds_bytes(int m, int64_t k) {
  const int ng = (m + 3) / 4;
  return size_t(4 * ng) * size_t(x_stride(int(k))) * 2;
}

int multi_mfma_launch(const uint8_t* nib, const uint16_t* scl, int64_t n, int64_t k, const uint16_t* x, int m,
                      float* y, hipStream_t stream) {
  const MultiPlan p = multi_plan<kMultiGemv>(n, k, m);
  if (!p.fn) return fail(Q4DEC_ERR_UNSUPPORTED, "q4_gemv_multi: no kernel for k=%lld", (long long)k);
  return multi_run(p, nib, scl, n, k, x, m, y, nullptr, stream, "q4_gemv_multi");
}

}  // namespace q4dec

extern "C" size_t lmhead_multi_workspace_bytes(int64_t vocab, int64_t k, int64_t m) {
  (void)vocab;
  (void)k;
  (void)m;
  return size_t(q4dec::kMultiPartials) * q4dec::kMultiVecs * sizeof(uint2);
}

extern "C" int lmhead_softcap_argmax_multi(const void* packed, int64_t vocab, int64_t k, const uint16_t* x,
                                           int64_t m, float cap, void* ws, size_t ws_bytes, int32_t* idx_out,
                                           float* val_out, void* stream) {
  using namespace q4dec;
  const char* name = "lmhead_softcap_argmax_multi";
  if (!packed) return fail(Q4DEC_ERR_NULL, "%s: packed is NULL", name);
  if (!x) return fail(Q4DEC_ERR_NULL, "%s: x is NULL", name);
  if (!ws) return fail(Q4DEC_ERR_NULL, "%s: ws is NULL", name);
  if (!idx_out) return fail(Q4DEC_ERR_NULL, "%s: idx_out is NULL", name);
  if (!val_out) return fail(Q4DEC_ERR_NULL, "%s: val_out is NULL", name);
  if (vocab <= 0 || vocab >= (int64_t(1) << 31))
    return fail(Q4DEC_ERR_SHAPE, "%s: vocab must be in [1, 2^31) (got %lld)", name, (long long)vocab);
  if (k <= 0 || k % 32)
    return fail(Q4DEC_ERR_SHAPE, "%s: k must be a positive multiple of 32 (got %lld)", name, (long long)k);
  if (k > Q4DEC_MAX_K)
    return fail(Q4DEC_ERR_UNSUPPORTED, "%s: k must be <= %d (got %lld)", name, Q4DEC_MAX_K, (long long)k);
  if (m < 1 || m > kMultiVecs)
    return fail(Q4DEC_ERR_SHAPE, "%s: m must be in [1, %d] (got %lld)", name, kMultiVecs, (long long)m);
  if (!aligned(packed, 16)) return fail(Q4DEC_ERR_ALIGN, "%s: packed must be 16-byte aligned", name);
  if (!aligned(x, 16)) return fail(Q4DEC_ERR_ALIGN, "%s: x must be 16-byte aligned", name);
  if (!aligned(ws, 8)) return fail(Q4DEC_ERR_ALIGN, "%s: ws must be 8-byte aligned", name);
  if (!aligned(idx_out, 4) || !aligned(val_out, 4))
    return fail(Q4DEC_ERR_ALIGN, "%s: idx_out and val_out must be 4-byte aligned", name);
  const size_t need = lmhead_multi_workspace_bytes(vocab, k, m);
  if (ws_bytes < need) return fail(Q4DEC_ERR_WORKSPACE, "%s: ws_bytes %zu < required %zu", name, ws_bytes, need);
  const size_t lds = multi_mfma_lds_bytes(int(m), k);
  if (lds > max_lds_per_block_bytes())
    return fail(Q4DEC_ERR_UNSUPPORTED, "%s: m * k too large (%zu bytes of LDS, device allows %zu)", name, lds,
                max_lds_per_block_bytes());
  const MultiPlan p = multi_plan<kMultiHead>(vocab, k, int(m));
  if (!p.fn) return fail(Q4DEC_ERR_UNSUPPORTED, "%s: no kernel for k=%lld", name, (long long)k);
  if (p.grid > kMultiPartials) return fail(Q4DEC_ERR_UNSUPPORTED, "%s: too many workgroups", name);
  const uint8_t* nib = static_cast<const uint8_t*>(packed);
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(nib + nib_plane_bytes(vocab, k));
  uint2* partials = static_cast<uint2*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int rc = multi_run(p, nib, scl, vocab, k, x, int(m), nullptr, partials, st, name);
  if (rc) return rc;
  reduce_argmax_partials(partials, p.grid, kMultiVecs, int(m), cap, idx_out, val_out, st);
  return launch_status(name);
}
