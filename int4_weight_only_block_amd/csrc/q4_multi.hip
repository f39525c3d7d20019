// q4_multi: multi-vector q4_0 GEMV on the matrix cores, y[v, r] = W[r, :] .
// x[v, :] for 2 <= m <= 8 activation vectors ("visible-cx/gemma-4-E2B-CoreAI",
// speculative verify: the weights are read once for the few rows a verify
// step checks).
//
// Mapping. v_mfma_f32_4x4x4_16b_f16 runs 16 independent 4x4x4 products per
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
// Codes. q4_pack's dword d of a block unpacks (fp16 magic number) into the
// consecutive k pairs 8d .. 8d+7, so one MFMA takes 4 codes in k order and the
// matching 4 activations straight from LDS, where each vector is stored as
// fp16 in k order, scaled by one power of two per vector (its largest bf16
// exponent lands at 2^14, as the prefill GEMM's per-token factor).
#include <math.h>

#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>

#include "q4dec_internal.h"

namespace q4dec {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMWaves = 4;
constexpr int kMThreads = 64 * kMWaves;
constexpr int kMaxBpl = 6;  // blocks per lane per row segment

// halves per activation row in LDS: k plus 8 (16 bytes), so the 4 vectors a
// 4-lane group reads sit in different bank quads
__device__ __host__ inline int x_stride(int k) { return k + 8; }

template <int BPL, int NG, bool FULL>
__global__ __launch_bounds__(kMThreads) void q4_multi_kernel(const uint8_t* __restrict__ nib,
                                                             const uint16_t* __restrict__ scl,
                                                             const uint16_t* __restrict__ x, int n, int k, int m,
                                                             int nseg, int ipw, float* __restrict__ y) {
  extern __shared__ uint32_t dyn_lds[];
  const int B = k >> 5;
  const int xsn = x_stride(k);
  _Float16* xs = reinterpret_cast<_Float16*>(dyn_lds);  // [4 * NG][xsn]
  __shared__ uint32_t red[kMWaves][4 * NG];
  __shared__ float ef[4 * NG];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 2;  // which of the 16 blocks of a step
  const int j = lane & 3;     // weight row of the 4-row group, and activation vector within a group of 4
  const int RG = (n + 3) / 4;
  const int rg_base = blockIdx.x * kMWaves * ipw + wave;
  const int iters = rg_base < RG ? min(ipw, (RG - rg_base + kMWaves - 1) / kMWaves) : 0;
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
  // the first weights do not depend on x: in flight before the staging
  if (units > 0) load(0);

  // Stage x: the raw bf16 rows go to LDS while each vector's largest bf16
  // exponent is found; then each row is rewritten in place as fp16 scaled by
  // the power of two that puts its largest value at 2^14 (x is read from
  // memory once). Rows v >= m are zeros.
  const int k8 = k >> 3;
  for (int v = 0; v < m; ++v) {
    const uint4* s4 = reinterpret_cast<const uint4*>(x + size_t(v) * size_t(k));
    uint32_t emax = 1;
    for (int i = threadIdx.x; i < k8; i += kMThreads) {
      const uint4 w = s4[i];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) emax = max(emax, max((ws[e] >> 7) & 0xFFu, (ws[e] >> 23) & 0xFFu));
      *reinterpret_cast<uint4*>(xs + size_t(v) * xsn + 8 * i) = w;
    }
    for (int off = 32; off >= 1; off >>= 1) emax = max(emax, uint32_t(__shfl_xor(int(emax), off)));
    if (lane == 0) red[wave][v] = emax;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 4 * NG * k8; idx += kMThreads) {
    const int v = idx / k8, i = idx - v * k8;
    uint4* slot = reinterpret_cast<uint4*>(xs + size_t(v) * xsn + 8 * i);
    uint4 o = make_uint4(0u, 0u, 0u, 0u);
    if (v < m) {
      const uint32_t emax = max(max(red[0][v], red[1][v]), max(red[2][v], red[3][v]));
      const int e = int(emax) - 127 - 14;
      const uint4 w = *slot;
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      uint32_t h[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const half2_t p = {(_Float16)ldexpf(bf16_to_f32(ws[c] & 0xFFFFu), -e),
                           (_Float16)ldexpf(bf16_to_f32(ws[c] >> 16), -e)};
        h[c] = __builtin_bit_cast(uint32_t, p);
      }
      o = make_uint4(h[0], h[1], h[2], h[3]);
      if (i == 0) ef[v] = ldexpf(1.0f, e);
    }
    *slot = o;
  }
  // LDS writes done and visible; the weight loads above stay in flight
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  uint32_t m_lo, m_hi, magic;
  asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(m_lo));
  asm volatile("v_mov_b32 %0, 0x00F000F0" : "=v"(m_hi));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

  float acc[NG][4];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[g][i] = 0.0f;

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
          const CodePairs cp = unpack_dword(wd[dd], m_lo, m_hi, magic);  // k = 8dd .. 8dd+7 in order
          const half4_t b_lo = {cp.p[0][0], cp.p[0][1], cp.p[1][0], cp.p[1][1]};
          const half4_t b_hi = {cp.p[2][0], cp.p[2][1], cp.p[3][0], cp.p[3][1]};
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const uint4 xa = *reinterpret_cast<const uint4*>(xs + size_t(4 * g + j) * xsn + 32 * b + 8 * dd);
            const half4_t a_lo = __builtin_bit_cast(half4_t, make_uint2(xa.x, xa.y));
            const half4_t a_hi = __builtin_bit_cast(half4_t, make_uint2(xa.z, xa.w));
            c[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(a_lo, b_lo, c[g], 0, 0, 0);
            c[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(a_hi, b_hi, c[g], 0, 0, 0);
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
    if (u % nseg == nseg - 1) {
      // sum the 16 lane groups (lanes 4g + j for fixed j); lanes 0..3 hold
      // the row group's results, vector 4 * g + i of row j in acc[g][i]
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
          if (grp == 0 && row < n && v < m) y[size_t(v) * size_t(n) + row] = s * ef[v];
          acc[g][i] = 0.0f;
        }
    }
  };
  for (int u = 0; u + 1 < units; ++u) step(u, std::true_type{});
  if (units > 0) step(units - 1, std::false_type{});
}

template <int NG, bool FULL>
const void* pick_multi(int bpl) {
  switch (bpl) {
    case 1: return reinterpret_cast<const void*>(&q4_multi_kernel<1, NG, FULL>);
    case 2: return reinterpret_cast<const void*>(&q4_multi_kernel<2, NG, FULL>);
    case 3: return reinterpret_cast<const void*>(&q4_multi_kernel<3, NG, FULL>);
    case 4: return reinterpret_cast<const void*>(&q4_multi_kernel<4, NG, FULL>);
    case 5: return reinterpret_cast<const void*>(&q4_multi_kernel<5, NG, FULL>);
    case 6: return reinterpret_cast<const void*>(&q4_multi_kernel<6, NG, FULL>);
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

}  // namespace

size_t multi_mfma_lds_bytes(int m, int64_t k) {
  const int ng = (m + 3) / 4;
  return size_t(4 * ng) * size_t(x_stride(int(k))) * 2;
}

int multi_mfma_launch(const uint8_t* nib, const uint16_t* scl, int64_t n, int64_t k, const uint16_t* x, int m,
                      float* y, hipStream_t stream) {
  const int B = int(k / 32);
  const int nseg = (B + 16 * kMaxBpl - 1) / (16 * kMaxBpl);
  const int bpl = (B + 16 * nseg - 1) / (16 * nseg);
  const bool full = B == 16 * bpl * nseg;
  const int ng = (m + 3) / 4;
  const void* fn = ng == 1 ? (full ? pick_multi<1, true>(bpl) : pick_multi<1, false>(bpl))
                           : (full ? pick_multi<2, true>(bpl) : pick_multi<2, false>(bpl));
  if (!fn) return fail(Q4DEC_ERR_UNSUPPORTED, "q4_gemv_multi: no kernel for k=%lld", (long long)k);
  const size_t lds = multi_mfma_lds_bytes(m, k);
  const int rg = int((n + 3) / 4);
  const int cus = device_cu_count();
  const int waves_max = cus * multi_blocks_per_cu(fn, lds) * kMWaves;
  int ipw = (rg + waves_max - 1) / waves_max;
  // every workgroup stages all m vectors: a wave walks up to three row
  // groups while the grid still covers 80% of the CUs, to spread that cost
  for (int want = 3; want > ipw; --want) {
    const int64_t g = ((rg + want - 1) / want + kMWaves - 1) / kMWaves;
    if (g * 5 >= int64_t(cus) * 4) {
      ipw = want;
      break;
    }
  }
  const int waves = (rg + ipw - 1) / ipw;
  const int grid = (waves + kMWaves - 1) / kMWaves;
  int ni = int(n), ki = int(k), mi = m, ns = nseg, ip = ipw;
  void* args[] = {&nib, &scl, &x, &ni, &ki, &mi, &ns, &ip, &y};
  hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(kMThreads), args, lds, stream);
  if (e != hipSuccess) return fail(Q4DEC_ERR_HIP, "q4_gemv_multi: kernel launch failed: %s", hipGetErrorString(e));
  return launch_status("q4_gemv_multi");
}

}  // namespace q4dec
