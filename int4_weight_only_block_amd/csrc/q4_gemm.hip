// q4_gemm_s64: S<=64 chunked-prefill product Y[s, r] = sum_k X[s, k] * w[r, k]
// on the matrix cores ("visible-cx/gemma-4-E2B-CoreAI": the prefill entry
// point has a static query width of 64 and reads the weights once per 64
// tokens).
//
// Numerics. Codes and activations meet in v_mfma_f32_16x16x32_bf16, one MFMA
// per 32-wide block and 16x16 (token, row) tile: the B operand holds 16 * c
// for the block's codes (exact in bf16), the A operand the activations as
// stored (bf16), so every product is exact and the matrix core sums one
// block in fp32. Each block's tile is then folded into fp32 accumulators
// with the row's scale d, one FMA per output and block, and the factor 1/16
// is applied once at the end (exact). There is no activation conversion and
// no range limit on X beyond fp32's own.
//
// Codes. q4_pack's dword q of a block holds the codes of k = 8q .. 8q+7,
// which is one lane's B operand (lane group q supplies k = 8q .. 8q+7 of the
// MFMA's 32). XOR with 0x88888888 turns the nibbles into 4-bit two's
// complement codes; moved to the top half of each byte they read as signed
// bytes 16 * c, which convert to fp32 one byte at a time and to bf16 in
// pairs.
//
// Work split. When k is a multiple of 256 (every model shape) the chunked
// kernel runs: the 4 waves of a workgroup own consecutive groups of rows and
// share each chunk of 8 blocks of activations through LDS, whole 16-byte
// blocks of codes are loaded two chunks ahead and transposed across lane
// groups for the MFMAs (see below). Otherwise a workgroup owns one row tile
// and its 4 waves take quarters of its K range, adding their partial tiles
// in LDS in a fixed order. Matrices with too few row tiles to occupy the
// chip also split K across workgroups: their partial tiles go to the
// workspace and a second kernel adds them in slice order, so results are
// deterministic.
//
// The same kernel, with an argmax epilogue instead of the output store, is
// the LM head over a chunk of up to 64 tokens: each workgroup keeps, per
// token, the best (logit, row) of its rows, and a second launch reduces
// those per token and caps the winner, so no logits are written.
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "q4_codes.h"
#include "q4dec_internal.h"

namespace q4dec {
Q4DEC_DEBUG_READER(q4_gemm)

typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kTok = 64;   // token slots
constexpr int kChunk = 8;  // blocks per activation chunk of the chunked kernel
constexpr int kGWaves = 4;
constexpr int kGThreads = 64 * kGWaves;

struct GemmPlan {
  bool chunked;  // k % 256 == 0: the chunked kernel (rows per workgroup = 64 * sub + 16 * extra)
  int sub;       // 16-row MFMA tiles per wave
  int extra;     // chunked, sub 1: a fifth 16-row tile whose blocks the four waves share
  int tiles;     // row tiles
  int slices;    // K slices across workgroups
  int bps;       // blocks per slice
  size_t total;  // workspace bytes (partials of split matrices)
};

// what the kernel does with its output tile
enum GemmMode : int {
  kGemmOut = 0,     // Y[s, r] (fp32)
  kGemmSlices = 1,  // the K slice's partial Y into the workspace
  kGemmHead = 2,    // per token, the tile's best (logit, row) into the workspace
};

// Row tile width and K split, from timings of the model shapes on MI355X.
// Very tall matrices (the heads) take two 16-row tiles per wave; otherwise
// one. When the row tiles alone give fewer workgroups than CUs, K is split
// across workgroups so that about one workgroup runs per CU (smaller splits
// leave CUs idle; larger ones gain nothing and add partial-sum traffic).
static GemmPlan gemm_plan_rows(int64_t n, int64_t k, bool split, int extra);

// The chunked kernel with one 16-row tile per wave can take a fifth tile per
// workgroup, its blocks shared out among the four waves (each wave 1.25 times
// the work). Without a K split it is taken when it lowers the resident
// rounds times the work per workgroup: the E4B gate+up runs 256 workgroups
// of 80 rows in one round instead of 320 of 64 in two (27.7 to 24.6-25.0 us).
// Split shapes keep 64 rows: the E4B down as 8 slices of 80-row tiles took
// 19.6-19.8 us against 18.1 as 6 slices of 64-row tiles.
static GemmPlan gemm_plan(int64_t n, int64_t k, bool split = true) {
  const GemmPlan p0 = gemm_plan_rows(n, k, split, 0);
  if (!p0.chunked || p0.sub != 1 || !split || p0.slices != 1) return p0;
  const GemmPlan p1 = gemm_plan_rows(n, k, split, 1);
  if (p1.slices != 1) return p0;
  const int64_t cus = std::max(1, device_cu_count());
  auto cost = [&](const GemmPlan& p) {
    const int64_t rounds = (int64_t(p.tiles) * p.slices + cus - 1) / cus;
    return double(rounds) * p.bps * (4 + p.extra);
  };
  return cost(p1) < cost(p0) ? p1 : p0;
}

static GemmPlan gemm_plan_rows(int64_t n, int64_t k, bool split, int extra) {
  const int64_t B = k / 32;
  const int64_t cus = std::max(1, device_cu_count());
  GemmPlan p{};
  p.chunked = B % kChunk == 0;
  // rows per workgroup: chunked 64 * sub (4 waves side by side), otherwise
  // 16 * sub (4 waves over K quarters)
  const int64_t base = p.chunked ? 64 : 16;
  const int subs[3] = {p.chunked ? 2 : 4, p.chunked ? 1 : 2, 1};
  p.sub = subs[2];
  if ((n + base * subs[0] - 1) / (base * subs[0]) >= 2 * cus)
    p.sub = subs[0];
  else if ((n + base * subs[1] - 1) / (base * subs[1]) >= cus)
    p.sub = subs[1];
  p.extra = extra;
  const int64_t rows = base * p.sub + 16 * p.extra;
  p.tiles = int((n + rows - 1) / rows);
  int64_t want = 1;
  if (split && p.tiles < cus) {
    const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(16, B / (p.chunked ? 2 * kChunk : 8)));
    want = std::min<int64_t>(smax, std::max<int64_t>(1, (cus + p.tiles / 2) / p.tiles));
  }
  const int64_t unit = p.chunked ? kChunk : 1;
  p.bps = int(((B + want - 1) / want + unit - 1) / unit * unit);
  p.slices = int((B + p.bps - 1) / p.bps);
  p.total = p.slices > 1 ? align256(size_t(p.slices) * kTok * size_t(n) * 4) : 256;
  return p;
}

// One block's registers for one lane: the activations of its 4 token tiles
// (A operands) and, per row tile, the code dword and the fp16 scale.
template <int SUB>
struct BlockRegs {
  uint4 a[4];
  uint32_t w[SUB];
  uint32_t s[SUB];
};

template <int SUB, int MODE>
__global__ __launch_bounds__(kGThreads) void q4_gemm_kernel(const uint8_t* __restrict__ nib,
                                                            const uint16_t* __restrict__ scl,
                                                            const uint16_t* __restrict__ x, int n, int k, int n_tok,
                                                            int bps, void* __restrict__ out) {
  constexpr int kRows = 16 * SUB;
  __shared__ float4_t red[2][SUB * 4][64];  // two partial tiles (SUB = 4: 32 KB)
  const int B = k >> 5;
  Q4_DCHECK(bps > 0 && int64_t(gridDim.y) * bps >= B && int64_t(gridDim.y - 1) * bps < B, kDbgGemmSlices);
  Q4_DCHECK(int64_t(gridDim.x) * kRows >= n, kDbgGemmTiles);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;    // lane group: k = 8q .. 8q+7 of a block; tokens 4q .. 4q+3 of a C tile
  const int col = lane & 15;  // row of a 16-row tile (B, C) and token of a 16-token tile (A)

  // this wave's K range: a quarter of the workgroup's slice (may be empty)
  const int s0 = blockIdx.y * bps;
  const int s1 = min(B, s0 + bps);
  const int per = (s1 - s0 + kGWaves - 1) / kGWaves;
  const int wb0 = min(s1, s0 + wave * per);
  const int wb1 = min(s1, wb0 + per);

  // Byte offsets from uniform bases (the tile's first row, the call's first
  // token), so each load is a scalar base plus a 32-bit lane offset.
  const int r0 = blockIdx.x * kRows;
  const uint8_t* wt = nib + size_t(r0) * size_t(k >> 1);
  const uint8_t* st = reinterpret_cast<const uint8_t*>(scl) + size_t(r0) * size_t(B) * 2;
  const uint8_t* xt = reinterpret_cast<const uint8_t*>(x);
  uint32_t woff[SUB], soff[SUB], xoff[4];
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    const int rl = min(r0 + 16 * u + col, n - 1) - r0;  // rows past n repeat the last row; never stored
    woff[u] = uint32_t(rl) * uint32_t(k >> 1) + 4u * uint32_t(q);
    soff[u] = uint32_t(rl) * uint32_t(B) * 2u;
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int tok = min(16 * m + col, n_tok - 1);  // slots past n_tok repeat a real token; never stored
    xoff[m] = (uint32_t(tok) * uint32_t(k) + 8u * uint32_t(q)) * 2u;
  }

  // a block past the wave's range reloads its last block (cache hits) and is
  // never computed
  const int blast = wb1 > wb0 ? wb1 - 1 : min(wb0, B - 1);
  auto load = [&](BlockRegs<SUB>& R, int b) {
    const uint32_t bc = uint32_t(min(b, blast));
#pragma unroll
    for (int m = 0; m < 4; ++m) R.a[m] = *reinterpret_cast<const uint4*>(xt + size_t(bc * 64u) + xoff[m]);
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      R.w[u] = *reinterpret_cast<const uint32_t*>(wt + size_t(bc * 16u) + woff[u]);
      R.s[u] = *reinterpret_cast<const uint16_t*>(st + size_t(bc * 2u) + soff[u]);
    }
  };

  float4_t acc[SUB][4];
#pragma unroll
  for (int u = 0; u < SUB; ++u)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[u][m] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](const BlockRegs<SUB>& R) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const float d = float(__builtin_bit_cast(_Float16, uint16_t(R.s[u])));
      const bf16x8_t bc = codes16_bf16(R.w[u]);
      float4_t c[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        c[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, R.a[m]), bc,
                                                       float4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[u][m][i] = fmaf(d, c[m][i], acc[u][m][i]);
    }
  };

  // two blocks in flight: ra holds blocks wb0, wb0 + 2, ..., rb the odd ones;
  // each set is refilled two blocks ahead right after its use. The loop body
  // has no condition, so every refill feeds an unconditional use and stays
  // where it is issued; an odd last block runs after the loop.
  BlockRegs<SUB> ra, rb;
  load(ra, wb0);
  load(rb, wb0 + 1);
  int b = wb0;
  // the scheduling fences keep each refill where it is written: left to
  // itself the scheduler sinks loads next to their use
  for (; b + 1 < wb1; b += 2) {
    compute(ra);
    __builtin_amdgcn_sched_barrier(0);
    load(ra, b + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(rb);
    __builtin_amdgcn_sched_barrier(0);
    load(rb, b + 3);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (b < wb1) compute(ra);

  // partial tiles of the 4 waves, added as (w0 + w2) + (w1 + w3)
  if (wave < 2) {
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int m = 0; m < 4; ++m) red[wave][4 * u + m][lane] = acc[u][m];
  }
  __syncthreads();
  if (wave >= 2) {
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int m = 0; m < 4; ++m) red[wave - 2][4 * u + m][lane] += acc[u][m];
  }
  __syncthreads();
  // wave w finishes token tile m = w for every row tile: lane holds tokens
  // 16w + 4q + i of rows r0 + 16u + col
  float4_t v[SUB];
#pragma unroll
  for (int u = 0; u < SUB; ++u) v[u] = (red[0][4 * u + wave][lane] + red[1][4 * u + wave][lane]) * 0.0625f;

  if constexpr (MODE == kGemmHead) {
    uint2* part = static_cast<uint2*>(out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float bv = -INFINITY;
      int br = INT_MAX;
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const int row = r0 + 16 * u + col;
        const float val = v[u][i];
        if (row < n && !(val != val) && better(val, row, bv, br)) {  // NaN never wins
          bv = val;
          br = row;
        }
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {  // the 16 lanes of the lane group
        const float ov = __shfl_xor(bv, off);
        const int orow = __shfl_xor(br, off);
        if (better(ov, orow, bv, br)) {
          bv = ov;
          br = orow;
        }
      }
      const int s = 16 * wave + 4 * q + i;
      if (col == 0 && s < n_tok)
        part[size_t(blockIdx.x) * kTok + s] = make_uint2(__builtin_bit_cast(uint32_t, bv), uint32_t(br));
    }
  } else {
    float* y = static_cast<float*>(out);
    if (MODE == kGemmSlices) y += size_t(blockIdx.y) * kTok * size_t(n);
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int row = r0 + 16 * u + col;
      if (row >= n) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * wave + 4 * q + i;
        if (s < n_tok) y[size_t(s) * size_t(n) + row] = v[u][i];
      }
    }
  }
}


// --------------------------------------------------------- chunked kernel
// For k a multiple of 256 (8 blocks): the 4 waves of a workgroup own
// consecutive groups of 16 * SUB rows and walk the same K range, so the
// activations of a chunk of 8 blocks are loaded once per workgroup and
// shared through LDS. A lane loads whole 16-byte blocks (lane group q: block
// 4h + q of its row) and the 8 scales of its row for the chunk in one
// 16-byte load; a 4 x 4 transpose across the lane groups then gives each
// lane the dword of every block that its MFMA needs. The next chunk's
// activations and the chunk after that's weights are in flight while a
// chunk runs (the activations are issued first, so waiting for them does
// not wait for the weights issued after them).
// LDS slot of activation quarter qq of token tok, swizzled so that the 16
// lanes of one ds_read_b128 (16 tokens, one quarter) hit distinct banks.
__device__ __forceinline__ int xslot(int tok, int qq) { return qq ^ ((tok >> 2) & 3); }

// On entry lane group g holds dword j of block g in r[j]; on exit lane group
// g holds dword g of block j in r[j], which is block j's B operand.
__device__ __forceinline__ void transpose_groups(uint32_t (&r)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);  // groups 0,1 <-> 2,3
  const auto b = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);  // groups 0 <-> 1, 2 <-> 3
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r[0] = c[0];
  r[1] = c[1];
  r[2] = d[0];
  r[3] = d[1];
}

struct ChunkX {
  u32x4 v[kChunk];  // thread t: token t / 4, quarter t % 4 of each block of a chunk
};

// A copy of v in a register of its own, made where it is written: the
// register set it came from is refilled right after, and the refill then
// lands in that set's registers instead of being moved back at the end of
// the loop (which would wait for it), and the uses of the copy cannot be
// hoisted into the previous chunk (which would wait for its loads early).
__device__ __forceinline__ uint32_t fresh_copy(uint32_t v) {
  uint32_t o;
  asm volatile("v_mov_b32 %0, %1" : "=&v"(o) : "v"(v));
  return o;
}

template <int SUB, int EXTRA>
struct ChunkW {
  u32x4 w[SUB][2];  // lane group q: block 4h + q of the lane's row, h = 0, 1
  u32x4 sc[SUB];    // the row's 8 fp16 scales of the chunk
  // the shared fifth tile: the wave's blocks wave and wave + 4 of the chunk,
  // dword q of the lane's row of that tile, and their fp16 scales
  uint32_t ew[EXTRA ? 2 : 1];
  uint16_t es[EXTRA ? 2 : 1];
};

template <int SUB, int MODE, int EXTRA>
__global__ __launch_bounds__(kGThreads) void q4_gemm_chunk_kernel(const uint8_t* __restrict__ nib,
                                                                  const uint16_t* __restrict__ scl,
                                                                  const uint16_t* __restrict__ x, int n, int k,
                                                                  int n_tok, int bps, void* __restrict__ out) {
  __shared__ u32x4 xs[kChunk][kTok][4];  // [block][token][quarter, swizzled], 32 KB
  const int B = k >> 5;
  Q4_DCHECK(B % kChunk == 0 && bps > 0 && bps % kChunk == 0, kDbgGemmChunks);
  Q4_DCHECK(int64_t(gridDim.y) * bps >= B && int64_t(gridDim.y - 1) * bps < B, kDbgGemmSlices);
  Q4_DCHECK(int64_t(gridDim.x) * (64 * SUB + 16 * EXTRA) >= n, kDbgGemmTiles);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int col = lane & 15;
  const int b_begin = blockIdx.y * bps;
  const int nch = (min(B, b_begin + bps) - b_begin) / kChunk;  // >= 1: B and bps are multiples of 8
  const int rwg = blockIdx.x * (64 * SUB + 16 * EXTRA);          // the workgroup's first row
  const int r0 = rwg + wave * 16 * SUB;                          // the wave's first row
  const int re = rwg + 64 * SUB;                                 // the shared tile's first row

  const uint8_t* wrow[SUB];
  const uint8_t* srow[SUB];
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    const int rc = min(r0 + 16 * u + col, n - 1);  // rows past n repeat the last row; never stored
    wrow[u] = nib + size_t(rc) * size_t(k >> 1) + 16 * q;
    srow[u] = reinterpret_cast<const uint8_t*>(scl) + size_t(rc) * size_t(B) * 2;
  }
  const int rce = min(re + col, n - 1);
  const uint8_t* wrow_e = nib + size_t(rce) * size_t(k >> 1) + 4 * q;
  const uint16_t* srow_e = scl + size_t(rce) * size_t(B);
  // activation staging: thread t holds token t / 4, quarter t % 4 of each block
  const int sx = threadIdx.x >> 2, qq = threadIdx.x & 3;
  const uint8_t* xrow = reinterpret_cast<const uint8_t*>(x) + size_t(min(sx, n_tok - 1)) * size_t(k) * 2 + 16 * qq;

  auto load_w = [&](ChunkW<SUB, EXTRA>& R, int ci) {
    const size_t b0 = size_t(b_begin + ci * kChunk);
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h) R.w[u][h] = *reinterpret_cast<const u32x4*>(wrow[u] + (b0 + 4 * h) * 16);
      R.sc[u] = *reinterpret_cast<const u32x4*>(srow[u] + b0 * 2);
    }
#pragma unroll
    for (int h = 0; h < EXTRA * 2; ++h) {
      R.ew[h] = *reinterpret_cast<const uint32_t*>(wrow_e + (b0 + 4 * h + wave) * 16);
      R.es[h] = srow_e[b0 + 4 * h + wave];
    }
  };
  auto load_x = [&](ChunkX& X, int ci) {
    const size_t b0 = size_t(b_begin + ci * kChunk);
#pragma unroll
    for (int c = 0; c < kChunk; ++c) X.v[c] = *reinterpret_cast<const u32x4*>(xrow + (b0 + c) * 64);
  };

  float4_t acc[SUB][4];
#pragma unroll
  for (int u = 0; u < SUB; ++u)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[u][m] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float4_t acc_e[EXTRA ? 4 : 1];
#pragma unroll
  for (int m = 0; m < (EXTRA ? 4 : 1); ++m) acc_e[m] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto load_a = [&](u32x4 (&a)[4], int c) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int tok = 16 * m + col;
      a[m] = xs[c][tok][xslot(tok, q)];
    }
  };

  // One chunk: stage its activations into LDS, take the weights out of the
  // register set (transposed), refill the set two chunks ahead and the
  // activation staging one chunk ahead, then run the 8 blocks.
  auto run = [&](ChunkW<SUB, EXTRA>& R, ChunkX& X, int ci) {
    __syncthreads();  // every wave is done with the previous chunk
#pragma unroll
    for (int c = 0; c < kChunk; ++c) xs[c][sx][xslot(sx, qq)] = X.v[c];
    uint32_t wt[SUB][2][4];
    uint32_t sc[SUB][4];
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = fresh_copy(R.w[u][h][j]);
        transpose_groups(r);
#pragma unroll
        for (int j = 0; j < 4; ++j) wt[u][h][j] = r[j];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[u][j] = fresh_copy(R.sc[u][j]);
    }
    uint32_t ewt[EXTRA ? 2 : 1], est[EXTRA ? 2 : 1];
#pragma unroll
    for (int h = 0; h < 2 * EXTRA; ++h) {
      ewt[h] = fresh_copy(R.ew[h]);
      est[h] = fresh_copy(R.es[h]);
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    load_x(X, ci + 1 < nch ? ci + 1 : ci);  // past the end: this chunk again (cache hits, never used)
    load_w(R, ci + 2 < nch ? ci + 2 : ci);
    __builtin_amdgcn_sched_barrier(0);
    // The chunk as a fixed sequence of steps: its 8 blocks of the wave's own
    // tiles, then (fifth tile) the wave's two blocks of the shared tile. The
    // activations of step s + 2 are read from LDS while step s is issued,
    // and step s's products are folded after step s + 1's MFMAs are issued,
    // so the wave waits on neither the LDS nor the matrix cores' latency.
    // Every accumulator still takes its blocks in K order.
    constexpr int NS = kChunk + 2 * EXTRA;
    u32x4 a[3][4];
    float4_t pr[2][SUB][4];
    float pd[2][SUB];
    auto ablock = [&](int s) { return s < kChunk ? s : 4 * (s - kChunk) + wave; };
    auto issue = [&](int s, float4_t (&r)[SUB][4], float (&d)[SUB]) {
      const u32x4 (&av)[4] = a[s % 3];
      if (s < kChunk) {
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
          const bf16x8_t bc = codes16_bf16(wt[u][s >> 2][s & 3]);
          const uint32_t sw = sc[u][s >> 1];
          d[u] = float(__builtin_bit_cast(_Float16, uint16_t((s & 1) ? sw >> 16 : sw & 0xFFFFu)));
#pragma unroll
          for (int m = 0; m < 4; ++m)
            r[u][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[m]), bc,
                                                              float4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        }
      } else {
        const bf16x8_t bc = codes16_bf16(ewt[(s - kChunk) & 1]);
        d[0] = float(__builtin_bit_cast(_Float16, uint16_t(est[(s - kChunk) & 1])));
#pragma unroll
        for (int m = 0; m < 4; ++m)
          r[0][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[m]), bc,
                                                            float4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
      }
    };
    auto fold = [&](int s, const float4_t (&r)[SUB][4], const float (&d)[SUB]) {
      if (s < kChunk) {
#pragma unroll
        for (int u = 0; u < SUB; ++u)
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[u][m][i] = fmaf(d[u], r[u][m][i], acc[u][m][i]);
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc_e[m][i] = fmaf(d[0], r[0][m][i], acc_e[m][i]);
      }
    };
    load_a(a[0], ablock(0));
    load_a(a[1], ablock(1));
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + 2 < NS) load_a(a[(s + 2) % 3], ablock(s + 2));
      issue(s, pr[s & 1], pd[s & 1]);
      if (s > 0) fold(s - 1, pr[(s - 1) & 1], pd[(s - 1) & 1]);
    }
    fold(NS - 1, pr[(NS - 1) & 1], pd[(NS - 1) & 1]);
  };

  ChunkW<SUB, EXTRA> ra, rb;
  ChunkX xr;
  load_w(ra, 0);
  load_w(rb, nch > 1 ? 1 : 0);
  load_x(xr, 0);
  int ci = 0;
  for (; ci + 1 < nch; ci += 2) {
    run(ra, xr, ci);
    run(rb, xr, ci + 1);
  }
  if (ci < nch) run(ra, xr, ci);

  // lane holds tokens 16m + 4q + i of rows r0 + 16u + col
  if constexpr (MODE == kGemmHead) {
    __shared__ float hv[4][kTok];
    __shared__ int hr[4][kTok];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float bv = -INFINITY;
        int br = INT_MAX;
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
          const int row = r0 + 16 * u + col;
          const float val = acc[u][m][i] * 0.0625f;
          if (row < n && !(val != val) && better(val, row, bv, br)) {  // NaN never wins
            bv = val;
            br = row;
          }
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          const float ov = __shfl_xor(bv, off);
          const int orow = __shfl_xor(br, off);
          if (better(ov, orow, bv, br)) {
            bv = ov;
            br = orow;
          }
        }
        if (col == 0) {
          hv[wave][16 * m + 4 * q + i] = bv;
          hr[wave][16 * m + 4 * q + i] = br;
        }
      }
    }
    __syncthreads();
    if (int(threadIdx.x) < n_tok) {
      const int s = threadIdx.x;
      float bv = hv[0][s];
      int br = hr[0][s];
#pragma unroll
      for (int w = 1; w < 4; ++w)
        if (better(hv[w][s], hr[w][s], bv, br)) {
          bv = hv[w][s];
          br = hr[w][s];
        }
      static_cast<uint2*>(out)[size_t(blockIdx.x) * kTok + s] = make_uint2(__builtin_bit_cast(uint32_t, bv),
                                                                            uint32_t(br));
    }
  } else {
    float* y = static_cast<float*>(out);
    if (MODE == kGemmSlices) y += size_t(blockIdx.y) * kTok * size_t(n);
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int row = r0 + 16 * u + col;
      if (row >= n) continue;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * m + 4 * q + i;
          if (s < n_tok) y[size_t(s) * size_t(n) + row] = acc[u][m][i] * 0.0625f;
        }
    }
    if constexpr (EXTRA != 0) {
      // the shared tile's four partial sums (one per wave), added in wave
      // order through LDS (the activation buffer, free once every wave is
      // past its last chunk)
      float4_t* red = reinterpret_cast<float4_t*>(&xs[0][0][0]);  // [wave][m][lane]
      __syncthreads();
#pragma unroll
      for (int m = 0; m < 4; ++m) red[(wave * 4 + m) * 64 + lane] = acc_e[m];
      __syncthreads();
      if (wave == 0) {
        const int row = re + col;
        if (row < n) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float4_t v = ((red[m * 64 + lane] + red[(4 + m) * 64 + lane]) + red[(8 + m) * 64 + lane]) +
                               red[(12 + m) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int s = 16 * m + 4 * q + i;
              if (s < n_tok) y[size_t(s) * size_t(n) + row] = v[i] * 0.0625f;
            }
          }
        }
      }
    }
  }
}

template <int MODE>
static void launch_gemm(const GemmPlan& p, hipStream_t st, const uint8_t* nib, const uint16_t* scl,
                        const uint16_t* x, int n, int k, int n_tok, void* out) {
  const dim3 grid(unsigned(p.tiles), unsigned(p.slices));
  const dim3 block(kGThreads);
  if (p.chunked) {
    if (p.sub == 2)
      hipLaunchKernelGGL((q4_gemm_chunk_kernel<2, MODE, 0>), grid, block, 0, st, nib, scl, x, n, k, n_tok, p.bps,
                         out);
    else if (MODE != kGemmHead && p.extra)
      hipLaunchKernelGGL((q4_gemm_chunk_kernel<1, MODE == kGemmHead ? kGemmOut : MODE, 1>), grid, block, 0, st, nib,
                         scl, x, n, k, n_tok, p.bps, out);
    else
      hipLaunchKernelGGL((q4_gemm_chunk_kernel<1, MODE, 0>), grid, block, 0, st, nib, scl, x, n, k, n_tok, p.bps,
                         out);
    return;
  }
  switch (p.sub) {
    case 4:
      hipLaunchKernelGGL((q4_gemm_kernel<4, MODE>), grid, block, 0, st, nib, scl, x, n, k, n_tok, p.bps, out);
      break;
    case 2:
      hipLaunchKernelGGL((q4_gemm_kernel<2, MODE>), grid, block, 0, st, nib, scl, x, n, k, n_tok, p.bps, out);
      break;
    default:
      hipLaunchKernelGGL((q4_gemm_kernel<1, MODE>), grid, block, 0, st, nib, scl, x, n, k, n_tok, p.bps, out);
      break;
  }
}

// y[s, r] = sum over slices, in slice order. Every slice's value is loaded
// before the first add, so a thread has all of its loads in flight at once.
constexpr int kMaxSlices = 16;
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part, int slices, int n,
                                                          int n_tok, float* __restrict__ y) {
  const size_t total = size_t(n_tok) * size_t(n);
  const size_t stride = size_t(kTok) * size_t(n);
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += size_t(gridDim.x) * 256) {
    float v[kMaxSlices];
#pragma unroll
    for (int sl = 0; sl < kMaxSlices; ++sl) v[sl] = sl < slices ? part[size_t(sl) * stride + i] : 0.0f;
    float acc = v[0];
#pragma unroll
    for (int sl = 1; sl < kMaxSlices; ++sl)
      if (sl < slices) acc += v[sl];
    y[i] = acc;
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
  if (n <= 0 || n >= (int64_t(1) << 31))
    return fail(Q4DEC_ERR_SHAPE, "q4_gemm_s64: n must be in [1, 2^31) (got %lld)", (long long)n);
  if (k <= 0 || k % 32)
    return fail(Q4DEC_ERR_SHAPE, "q4_gemm_s64: k must be a positive multiple of 32 (got %lld)", (long long)k);
  if (k > Q4DEC_MAX_K)
    return fail(Q4DEC_ERR_UNSUPPORTED, "q4_gemm_s64: k must be <= %d (got %lld)", Q4DEC_MAX_K, (long long)k);
  if (n_tok < 1 || n_tok > 64)
    return fail(Q4DEC_ERR_SHAPE, "q4_gemm_s64: n_tok must be in [1, 64] (got %lld)", (long long)n_tok);
  if (!aligned(packed, 16)) return fail(Q4DEC_ERR_ALIGN, "q4_gemm_s64: packed must be 16-byte aligned");
  if (!aligned(x, 16)) return fail(Q4DEC_ERR_ALIGN, "q4_gemm_s64: x must be 16-byte aligned");
  if (!aligned(y, 4)) return fail(Q4DEC_ERR_ALIGN, "q4_gemm_s64: y must be 4-byte aligned");
  if (!ws) return fail(Q4DEC_ERR_NULL, "q4_gemm_s64: ws is NULL");
  if (!aligned(ws, 256)) return fail(Q4DEC_ERR_ALIGN, "q4_gemm_s64: ws must be 256-byte aligned");
  const GemmPlan p = gemm_plan(n, k);
  if (ws_bytes < p.total)
    return fail(Q4DEC_ERR_WORKSPACE, "q4_gemm_s64: ws_bytes %zu < required %zu", ws_bytes, p.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* nib = static_cast<const uint8_t*>(packed);
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(nib + nib_plane_bytes(n, k));
  if (p.slices == 1) {
    launch_gemm<kGemmOut>(p, st, nib, scl, x, int(n), int(k), int(n_tok), y);
  } else {
    float* part = static_cast<float*>(ws);
    launch_gemm<kGemmSlices>(p, st, nib, scl, x, int(n), int(k), int(n_tok), part);
    const size_t total = size_t(n_tok) * size_t(n);
    const unsigned rgrid = unsigned(std::min<size_t>((total + 255) / 256, 4096));
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3(rgrid), dim3(256), 0, st, part, p.slices, int(n), int(n_tok), y);
  }
  return launch_status("q4_gemm_s64");
}

// ------------------------------------------------------ head over 64 tokens
namespace q4dec {
// workspace of the head over S tokens: one (logit, row) partial per row tile
// and token slot (the head is never split along K)
static size_t head_s64_ws_bytes(int64_t vocab, int64_t k) {
  const GemmPlan p = gemm_plan(vocab, k, false);
  return align256(size_t(p.tiles) * kTok * sizeof(uint2));
}
}  // namespace q4dec

extern "C" size_t lmhead_s64_workspace_bytes(int64_t vocab, int64_t k) {
  if (vocab <= 0 || vocab >= (int64_t(1) << 31) || k <= 0 || k % 32 || k > Q4DEC_MAX_K) return 0;
  return q4dec::head_s64_ws_bytes(vocab, k);
}

extern "C" int lmhead_softcap_argmax_s64(const void* packed, int64_t vocab, int64_t k, const uint16_t* x,
                                         int64_t n_tok, float cap, void* ws, size_t ws_bytes, int32_t* idx_out,
                                         float* val_out, void* stream) {
  using namespace q4dec;
  const char* name = "lmhead_softcap_argmax_s64";
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
  if (n_tok < 1 || n_tok > kTok)
    return fail(Q4DEC_ERR_SHAPE, "%s: n_tok must be in [1, %d] (got %lld)", name, kTok, (long long)n_tok);
  if (!aligned(packed, 16)) return fail(Q4DEC_ERR_ALIGN, "%s: packed must be 16-byte aligned", name);
  if (!aligned(x, 16)) return fail(Q4DEC_ERR_ALIGN, "%s: x must be 16-byte aligned", name);
  if (!aligned(ws, 256)) return fail(Q4DEC_ERR_ALIGN, "%s: ws must be 256-byte aligned", name);
  if (!aligned(idx_out, 4) || !aligned(val_out, 4))
    return fail(Q4DEC_ERR_ALIGN, "%s: idx_out and val_out must be 4-byte aligned", name);
  const size_t need = head_s64_ws_bytes(vocab, k);
  if (ws_bytes < need) return fail(Q4DEC_ERR_WORKSPACE, "%s: ws_bytes %zu < required %zu", name, ws_bytes, need);
  const GemmPlan p = gemm_plan(vocab, k, false);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint2* part = static_cast<uint2*>(ws);
  const uint8_t* nib = static_cast<const uint8_t*>(packed);
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(nib + nib_plane_bytes(vocab, k));
  launch_gemm<kGemmHead>(p, st, nib, scl, x, int(vocab), int(k), int(n_tok), part);
  reduce_argmax_partials(part, p.tiles, kTok, int(n_tok), cap, idx_out, val_out, st);
  return launch_status(name);
}
