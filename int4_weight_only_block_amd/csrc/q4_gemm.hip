// q4_gemm_s64: S<=64 chunked-prefill product Y[s, r] = sum_k X[s, k] * w[r, k]
// on the matrix cores ("visible-cx/gemma-4-E2B-CoreAI": the prefill entry
// point has a static query width of 64 and reads the weights once per 64
// tokens).
//
// Numerics. A single fp16 or bf16 copy of c * d would round the 15-bit
// product, so each fp16 block scale d is split into d_hi (its top 7
// significant bits) and d_lo = d - d_hi (at most 4 bits). Both c * d_hi and
// c * d_lo are exact in fp16, and the two v_mfma_f32_16x16x32_f16 products
// accumulate straight into fp32, so the sum is exact up to fp32 accumulation
// and no per-block fold runs on the VALU. Activations are converted once per
// call into fp16 scaled by a per-token power of two (the token's largest
// magnitude lands in [2^14, 2^15)) by a small prep kernel, so the conversion
// is not repeated by every workgroup; a row whose largest scale would let
// c * d_hi overflow fp16 is scaled down by a power of two. Both factors are
// undone on the output.
//
// Work split. A workgroup (4 waves) owns 128 output rows (32 per wave, two
// MFMA column tiles) for all 64 token slots and one K slice. Activations move
// through LDS in chunks of 8 blocks shared by the 4 waves; the weights and
// activations of the next two chunks are in flight in registers while the
// current chunk runs on the matrix cores. Small-N matrices split K over
// several workgroups; their partial sums go to the workspace and a second
// kernel adds them in a fixed order, so results are deterministic.
//
// The same kernel, with an argmax epilogue instead of the output store, is
// the LM head over a chunk of up to 64 tokens: each workgroup keeps, per
// token, the best (logit, row) of its 128 rows, and a second launch reduces
// those per token and caps the winner, so no logits are written.
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "q4dec_internal.h"

namespace q4dec {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kTok = 64;     // token slots
constexpr int kSub = 2;      // 16-row MFMA column tiles per wave
constexpr int kTileN = 128;  // weight rows per workgroup (4 waves x kSub x 16)
constexpr int kChunk = 8;    // 32-wide blocks per LDS chunk

struct GemmPlan {
  int slices;  // K slices
  int bps;     // blocks per slice
  size_t xh_off, xf_off, part_off, total;  // workspace: fp16 activations, token factors, partials
};

// what the MFMA kernel does with its output tile
enum GemmMode : int {
  kGemmOut = 0,     // Y[s, r] (fp32)
  kGemmSlices = 1,  // the K slice's partial Y into the workspace
  kGemmHead = 2,    // per token, the tile's best (logit, row) into the workspace
};

static GemmPlan gemm_plan(int64_t n, int64_t k, bool split = true) {
  GemmPlan p{};
  const int B = int(k / 32);
  const int64_t tiles = (n + kTileN - 1) / kTileN;
  // About one workgroup per CU: split K when the row tiles alone leave CUs
  // idle, in slices of whole chunks (a partial last chunk runs its MFMAs on
  // zeroed scales). Matrices with >= 128 tiles are not split, so they need
  // no second launch.
  const int64_t s_target = split ? std::max<int64_t>(1, 256 / tiles) : 1;
  const int per = int((B + s_target - 1) / s_target);
  p.bps = ((per + kChunk - 1) / kChunk) * kChunk;
  p.slices = (B + p.bps - 1) / p.bps;
  p.xh_off = 0;
  p.xf_off = align256(size_t(kTok) * size_t(k) * 2);
  p.part_off = p.xf_off + 256;
  p.total = p.part_off + (p.slices > 1 ? align256(size_t(p.slices) * kTok * size_t(n) * 4) : 0);
  return p;
}

// One workgroup per token slot: find the token's largest exponent, convert
// its row to scaled fp16, store 2^E. Slots >= n_tok are zero-filled. Rows are
// read and written 8 values (16 bytes) at a time (x is 16-byte aligned and
// k % 32 == 0); a thread keeps its at most kPrepVec vectors in registers
// between the exponent scan and the conversion, so the row is read once.
constexpr int kPrepVec = Q4DEC_MAX_K / 8 / 256;
__global__ __launch_bounds__(256) void gemm_x_prep_kernel(const uint16_t* __restrict__ x, int k, int n_tok,
                                                          _Float16* __restrict__ xh, float* __restrict__ xf) {
  const int s = blockIdx.x;
  uint4* dst = reinterpret_cast<uint4*>(xh + size_t(s) * size_t(k));
  const int k8 = k >> 3;
  if (s >= n_tok) {
    for (int i = threadIdx.x; i < k8; i += 256) dst[i] = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x == 0) xf[s] = 0.0f;
    return;
  }
  const uint4* s4 = reinterpret_cast<const uint4*>(x + size_t(s) * size_t(k));
  uint4 v[kPrepVec];
#pragma unroll
  for (int r = 0; r < kPrepVec; ++r) {
    const int i = threadIdx.x + 256 * r;
    v[r] = i < k8 ? s4[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  uint32_t emax = 1, emin = 255;
#pragma unroll
  for (int r = 0; r < kPrepVec; ++r) {
    const uint32_t w[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      emax = max(emax, max((w[j] >> 7) & 0xFFu, (w[j] >> 23) & 0xFFu));
      emin = min(emin, min(bf16_exp_nz(w[j] & 0xFFFFu), bf16_exp_nz(w[j] >> 16)));
    }
  }
  for (int off = 32; off >= 1; off >>= 1) {
    emax = max(emax, uint32_t(__shfl_xor(int(emax), off)));
    emin = min(emin, uint32_t(__shfl_xor(int(emin), off)));
  }
  __shared__ uint32_t wm[4], wn[4];
  if ((threadIdx.x & 63) == 0) {
    wm[threadIdx.x >> 6] = emax;
    wn[threadIdx.x >> 6] = emin;
  }
  __syncthreads();
  emax = max(max(wm[0], wm[1]), max(wm[2], wm[3]));
  emin = min(min(wn[0], wn[1]), min(wn[2], wn[3]));
  const int e = int(emax) - 127 - 14;
#pragma unroll
  for (int r = 0; r < kPrepVec; ++r) {
    const int i = threadIdx.x + 256 * r;
    if (i >= k8) break;
    const uint32_t w[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half2_t h = {(_Float16)ldexpf(bf16_to_f32(w[j] & 0xFFFFu), -e),
                         (_Float16)ldexpf(bf16_to_f32(w[j] >> 16), -e)};
      o[j] = __builtin_bit_cast(uint32_t, h);
    }
    dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  // a token whose nonzero values span more binades than its scaled fp16
  // copy keeps is marked by a negative factor: the GEMM then reads X as
  // stored (exact path)
  if (threadIdx.x == 0) xf[s] = int(emax) - int(emin) > kMaxSpan ? -1.0f : ldexpf(1.0f, e);
}

__device__ __forceinline__ half8_t codes_f16x8(uint32_t w, uint32_t m_lo, uint32_t m_hi, uint32_t magic) {
  const CodePairs cp = unpack_dword(w, m_lo, m_hi, magic);
  half8_t r;
  r[0] = cp.p[0][0]; r[1] = cp.p[0][1]; r[2] = cp.p[1][0]; r[3] = cp.p[1][1];
  r[4] = cp.p[2][0]; r[5] = cp.p[2][1]; r[6] = cp.p[3][0]; r[7] = cp.p[3][1];
  return r;
}

// Registers of one chunk (kChunk = 8 blocks = 2 groups of 4). Lane (col, q)
// holds block 4g + q of its rows: the k-slots of lane group q inside one MFMA
// then come from block 4g + q, and the A operand follows the same mapping.
// Mixing blocks inside one MFMA is exact because the scale is already inside
// the fp16 B operand (c * d_hi, c * d_lo).
struct ChunkRegs {
  uint4 w[kSub][2];      // full 16-byte block (32 codes) per column tile and group
  uint32_t sd[kSub][2];  // its fp16 scale bits
  uint4 xr[(kChunk * kTok * 4) / 256];  // scaled fp16 activations
};

// LDS slot of activation quarter qq of a token: swizzled so the 16 lanes of a
// ds_read_b128 (16 tokens, same quarter) hit 16 distinct bank groups.
__device__ __forceinline__ int xslot(int tok, int qq) { return qq ^ ((tok >> 2) & 3); }

// Thread tid stages token tid / 4, quarter tid % 4 of each block of a chunk.
__device__ __forceinline__ void load_chunk(ChunkRegs& R, const uint4* const (&wrow)[kSub],
                                           const uint16_t* const (&srow)[kSub], const _Float16* __restrict__ xh,
                                           int k, int q, int b0, int b_end) {
  // Every load is issued unconditionally and nothing is computed from the
  // loaded values here, so the number of loads in flight is the same on
  // every path and the wait before a chunk's first use only covers that
  // chunk, not the chunk loaded after it. A block past the slice's end reads
  // a valid block instead; its weight scale is zeroed when the chunk is used,
  // which zeroes its products with the (finite) activations as well.
#pragma unroll
  for (int u = 0; u < kSub; ++u)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int bb = b0 + 4 * g + q;
      const int bc = bb < b_end ? bb : b0;  // ragged tail: any valid block, zeroed by its scale
      R.w[u][g] = wrow[u][bc];
      R.sd[u][g] = srow[u][bc];  // zeroed at use when bb >= b_end
    }
  const int sx = threadIdx.x >> 2, qq = threadIdx.x & 3;
#pragma unroll
  for (int c = 0; c < kChunk; ++c) {
    const int bb = b0 + c;
    const int bc = bb < b_end ? bb : b0;
    R.xr[c] = *reinterpret_cast<const uint4*>(xh + size_t(sx) * size_t(k) + size_t(bc) * 32 + qq * 8);
  }
}

// Writes the staged chunk to LDS (thread tid: token tid / 4, quarter tid % 4).
__device__ __forceinline__ void store_chunk(const ChunkRegs& R, uint4 (*xs)[kTok][4]) {
  const int sx = threadIdx.x >> 2, qq = threadIdx.x & 3;
#pragma unroll
  for (int c = 0; c < kChunk; ++c) xs[c][sx][xslot(sx, qq)] = R.xr[c];
}

// exact split of one fp16 scale (already shifted into range): hi keeps the
// top 7 significant bits, lo = d - hi
__device__ __forceinline__ void split_scale(uint32_t dbits, half2_t& hi, half2_t& lo) {
  const _Float16 d = __builtin_bit_cast(_Float16, uint16_t(dbits));
  const _Float16 h = __builtin_bit_cast(_Float16, uint16_t(dbits & 0xFFF0u));
  const _Float16 l = d - h;
  hi = half2_t{h, h};
  lo = half2_t{l, l};
}

// Activation tiles of step (g, j): the 4 token tiles' A operands.
__device__ __forceinline__ void load_a(half8_t (&a)[4], const uint4 (*xs)[kTok][4], int g, int j, int q, int col) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int tok = 16 * m + col;
    a[m] = __builtin_bit_cast(half8_t, xs[4 * g + q][tok][xslot(tok, j)]);
  }
}

// One chunk on the matrix cores: 2 groups x 4 k-slices x kSub column tiles x
// 4 token tiles x (hi, lo), accumulated into t. The A operands of the next
// step are read from LDS before this step's products are issued, so the LDS
// latency runs under the matrix-core work.
__device__ __forceinline__ void mma_chunk(float4_t (&t)[kSub][4], const uint4 (&w)[kSub][2],
                                          const uint32_t (&sd)[kSub][2], const int (&shift)[kSub],
                                          const uint4 (*xs)[kTok][4], int q, int col, int ngroups,
                                          uint32_t m_lo, uint32_t m_hi, uint32_t magic) {
  half8_t a0[4], a1[4];
  load_a(a0, xs, 0, 0, q, col);
  half2_t dh[kSub], dl[kSub];
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    const int g = st >> 2, j = st & 3;
    if (g >= ngroups) break;
    half8_t(&cur)[4] = (st & 1) ? a1 : a0;
    half8_t(&nxt)[4] = (st & 1) ? a0 : a1;
    // the tiles past the last used group are valid LDS, read and ignored
    if (st + 1 < 8) load_a(nxt, xs, (st + 1) >> 2, (st + 1) & 3, q, col);
    if (j == 0) {
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        uint32_t dbits = sd[u][g];
        if (shift[u] > 0) {  // rare: rows with scales >= 2^11
          const float df = ldexpf(float(__builtin_bit_cast(_Float16, uint16_t(dbits))), -shift[u]);
          dbits = __builtin_bit_cast(uint16_t, (_Float16)df);
        }
        split_scale(dbits, dh[u], dl[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      const uint32_t wd = j == 0 ? w[u][g].x : j == 1 ? w[u][g].y : j == 2 ? w[u][g].z : w[u][g].w;
      const CodePairs cp = unpack_dword(wd, m_lo, m_hi, magic);
      half8_t bh, bl;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const half2_t ph = cp.p[jj] * dh[u];
        const half2_t pl = cp.p[jj] * dl[u];
        bh[2 * jj] = ph[0]; bh[2 * jj + 1] = ph[1];
        bl[2 * jj] = pl[0]; bl[2 * jj + 1] = pl[1];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) t[u][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur[m], bh, t[u][m], 0, 0, 0);
#pragma unroll
      for (int m = 0; m < 4; ++m) t[u][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur[m], bl, t[u][m], 0, 0, 0);
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void q4_gemm_kernel(const uint8_t* __restrict__ nib, const uint16_t* __restrict__ scl,
                                                      const uint8_t* __restrict__ rexp, const _Float16* __restrict__ xh,
                                                      const float* __restrict__ xf, const uint16_t* __restrict__ x,
                                                      int n, int k, int n_tok, int bps, void* __restrict__ out) {
  __shared__ uint4 xs[kChunk][kTok][4];  // [block][token][k quarter, swizzled], 32 KB
  const int B = k >> 5;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4;    // lane group: block 4g + q of a chunk
  const int col = lane & 15;  // row within a 16-row MFMA column tile
  const int b_begin = blockIdx.y * bps;
  const int b_end = min(B, b_begin + bps);

  const uint4* wrow[kSub];
  const uint16_t* srow[kSub];
  int rows[kSub];
  int shift[kSub];  // power-of-two range shift of the row's scales
#pragma unroll
  for (int u = 0; u < kSub; ++u) {
    rows[u] = blockIdx.x * kTileN + (wave * kSub + u) * 16 + col;
    const int rc = rows[u] < n ? rows[u] : n - 1;
    wrow[u] = reinterpret_cast<const uint4*>(nib + size_t(rc) * size_t(k >> 1));
    srow[u] = scl + size_t(rc) * size_t(B);
    // largest fp16 exponent field of the row's scales (computed by q4_pack);
    // keep every scale below 2^11 so |c * d_hi| < 2^14 stays finite in fp16
    shift[u] = max(0, int(rexp[rc]) - 15 - 10);
  }

  uint32_t m_lo, m_hi, magic;
  asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(m_lo));
  asm volatile("v_mov_b32 %0, 0x00F000F0" : "=v"(m_hi));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

  // the lane's 16 token factors, loaded now so they arrive under the main
  // loop instead of one dependent load per output at the end
  float tf[16];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) tf[4 * m + i] = xf[16 * m + 4 * q + i];

  float4_t acc[kSub][4];
#pragma unroll
  for (int u = 0; u < kSub; ++u)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[u][m] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // A wide token (negative factor from the prep kernel) puts the whole
  // workgroup on the exact path.
  __shared__ int wide_w[4];
  {
    const bool wide_t = int(threadIdx.x) < n_tok && xf[threadIdx.x & (kTok - 1)] < 0.0f;
    const bool wide_wave = __ballot(wide_t) != 0;
    if (lane == 0) wide_w[wave] = wide_wave;
  }
  __syncthreads();
  // uniform by construction; readfirstlane lets the compiler branch on it
  // as a scalar, so the two paths do not hold registers at the same time
  const bool exact = __builtin_amdgcn_readfirstlane(wide_w[0] | wide_w[1] | wide_w[2] | wide_w[3]) != 0;
  if (exact) {
    // Each lane's outputs (rows rows[u], tokens 16m + 4q + i) summed over the
    // slice's blocks in fp32 with X as stored: every code-activation product
    // is exact, each block sum is scaled by its fp16 d. One block at a time.
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) tf[4 * m + i] = 1.0f;
#pragma unroll
    for (int u = 0; u < kSub; ++u) shift[u] = 0;
#pragma unroll 1
    for (int b = b_begin; b < b_end; ++b) {
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        const uint4 wq = wrow[u][b];
        const uint32_t wd[4] = {wq.x, wq.y, wq.z, wq.w};
        const float d = float(__builtin_bit_cast(_Float16, srow[u][b]));
#pragma unroll 1
        for (int mi = 0; mi < 16; ++mi) {
          const int tok = 16 * (mi >> 2) + 4 * q + (mi & 3);
          if (tok >= n_tok) continue;
          const uint4* xb = reinterpret_cast<const uint4*>(x + size_t(tok) * size_t(k) + size_t(b) * 32);
          float sum = 0.0f;
#pragma unroll
          for (int dd = 0; dd < 4; ++dd) {
            const uint4 xv = xb[dd];
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
            const CodePairs cp = unpack_dword(wd[dd], m_lo, m_hi, magic);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              sum = fmaf(float(cp.p[jj][0]), bf16_to_f32(xw[jj] & 0xFFFFu), sum);
              sum = fmaf(float(cp.p[jj][1]), bf16_to_f32(xw[jj] >> 16), sum);
            }
          }
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * m + i == mi) acc[u][m][i] = fmaf(d, sum, acc[u][m][i]);
        }
      }
    }
  } else {
  // two chunks in flight: A holds chunks 0, 2, 4, ..., B holds 1, 3, 5, ...
  // (every slice holds at least one block; a chunk past the slice's end is
  // replaced by its first chunk, which is loaded but never used)
  ChunkRegs ra, rb;
  load_chunk(ra, wrow, srow, xh, k, q, b_begin, b_end);
  load_chunk(rb, wrow, srow, xh, k, q, b_begin + kChunk < b_end ? b_begin + kChunk : b_begin, b_end);

  auto run = [&](ChunkRegs& R, int b0) {
    __syncthreads();  // previous chunk fully consumed
    store_chunk(R, xs);
    uint4 w[kSub][2];
    uint32_t sd[kSub][2];
#pragma unroll
    for (int u = 0; u < kSub; ++u)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        w[u][g] = R.w[u][g];
        sd[u][g] = b0 + 4 * g + q < b_end ? R.sd[u][g] : 0u;
        // opaque copy: w gets registers of its own, so the refill below
        // lands in R's registers in place (otherwise the compiler reuses R's
        // registers for w and moves the refilled values back at the end of
        // the loop, waiting on their loads)
        asm volatile("" : "+v"(w[u][g].x), "+v"(w[u][g].y), "+v"(w[u][g].z), "+v"(w[u][g].w));
      }
    __syncthreads();
    // refill this register set with the chunk after next (or, past the end,
    // with the current chunk again: cache hits, never used)
    load_chunk(R, wrow, srow, xh, k, q, b0 + 2 * kChunk < b_end ? b0 + 2 * kChunk : b0, b_end);
    const int ngroups = (min(kChunk, b_end - b0) + 3) / 4;
    mma_chunk(acc, w, sd, shift, xs, q, col, ngroups, m_lo, m_hi, magic);
  };
  // pairs of chunks with no conditional inside, so both register sets stay
  // in place across iterations (no copies that would wait on their loads)
  int b0 = b_begin;
  for (; b0 + kChunk < b_end; b0 += 2 * kChunk) {
    run(ra, b0);
    run(rb, b0 + kChunk);
  }
  if (b0 < b_end) run(ra, b0);
  }

  // lane holds tokens s = 16m + 4q + i of output rows rows[u]
  if constexpr (MODE == kGemmHead) {
    // per token: the best (logit, row) of the lane's two rows, then of the
    // 16 lanes of its lane group (the tile's 16 columns), then of the waves
    __shared__ float hv[4][kTok];
    __shared__ int hr[4][kTok];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float bv = -INFINITY;
        int br = INT_MAX;
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
          const float v = acc[u][m][i] * (tf[4 * m + i] * ldexpf(1.0f, shift[u]));
          if (rows[u] < n && better(v, rows[u], bv, br)) {
            bv = v;
            br = rows[u];
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
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      if (rows[u] >= n) continue;
      const float rf = ldexpf(1.0f, shift[u]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * m + 4 * q + i;
          const float v = acc[u][m][i] * (tf[4 * m + i] * rf);
          if (MODE == kGemmSlices) {
            y[(size_t(blockIdx.y) * kTok + s) * size_t(n) + rows[u]] = v;
          } else if (s < n_tok) {
            y[size_t(s) * size_t(n) + rows[u]] = v;
          }
        }
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
    // slices added left to right; the loads of four slices are issued
    // before their adds so they are in flight together
    float v = part[i];
    int sl = 1;
    for (; sl + 4 <= slices; sl += 4) {
      const float a = part[size_t(sl) * stride + i], b = part[size_t(sl + 1) * stride + i];
      const float c = part[size_t(sl + 2) * stride + i], d = part[size_t(sl + 3) * stride + i];
      v += a;
      v += b;
      v += c;
      v += d;
    }
    for (; sl < slices; ++sl) v += part[size_t(sl) * stride + i];
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
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  _Float16* xh = reinterpret_cast<_Float16*>(w8 + p.xh_off);
  float* xf = reinterpret_cast<float*>(w8 + p.xf_off);
  float* part = reinterpret_cast<float*>(w8 + p.part_off);
  const uint8_t* nib = static_cast<const uint8_t*>(packed);
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(nib + nib_plane_bytes(n, k));
  const uint8_t* rexp = nib + nib_plane_bytes(n, k) + scale_plane_bytes(n, k);
  hipLaunchKernelGGL(gemm_x_prep_kernel, dim3(kTok), dim3(256), 0, st, x, int(k), int(n_tok), xh, xf);
  const dim3 grid(unsigned((n + kTileN - 1) / kTileN), unsigned(p.slices));
  if (p.slices == 1) {
    hipLaunchKernelGGL(q4_gemm_kernel<kGemmOut>, grid, dim3(256), 0, st, nib, scl, rexp, xh, xf, x, int(n),
                       int(k), int(n_tok), p.bps, static_cast<void*>(y));
  } else {
    hipLaunchKernelGGL(q4_gemm_kernel<kGemmSlices>, grid, dim3(256), 0, st, nib, scl, rexp, xh, xf, x, int(n),
                       int(k), int(n_tok), p.bps, static_cast<void*>(part));
    const size_t total = size_t(n_tok) * size_t(n);
    const unsigned rgrid = unsigned(std::min<size_t>((total + 255) / 256, 4096));
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3(rgrid), dim3(256), 0, st, part, p.slices, int(n), int(n_tok), y);
  }
  return launch_status("q4_gemm_s64");
}

// ------------------------------------------------------ head over 64 tokens
namespace q4dec {
// workspace of the head over S tokens: the scaled activations and token
// factors as for q4_gemm_s64, then one (logit, row) partial per row tile and
// token slot
static size_t head_s64_partials_off(int64_t vocab, int64_t k) { return gemm_plan(vocab, k, false).part_off; }
static size_t head_s64_ws_bytes(int64_t vocab, int64_t k) {
  const int64_t tiles = (vocab + kTileN - 1) / kTileN;
  return head_s64_partials_off(vocab, k) + align256(size_t(tiles) * kTok * sizeof(uint2));
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
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  _Float16* xh = reinterpret_cast<_Float16*>(w8 + p.xh_off);
  float* xf = reinterpret_cast<float*>(w8 + p.xf_off);
  uint2* part = reinterpret_cast<uint2*>(w8 + head_s64_partials_off(vocab, k));
  const uint8_t* nib = static_cast<const uint8_t*>(packed);
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(nib + nib_plane_bytes(vocab, k));
  const uint8_t* rexp = nib + nib_plane_bytes(vocab, k) + scale_plane_bytes(vocab, k);
  const int tiles = int((vocab + kTileN - 1) / kTileN);
  hipLaunchKernelGGL(gemm_x_prep_kernel, dim3(kTok), dim3(256), 0, st, x, int(k), int(n_tok), xh, xf);
  hipLaunchKernelGGL(q4_gemm_kernel<kGemmHead>, dim3(unsigned(tiles), 1u), dim3(256), 0, st, nib, scl, rexp, xh, xf,
                     x, int(vocab), int(k), int(n_tok), p.bps, static_cast<void*>(part));
  reduce_argmax_partials(part, tiles, kTok, int(n_tok), cap, idx_out, val_out, st);
  return launch_status(name);
}
