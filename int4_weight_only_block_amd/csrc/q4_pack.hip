// q4_pack: int8 codes + fp16 scales -> packed nibble plane + scale plane.
// Stored nibble = code + 8 (unsigned code minus the midpoint, mixed-bit QAT
// page, P6 section). One thread packs one 32-weight block.
#include "q4dec_internal.h"

namespace q4dec {
Q4DEC_DEBUG_READER(q4_pack)

__global__ __launch_bounds__(256) void q4_pack_kernel(const int8_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales,
                                                      int64_t n_blocks, uint8_t* __restrict__ nib,
                                                      uint16_t* __restrict__ scl, int32_t* __restrict__ err) {
  Q4_DCHECK(int64_t(gridDim.x) * blockDim.x >= n_blocks, kDbgPackGrid);
  const int64_t blk = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  // codes of a block are 32 contiguous bytes (row-major [n, k], k % 32 == 0)
  const int8_t* c = codes + blk * 32;
  int8_t cb[32];
  bool bad = false;
  if ((reinterpret_cast<uintptr_t>(c) & 15) == 0) {
    const uint4* c4 = reinterpret_cast<const uint4*>(c);
    uint4 a = c4[0], b = c4[1];
    const uint32_t wv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 32; ++i) cb[i] = int8_t((wv[i >> 2] >> (8 * (i & 3))) & 0xFF);
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) cb[i] = c[i];
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) bad |= (cb[i] < -8) | (cb[i] > 7);
  uint4 out;
  out.x = pack_dword(cb + 0);
  out.y = pack_dword(cb + 8);
  out.z = pack_dword(cb + 16);
  out.w = pack_dword(cb + 24);
  reinterpret_cast<uint4*>(nib)[blk] = out;
  scl[blk] = scales[blk];
  if (bad && err) *err = 1;
}

}  // namespace q4dec

extern "C" int q4_pack(const int8_t* codes, const uint16_t* scales, int64_t n, int64_t k, void* packed,
                       int32_t* err_flag, void* stream) {
  using namespace q4dec;
  if (!codes) return fail(Q4DEC_ERR_NULL, "q4_pack: codes is NULL");
  if (!scales) return fail(Q4DEC_ERR_NULL, "q4_pack: scales is NULL");
  if (!packed) return fail(Q4DEC_ERR_NULL, "q4_pack: packed is NULL");
  if (n <= 0) return fail(Q4DEC_ERR_SHAPE, "q4_pack: n must be > 0 (got %lld)", (long long)n);
  if (k <= 0 || k % 32) return fail(Q4DEC_ERR_SHAPE, "q4_pack: k must be a positive multiple of 32 (got %lld)", (long long)k);
  if (!aligned(packed, 16)) return fail(Q4DEC_ERR_ALIGN, "q4_pack: packed must be 16-byte aligned");
  if (!aligned(scales, 2)) return fail(Q4DEC_ERR_ALIGN, "q4_pack: scales must be 2-byte aligned");
  const int64_t n_blocks = n * (k / 32);
  uint8_t* nib = static_cast<uint8_t*>(packed);
  uint16_t* scl = reinterpret_cast<uint16_t*>(nib + nib_plane_bytes(n, k));
  const int64_t grid = (n_blocks + 255) / 256;
  if (grid > 0x7FFFFFFF) return fail(Q4DEC_ERR_SHAPE, "q4_pack: matrix too large");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(q4_pack_kernel, dim3(unsigned(grid)), dim3(256), 0, st, codes, scales, n_blocks, nib, scl,
                     err_flag);
  return launch_status("q4_pack");
}
