// Exact bf16 form of q4_0 codes for the matrix-core kernels (the S=64 GEMM
// and the multi-vector GEMV): q4_pack's dword of a block holds the codes of
// eight consecutive k (block dword d: k = 8d .. 8d+7), stored as nibbles
// code + 8 ("Gemma-4 E2B mobile mixed-bit QAT weights": q4_0 grid, stored
// code = unsigned nibble - 8).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace q4dec {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_codes __attribute__((ext_vector_type(2)));
typedef float float2_codes __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_codes __attribute__((ext_vector_type(4)));

// 16 * c for the 8 codes of one packed dword, in k order, as bf16 (exact:
// 16 * c is a signed byte). XOR with 0x88888888 turns the nibbles into
// 4-bit two's complement codes; moved to the top half of each byte they read
// as signed bytes 16 * c, which convert to fp32 one byte at a time and to
// bf16 in pairs.
__device__ __forceinline__ bf16x8_t codes16_bf16(uint32_t w) {
  const uint32_t t = w ^ 0x88888888u;  // two's complement 4-bit codes
  const uint32_t lo = (t << 4) & 0xF0F0F0F0u, hi = t & 0xF0F0F0F0u;
  // byte j of the dword: low nibble k = 8d + {0, 4, 1, 5}[j], high nibble
  // k = 8d + {2, 6, 3, 7}[j]; as signed bytes in the top half, 16 * c
  bf16x8_t r;
  r[0] = (__bf16)(float)(int8_t)(lo);
  r[1] = (__bf16)(float)(int8_t)(lo >> 16);
  r[2] = (__bf16)(float)(int8_t)(hi);
  r[3] = (__bf16)(float)(int8_t)(hi >> 16);
  r[4] = (__bf16)(float)(int8_t)(lo >> 8);
  r[5] = (__bf16)(float)(int8_t)(lo >> 24);
  r[6] = (__bf16)(float)(int8_t)(hi >> 8);
  r[7] = (__bf16)(float)(int8_t)(hi >> 24);
  return r;
}

// The same 8 values as 4 dwords, each the bf16 pair (k = 8d + 2i, 8d + 2i + 1)
// (low half first), converted two at a time.
__device__ __forceinline__ u32x4_codes codes16_bf16_pairs(uint32_t w) {
  const uint32_t t = w ^ 0x88888888u;
  const uint32_t lo = (t << 4) & 0xF0F0F0F0u, hi = t & 0xF0F0F0F0u;
  auto pair = [](uint32_t a, uint32_t b) {
    const bf16x2_codes v = __builtin_convertvector(
        (float2_codes){(float)(int8_t)a, (float)(int8_t)b}, bf16x2_codes);
    return __builtin_bit_cast(uint32_t, v);
  };
  return u32x4_codes{pair(lo, lo >> 16), pair(hi, hi >> 16), pair(lo >> 8, lo >> 24), pair(hi >> 8, hi >> 24)};
}

}  // namespace q4dec
