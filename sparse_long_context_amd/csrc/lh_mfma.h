// MFMA helpers for gfx950 (CDNA4): v_mfma_f32_32x32x16_bf16 operand types,
// packing, and the lane layout the attention kernels rely on.
//
// For C[32x32] += A[32x16] * B[16x32] with 64 lanes, lane l (h = l / 32):
//   A operand: row l % 32, k = 8h .. 8h+7   (8 bf16)
//   B operand: col l % 32, k = 8h .. 8h+7   (8 bf16)
//   C (16 f32): acc[4*I + J] = C[8*I + 4*h + J][l % 32], I, J in 0..3
// Because k is a summation index, A and B may present their k slots in any
// order as long as both use the same one; the kernels exploit this to feed
// an accumulator tile straight back in as the next product's operand.
#pragma once

#include "lh_internal.h"

namespace lh {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // 16 raw bytes
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

// two 4-element (8-byte) pieces -> one operand
__device__ __forceinline__ bf16x8 ld_bf16x4x2(const bf16_t *p0, const bf16_t *p1) {
  const uint2 a = *reinterpret_cast<const uint2 *>(p0);
  const uint2 b = *reinterpret_cast<const uint2 *>(p1);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// 8 accumulator values acc[o .. o+7] -> bf16 operand (round to nearest even)
__device__ __forceinline__ bf16x8 pack_bf16x8(const f32x16 &acc, int o) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)acc[o + e];
  return r;
}

// the same values as a two-term split: hi = bf16(x), lo = bf16(x - hi); the
// pair carries about 16 significant bits, so a product taken as
// hi*B + lo*B loses far less than one rounding of x to bf16
__device__ __forceinline__ void pack_split(const f32x16 &acc, int o, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = (__bf16)acc[o + e];
    hi[e] = h;
    lo[e] = (__bf16)(acc[o + e] - (float)h);
  }
}

}  // namespace lh
