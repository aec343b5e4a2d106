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
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const f2 x = {acc[o + e], acc[o + e + 1]};
    const b2 h = __builtin_convertvector(x, b2);   // one packed convert per pair
    const uint32_t hb = __builtin_bit_cast(uint32_t, h);
    const f2 hf = {__uint_as_float(hb << 16), __uint_as_float(hb & 0xffff0000u)};
    const b2 l = __builtin_convertvector(x - hf, b2);
    hi[e] = h[0];
    hi[e + 1] = h[1];
    lo[e] = l[0];
    lo[e + 1] = l[1];
  }
}

// ---------------------------------------------------------------- row tiles
// A row tile X[r][n] (16-bit, D columns) in LDS is read two ways: as the
// "row" operand (lane % 32 = row r, k = columns 16s + 8h .. +7) and as the
// "column" operand (lane % 32 = column n, k = rows) with ds_read_b64_tr_b16.
// The transposing read hands lane 4a+b of each 16-lane group element b of
// the 8-byte pieces addressed by lanes a, a+4, a+8, a+12 of that group, so a
// group whose lane j points at row kbase + j/4, columns n0 + 4(j%4) receives
// column n0 + i of rows kbase..kbase+3 in its lane i.  16-byte chunks are
// XOR-swizzled per row so that both reads stay free of bank conflicts.
typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));

template <int D>
__device__ __forceinline__ int swz_r(int r) {
  int f = ((r & 3) << 1) | ((r >> 2) & 1);
  if (D == 128) f |= ((r >> 3) & 1) << 3;
  return f;
}
// element offset of (row r, column n) in a swizzled row tile
template <int D>
__device__ __forceinline__ int toff(int r, int n) {
  return r * D + ((((n >> 3) ^ swz_r<D>(r))) << 3) + (n & 7);
}
// row operand: row r, k-step s (columns 16s + 8h .. +7)
template <int D>
__device__ __forceinline__ bf16x8 ld_rowop(const bf16_t *X, int r, int s, int h) {
  return ld_bf16x8(X + toff<D>(r, 16 * s + 8 * h));
}
// column operand over the 32 columns nb .. nb+31, k-step s over rows, with
// k-slot 8h + 4u + J <-> row 16s + 8u + 4h + J (the order pack_split uses for
// an accumulator tile whose rows are 8I + 4h + J)
template <int D>
__device__ __forceinline__ bf16x8 ld_colop(const bf16_t *X, int s, int nb, int lane) {
  const int j = lane & 15, g = lane >> 4, h = lane >> 5;
  const int n = nb + 16 * (g & 1) + 4 * (j & 3);
  const int r = 16 * s + 4 * h + (j >> 2);
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16 *)(X + toff<D>(r, n)));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16 *)(X + toff<D>(r + 8, n)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Workgroup barrier for LDS traffic: waits for this wavefront's LDS
// operations only.  Outstanding global->LDS loads are not waited for here
// (a full __syncthreads fence would drain them all); callers wait for the
// loads they need with an explicit vmcnt first.  LDS data read after the
// barrier should be read through native vector types (f32x4, bf16x8): a
// read the backend splits and re-merges loses the memory information that
// tells it the read cannot overlap a pending global->LDS load, and it then
// waits for every such load.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// async global -> LDS copy of ROWS rows of a [*, D] bf16 matrix (row stride
// D) into a swizzled row tile, by the NTHR threads t = 0..NTHR-1 (whole
// wavefronts, each issuing the same number of 1 KB pieces); rows past `rmax`
// repeat row rmax
template <int D, int ROWS, int NTHR>
__device__ __forceinline__ void tile_load(bf16_t *dst, const bf16_t *src, int64_t row0,
                                          int64_t rmax, int t) {
  constexpr int PIECES = ROWS * D / 8 / 64;
  constexpr int WAVES = NTHR / 64;
  static_assert(PIECES % WAVES == 0, "pieces split evenly over the wavefronts");
  const int lane = t & 63, w = t >> 6;
#pragma unroll
  for (int i = 0; i < PIECES / WAVES; ++i) {
    const int j = w + i * WAVES;
    const int chunk = j * 64 + lane;
    const int r = chunk / (D / 8), p = chunk % (D / 8);
    const int c = p ^ swz_r<D>(r);
    const int64_t row = min(row0 + r, rmax);
    __builtin_amdgcn_global_load_lds((const void *)(src + row * D + c * 8),
                                     (lds_void *)(reinterpret_cast<unsigned char *>(dst) + j * 1024),
                                     16, 0, 0);
  }
}

}  // namespace lh
