// Internal declarations shared by the HIP sources of liblighthouse.
// Host geometry, element-type helpers and the kernel launchers each source
// file provides.  Not part of the public ABI (include/lighthouse.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "../../include/lighthouse.h"

namespace lh {

constexpr int kMaxLevels = 32;

// Everything a kernel needs to know about one call's shapes.  Filled on the
// host by make_geo() from a validated lh_dims and passed to kernels by value.
struct Geo {
  int64_t B, N, K, S, E, n_c, T, k_s, Bc, Sp;
  int32_t H, d, p, L;
  int32_t io, out;
  int64_t Nreal;                 // the caller's sequence length (N is it rounded up to
                                 // whole coarsest cells: the layer pads with zero rows)
  int32_t mode;                  // LH_SCATTER_HOLD or LH_SCATTER_SPAN
  int32_t sigma;                 // LH_SIGMA_SUM, LH_SIGMA_MAX or LH_SIGMA_PRODUCT
  int32_t strata;                // LH_STRATA_JOINT or LH_STRATA_PER_LEVEL
  int64_t quota[kMaxLevels];     // per-level quotas of k_s (LH_STRATA_PER_LEVEL)
  float scale;                   // softmax scale (1/sqrt(d) when dims say 0)
  int64_t lsize[kMaxLevels];     // N / p^l
  int64_t loff[kMaxLevels];      // flat offset of level l
  int64_t pw[kMaxLevels + 1];    // p^l
  int64_t BH() const { return B * (int64_t)H; }
};

lh_status make_geo(const lh_dims *dims, Geo *g);

inline size_t el_size(int32_t dt) { return dt == LH_BF16 ? 2 : 4; }

// ---------------------------------------------------------------- device helpers
typedef uint16_t bf16_t;   // raw bfloat16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// float32 -> bfloat16, round-to-nearest-even, with the hardware packed
// convert (v_cvt_pk_bf16_f32); it matches a software RNE on every non-NaN
// input and maps NaN to a quiet NaN
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const f32x2_hw v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float load(const float *p) { return *p; }
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  __device__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// load / store 8 consecutive elements as float
__device__ __forceinline__ void load8(const float *p, float *x) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t *p, float *x) {
  const uint4 a = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void store8(float *p, const float *x) {
  *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4 *>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void store8(bf16_t *p, const float *x) {
  *reinterpret_cast<uint4 *>(p) = make_uint4(pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]),
                                             pack2_bf16(x[4], x[5]), pack2_bf16(x[6], x[7]));
}

// Streaming (nontemporal) stores, for the large outputs that no later kernel
// of the layer reads back: the layer output and the input gradients.  Plain
// stores leave them dirty in the chip's caches, and the next kernel that
// streams its own input then waits behind their write-back (on MI355X a
// 256 MiB read right after a 1 GiB plain write ran at 2.1 TB/s, after a
// nontemporal one at 6.3 TB/s).
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_nt(void *p, uint4 v) {
  __builtin_nontemporal_store(nt_u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_u32x4 *>(p));
}
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store8b_nt(void *p, uint2 v) {
  __builtin_nontemporal_store(nt_u32x2{v.x, v.y}, reinterpret_cast<nt_u32x2 *>(p));
}
__device__ __forceinline__ void store8_nt(float *p, const float *x) {
  store16_nt(p, make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                           __float_as_uint(x[3])));
  store16_nt(p + 4, make_uint4(__float_as_uint(x[4]), __float_as_uint(x[5]),
                               __float_as_uint(x[6]), __float_as_uint(x[7])));
}
__device__ __forceinline__ void store8_nt(bf16_t *p, const float *x) {
  store16_nt(p, make_uint4(pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]),
                           pack2_bf16(x[4], x[5]), pack2_bf16(x[6], x[7])));
}

// two-term bf16 split of 8 floats: hi = bf16(x), lo = bf16(x - hi), so that
// hi + lo carries about 16 significant bits of x
__device__ __forceinline__ void store8_split(bf16_t *hi, bf16_t *lo, const float *x) {
  float h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = bf16_to_f32(f32_to_bf16(x[i]));
    l[i] = x[i] - h[i];
  }
  store8(hi, h);
  store8(lo, l);
}

// ---------------------------------------------------------------- launchers
// Each returns LH_OK or LH_ERR_HIP / LH_ERR_UNSUPPORTED; none allocates.
// rows of row_bytes bytes (a multiple of 16) per (b, h): dst row r takes src
// row r for r < rows_src and zeros after it (pads or truncates a sequence)
lh_status launch_copy_rows(const Geo &g, const void *src, void *dst, int64_t rows_src,
                           int64_t rows_dst, int64_t row_bytes, hipStream_t st);
lh_status launch_pyramid_score(const Geo &g, const void *q, const void *k, const void *v,
                               void *pq, void *pk, void *pv, float *sq, float *sk,
                               hipStream_t st);
lh_status check_pyramid_supported(const Geo &g);

lh_status launch_select(const Geo &g, const float *sq, const float *sk, int32_t *sel_idx,
                        int32_t *sel_anchor, uint8_t *sel_flags, int32_t *row_of,
                        hipStream_t st);
lh_status check_select_supported(const Geo &g);
// launch limits of the other kernel families (grid sizes, LDS budgets,
// buffer-resource ranges), so that lh_validate rejects every geometry a
// launch would reject
lh_status check_rows_supported(const Geo &g);
lh_status check_attn_f32_supported(const Geo &g);
lh_status check_attn_fwd_supported(const Geo &g);
lh_status check_attn_dkv_supported(const Geo &g);
lh_status check_attn_dq_supported(const Geo &g);

// tensors z0 .. z0 + nz - 1 of the three (0 q, 1 k, 2 v)
lh_status launch_gather(const Geo &g, const void *const src[3], const void *const psrc[3],
                        const int32_t *sel_idx, void *const dst[3], hipStream_t st, int z0 = 0,
                        int nz = 3);
// rows [BH, S, d] bf16 -> [BH, d, Sp] bf16 with zeroed padding
lh_status launch_transpose(const Geo &g, const void *rows, void *tr, hipStream_t st);
// os is float32; o has the output type
lh_status launch_scatter(const Geo &g, const float *os, const int32_t *sel_anchor,
                         const uint8_t *sel_flags, void *o, hipStream_t st);
// Scatter adjoint.  dos (float32) may be NULL; dos_hi/dos_lo (bf16, may be
// NULL) receive the two-term split dos ~= hi + lo; drow[j] = <dos_j, os_j>
// when os (float32) and drow are not NULL, which needs float32 rows [B*H, S,
// d] to keep dos in: dos itself, else `scratch` (overwritten).  dout has the
// output type.
lh_status launch_scatter_bwd(const Geo &g, const void *dout, const int32_t *sel_anchor,
                             const uint8_t *sel_flags, float *dos, bf16_t *dos_hi,
                             bf16_t *dos_lo, const float *os, float *drow, float *scratch,
                             hipStream_t st);
// span broadcast: owner[BH, N] int32 (finest selected entry per token), the
// copy O[t] = OS[owner[t]], and its adjoint (outputs as launch_scatter_bwd)
lh_status launch_owner(const Geo &g, const int32_t *row_of, int32_t *owner, hipStream_t st);
lh_status launch_scatter_span(const Geo &g, const float *os, const int32_t *owner, void *o,
                              hipStream_t st);
lh_status launch_scatter_span_bwd(const Geo &g, const void *dout, const int32_t *sel_idx,
                                  const uint8_t *sel_flags, const int32_t *owner, float *dos,
                                  bf16_t *dos_hi, bf16_t *dos_lo, const float *os, float *drow,
                                  hipStream_t st);
// the gather + pooling adjoints of nt (1..3) tensors: dxs[i] rows -> dx[i] tokens
lh_status launch_unpool(const Geo &g, const float *const dxs[], const int32_t *row_of,
                        void *const dx[], int nt, hipStream_t st);

// attention, float32 I/O (VALU)
lh_status launch_attn_fwd_f32(const Geo &g, const float *qs, const float *ks, const float *vs,
                              const uint8_t *flags, float *os, float *lse, hipStream_t st);
lh_status launch_attn_bwd_f32(const Geo &g, const float *qs, const float *ks, const float *vs,
                              const float *os, const float *lse, const uint8_t *flags,
                              const float *dos, float *drow_ws, float *dqs, float *dks,
                              float *dvs, hipStream_t st);

// attention, bf16 I/O (MFMA), on the gathered rows [BH, S, d].  dO enters
// the backward as a two-term bf16 split (hi + lo).  With `o` given, the
// forward also writes the layer output o [BH, N, d] (out type) under the
// causal hold from sel_anchor, as launch_scatter would.
lh_status launch_attn_fwd_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                               const bf16_t *vs, const uint8_t *flags, float *os, float *lse,
                               hipStream_t st, const int32_t *sel_anchor = nullptr,
                               void *o = nullptr);
lh_status launch_attn_bwd_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                               const bf16_t *vs, const bf16_t *dos_hi, const bf16_t *dos_lo,
                               const float *lse, const float *drow, const uint8_t *flags,
                               float *dqs, float *dks, float *dvs, hipStream_t st);
lh_status launch_attn_bwd_dkv_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                                   const bf16_t *vs, const bf16_t *dos_hi, const bf16_t *dos_lo,
                                   const float *lse, const float *drow, const uint8_t *flags,
                                   float *dks, float *dvs, hipStream_t st);
lh_status launch_attn_bwd_dq_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                                  const bf16_t *vs, const bf16_t *dos_hi, const bf16_t *dos_lo,
                                  const float *lse, const float *drow, const uint8_t *flags,
                                  float *dqs, hipStream_t st);
// The same dQ kernel with the gather + pooling adjoint of its own rows in
// the epilogue (the layer backward): dq [BH, N, d] of the output type
// instead of the float32 subsequence rows.  Only at d = 64, where every
// workgroup's 128 rows are whole strata and the epilogue's LDS fits
// (dq_can_unpool).
bool dq_can_unpool(const Geo &g);
lh_status launch_attn_bwd_dq_unpool(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                                    const bf16_t *vs, const bf16_t *dos_hi,
                                    const bf16_t *dos_lo, const float *lse, const float *drow,
                                    const uint8_t *flags, const int32_t *row_of, void *dq,
                                    hipStream_t st);
// float32 dos [BH,S,d] -> optional bf16 split (hi, lo) and drow = rowsum(dos * os)
lh_status launch_dos_prep(const Geo &g, const float *dos, const float *os, bf16_t *dos_hi,
                          bf16_t *dos_lo, float *drow, hipStream_t st);

inline lh_status hip_status() {
  return hipGetLastError() == hipSuccess ? LH_OK : LH_ERR_HIP;
}

inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// a one-dimensional launch of `blocks` workgroups of `threads` work-items:
// the work-item count along x must fit 32 bits
inline bool grid_fits(int64_t blocks, int64_t threads) {
  return blocks >= 0 && blocks <= (int64_t)UINT32_MAX / threads;
}

}  // namespace lh
