// The gather and pooling adjoint (unpool) of whole strata, shared by the
// unpool kernel and the epilogue of the dQ kernel, whose workgroups hold
// whole strata's subsequence rows (gist.science explainer "Long Context
// Pre-Training with Lighthouse Attention", technical summary 2.B: gradients
// reach the pooled inputs through gather and pooling only):
//   dx[t] = sum over levels l of dxs[row_of(l, t / p^l)] / p^l,
// over the selected ancestors of token t (rows of -1 skipped).
//
// The row_of entries of the strata are staged in LDS level by level (level
// l of strata m0 .. m0+spw-1 is one contiguous run of row_of), so the level-l
// ancestor of workgroup-local token u sits at lb[l] + u / p^l.  A group of
// CPR lanes (8 columns each) owns a contiguous run of level-1 entries.
// Levels L-1 .. 2 are summed once per level-2 cell (coarsest first) and
// kept; each entry adds its level-1 row, converts that sum once, and every
// token without a level-0 row of its own stores it unchanged; the others
// add their row.  The summation order is fixed, so results are reproducible
// and equal wherever the rows come from.
#pragma once

#include "lh_internal.h"

namespace lh {

constexpr int kUnpoolThreads = 256;
constexpr int kUnpoolLdsEntries = 8192;   // row_of entries staged per workgroup

struct UnpoolArgs {
  const float *dxs[3];
  void *dx[3];
  const int32_t *row_of;
  int64_t N, E, S, Bc;
  int32_t d, L, p, spw, lgp;    // lgp = log2(p) when p is a power of two, else -1
  int32_t parts;                // workgroups per group of spw strata (each a run of entries)
  int64_t loff[kMaxLevels];
  int32_t per[kMaxLevels];      // entries of level l per stratum (Bc / p^l)
  int32_t pw[kMaxLevels];       // p^l
  int32_t lb[kMaxLevels];       // first LDS slot of level l (spw * entries below it)
  float inv[kMaxLevels];
};

// the geometry fields of UnpoolArgs for `spw` strata per workgroup
UnpoolArgs make_unpool_args(const Geo &g, int spw);

// 8 output values in the output dtype, as stored by one 16- or 32-byte write
template <typename TO> struct Pack8;
template <> struct Pack8<bf16_t> {
  uint4 w;
  __device__ void set(const float *x) {
    w = make_uint4(pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]), pack2_bf16(x[4], x[5]),
                   pack2_bf16(x[6], x[7]));
  }
  __device__ void put(bf16_t *p) const { store16_nt(p, w); }   // gradients: streamed out
  // columns 0-3 at p, 4-7 at p + half
  __device__ void put(bf16_t *p, int half) const {
    store8b_nt(p, make_uint2(w.x, w.y));
    store8b_nt(p + half, make_uint2(w.z, w.w));
  }
};
template <> struct Pack8<float> {
  float4 a, b;
  __device__ void set(const float *x) {
    a = make_float4(x[0], x[1], x[2], x[3]);
    b = make_float4(x[4], x[5], x[6], x[7]);
  }
  __device__ void put(float *p) const {
    store16_nt(p, make_uint4(__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z),
                             __float_as_uint(a.w)));
    store16_nt(p + 4, make_uint4(__float_as_uint(b.x), __float_as_uint(b.y),
                                 __float_as_uint(b.z), __float_as_uint(b.w)));
  }
  __device__ void put(float *p, int half) const {
    store16_nt(p, make_uint4(__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z),
                             __float_as_uint(a.w)));
    store16_nt(p + half, make_uint4(__float_as_uint(b.x), __float_as_uint(b.y),
                                    __float_as_uint(b.z), __float_as_uint(b.w)));
  }
};

// row_of of strata m0 .. m0+spw-1 (rog: this (b, h)'s row_of) into ro;
// rows outside [row_lo, row_hi) become -1.  Readers need a barrier.
template <int NTHR>
__device__ __forceinline__ void unpool_stage_ro(const UnpoolArgs &a, int32_t *ro,
                                                const int32_t *rog, int64_t m0, int spw,
                                                int64_t row_lo, int64_t row_hi, int tid) {
  for (int l = 0; l < a.L; ++l) {
    const int cnt = spw * a.per[l];
    const int32_t *src = rog + a.loff[l] + m0 * a.per[l];
    for (int i = tid; i < cnt; i += NTHR) {
      const int32_t r = src[i];
      ro[a.lb[l] + i] = (r >= row_lo && r < row_hi) ? r : -1;
    }
  }
}

// The tokens of the spw staged strata: out points at the first token row of
// stratum m0 ([*, d], output type), rows(r, x) loads this lane's 8 columns of
// subsequence row r (any r that ro holds).  NTHR threads, CPR lanes per row.
// SPLIT: the lane's 8 columns are 4 at c*4 and 4 at d/2 + c*4 instead of 8
// at c*8 (rows must load them in that order), and they are stored the same
// way: every 16-byte-per-lane load of a float32 row by a lane group then
// covers whole 128-byte lines (with 8 contiguous columns per lane each load
// instruction covers half of every line of the row).
// part, parts: this workgroup takes the part-th of `parts` equal runs of the
// strata's level-1 entries (whole strata: part 0 of 1).
template <typename TO, int CPR, int NTHR, bool SPLIT, typename Rows>
__device__ __forceinline__ void unpool_strata(const UnpoolArgs &a, const int32_t *ro, Rows rows,
                                              TO *out, int spw, int tid, int part = 0,
                                              int parts = 1) {
  const int c = tid % CPR;
  constexpr int LANES = NTHR / CPR;   // lanes along the tokens
  const int d = a.d;
  out += SPLIT ? c * 4 : c * 8;
  auto put = [&](const Pack8<TO> &v, TO *dst) {
    if constexpr (SPLIT) v.put(dst, d / 2);
    else v.put(dst);
  };
  const int ntok = spw * (int)a.Bc;
  const int P1 = a.L >= 2 ? a.p : 1;    // tokens per level-1 entry
  const int nall = ntok / P1;
  const int per_part = (nall + parts - 1) / parts;
  const int p_begin = part * per_part, nent = min(nall, p_begin + per_part);
  const int span = (nent - p_begin + LANES - 1) / LANES;
  const int e_begin = p_begin + (tid / CPR) * span, e_end = min(nent, e_begin + span);
  auto anc = [&](int u, int l) { return a.lgp >= 0 ? (u >> (a.lgp * l)) : u / a.pw[l]; };
  float A2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) A2[i] = 0.f;
  int cell = -1;
  for (int e = e_begin; e < e_end; ++e) {
    const int u0 = e * P1;
    if (a.L >= 3 && anc(u0, 2) != cell) {   // levels L-1 .. 2, coarsest first
      cell = anc(u0, 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) A2[i] = 0.f;
      for (int l = a.L - 1; l >= 2; --l) {
        const int32_t r = ro[a.lb[l] + anc(u0, l)];
        if (r >= 0) {
          float x[8];
          rows(r, x);
          const float w = a.inv[l];
#pragma unroll
          for (int i = 0; i < 8; ++i) A2[i] += x[i] * w;
        }
      }
    }
    float A[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) A[i] = A2[i];
    if (a.L >= 2) {
      const int32_t r = ro[a.lb[1] + e];
      if (r >= 0) {
        float x[8];
        rows(r, x);
        const float w = a.inv[1];
#pragma unroll
        for (int i = 0; i < 8; ++i) A[i] += x[i] * w;
      }
    }
    Pack8<TO> shared_row;
    shared_row.set(A);
    TO *orow = out + (int64_t)u0 * d;
    for (int k0 = 0; k0 < P1; k0 += 4) {
      float x[4][8];
      int32_t r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        r[k] = k0 + k < P1 ? ro[u0 + k0 + k] : -1;   // level 0 starts at slot 0
        if (r[k] >= 0) rows(r[k], x[k]);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k0 + k >= P1) break;
        TO *dst = orow + (k0 + k) * d;
        if (r[k] >= 0) {
          float o[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = A[i] + x[k][i];
          Pack8<TO> v;
          v.set(o);
          put(v, dst);
        } else {
          put(shared_row, dst);
        }
      }
    }
  }
}

}  // namespace lh
