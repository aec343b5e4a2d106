// Stage 3b backward for bf16 I/O on MFMA: the standard SDPA backward on the
// subsequence with the forward's mask (gist.science explainer "Long Context
// Pre-Training with Lighthouse Attention", technical summary 2.B and 2.C:
// gradients flow through the dense attention; the selection carries none).
//
//   P = exp(scale Q K^T - lse)      (from the forward's saved lse)
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - drow),  drow = rowsum(dO * O)
//   dQ = scale dS K,  dK = scale dS^T Q
//
// Two kernels, so that no sum needs atomics and results are bitwise
// reproducible:
//  * dK/dV: a workgroup owns 128 keys (4 wavefronts x 32) and walks the query
//    blocks of 64 from its diagonal to the end.  S = Q K^T and dP = dO V^T are
//    formed with the key as the MFMA column, so the lanes holding P and dS
//    are already the A operands of dV += P^T dO and dK += dS^T Q; the B
//    operands dO and Q come from their transposed copies in LDS.
//  * dQ: a workgroup owns 128 queries and walks the key blocks of 64 up to
//    its diagonal; S^T = K Q^T and dP^T = V dO^T put the query on the
//    column, and dS^T is the B operand of dQ^T += K^T dS^T (K^T from the
//    transposed copy of KS).
// Products accumulate in float32.  dO, P and dS enter the MFMAs as two-term
// bf16 splits (hi + lo; the lo*lo term is dropped), so their rounding stays
// near 2^-17 relative; Q, K and V are exact bf16 values already.
// Skips are decided per wavefront (MFMA mixes all 64 lanes, so a lane may
// never sit out an MFMA whose result other lanes use); a dead key column is
// zeroed instead.
#include "lh_mfma.h"

namespace lh {

constexpr int kPad = 8;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- dK / dV
constexpr int kKvBK = 128;   // keys per workgroup
constexpr int kKvBQ = 64;    // queries per step

template <int D>
struct KvSmem {
  bf16_t q[kKvBQ][D + kPad];      // Q rows
  bf16_t dOh[kKvBQ][D + kPad];    // dO rows, hi and lo parts
  bf16_t dOl[kKvBQ][D + kPad];
  bf16_t qt[D][kKvBQ + kPad];     // Q^T
  bf16_t dOth[D][kKvBQ + kPad];   // dO^T, hi and lo parts
  bf16_t dOtl[D][kKvBQ + kPad];
  float lse2[kKvBQ];              // lse in log2 units (+inf past S)
  float drow[kKvBQ];
};

template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkv_kernel(
    const bf16_t *__restrict__ qs, const bf16_t *__restrict__ ks, const bf16_t *__restrict__ vs,
    const bf16_t *__restrict__ qst, const bf16_t *__restrict__ doh,
    const bf16_t *__restrict__ dol, const bf16_t *__restrict__ doth,
    const bf16_t *__restrict__ dotl, const float *__restrict__ lse,
    const float *__restrict__ drow, const uint8_t *__restrict__ flags, float *__restrict__ dks,
    float *__restrict__ dvs, int64_t S, int64_t Sp, float scale) {
  extern __shared__ __align__(16) unsigned char smraw[];
  KvSmem<D> &sm = *reinterpret_cast<KvSmem<D> *>(smraw);
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int RPASS = kKvBQ * D / 8 / 256;    // row tiles: 16-byte chunks per thread
  constexpr int TPASS = D * kKvBQ / 8 / 256;    // transposed tiles

  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int col = lane & 31, h = lane >> 5;
  const int kb = (int)blockIdx.x;               // longest query range first
  const int64_t kw0 = (int64_t)kb * kKvBK + w * 32;
  const int64_t key = kw0 + col;
  const float sl2 = scale * kLog2e;

  const bf16_t *Q = qs + bh * S * D, *dOH = doh + bh * S * D, *dOL = dol + bh * S * D;
  const bf16_t *Qt = qst + bh * (int64_t)D * Sp;
  const bf16_t *dOtH = doth + bh * (int64_t)D * Sp, *dOtL = dotl + bh * (int64_t)D * Sp;
  const float *LSE = lse + bh * S, *DR = drow + bh * S;
  const bool dead = key >= S || (flags[bh * S + min(key, S - 1)] & LH_ROW_REDUNDANT);
  const bool all_dead = __all(dead);

  bf16x8 kreg[KSTEPS], vreg[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    if (key < S) {
      kreg[s] = ld_bf16x8(ks + (bh * S + key) * D + s * 16 + 8 * h);
      vreg[s] = ld_bf16x8(vs + (bh * S + key) * D + s * 16 + 8 * h);
    } else {
      kreg[s] = vreg[s] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
  }
  f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc_dk[b] = acc_dv[b] = zero16();

  const int64_t kfirst = (int64_t)kb * kKvBK;
  const int qb0 = (int)(kfirst / kKvBQ);
  const int nqb = (int)((S + kKvBQ - 1) / kKvBQ);
  for (int qb = qb0; qb < nqb; ++qb) {
    const int64_t q0 = (int64_t)qb * kKvBQ;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RPASS; ++i) {
      const int idx = i * 256 + tid;
      const int r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
      const int64_t qq = q0 + r;
      // rows past S repeat row S-1: their lse2 is +inf, so P = dS = 0
      const int64_t qc = min(qq, S - 1);
      const u32x4 a = *reinterpret_cast<const u32x4 *>(Q + qc * D + c8);
      const u32x4 b = *reinterpret_cast<const u32x4 *>(dOH + qc * D + c8);
      const u32x4 e = *reinterpret_cast<const u32x4 *>(dOL + qc * D + c8);
      *reinterpret_cast<u32x4 *>(&sm.q[r][c8]) = a;
      *reinterpret_cast<u32x4 *>(&sm.dOh[r][c8]) = b;
      *reinterpret_cast<u32x4 *>(&sm.dOl[r][c8]) = e;
    }
#pragma unroll
    for (int i = 0; i < TPASS; ++i) {
      const int idx = i * 256 + tid;
      const int r = idx / (kKvBQ / 8), c8 = (idx % (kKvBQ / 8)) * 8;
      *reinterpret_cast<u32x4 *>(&sm.qt[r][c8]) =
          *reinterpret_cast<const u32x4 *>(Qt + (int64_t)r * Sp + q0 + c8);
      *reinterpret_cast<u32x4 *>(&sm.dOth[r][c8]) =
          *reinterpret_cast<const u32x4 *>(dOtH + (int64_t)r * Sp + q0 + c8);
      *reinterpret_cast<u32x4 *>(&sm.dOtl[r][c8]) =
          *reinterpret_cast<const u32x4 *>(dOtL + (int64_t)r * Sp + q0 + c8);
    }
    if (tid < kKvBQ) {
      const int64_t qq = q0 + tid;
      sm.lse2[tid] = qq < S ? LSE[qq] * kLog2e : INFINITY;
      sm.drow[tid] = qq < S ? DR[qq] : 0.f;
    }
    __syncthreads();
    // wavefront-uniform skip: no query of the block sees a key of this
    // wavefront, or every key of the wavefront is dead
    if (all_dead || q0 + kKvBQ - 1 < kw0) continue;
    const bool diag = q0 < kw0 + 32;

    // the block's two 32-query halves one after the other: S and dP of a
    // half (lane: key column; rows: queries qq*32 + 8I + 4h + J) feed dV and
    // dK at once, so only one half's logits are live
#pragma unroll 1
    for (int qq = 0; qq < 2; ++qq) {
      f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8 aq = ld_bf16x8(&sm.q[qq * 32 + col][s * 16 + 8 * h]);
        sacc = mfma32(aq, kreg[s], sacc);
      }
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8 adh = ld_bf16x8(&sm.dOh[qq * 32 + col][s * 16 + 8 * h]);
        const bf16x8 adl = ld_bf16x8(&sm.dOl[qq * 32 + col][s * 16 + 8 * h]);
        dpacc = mfma32(adh, vreg[s], dpacc);
        dpacc = mfma32(adl, vreg[s], dpacc);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ql = qq * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        float p = exp2f(sacc[v] * sl2 - sm.lse2[ql]);
        if (dead || (diag && q0 + ql < key)) p = 0.f;
        sacc[v] = p;
        dpacc[v] = p * (dpacc[v] - sm.drow[ql]);
      }
      // dV += P^T dO, dK += dS^T Q over the half's two 16-query steps
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int s = 2 * qq + s2;
        bf16x8 aph, apl, ash, asl;
        pack_split(sacc, 8 * s2, aph, apl);
        pack_split(dpacc, 8 * s2, ash, asl);
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const bf16_t *rdh = &sm.dOth[b * 32 + col][0];
          const bf16_t *rdl = &sm.dOtl[b * 32 + col][0];
          const bf16_t *rq = &sm.qt[b * 32 + col][0];
          const bf16x8 bdh = ld_bf16x4x2(rdh + 16 * s + 4 * h, rdh + 16 * s + 8 + 4 * h);
          const bf16x8 bdl = ld_bf16x4x2(rdl + 16 * s + 4 * h, rdl + 16 * s + 8 + 4 * h);
          const bf16x8 bq = ld_bf16x4x2(rq + 16 * s + 4 * h, rq + 16 * s + 8 + 4 * h);
          acc_dv[b] = mfma32(aph, bdh, acc_dv[b]);
          acc_dv[b] = mfma32(aph, bdl, acc_dv[b]);
          acc_dv[b] = mfma32(apl, bdh, acc_dv[b]);
          acc_dk[b] = mfma32(ash, bq, acc_dk[b]);
          acc_dk[b] = mfma32(asl, bq, acc_dk[b]);
        }
      }
    }
  }

  // lane: head-dim column b*32 + col; rows are keys kw0 + 8I + 4h + J
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t kr = kw0 + 8 * (v >> 2) + 4 * h + (v & 3);
      if (kr < S) {
        dks[(bh * S + kr) * D + b * 32 + col] = acc_dk[b][v] * scale;
        dvs[(bh * S + kr) * D + b * 32 + col] = acc_dv[b][v];
      }
    }
}

// ---------------------------------------------------------------- dQ
constexpr int kQBQ = 128;   // queries per workgroup
constexpr int kQBK = 64;    // keys per step

template <int D>
struct QSmem {
  bf16_t k[kQBK][D + kPad];
  bf16_t v[kQBK][D + kPad];
  bf16_t kt[D][kQBK + kPad];
  float bias[kQBK];
};

template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_kernel(
    const bf16_t *__restrict__ qs, const bf16_t *__restrict__ ks, const bf16_t *__restrict__ vs,
    const bf16_t *__restrict__ kst, const bf16_t *__restrict__ doh,
    const bf16_t *__restrict__ dol, const float *__restrict__ lse, const float *__restrict__ drow,
    const uint8_t *__restrict__ flags, float *__restrict__ dqs, int64_t S, int64_t Sp,
    float scale) {
  __shared__ QSmem<D> sm;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int RPASS = kQBK * D / 8 / 256;
  constexpr int TPASS = D * kQBK / 8 / 256;

  const int nqb = (int)((S + kQBQ - 1) / kQBQ);
  const int qb = nqb - 1 - (int)blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int col = lane & 31, h = lane >> 5;
  const int64_t q0w = (int64_t)qb * kQBQ + w * 32;
  const int64_t q = q0w + col;
  const float sl2 = scale * kLog2e;

  const bf16_t *Kg = ks + bh * S * D, *Vg = vs + bh * S * D;
  const bf16_t *Kt = kst + bh * (int64_t)D * Sp;
  const uint8_t *fl = flags + bh * S;

  bf16x8 qreg[KSTEPS], dregh[KSTEPS], dregl[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    if (q < S) {
      qreg[s] = ld_bf16x8(qs + (bh * S + q) * D + s * 16 + 8 * h);
      dregh[s] = ld_bf16x8(doh + (bh * S + q) * D + s * 16 + 8 * h);
      dregl[s] = ld_bf16x8(dol + (bh * S + q) * D + s * 16 + 8 * h);
    } else {
      qreg[s] = dregh[s] = dregl[s] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
  }
  const float lse2 = q < S ? lse[bh * S + q] * kLog2e : INFINITY;
  const float dr = q < S ? drow[bh * S + q] : 0.f;

  f32x16 acc_dq[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc_dq[b] = zero16();

  const int64_t kend = min(S, (int64_t)(qb + 1) * kQBQ);
  const int nkb = (int)((kend + kQBK - 1) / kQBK);
  for (int kb = 0; kb < nkb; ++kb) {
    const int64_t k0 = (int64_t)kb * kQBK;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RPASS; ++i) {
      const int idx = i * 256 + tid;
      const int r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
      // rows past S repeat row S-1: those keys carry a -inf bias
      const int64_t kk = min(k0 + r, S - 1);
      *reinterpret_cast<u32x4 *>(&sm.k[r][c8]) = *reinterpret_cast<const u32x4 *>(Kg + kk * D + c8);
      *reinterpret_cast<u32x4 *>(&sm.v[r][c8]) = *reinterpret_cast<const u32x4 *>(Vg + kk * D + c8);
    }
#pragma unroll
    for (int i = 0; i < TPASS; ++i) {
      const int idx = i * 256 + tid;
      const int r = idx / (kQBK / 8), c8 = (idx % (kQBK / 8)) * 8;
      *reinterpret_cast<u32x4 *>(&sm.kt[r][c8]) =
          *reinterpret_cast<const u32x4 *>(Kt + (int64_t)r * Sp + k0 + c8);
    }
    if (tid < kQBK) {
      const int64_t kk = k0 + tid;
      sm.bias[tid] = (kk < S && !(fl[kk] & LH_ROW_REDUNDANT)) ? 0.f : -INFINITY;
    }
    __syncthreads();
    if (k0 > q0w + 31) continue;
    const bool diag = k0 + kQBK - 1 > q0w;

    f32x16 acc_ds[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8 ak = ld_bf16x8(&sm.k[kk * 32 + col][s * 16 + 8 * h]);
        const bf16x8 av = ld_bf16x8(&sm.v[kk * 32 + col][s * 16 + 8 * h]);
        sacc = mfma32(ak, qreg[s], sacc);
        dpacc = mfma32(av, dregh[s], dpacc);
        dpacc = mfma32(av, dregl[s], dpacc);
      }
      // lane: query column; rows are keys kk*32 + 8I + 4h + J
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kl = kk * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        float p = exp2f(sacc[v] * sl2 + sm.bias[kl] - lse2);
        if (diag && k0 + kl > q) p = 0.f;
        dpacc[v] = p * (dpacc[v] - dr);
      }
      acc_ds[kk] = dpacc;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 bsh, bsl;
      pack_split(acc_ds[s >> 1], 8 * (s & 1), bsh, bsl);
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const bf16_t *rk = &sm.kt[b * 32 + col][0];
        const bf16x8 a = ld_bf16x4x2(rk + 16 * s + 4 * h, rk + 16 * s + 8 + 4 * h);
        acc_dq[b] = mfma32(a, bsh, acc_dq[b]);
        acc_dq[b] = mfma32(a, bsl, acc_dq[b]);
      }
    }
  }
  if (q < S) {
    float *out = dqs + (bh * S + q) * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int dd = b * 32 + 8 * I + 4 * h;
        *reinterpret_cast<float4 *>(out + dd) =
            make_float4(acc_dq[b][4 * I] * scale, acc_dq[b][4 * I + 1] * scale,
                        acc_dq[b][4 * I + 2] * scale, acc_dq[b][4 * I + 3] * scale);
      }
  }
}

// the dK/dV kernel's LDS exceeds the 64 KB default of a launch
static void set_smem(const void *fn, size_t bytes) {
  (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

lh_status launch_attn_bwd_dkv_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                                   const bf16_t *vs, const bf16_t *qst, const bf16_t *dos_hi,
                                   const bf16_t *dos_lo, const bf16_t *dost_hi,
                                   const bf16_t *dost_lo, const float *lse, const float *drow,
                                   const uint8_t *flags, float *dks, float *dvs, hipStream_t st) {
  dim3 grid(cdiv(g.S, kKvBK), (unsigned)g.BH());
#define LH_DKV(D)                                                                          \
  do {                                                                                     \
    const size_t shm = sizeof(KvSmem<D>);                                                  \
    set_smem((const void *)attn_bwd_dkv_kernel<D>, shm);                                   \
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<D>, grid, dim3(256), shm, st, qs, ks, vs, qst,  \
                       dos_hi, dos_lo, dost_hi, dost_lo, lse, drow, flags, dks, dvs, g.S,   \
                       g.Sp, g.scale);                                                     \
  } while (0)
  if (g.d == 128) LH_DKV(128); else LH_DKV(64);
#undef LH_DKV
  return hip_status();
}

lh_status launch_attn_bwd_dq_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                                  const bf16_t *vs, const bf16_t *kst, const bf16_t *dos_hi,
                                  const bf16_t *dos_lo, const float *lse, const float *drow,
                                  const uint8_t *flags, float *dqs, hipStream_t st) {
  dim3 grid(cdiv(g.S, kQBQ), (unsigned)g.BH());
  if (g.d == 128)
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, grid, dim3(256), 0, st, qs, ks, vs, kst, dos_hi, dos_lo, lse, drow, flags, dqs, g.S, g.Sp, g.scale);
  else
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, grid, dim3(256), 0, st, qs, ks, vs, kst, dos_hi, dos_lo, lse, drow, flags, dqs, g.S, g.Sp, g.scale);
  return hip_status();
}

lh_status launch_attn_bwd_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                               const bf16_t *vs, const bf16_t *qst, const bf16_t *kst,
                               const bf16_t *dos_hi, const bf16_t *dos_lo,
                               const bf16_t *dost_hi, const bf16_t *dost_lo, const float *lse,
                               const float *drow, const uint8_t *flags, float *dqs,
                               float *dks, float *dvs, hipStream_t st) {
  lh_status s = launch_attn_bwd_dkv_bf16(g, qs, ks, vs, qst, dos_hi, dos_lo, dost_hi, dost_lo,
                                         lse, drow, flags, dks, dvs, st);
  if (s != LH_OK) return s;
  return launch_attn_bwd_dq_bf16(g, qs, ks, vs, kst, dos_hi, dos_lo, lse, drow, flags, dqs, st);
}

}  // namespace lh
