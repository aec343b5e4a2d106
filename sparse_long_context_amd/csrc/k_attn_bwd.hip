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
//  * dK/dV: a workgroup owns 128 keys; its 8 wavefronts form two groups of
//    4 (32 keys per wavefront) that take alternate 32-query blocks, from the
//    diagonal to the end, and add their partial dK, dV in LDS at the end.
//    S = Q K^T and dP = dO V^T have the key as the MFMA column, so the lanes
//    holding P and dS are already the A operands of dV += P^T dO and
//    dK += dS^T Q; the B operands dO and Q are read from the same row tiles
//    with the LDS transposing read.  K sits in registers, V in LDS.
//  * dQ: a workgroup owns 128 queries; two groups take alternate 32-key
//    blocks up to the diagonal.  S^T = K Q^T and dP^T = V dO^T have the query
//    as the column, and dS^T is the B operand of dQ^T += K^T dS^T, K^T again
//    from the K row tile through the transposing read.
// Row tiles arrive by direct global->LDS loads, double-buffered per group.
// Grids are one-dimensional, heaviest blocks first over all heads.
//
// Products accumulate in float32.  dO, P and dS enter the MFMAs as two-term
// bf16 splits (hi + lo; the lo*lo term is dropped), so their rounding stays
// near 2^-17 relative; Q, K and V are exact bf16 values already.
// Skips are decided per wavefront (MFMA mixes all 64 lanes, so a lane may
// never sit out an MFMA whose result other lanes use); a dead key column is
// zeroed instead.
#include "lh_mfma.h"

namespace lh {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBwdThreads = 512;

// ---------------------------------------------------------------- dK / dV
constexpr int kKvBK = 128;   // keys per workgroup
constexpr int kKvBQ = 32;    // queries per block

template <int D>
struct KvSmem {
  bf16_t v[kKvBK * D];                 // V rows of the workgroup's keys
  bf16_t q[2][2][kKvBQ * D];           // [group][buffer] Q rows
  bf16_t dh[2][2][kKvBQ * D];          // dO rows, hi part
  bf16_t dl[2][2][kKvBQ * D];          // dO rows, lo part
  float lse2[2][2][kKvBQ];             // lse in log2 units (+inf past S)
  float drow[2][2][kKvBQ];
};

template <int D>
__global__ __launch_bounds__(kBwdThreads, 1) void attn_bwd_dkv_kernel(
    const bf16_t *__restrict__ qs, const bf16_t *__restrict__ ks, const bf16_t *__restrict__ vs,
    const bf16_t *__restrict__ doh, const bf16_t *__restrict__ dol,
    const float *__restrict__ lse, const float *__restrict__ drow,
    const uint8_t *__restrict__ flags, float *__restrict__ dks, float *__restrict__ dvs,
    int64_t S, int32_t BH, float scale) {
  extern __shared__ __align__(16) unsigned char smraw[];
  KvSmem<D> &sm = *reinterpret_cast<KvSmem<D> *>(smraw);
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;

  const int item = (int)blockIdx.x;
  const int kb = item / BH;                      // small kb: longest query range
  const int64_t bh = item % BH;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = wave >> 2, w = wave & 3, gtid = tid & 255;
  const int col = lane & 31, h = lane >> 5;
  const int64_t kw0 = (int64_t)kb * kKvBK + w * 32;
  const int64_t key = kw0 + col;
  const float sl2 = scale * kLog2e;

  const bf16_t *Q = qs + bh * S * D, *DH = doh + bh * S * D, *DL = dol + bh * S * D;
  const float *LSE = lse + bh * S, *DR = drow + bh * S;
  const bool dead = key >= S || (flags[bh * S + min(key, S - 1)] & LH_ROW_REDUNDANT);
  const bool all_dead = __all(dead);

  // K of this lane's key (B operand of S = Q K^T).  It is re-read from
  // global memory (cache-resident) at the end of every block through a
  // pointer the compiler cannot see through, so it is not held in registers
  // across the accumulator-heavy dV/dK phase.
  const bf16_t *kptr = ks + (bh * S + min(key, S - 1)) * D + 8 * h;
  bf16x8 kreg[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) kreg[s] = ld_bf16x8(kptr + s * 16);
  tile_load<D>(sm.v, vs + bh * S * D, (int64_t)kb * kKvBK, S - 1, kKvBK, tid, kBwdThreads);

  f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc_dk[b] = acc_dv[b] = zero16();

  const int qb0 = (int)((int64_t)kb * kKvBK / kKvBQ);
  const int nqb = (int)((S + kKvBQ - 1) / kKvBQ);
  const int niter = (nqb - qb0 + 1) / 2;

#define LH_KV_ISSUE(qb_, buf_)                                                                  \
  do {                                                                                          \
    const int64_t r0 = (int64_t)(qb_) * kKvBQ;                                                  \
    tile_load<D>(sm.q[grp][buf_], Q, r0, S - 1, kKvBQ, gtid, 256);                             \
    tile_load<D>(sm.dh[grp][buf_], DH, r0, S - 1, kKvBQ, gtid, 256);                           \
    tile_load<D>(sm.dl[grp][buf_], DL, r0, S - 1, kKvBQ, gtid, 256);                           \
  } while (0)

  float nl = INFINITY, nd = 0.f;   // this thread's lse2 / drow of the next block
  {
    const int qb = qb0 + grp;
    if (qb < nqb) {
      LH_KV_ISSUE(qb, 0);
      if (gtid < kKvBQ) {
        const int64_t qq = (int64_t)qb * kKvBQ + gtid;
        sm.lse2[grp][0][gtid] = qq < S ? LSE[qq] * kLog2e : INFINITY;
        sm.drow[grp][0][gtid] = qq < S ? DR[qq] : 0.f;
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int it = 0; it < niter; ++it) {
    const int qb = qb0 + 2 * it + grp, qbn = qb + 2, buf = it & 1;
    if (qbn < nqb) {
      LH_KV_ISSUE(qbn, buf ^ 1);
      if (gtid < kKvBQ) {
        const int64_t qq = (int64_t)qbn * kKvBQ + gtid;
        nl = qq < S ? LSE[qq] * kLog2e : INFINITY;
        nd = qq < S ? DR[qq] : 0.f;
      }
    }
    const int64_t q0 = (int64_t)qb * kKvBQ;
    if (qb < nqb && !all_dead && q0 + kKvBQ - 1 >= kw0) {   // wavefront-uniform
      const bf16_t *tq = sm.q[grp][buf], *th = sm.dh[grp][buf], *tl = sm.dl[grp][buf];
      const float *l2 = sm.lse2[grp][buf], *dr = sm.drow[grp][buf];
      // S = Q K^T and dP = dO V^T (lane: key column; rows: queries 8I + 4h + J)
      f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        sacc = mfma32(ld_rowop<D>(tq, col, s, h), kreg[s], sacc);
        const bf16x8 bv = ld_rowop<D>(sm.v, w * 32 + col, s, h);
        dpacc = mfma32(ld_rowop<D>(th, col, s, h), bv, dpacc);
        dpacc = mfma32(ld_rowop<D>(tl, col, s, h), bv, dpacc);
      }
      const bool diag = q0 < kw0 + 32;
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int ql = 8 * I + 4 * h;
        const float4 lv = *reinterpret_cast<const float4 *>(l2 + ql);
        const float4 dv = *reinterpret_cast<const float4 *>(dr + ql);
        const float lj[4] = {lv.x, lv.y, lv.z, lv.w}, dj[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          const int v = 4 * I + J;
          float p = __builtin_amdgcn_exp2f(sacc[v] * sl2 - lj[J]);
          if (dead || (diag && q0 + ql + J < key)) p = 0.f;
          sacc[v] = p;
          dpacc[v] = p * (dpacc[v] - dj[J]);
        }
      }
      // dV += P^T dO, dK += dS^T Q over two 16-query steps
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 aph, apl, ash, asl;
        pack_split(sacc, 8 * s2, aph, apl);
        pack_split(dpacc, 8 * s2, ash, asl);
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const bf16x8 bdh = ld_colop<D>(th, s2, 32 * b, lane);
          const bf16x8 bdl = ld_colop<D>(tl, s2, 32 * b, lane);
          const bf16x8 bq = ld_colop<D>(tq, s2, 32 * b, lane);
          acc_dv[b] = mfma32(aph, bdh, acc_dv[b]);
          acc_dv[b] = mfma32(aph, bdl, acc_dv[b]);
          acc_dv[b] = mfma32(apl, bdh, acc_dv[b]);
          acc_dk[b] = mfma32(ash, bq, acc_dk[b]);
          acc_dk[b] = mfma32(asl, bq, acc_dk[b]);
        }
      }
    }
    {
      const bf16_t *kp = kptr;
      asm volatile("" : "+v"(kp));
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) kreg[s] = ld_bf16x8(kp + s * 16);
    }
    if (qbn < nqb && gtid < kKvBQ) {
      sm.lse2[grp][buf ^ 1][gtid] = nl;
      sm.drow[grp][buf ^ 1][gtid] = nd;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
#undef LH_KV_ISSUE

  // group 1 adds its partials to group 0's through LDS (dK, then dV)
  float *xo = reinterpret_cast<float *>(smraw);   // [DB*16][256]
#define LH_KV_MERGE(ACC, OUT, F)                                                              \
  do {                                                                                        \
    if (grp == 1) {                                                                           \
      _Pragma("unroll") for (int b = 0; b < DB; ++b)                                          \
      _Pragma("unroll") for (int v = 0; v < 16; ++v) xo[(b * 16 + v) * 256 + gtid] = ACC[b][v]; \
    }                                                                                         \
    __syncthreads();                                                                          \
    if (grp == 0) {                                                                           \
      /* lane: head-dim column b*32 + col; rows are keys kw0 + 8I + 4h + J */                 \
      _Pragma("unroll") for (int b = 0; b < DB; ++b)                                          \
      _Pragma("unroll") for (int v = 0; v < 16; ++v) {                                        \
        const int64_t kr = kw0 + 8 * (v >> 2) + 4 * h + (v & 3);                              \
        const float x = (ACC[b][v] + xo[(b * 16 + v) * 256 + gtid]) * (F);                    \
        if (kr < S) OUT[(bh * S + kr) * D + b * 32 + col] = x;                                \
      }                                                                                       \
    }                                                                                         \
    __syncthreads();                                                                          \
  } while (0)
  LH_KV_MERGE(acc_dk, dks, scale);
  LH_KV_MERGE(acc_dv, dvs, 1.f);
#undef LH_KV_MERGE
}

// ---------------------------------------------------------------- dQ
constexpr int kQBQ = 128;   // queries per workgroup
constexpr int kQBK = 32;    // keys per block

template <int D>
struct QSmem {
  bf16_t k[2][2][kQBK * D];   // [group][buffer] K rows
  bf16_t v[2][2][kQBK * D];   // V rows
  float bias[2][2][kQBK];
};

template <int D>
__global__ __launch_bounds__(kBwdThreads, 1) void attn_bwd_dq_kernel(
    const bf16_t *__restrict__ qs, const bf16_t *__restrict__ ks, const bf16_t *__restrict__ vs,
    const bf16_t *__restrict__ doh, const bf16_t *__restrict__ dol,
    const float *__restrict__ lse, const float *__restrict__ drow,
    const uint8_t *__restrict__ flags, float *__restrict__ dqs, int64_t S, int32_t BH,
    float scale) {
  extern __shared__ __align__(16) unsigned char smraw[];
  QSmem<D> &sm = *reinterpret_cast<QSmem<D> *>(smraw);
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;

  const int nqb = (int)((S + kQBQ - 1) / kQBQ);
  const int item = (int)blockIdx.x;
  const int qb = nqb - 1 - item / BH;             // heaviest first
  const int64_t bh = item % BH;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = wave >> 2, w = wave & 3, gtid = tid & 255;
  const int col = lane & 31, h = lane >> 5;
  const int64_t q0w = (int64_t)qb * kQBQ + w * 32;
  const int64_t q = q0w + col;
  const float sl2 = scale * kLog2e;

  const bf16_t *Kg = ks + bh * S * D, *Vg = vs + bh * S * D;
  const uint8_t *fl = flags + bh * S;

  bf16x8 qreg[KSTEPS], dregh[KSTEPS], dregl[KSTEPS];
  {
    const int64_t qc = min(q, S - 1);   // rows past S are never stored
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      qreg[s] = ld_bf16x8(qs + (bh * S + qc) * D + s * 16 + 8 * h);
      dregh[s] = ld_bf16x8(doh + (bh * S + qc) * D + s * 16 + 8 * h);
      dregl[s] = ld_bf16x8(dol + (bh * S + qc) * D + s * 16 + 8 * h);
    }
  }
  const float lse2 = q < S ? lse[bh * S + q] * kLog2e : INFINITY;
  const float dr = q < S ? drow[bh * S + q] : 0.f;

  f32x16 acc_dq[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc_dq[b] = zero16();

  const int64_t kend = min(S, (int64_t)(qb + 1) * kQBQ);
  const int nkb = (int)((kend + kQBK - 1) / kQBK);
  const int niter = (nkb + 1) / 2;

#define LH_Q_ISSUE(kb_, buf_)                                                                 \
  do {                                                                                        \
    const int64_t r0 = (int64_t)(kb_) * kQBK;                                                 \
    tile_load<D>(sm.k[grp][buf_], Kg, r0, S - 1, kQBK, gtid, 256);                           \
    tile_load<D>(sm.v[grp][buf_], Vg, r0, S - 1, kQBK, gtid, 256);                           \
  } while (0)
#define LH_Q_BIAS(kb_)                                                                        \
  ([&]() -> float {                                                                           \
    const int64_t kk_ = (int64_t)(kb_) * kQBK + (gtid & 31);                                  \
    return (kk_ < S && !(fl[kk_] & LH_ROW_REDUNDANT)) ? 0.f : -INFINITY;                      \
  }())

  if (grp < nkb) {
    LH_Q_ISSUE(grp, 0);
    const float bv = LH_Q_BIAS(grp);
    if (gtid < kQBK) sm.bias[grp][0][gtid] = bv;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int it = 0; it < niter; ++it) {
    const int kb = 2 * it + grp, kbn = kb + 2, buf = it & 1;
    float bnext = 0.f;
    if (kbn < nkb) {
      LH_Q_ISSUE(kbn, buf ^ 1);
      bnext = LH_Q_BIAS(kbn);
    }
    const int64_t k0 = (int64_t)kb * kQBK;
    if (kb < nkb && k0 <= q0w + 31) {   // wavefront-uniform
      const bf16_t *tk = sm.k[grp][buf], *tv = sm.v[grp][buf];
      const float *bias = sm.bias[grp][buf];
      // S^T = K Q^T, dP^T = V dO^T (lane: query column; rows: keys 8I + 4h + J)
      f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        sacc = mfma32(ld_rowop<D>(tk, col, s, h), qreg[s], sacc);
        const bf16x8 av = ld_rowop<D>(tv, col, s, h);
        dpacc = mfma32(av, dregh[s], dpacc);
        dpacc = mfma32(av, dregl[s], dpacc);
      }
      const bool diag = k0 + kQBK - 1 > q0w;
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int kl = 8 * I + 4 * h;
        const float4 bv = *reinterpret_cast<const float4 *>(bias + kl);
        const float bj[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          const int v = 4 * I + J;
          float p = __builtin_amdgcn_exp2f(sacc[v] * sl2 + bj[J] - lse2);
          if (diag && k0 + kl + J > q) p = 0.f;
          dpacc[v] = p * (dpacc[v] - dr);
        }
      }
      // dQ^T += K^T dS^T over two 16-key steps (K^T through the transposing read)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 bsh, bsl;
        pack_split(dpacc, 8 * s2, bsh, bsl);
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const bf16x8 a = ld_colop<D>(tk, s2, 32 * b, lane);
          acc_dq[b] = mfma32(a, bsh, acc_dq[b]);
          acc_dq[b] = mfma32(a, bsl, acc_dq[b]);
        }
      }
    }
    if (kbn < nkb && gtid < kQBK) sm.bias[grp][buf ^ 1][gtid] = bnext;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
#undef LH_Q_ISSUE
#undef LH_Q_BIAS

  // group 1 adds its partial to group 0's through LDS
  float *xo = reinterpret_cast<float *>(smraw);   // [DB*16][256]
  if (grp == 1) {
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) xo[(b * 16 + v) * 256 + gtid] = acc_dq[b][v];
  }
  __syncthreads();
  if (grp == 0 && q < S) {
    float *out = dqs + (bh * S + q) * D;
    // lane: query column; rows are head-dim 8I + 4h + J
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        float o4[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          const int v = 4 * I + J;
          o4[J] = (acc_dq[b][v] + xo[(b * 16 + v) * 256 + gtid]) * scale;
        }
        *reinterpret_cast<float4 *>(out + b * 32 + 8 * I + 4 * h) =
            make_float4(o4[0], o4[1], o4[2], o4[3]);
      }
  }
}

template <typename Smem>
static size_t smem_bytes(size_t merge) {
  return sizeof(Smem) > merge ? sizeof(Smem) : merge;
}

lh_status launch_attn_bwd_dkv_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                                   const bf16_t *vs, const bf16_t *dos_hi, const bf16_t *dos_lo,
                                   const float *lse, const float *drow, const uint8_t *flags,
                                   float *dks, float *dvs, hipStream_t st) {
  const unsigned items = cdiv(g.S, kKvBK) * (unsigned)g.BH();
#define LH_DKV(D)                                                                             \
  do {                                                                                        \
    const size_t shm = smem_bytes<KvSmem<D>>((size_t)(D / 32) * 16 * 256 * 4);              \
    (void)hipFuncSetAttribute((const void *)attn_bwd_dkv_kernel<D>,                           \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);          \
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<D>, dim3(items), dim3(kBwdThreads), shm, st, qs,   \
                       ks, vs, dos_hi, dos_lo, lse, drow, flags, dks, dvs, g.S,               \
                       (int32_t)g.BH(), g.scale);                                             \
  } while (0)
  if (g.d == 128) LH_DKV(128); else LH_DKV(64);
#undef LH_DKV
  return hip_status();
}

lh_status launch_attn_bwd_dq_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                                  const bf16_t *vs, const bf16_t *dos_hi, const bf16_t *dos_lo,
                                  const float *lse, const float *drow, const uint8_t *flags,
                                  float *dqs, hipStream_t st) {
  const unsigned items = cdiv(g.S, kQBQ) * (unsigned)g.BH();
#define LH_DQ(D)                                                                              \
  do {                                                                                        \
    const size_t shm = smem_bytes<QSmem<D>>((size_t)(D / 32) * 16 * 256 * 4);               \
    (void)hipFuncSetAttribute((const void *)attn_bwd_dq_kernel<D>,                            \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);          \
    hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, dim3(items), dim3(kBwdThreads), shm, st, qs,    \
                       ks, vs, dos_hi, dos_lo, lse, drow, flags, dqs, g.S, (int32_t)g.BH(),   \
                       g.scale);                                                              \
  } while (0)
  if (g.d == 128) LH_DQ(128); else LH_DQ(64);
#undef LH_DQ
  return hip_status();
}

lh_status launch_attn_bwd_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                               const bf16_t *vs, const bf16_t *dos_hi, const bf16_t *dos_lo,
                               const float *lse, const float *drow, const uint8_t *flags,
                               float *dqs, float *dks, float *dvs, hipStream_t st) {
  lh_status s = launch_attn_bwd_dkv_bf16(g, qs, ks, vs, dos_hi, dos_lo, lse, drow, flags, dks,
                                         dvs, st);
  if (s != LH_OK) return s;
  return launch_attn_bwd_dq_bf16(g, qs, ks, vs, dos_hi, dos_lo, lse, drow, flags, dqs, st);
}

}  // namespace lh
