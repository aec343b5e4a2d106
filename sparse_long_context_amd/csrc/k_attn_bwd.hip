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
#include <type_traits>

#include "lh_mfma.h"

namespace lh {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBwdThreads = 512;

// ---------------------------------------------------------------- dK / dV
constexpr int kKvBK = 128;    // keys per workgroup (32 per wavefront)
constexpr int kKvBQ = 32;     // queries per block
constexpr int kKvThreads = 256;
constexpr int kKvStages = 4;  // LDS ring: two blocks in use, two loading

template <int D>
struct KvStage {
  bf16_t q[kKvBQ * D];    // Q rows of the block
  bf16_t dh[kKvBQ * D];   // dO rows, hi part
  bf16_t dl[kKvBQ * D];   // dO rows, lo part
  float lse[kKvBQ];       // then drow: one 64-lane dword load fills both
  float drow[kKvBQ];
};

// global -> LDS loads one workgroup issues for a block: the three row tiles,
// split over the four wavefronts, plus one dword load (wavefront 0) of the
// block's lse and drow
template <int D>
__device__ __forceinline__ void kv_issue(KvStage<D> &st, const bf16_t *Q, const bf16_t *DH,
                                         const bf16_t *DL, const float *LSE, const float *DR,
                                         int64_t q0, int64_t S, int tid) {
  tile_load<D, kKvBQ, kKvThreads>(st.q, Q, q0, S - 1, tid);
  tile_load<D, kKvBQ, kKvThreads>(st.dh, DH, q0, S - 1, tid);
  tile_load<D, kKvBQ, kKvThreads>(st.dl, DL, q0, S - 1, tid);
  if (tid < 64) {
    const int64_t qq = min(q0 + (tid & 31), S - 1);
    __builtin_amdgcn_global_load_lds((const void *)(tid < 32 ? LSE + qq : DR + qq),
                                     (lds_void *)st.lse, 4, 0, 0);
  }
}

// vmcnt of a wavefront once the block being waited for has landed, given
// whether one more block was issued after it
template <int D>
__device__ __forceinline__ void kv_wait(bool later, bool wave0) {
  constexpr int L = 3 * (kKvBQ * D / 8 / 64) / 4;   // tile loads per wavefront per block
  if (!later) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else if (wave0) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L + 1) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
  }
}

template <int D>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_dkv_kernel(
    const bf16_t *__restrict__ qs, const bf16_t *__restrict__ ks, const bf16_t *__restrict__ vs,
    const bf16_t *__restrict__ doh, const bf16_t *__restrict__ dol,
    const float *__restrict__ lse, const float *__restrict__ drow,
    const uint8_t *__restrict__ flags, float *__restrict__ dks, float *__restrict__ dvs,
    int64_t S, int32_t BH, float scale) {
  static_assert(kKvStages == 4, "block qb + 3 is issued into the slot of block qb - 1");
  extern __shared__ __align__(16) unsigned char smraw[];
  KvStage<D> *stg = reinterpret_cast<KvStage<D> *>(smraw);
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;

  const int item = (int)blockIdx.x;
  const int kb = item / BH;                      // small kb: longest query range
  const int64_t bh = item % BH;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int col = lane & 31, h = lane >> 5;
  const int64_t kw0 = (int64_t)kb * kKvBK + w * 32;
  const int64_t key = kw0 + col;
  const float sl2 = scale * kLog2e;

  const bf16_t *Q = qs + bh * S * D, *DH = doh + bh * S * D, *DL = dol + bh * S * D;
  const float *LSE = lse + bh * S, *DR = drow + bh * S;
  const bool dead = key >= S || (flags[bh * S + min(key, S - 1)] & LH_ROW_REDUNDANT);
  const bool all_dead = __all(dead);

  const int qb0 = (int)((int64_t)kb * kKvBK / kKvBQ);
  const int nqb = (int)((S + kKvBQ - 1) / kKvBQ);
  for (int j = 0; j < 2; ++j)
    if (qb0 + j < nqb)
      kv_issue<D>(stg[(qb0 + j) % kKvStages], Q, DH, DL, LSE, DR, (int64_t)(qb0 + j) * kKvBQ, S, tid);

  // K and V of this lane's key: the B operands of S = Q K^T and dP = dO V^T
  bf16x8 kreg[KSTEPS], vreg[KSTEPS];
  {
    const int64_t kc = (bh * S + min(key, S - 1)) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      kreg[s] = ld_bf16x8(ks + kc + s * 16);
      vreg[s] = ld_bf16x8(vs + kc + s * 16);
    }
  }
  f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc_dk[b] = acc_dv[b] = zero16();

  // Iteration qb (qb0 - 1 .. nqb - 1) waits for block qb + 1, then issues
  // block qb + 3 into the slot of block qb - 1 (every wavefront is past it
  // after the barrier).  A wavefront computes S and dP of block qb + 1 while
  // it turns block qb's S and dP into P and dS and adds block qb's dV and dK:
  // the two halves are independent, so MFMAs overlap the exponentials.
  auto step = [&](int qb) {
    kv_wait<D>(qb + 2 < nqb, w == 0);
    __syncthreads();
    if (qb + 3 < nqb)
      kv_issue<D>(stg[(qb + 3) % kKvStages], Q, DH, DL, LSE, DR, (int64_t)(qb + 3) * kKvBQ, S,
                  tid);
  };
  // S = Q K^T and dP = dO V^T of block qb (lane: key column; rows: queries 8I + 4h + J)
  auto sdp = [&](int qb, f32x16 &sa, f32x16 &dp) {
    const KvStage<D> &sb = stg[qb % kKvStages];
    sa = zero16();
    dp = zero16();
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      sa = mfma32(ld_rowop<D>(sb.q, col, s, h), kreg[s], sa);
      dp = mfma32(ld_rowop<D>(sb.dh, col, s, h), vreg[s], dp);
      dp = mfma32(ld_rowop<D>(sb.dl, col, s, h), vreg[s], dp);
    }
  };
  // P, dS of block qb from its S, dP (in place).  EDGE blocks (the one on
  // the wavefront's diagonal, the one crossing S) mask by index; inside the
  // range only dead keys are masked, through an infinite lse.
  const float dead_lse = dead ? INFINITY : 0.f;
  auto softmax = [&](auto edge_tag, int qb, f32x16 &sa, f32x16 &dp) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const KvStage<D> &sb = stg[qb % kKvStages];
    const int64_t q0 = (int64_t)qb * kKvBQ;
    const int kr = (int)(key - q0);                       // causal: query index >= kr
    const int qn = (int)min((int64_t)kKvBQ, S - q0);      // queries of the block inside S
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const int ql = 8 * I + 4 * h;
      const float4 lv = *reinterpret_cast<const float4 *>(sb.lse + ql);
      const float4 dv = *reinterpret_cast<const float4 *>(sb.drow + ql);
      const float lj[4] = {lv.x, lv.y, lv.z, lv.w}, dj[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const int v = 4 * I + J;
        // masked entries take exp2(-inf) = 0 (selects, so the exponential
        // stays unconditional and the block stays one basic block)
        float x = sa[v] * sl2 - (lj[J] * kLog2e + dead_lse);
        if constexpr (EDGE) x = (ql + J < kr || ql + J >= qn) ? -INFINITY : x;
        const float p = __builtin_amdgcn_exp2f(x);
        sa[v] = p;
        dp[v] = p * (dp[v] - dj[J]);
      }
    }
  };
  // the B operands of one 16-query step of block qb: dO hi, dO lo, Q
  // columns for every 32-column block of the head dimension
  struct ColOps { bf16x8 dh[DB], dl[DB], q[DB]; };
  auto colops = [&](int qb, int s2, ColOps &c) {
    const KvStage<D> &sb = stg[qb % kKvStages];
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      c.dh[b] = ld_colop<D>(sb.dh, s2, 32 * b, lane);
      c.dl[b] = ld_colop<D>(sb.dl, s2, 32 * b, lane);
      c.q[b] = ld_colop<D>(sb.q, s2, 32 * b, lane);
    }
  };
  // dV += P^T dO and dK += dS^T Q over one 16-query step
  auto accum = [&](const f32x16 &pa, const f32x16 &ds, int s2, const ColOps &c) {
    bf16x8 aph, apl, ash, asl;
    pack_split(pa, 8 * s2, aph, apl);
    pack_split(ds, 8 * s2, ash, asl);
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      acc_dv[b] = mfma32(aph, c.dh[b], acc_dv[b]);
      acc_dv[b] = mfma32(aph, c.dl[b], acc_dv[b]);
      acc_dv[b] = mfma32(apl, c.dh[b], acc_dv[b]);
      acc_dk[b] = mfma32(ash, c.q[b], acc_dk[b]);
      acc_dk[b] = mfma32(asl, c.q[b], acc_dk[b]);
    }
  };
  auto grad = [&](int qb, f32x16 sa, f32x16 dp) {   // edge blocks only
    softmax(std::true_type(), qb, sa, dp);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      ColOps c;
      colops(qb, s2, c);
      accum(sa, dp, s2, c);
    }
  };

  // first block with queries at or past this wavefront's keys
  const int f = all_dead ? nqb : (int)(kw0 / kKvBQ);
  int qb = qb0 - 1;
  if (f >= nqb) {
    for (; qb < nqb; ++qb) step(qb);
  } else {
    for (; qb < f - 1; ++qb) step(qb);
    f32x16 sa, dp;
    step(qb);
    sdp(f, sa, dp);
    // block f (the diagonal) has the index mask; later blocks up to nqb - 2
    // lie inside the range; block nqb - 1 goes through grad below
    auto iter = [&](auto edge_tag) {
      constexpr bool EDGE = decltype(edge_tag)::value;
      step(qb);
      // One wavefront per SIMD: no other wavefront hides LDS latency or the
      // exponentials, so the iteration is laid out by hand in fenced regions:
      // (1) all row-operand reads of block qb + 1; (2) its S and dP MFMAs
      // with block qb's exponentials between them, and the column operands
      // of block qb's first query step; (3) that step's MFMAs with the second
      // step's reads; (4) the second step's MFMAs.
      const KvStage<D> &sn_ = stg[(qb + 1) % kKvStages];
      bf16x8 ra[KSTEPS], rh[KSTEPS], rl[KSTEPS];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        ra[s] = ld_rowop<D>(sn_.q, col, s, h);
        rh[s] = ld_rowop<D>(sn_.dh, col, s, h);
        rl[s] = ld_rowop<D>(sn_.dl, col, s, h);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 sn = zero16(), dn = zero16();
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        sn = mfma32(ra[s], kreg[s], sn);
        dn = mfma32(rh[s], vreg[s], dn);
        dn = mfma32(rl[s], vreg[s], dn);
      }
      softmax(edge_tag, qb, sa, dp);
      ColOps c0;
      colops(qb, 0, c0);
      __builtin_amdgcn_sched_barrier(0);
      ColOps c1;
      colops(qb, 1, c1);
      accum(sa, dp, 0, c0);
      __builtin_amdgcn_sched_barrier(0);
      accum(sa, dp, 1, c1);
      sa = sn;
      dp = dn;
    };
    qb = f;
    if (qb < nqb - 1) {
      iter(std::true_type());
      for (++qb; qb < nqb - 1; ++qb) iter(std::false_type());
    }
    step(qb);
    grad(qb, sa, dp);
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
    tile_load<D, kQBK, 256>(sm.k[grp][buf_], Kg, r0, S - 1, gtid);                             \
    tile_load<D, kQBK, 256>(sm.v[grp][buf_], Vg, r0, S - 1, gtid);                             \
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
    const size_t shm = sizeof(KvStage<D>) * kKvStages;                                        \
    (void)hipFuncSetAttribute((const void *)attn_bwd_dkv_kernel<D>,                           \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);          \
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<D>, dim3(items), dim3(kKvThreads), shm, st, qs,    \
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
