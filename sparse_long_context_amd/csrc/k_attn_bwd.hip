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
//  * dK/dV: a workgroup owns 128 keys and has 4 wavefronts, one per SIMD
//    (32 keys each, up to 512 registers); every wavefront walks the 32-query
//    blocks from its diagonal to the end.  S = Q K^T and dP = dO V^T have the
//    key as the MFMA column, so the lanes holding P and dS are already the A
//    operands of dV += P^T dO and dK += dS^T Q; the B operands dO and Q are
//    read from the same row tiles with the LDS transposing read.  K and V of
//    the wavefront's keys sit in registers.
//  * dQ (k_attn_bwd_dq.hip): a workgroup owns 128 queries (4 wavefronts, 32
//    queries each) and walks the 32-key blocks up to the diagonal.
// Row tiles arrive by direct buffer->LDS loads through a 5-slot ring, and
// each kernel's loop is a three-block software pipeline (below).  Grids are
// one-dimensional, heaviest blocks first over all heads.
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
constexpr int kKvStages = 5;  // LDS ring: three blocks resident, two loading

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
using KvMap = TileMap<D, kKvBQ, kKvThreads>;

// rows q0 .. q0 + 31 of Q, dO hi, dO lo and their lse, D into a stage (rows
// past S read as zeros; they are index-masked)
template <int D>
__device__ __forceinline__ void kv_issue(KvStage<D> &st, const KvMap<D> &map, brsrc Q, brsrc DH,
                                         brsrc DL, brsrc LSE, brsrc DR, int64_t q0, int tid) {
  map.load(st.q, Q, q0);
  map.load(st.dh, DH, q0);
  map.load(st.dl, DL, q0);
  // wavefront 0: lanes 0-31 copy lse, lanes 32-63 drow (which follows lse);
  // two loads, since a buffer resource is uniform over the wavefront
  if (tid < 64) {
    const uint32_t qq = (uint32_t)(q0 + (tid & 31)) * 4;
    if (tid < 32) {
      lds_dma<4>(LSE, st.lse, qq);
    } else {
      lds_dma<4>(DR, st.lse, qq);
    }
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
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L + 2) : "memory");
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
  static_assert(kKvStages == 5, "block qb + 4 is issued into the slot of block qb - 1");
  extern __shared__ __align__(16) unsigned char smraw[];
  KvStage<D> *stg = reinterpret_cast<KvStage<D> *>(smraw);
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;

  const int item = (int)blockIdx.x;
  const int kb = item / BH;                      // small kb: longest query range
  const int64_t bh = item % BH;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wavefront index, scalar
  const int col = lane & 31, h = lane >> 5;
  const int64_t kw0 = (int64_t)kb * kKvBK + w * 32;
  const int64_t key = kw0 + col;
  const float sl2 = scale * kLog2e;

  const uint32_t tb = (uint32_t)(S * D * 2), sb4 = (uint32_t)(S * 4);
  const brsrc Q = make_rsrc(qs + bh * S * D, tb), DH = make_rsrc(doh + bh * S * D, tb),
              DL = make_rsrc(dol + bh * S * D, tb);
  const brsrc LSE = make_rsrc(lse + bh * S, sb4), DR = make_rsrc(drow + bh * S, sb4);
  const bool dead = key >= S || (flags[bh * S + min(key, S - 1)] & LH_ROW_REDUNDANT);
  const bool all_dead = __all(dead);

  KvMap<D> kmap;
  kmap.init(tid);
  const int qb0 = (int)((int64_t)kb * kKvBK / kKvBQ);
  const int nqb = (int)((S + kKvBQ - 1) / kKvBQ);
  for (int j = 0; j < 3; ++j)
    if (qb0 + j < nqb)
      kv_issue<D>(stg[(qb0 + j) % kKvStages], kmap, Q, DH, DL, LSE, DR, (int64_t)(qb0 + j) * kKvBQ,
                  tid);

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

  // Iteration qb (qb0 - 1 .. nqb - 1) waits for block qb + 2, then issues
  // block qb + 4 into the slot of block qb - 1 (every wavefront is past it
  // after the barrier).  A wavefront computes S and dP of block qb + 1 while
  // it turns block qb's S and dP into P and dS and adds block qb's dV and dK,
  // and it reads block qb + 2's row operands for the next iteration: the
  // parts are independent, so MFMAs overlap the exponentials and the reads.
  auto sync = [&](int qb) {
    kv_wait<D>(qb + 3 < nqb, w == 0);
    lds_barrier();
  };
  auto issue = [&](KvStage<D> *st, int qb) {
    if (qb + 4 < nqb)
      kv_issue<D>(*st, kmap, Q, DH, DL, LSE, DR, (int64_t)(qb + 4) * kKvBQ, tid);
  };
  auto slot = [&](int qb) { return &stg[(qb + kKvStages) % kKvStages]; };
  // P, dS of block qb from its S, dP (in place).  EDGE blocks (the one on
  // the wavefront's diagonal, the one crossing S) mask by index; inside the
  // range only dead keys are masked, through an infinite lse.
  const float dead_lse = dead ? INFINITY : 0.f;
  // lse and D of the block's queries 8I + 4h + J (lanes of one half share them)
  struct RowStats { f32x4 l[4], d[4]; };
  auto rowstats = [&](const KvStage<D> *sb, RowStats &r) {
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      r.l[I] = *reinterpret_cast<const f32x4 *>(sb->lse + 8 * I + 4 * h);
      r.d[I] = *reinterpret_cast<const f32x4 *>(sb->drow + 8 * I + 4 * h);
    }
  };
  // HALF selects the rows of one 16-query step (I = 2 HALF, 2 HALF + 1)
  auto softmax = [&](auto edge_tag, auto half_tag, const RowStats &rs, int qb, f32x16 &sa,
                     f32x16 &dp) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    constexpr int HALF = decltype(half_tag)::value;
    const int64_t q0 = (int64_t)qb * kKvBQ;
    const int kr = (int)(key - q0);                       // causal: query index >= kr
    const int qn = (int)min((int64_t)kKvBQ, S - q0);      // queries of the block inside S
#pragma unroll
    for (int I = 2 * HALF; I < 2 * HALF + 2; ++I) {
      const int ql = 8 * I + 4 * h;
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const int v = 4 * I + J;
        // masked entries take exp2(-inf) = 0 (selects, so the exponential
        // stays unconditional and the block stays one basic block)
        float x = sa[v] * sl2 - (rs.l[I][J] * kLog2e + dead_lse);
        if constexpr (EDGE) x = (ql + J < kr || ql + J >= qn) ? -INFINITY : x;
        const float p = __builtin_amdgcn_exp2f(x);
        sa[v] = p;
        dp[v] = p * (dp[v] - rs.d[I][J]);
      }
    }
  };
  // the A operands of S and dP of a block: Q, dO hi, dO lo rows
  struct RowOps { bf16x8 q[KSTEPS], dh[KSTEPS], dl[KSTEPS]; };
  auto rows_q = [&](const KvStage<D> *sb, RowOps &r) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) r.q[s] = ld_rowop<D>(sb->q, col, s, h);
  };
  auto rows_d = [&](const KvStage<D> *sb, RowOps &r) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      r.dh[s] = ld_rowop<D>(sb->dh, col, s, h);
      r.dl[s] = ld_rowop<D>(sb->dl, col, s, h);
    }
  };
  // S = Q K^T and dP = dO V^T of a block (this wavefront's 32 keys)
  auto sdp = [&](const RowOps &r, f32x16 &sn, f32x16 &dn) {
    sn = zero16();
    dn = zero16();
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      sn = mfma32(r.q[s], kreg[s], sn);
      dn = mfma32(r.dh[s], vreg[s], dn);
      dn = mfma32(r.dl[s], vreg[s], dn);
    }
  };
  // the B operands of one 16-query step of a block: dO hi, dO lo, Q
  // columns for every 32-column block of the head dimension
  struct ColOps { bf16x8 dh[DB], dl[DB], q[DB]; };
  auto colops = [&](const KvStage<D> *sb, int s2, ColOps &c) {
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      c.dh[b] = ld_colop<D>(sb->dh, s2, 32 * b, lane);
      c.dl[b] = ld_colop<D>(sb->dl, s2, 32 * b, lane);
      c.q[b] = ld_colop<D>(sb->q, s2, 32 * b, lane);
    }
  };
  // P, dS of one 16-query step as two-term bf16 splits (the A operands)
  struct Packed { bf16x8 ph, pl, sh, sl; };
  auto pack = [&](const f32x16 &pa, const f32x16 &ds, int s2, Packed &k) {
    pack_split(pa, 8 * s2, k.ph, k.pl);
    pack_split(ds, 8 * s2, k.sh, k.sl);
  };
  // dV += P^T dO and dK += dS^T Q over one 16-query step
  auto accum = [&](const Packed &k, const ColOps &c) {
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      acc_dv[b] = mfma32(k.ph, c.dh[b], acc_dv[b]);
      acc_dv[b] = mfma32(k.ph, c.dl[b], acc_dv[b]);
      acc_dv[b] = mfma32(k.pl, c.dh[b], acc_dv[b]);
      acc_dk[b] = mfma32(k.sh, c.q[b], acc_dk[b]);
      acc_dk[b] = mfma32(k.sl, c.q[b], acc_dk[b]);
    }
  };

  using EdgeT = std::true_type;
  using InT = std::false_type;
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  // first block with queries at or past this wavefront's keys
  const int f = all_dead ? nqb : (int)(kw0 / kKvBQ);
  int qb = qb0 - 1;
  if (f >= nqb) {
    for (; qb < nqb; ++qb) {
      sync(qb);
      issue(slot(qb + 4), qb);
    }
  } else {
    for (; qb < f - 1; ++qb) {
      sync(qb);
      issue(slot(qb + 4), qb);
    }
    // qb == f - 1: blocks up to f + 1 have landed.  Prologue: P, dS of
    // block f (the diagonal, index-masked) and S, dP of block f + 1.
    sync(qb);
    issue(slot(qb + 4), qb);
    f32x16 sa, dp;   // S, dP of the block whose P, dS are formed next
    Packed k0, k1;   // P, dS of the block whose dV, dK are added next
    ColOps c0;       // that block's first-step column operands
    RowStats rs;     // lse, D of the block in sa, dp
    RowOps ro;
    rows_q(slot(f), ro);
    rows_d(slot(f), ro);
    sdp(ro, sa, dp);
    rowstats(slot(f), rs);
    softmax(EdgeT(), H0(), rs, f, sa, dp);
    softmax(EdgeT(), H1(), rs, f, sa, dp);
    pack(sa, dp, 0, k0);
    pack(sa, dp, 1, k1);
    if (f + 1 < nqb) {
      rows_q(slot(f + 1), ro);
      rows_d(slot(f + 1), ro);
      sdp(ro, sa, dp);
      rowstats(slot(f + 1), rs);
    }
    colops(slot(f), 0, c0);
    // Steady iteration qb (f .. nqb - 3), a three-block software pipeline:
    // dV and dK of block qb, P and dS of block qb + 1, S and dP of block
    // qb + 2.  The parts are independent, so the exponentials and splits
    // (VALU) run beside the dV/dK MFMAs instead of between dependent ones.
    // The slots are distinct, which the restrict qualifiers state, so the
    // compiler does not make LDS reads wait for the global->LDS loads into
    // `fill`; the explicit vmcnt before each barrier is what orders them.
    // Fenced regions with prescribed interleaves: (1) block qb's first
    // query step (20 MFMAs) with block qb + 1's first-step exponentials and
    // splits, and the reads of block qb's second-step columns and block
    // qb + 2's Q rows; (2) the second step with block qb + 1's second half
    // and the reads of block qb + 2's dO rows; (3) S and dP of block qb + 2
    // with the reads of block qb + 1's first-step columns and block qb + 2's
    // lse and D.  Blocks qb + 1 in this range lie inside the causal range
    // and inside S: no index masks.
    auto iter = [&](KvStage<D> *__restrict__ fill, const KvStage<D> *__restrict__ cur,
                    const KvStage<D> *__restrict__ nx, const KvStage<D> *__restrict__ nx2) {
      issue(fill, qb);
      __builtin_amdgcn_sched_barrier(0);
      ColOps c1;
      colops(cur, 1, c1);
      rows_q(nx2, ro);
      Packed n0, n1;
      accum(k0, c0);
      softmax(InT(), H0(), rs, qb + 1, sa, dp);
      pack(sa, dp, 0, n0);
      sched_mix<5 * DB, 8, (6 * DB + KSTEPS + 7) / 8, (120 + 5 * DB - 1) / (5 * DB)>();
      __builtin_amdgcn_sched_barrier(0);
      rows_d(nx2, ro);
      accum(k1, c1);
      softmax(InT(), H1(), rs, qb + 1, sa, dp);
      pack(sa, dp, 1, n1);
      sched_mix<5 * DB, 8, (2 * KSTEPS + 7) / 8, (120 + 5 * DB - 1) / (5 * DB)>();
      __builtin_amdgcn_sched_barrier(0);
      colops(nx, 0, c0);
      rowstats(nx2, rs);
      sdp(ro, sa, dp);
      sched_mix<3 * KSTEPS, 8, (6 * DB + 8 + 7) / 8, 0>();
      pin(sa);
      pin(dp);
      // keeps the reads under these MFMAs (otherwise they sink to the next
      // iteration, where their consumers would wait on them)
      asm volatile("" ::: "memory");
      k0 = n0;
      k1 = n1;
    };
    for (qb = f; qb < nqb - 2; ++qb) {
      sync(qb);
      iter(slot(qb + 4), slot(qb), slot(qb + 1), slot(qb + 2));
    }
    if (qb == nqb - 2) {
      // dV, dK of block nqb - 2; P, dS of the last block (it may cross S:
      // index-masked)
      sync(qb);
      ColOps c1;
      colops(slot(qb), 1, c1);
      Packed n0, n1;
      accum(k0, c0);
      softmax(EdgeT(), H0(), rs, qb + 1, sa, dp);
      pack(sa, dp, 0, n0);
      accum(k1, c1);
      softmax(EdgeT(), H1(), rs, qb + 1, sa, dp);
      pack(sa, dp, 1, n1);
      colops(slot(qb + 1), 0, c0);
      k0 = n0;
      k1 = n1;
      ++qb;
    }
    // qb == nqb - 1: dV, dK of the last block
    sync(qb);
    ColOps c1;
    colops(slot(qb), 1, c1);
    accum(k0, c0);
    accum(k1, c1);
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

// bf16 I/O: one head's rows fit a buffer resource and the grid's
// work-items fit 32 bits (the ring's LDS does not depend on the geometry)
lh_status check_attn_dkv_supported(const Geo &g) {
  static_assert(sizeof(KvStage<128>) * kKvStages <= kMaxLds, "the d = 128 ring fits");
  if (g.io != LH_BF16) return LH_OK;
  if (!rsrc_fits(g)) return LH_ERR_UNSUPPORTED;
  return grid_fits((int64_t)cdiv(g.S, kKvBK) * g.BH(), kKvThreads) ? LH_OK : LH_ERR_UNSUPPORTED;
}

lh_status launch_attn_bwd_dkv_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                                   const bf16_t *vs, const bf16_t *dos_hi, const bf16_t *dos_lo,
                                   const float *lse, const float *drow, const uint8_t *flags,
                                   float *dks, float *dvs, hipStream_t st) {
  if (check_attn_dkv_supported(g) != LH_OK) return LH_ERR_UNSUPPORTED;
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
