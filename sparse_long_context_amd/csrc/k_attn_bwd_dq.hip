// Stage 3b backward for bf16 I/O on MFMA, the dQ kernel (gist.science
// explainer "Long Context Pre-Training with Lighthouse Attention", technical
// summary 2.B and 2.C: gradients flow through the dense attention):
//   P = exp(scale Q K^T - lse),  dS = P * (dP - drow),  dQ = scale dS K,
// with S and dP recomputed here (the dK/dV kernel is k_attn_bwd.hip, which
// states the shared conventions: float32 accumulation, dO and dS as two-term
// bf16 splits, per-wavefront skips, no atomics).
//
// A workgroup owns 128 queries (4 wavefronts, one per SIMD, 32 queries each)
// and walks the 32-key blocks up to the diagonal.  S^T = K Q^T and
// dP^T = V dO^T have the query as the column, and dS^T is the B operand of
// dQ^T += K^T dS^T, K^T again from the K row tile through the transposing
// read.  Q and dO of the wavefront's queries are read only by MFMAs and are
// kept in AGPRs; this file is built with MFMA results in VGPRs, so that the
// softmax reads S^T and dP^T where the MFMAs leave them (with results in
// AGPRs every iteration began by copying both tiles across, with no MFMA
// in flight).
#include <type_traits>

#include "lh_mfma.h"
#include "lh_unpool.h"

namespace lh {

constexpr float kLog2eQ = 1.4426950408889634f;

// ---------------------------------------------------------------- dQ
constexpr int kQBQ = 128;      // queries per workgroup (32 per wavefront)
constexpr int kQBK = 32;       // keys per block
constexpr int kQThreads = 256;
constexpr int kQStages = 5;    // LDS ring: three blocks resident, two loading

static_assert(kQBK == kKeyBlock, "dQ streams the shared key blocks");
template <int D>
using QStage = KeyStage<D>;

// d = 128 needs more than 256 registers (one wavefront per SIMD); d = 64
// fits 256, so two workgroups share each CU
// EPI: 0 = dQS rows only; 1 (bf16) or 2 (float32) = instead, the layer's dQ
// of the workgroup's strata (its 128 rows are whole strata): the rows go to
// LDS and the gather + pooling adjoint runs from there (lh_unpool.h), so the
// token writes overlap other workgroups' MFMA work.
template <int D, int EPI>
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1)))
void attn_bwd_dq_kernel(
    const bf16_t *__restrict__ qs, const bf16_t *__restrict__ ks, const bf16_t *__restrict__ vs,
    const bf16_t *__restrict__ doh, const bf16_t *__restrict__ dol,
    const float *__restrict__ lse, const float *__restrict__ drow,
    const uint8_t *__restrict__ flags, float *__restrict__ dqs, int64_t S, int32_t BH,
    float scale, UnpoolArgs ua, int32_t rps) {
  static_assert(kQStages == 5, "block kb + 4 is issued into the slot of block kb - 1");
  extern __shared__ __align__(16) unsigned char smraw[];
  QStage<D> *stg = reinterpret_cast<QStage<D> *>(smraw);
  // REDUNDANT bits of keys 0 .. kend-1, one 64-bit word per 64 keys
  uint64_t *fl_bits = reinterpret_cast<uint64_t *>(smraw + sizeof(QStage<D>) * kQStages);
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int L = 2 * (kQBK * D / 8 / 64) / 4;   // tile loads per wavefront per block

  const int nqb = (int)((S + kQBQ - 1) / kQBQ);
  const int item = (int)blockIdx.x;
  const int qb = nqb - 1 - item / BH;             // heaviest first
  const int64_t bh = item % BH;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wavefront index, scalar
  const int col = lane & 31, h = lane >> 5;
  const int64_t q0w = (int64_t)qb * kQBQ + w * 32;
  const int64_t q = q0w + col;
  const float sl2 = scale * kLog2eQ;
  const brsrc Kg = make_rsrc(ks + bh * S * D, (uint32_t)(S * D * 2)),
              Vg = make_rsrc(vs + bh * S * D, (uint32_t)(S * D * 2));

  const int64_t kend = min(S, (int64_t)(qb + 1) * kQBQ);
  const int nkb = (int)((kend + kQBK - 1) / kQBK);
  stage_flag_bits<kQThreads>(fl_bits, flags + bh * S, kend, w, lane);

  // this lane's query: Q and dO (hi, lo) are the B operands of S^T = K Q^T
  // and dP^T = V dO^T
  bf16x8 qreg[KSTEPS], dregh[KSTEPS], dregl[KSTEPS];
  {
    const int64_t qc = (bh * S + min(q, S - 1)) * D + 8 * h;   // rows past S are never stored
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      qreg[s] = ld_bf16x8(qs + qc + s * 16);
      dregh[s] = ld_bf16x8(doh + qc + s * 16);
      dregl[s] = ld_bf16x8(dol + qc + s * 16);
    }
  }
  // read only by MFMAs: kept in AGPRs (an MFMA takes A/B from either file)
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    asm volatile("" : "+a"(qreg[s]));
    asm volatile("" : "+a"(dregh[s]));
    asm volatile("" : "+a"(dregl[s]));
  }
  const float lse2 = q < S ? lse[bh * S + q] * kLog2eQ : 0.f;
  const float dr = q < S ? drow[bh * S + q] : 0.f;
  // a wait the compiler sees: the register loads above are complete before
  // the loop (otherwise it re-waits for them inside every iteration)
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  TileMap<D, kQBK, kQThreads> qmap;
  qmap.init(tid);
  auto issue = [&](QStage<D> *st, int kb) {   // block kb + 4 into st
    if (kb + 4 < nkb) {
      qmap.load(st->k, Kg, (int64_t)(kb + 4) * kQBK);   // rows past S read as zeros (masked)
      qmap.load(st->v, Vg, (int64_t)(kb + 4) * kQBK);
    }
  };
  auto slot = [&](int kb) { return &stg[(kb + kQStages) % kQStages]; };
  for (int j = 0; j < 3; ++j) issue(slot(j), j - 4);
  f32x16 acc_dq[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc_dq[b] = zero16();

  // bias (0, or -inf for a redundant key or one past the range) of key
  // block kb, written into its slot by wavefront 0
  auto write_bias = [&](int kb) {
    if (w == 0 && lane < kQBK && kb < nkb)
      slot(kb)->bias[lane] = key_bias(fl_bits, (int64_t)kb * kQBK + lane, kend);
  };
  // Iteration kb (-1 .. nkb - 1) waits for block kb + 2, has wavefront 0
  // write block kb + 2's bias (read after the next barrier), and issues
  // block kb + 4 into the slot of block kb - 1.
  auto sync = [&](int kb) {
    if (kb + 3 >= nkb) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
    lds_barrier();
    write_bias(kb + 2);
  };
  // the bias of a block's keys 8I + 4h + J (lanes of one half share them)
  struct Bias { f32x4 b[4]; };
  auto biases = [&](const QStage<D> *sb, Bias &r) {
#pragma unroll
    for (int I = 0; I < 4; ++I) r.b[I] = *reinterpret_cast<const f32x4 *>(sb->bias + 8 * I + 4 * h);
  };
  // dS^T of block kb from its S^T, dP^T (in place), for the keys of one
  // 16-key step (HALF); EDGE: the block on the wavefront's diagonal (keys
  // past the query masked)
  auto softmax = [&](auto edge_tag, auto half_tag, const Bias &bs, int kb, f32x16 &sa,
                     f32x16 &dp) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    constexpr int HALF = decltype(half_tag)::value;
    const int qr = (int)(q - (int64_t)kb * kQBK);   // causal: key index <= qr
#pragma unroll
    for (int I = 2 * HALF; I < 2 * HALF + 2; ++I) {
      const int kl = 8 * I + 4 * h;
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const int v = 4 * I + J;
        float x = sa[v] * sl2 + (bs.b[I][J] - lse2);
        if constexpr (EDGE) x = kl + J > qr ? -INFINITY : x;
        const float p = __builtin_amdgcn_exp2f(x);
        dp[v] = p * (dp[v] - dr);
      }
    }
  };
  // the A operands of S^T and dP^T of a block: K and V rows
  struct RowOps { bf16x8 k[KSTEPS], v[KSTEPS]; };
  auto rows_k = [&](const QStage<D> *sb, RowOps &r) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) r.k[s] = ld_rowop<D>(sb->k, col, s, h);
  };
  auto rows_v = [&](const QStage<D> *sb, RowOps &r) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) r.v[s] = ld_rowop<D>(sb->v, col, s, h);
  };
  // S^T = K Q^T and dP^T = V dO^T of a block (this wavefront's 32 queries)
  auto sdp = [&](const RowOps &r, f32x16 &sn, f32x16 &dn) {
    sn = zero16();
    dn = zero16();
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      sn = mfma32(r.k[s], qreg[s], sn);
      dn = mfma32(r.v[s], dregh[s], dn);
      dn = mfma32(r.v[s], dregl[s], dn);
    }
  };
  // the A operands of one 16-key step: K^T through the transposing read
  auto colops = [&](const QStage<D> *sb, int s2, bf16x8 (&a)[DB]) {
#pragma unroll
    for (int b = 0; b < DB; ++b) a[b] = ld_colop<D>(sb->k, s2, 32 * b, lane);
  };
  // dQ^T += K^T dS^T over one 16-key step (dS^T as a two-term bf16 split)
  auto accum = [&](const bf16x8 &bsh, const bf16x8 &bsl, const bf16x8 (&a)[DB]) {
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      acc_dq[b] = mfma32(a[b], bsh, acc_dq[b]);
      acc_dq[b] = mfma32(a[b], bsl, acc_dq[b]);
    }
  };
  using EdgeT = std::true_type;
  using InT = std::false_type;
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;

  // block 0's bias is needed right after the first barrier
  write_bias(0);
  // last key block of this wavefront (its diagonal, or the last one of S)
  const int lw = q0w < S ? (int)min((int64_t)nkb - 1, (q0w + 31) / kQBK) : -1;
  int kb = -1;
  if (lw < 0) {
    for (; kb < nkb; ++kb) {
      sync(kb);
      issue(slot(kb + 4), kb);
    }
  } else {
    // kb == -1: blocks 0 and 1 have landed.  Prologue: dS of block 0 and
    // S, dP of block 1.
    sync(kb);
    issue(slot(kb + 4), kb);
    f32x16 sa, dp;               // S^T, dP^T of the block whose dS is formed next
    bf16x8 h0, l0, h1, l1;       // dS^T split of the block whose dQ is added next
    bf16x8 a0[DB];               // that block's first-step K^T operands
    Bias bs;                     // bias of the block in sa, dp
    RowOps ro;
    rows_k(slot(0), ro);
    rows_v(slot(0), ro);
    sdp(ro, sa, dp);
    biases(slot(0), bs);
    if (lw == 0) {
      softmax(EdgeT(), H0(), bs, 0, sa, dp);
      softmax(EdgeT(), H1(), bs, 0, sa, dp);
    } else {
      softmax(InT(), H0(), bs, 0, sa, dp);
      softmax(InT(), H1(), bs, 0, sa, dp);
    }
    pack_split(dp, 0, h0, l0);
    pack_split(dp, 8, h1, l1);
    if (lw >= 1) {
      rows_k(slot(1), ro);
      rows_v(slot(1), ro);
      sdp(ro, sa, dp);
    }
    colops(slot(0), 0, a0);
    // Steady iteration kb (0 .. lw - 2), a three-block software pipeline
    // as in the dK/dV kernel: dQ of block kb, dS of block kb + 1 (inside
    // the causal range: no index mask), S and dP of block kb + 2.  Fenced
    // regions: (1) block kb's first key step (8 MFMAs) with block kb + 1's
    // first-half exponentials and split, and the reads of block kb's
    // second-step K^T, block kb + 2's K rows and block kb + 1's bias; (2)
    // the second step with block kb + 1's second half and the reads of
    // block kb + 2's V rows; (3) S and dP of block kb + 2 with the reads of
    // block kb + 1's first-step K^T.  The restrict qualifiers state that the
    // slots are distinct.
    auto iter = [&](QStage<D> *__restrict__ fill, const QStage<D> *__restrict__ cur,
                    const QStage<D> *__restrict__ nx, const QStage<D> *__restrict__ nx2) {
      issue(fill, kb);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 a1[DB];
      colops(cur, 1, a1);
      biases(nx, bs);
      rows_k(nx2, ro);
      bf16x8 nh0, nl0, nh1, nl1;
      accum(h0, l0, a0);
      softmax(InT(), H0(), bs, kb + 1, sa, dp);
      pack_split(dp, 0, nh0, nl0);
      sched_mix<2 * DB, 2 * DB, (2 * DB + 4 + KSTEPS + 2 * DB - 1) / (2 * DB),
                (110 + 2 * DB - 1) / (2 * DB)>();
      __builtin_amdgcn_sched_barrier(0);
      rows_v(nx2, ro);
      accum(h1, l1, a1);
      softmax(InT(), H1(), bs, kb + 1, sa, dp);
      pack_split(dp, 8, nh1, nl1);
      sched_mix<2 * DB, 2 * DB, (KSTEPS + 2 * DB - 1) / (2 * DB), (110 + 2 * DB - 1) / (2 * DB)>();
      __builtin_amdgcn_sched_barrier(0);
      colops(nx, 0, a0);
      sdp(ro, sa, dp);
      sched_mix<3 * KSTEPS, 8, (2 * DB + 7) / 8, 0>();
      pin_v(sa);
      pin_v(dp);
      asm volatile("" ::: "memory");   // keeps the reads under these MFMAs
      h0 = nh0;
      l0 = nl0;
      h1 = nh1;
      l1 = nl1;
    };
    for (kb = 0; kb < lw - 1; ++kb) {
      sync(kb);
      iter(slot(kb + 4), slot(kb), slot(kb + 1), slot(kb + 2));
    }
    if (kb == lw - 1) {
      // dQ of block lw - 1; dS of the diagonal block lw
      sync(kb);
      issue(slot(kb + 4), kb);
      bf16x8 a1[DB], nh0, nl0, nh1, nl1;
      colops(slot(kb), 1, a1);
      biases(slot(kb + 1), bs);
      accum(h0, l0, a0);
      softmax(EdgeT(), H0(), bs, kb + 1, sa, dp);
      pack_split(dp, 0, nh0, nl0);
      accum(h1, l1, a1);
      softmax(EdgeT(), H1(), bs, kb + 1, sa, dp);
      pack_split(dp, 8, nh1, nl1);
      colops(slot(kb + 1), 0, a0);
      h0 = nh0;
      l0 = nl0;
      h1 = nh1;
      l1 = nl1;
      ++kb;
    }
    // kb == lw: dQ of the diagonal block
    sync(kb);
    issue(slot(kb + 4), kb);
    {
      bf16x8 a1[DB];
      colops(slot(kb), 1, a1);
      accum(h0, l0, a0);
      accum(h1, l1, a1);
    }
    for (++kb; kb < nkb; ++kb) {
      sync(kb);
      issue(slot(kb + 4), kb);
    }
  }

  if constexpr (EPI == 0) {
    if (q < S) {
      float *out = dqs + (bh * S + q) * D;
      // lane: query column; rows are head-dim 8I + 4h + J
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          float o4[4];
#pragma unroll
          for (int J = 0; J < 4; ++J) o4[J] = acc_dq[b][4 * I + J] * scale;
          *reinterpret_cast<float4 *>(out + b * 32 + 8 * I + 4 * h) =
              make_float4(o4[0], o4[1], o4[2], o4[3]);
        }
    }
  } else {
    // every wavefront is past its last ring read (and every copy into the
    // ring has landed: the last iterations wait for vmcnt(0))
    __syncthreads();
    using TO = typename std::conditional<EPI == 1, bf16_t, float>::type;
    const int64_t row0 = (int64_t)qb * kQBQ;
    const int nrows = (int)min((int64_t)kQBQ, S - row0);
    float *rows = reinterpret_cast<float *>(smraw);                          // [kQBQ][D]
    int32_t *ro = reinterpret_cast<int32_t *>(smraw + (size_t)kQBQ * D * 4);  // staged row_of
    if (q < S) {
      float *dst = rows + (q - row0) * D;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          float o4[4];
#pragma unroll
          for (int J = 0; J < 4; ++J) o4[J] = acc_dq[b][4 * I + J] * scale;
          *reinterpret_cast<f32x4 *>(dst + b * 32 + 8 * I + 4 * h) = {o4[0], o4[1], o4[2], o4[3]};
        }
    }
    const int64_t m0 = row0 / rps;
    const int spw = nrows / rps;
    unpool_stage_ro<kQThreads>(ua, ro, ua.row_of + bh * ua.E, m0, spw, row0, row0 + nrows, tid);
    __syncthreads();
    const float *lr = rows + (tid % (D / 8)) * 8;
    auto ld = [&](int32_t r, float *x) {   // r in [row0, row0 + nrows): staged so
      const float *p = lr + (int)(r - row0) * D;
      const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
      x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
      x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
    };
    unpool_strata<TO, D / 8, kQThreads, false>(
        ua, ro, ld, (TO *)ua.dx[0] + (bh * ua.N + m0 * ua.Bc) * D, spw, tid);
  }
}


// LDS of one dQ workgroup: the ring, then one REDUNDANT bit per key of the
// widest key range; with the pooling adjoint in the epilogue, at least the
// workgroup's rows and its strata's staged row_of
static size_t dq_lds(const Geo &g, bool unpool) {
  const size_t ring = g.d == 128 ? sizeof(QStage<128>) * kQStages : sizeof(QStage<64>) * kQStages;
  size_t b = ring + (size_t)((g.S + 63) / 64 * 8);
  if (unpool) {
    const size_t e = (size_t)kQBQ * g.d * 4 + (size_t)(kQBQ / (g.k_s + 1)) * g.T * 4;
    b = b > e ? b : e;
  }
  return b;
}

// bf16 I/O: one head's rows fit a buffer resource, the grid's work-items
// fit 32 bits, and the LDS fits
lh_status check_attn_dq_supported(const Geo &g) {
  if (g.io != LH_BF16) return LH_OK;
  if (!rsrc_fits(g)) return LH_ERR_UNSUPPORTED;
  if (!grid_fits((int64_t)cdiv(g.S, kQBQ) * g.BH(), kQThreads)) return LH_ERR_UNSUPPORTED;
  return dq_lds(g, false) <= kMaxLds ? LH_OK : LH_ERR_UNSUPPORTED;
}

// whether the dQ kernel runs the pooling adjoint of its own rows: d = 64
// (two workgroups per CU, so one's epilogue writes overlap the other's MFMA
// work; at d = 128 a workgroup holds its CU alone, and a separate unpool
// launch after the kernel was measured faster on both d = 128 workloads),
// every workgroup's 128 rows are whole strata, and the epilogue's LDS stays
// within the budget that keeps two workgroups per CU
bool dq_can_unpool(const Geo &g) {
  if (g.d != 64) return false;
  if (g.io != LH_BF16 || kQBQ % (g.k_s + 1) != 0 || g.T > kUnpoolLdsEntries) return false;
  return dq_lds(g, true) <= kMaxLds / 2 && dq_lds(g, false) <= kMaxLds / 2;
}

static lh_status launch_dq(const Geo &g, const bf16_t *qs, const bf16_t *ks, const bf16_t *vs,
                           const bf16_t *dos_hi, const bf16_t *dos_lo, const float *lse,
                           const float *drow, const uint8_t *flags, float *dqs,
                           const int32_t *row_of, void *dq, hipStream_t st) {
  if (check_attn_dq_supported(g) != LH_OK) return LH_ERR_UNSUPPORTED;
  const bool unpool = dq != nullptr;
  if (unpool && !dq_can_unpool(g)) return LH_ERR_UNSUPPORTED;
  const unsigned items = cdiv(g.S, kQBQ) * (unsigned)g.BH();
  const size_t shm = dq_lds(g, unpool);
  UnpoolArgs ua = make_unpool_args(g, unpool ? kQBQ / (int)(g.k_s + 1) : 1);
  ua.row_of = row_of;
  ua.dx[0] = dq;
  const int32_t rps = (int32_t)(g.k_s + 1);
  const int epi = unpool ? (g.out == LH_BF16 ? 1 : 2) : 0;
#define LH_DQ(D, E)                                                                           \
  do {                                                                                        \
    (void)hipFuncSetAttribute((const void *)attn_bwd_dq_kernel<D, E>,                         \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);          \
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, E>), dim3(items), dim3(kQThreads), shm, st, qs, \
                       ks, vs, dos_hi, dos_lo, lse, drow, flags, dqs, g.S, (int32_t)g.BH(),   \
                       g.scale, ua, rps);                                                     \
  } while (0)
  if (g.d == 128) {
    LH_DQ(128, 0);   // the epilogue forms run at d = 64 only (dq_can_unpool)
  } else {
    if (epi == 0) LH_DQ(64, 0); else if (epi == 1) LH_DQ(64, 1); else LH_DQ(64, 2);
  }
#undef LH_DQ
  return hip_status();
}

lh_status launch_attn_bwd_dq_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                                  const bf16_t *vs, const bf16_t *dos_hi, const bf16_t *dos_lo,
                                  const float *lse, const float *drow, const uint8_t *flags,
                                  float *dqs, hipStream_t st) {
  return launch_dq(g, qs, ks, vs, dos_hi, dos_lo, lse, drow, flags, dqs, nullptr, nullptr, st);
}

lh_status launch_attn_bwd_dq_unpool(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                                    const bf16_t *vs, const bf16_t *dos_hi,
                                    const bf16_t *dos_lo, const float *lse, const float *drow,
                                    const uint8_t *flags, const int32_t *row_of, void *dq,
                                    hipStream_t st) {
  return launch_dq(g, qs, ks, vs, dos_hi, dos_lo, lse, drow, flags, nullptr, row_of, dq, st);
}

}  // namespace lh
