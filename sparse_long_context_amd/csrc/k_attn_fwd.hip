// Stage 3b forward for bf16 I/O: causal attention on the gathered
// subsequence on MFMA (gist.science explainer "Long Context Pre-Training with
// Lighthouse Attention", technical summary 2.C: standard attention on the
// dense, contiguous subsequence; edge.aivizor.me news item: the cost moves
// from O(N S d) to O(S^2 d)).  This is the layer's only dense contraction
// in the forward.
//
// Mask: query j sees keys j' <= j whose row is not REDUNDANT (a per-key -inf
// bias staged in LDS next to each key block).
//
// Work decomposition.  A workgroup owns 128 queries of one (b, h) and has 8
// wavefronts in two groups of 4 (32 queries per wavefront, held in
// registers as the B operand of S^T = K Q^T); group g takes the key blocks
// of 32 with index = g (mod 2), so two wavefronts share each SIMD and one's
// softmax overlaps the other's MFMAs.  Key-block pairs (K, V rows and each
// key's bias) stream through an LDS ring of three pairs by direct
// buffer->LDS loads, two pairs ahead, with LDS-side barriers and explicit
// counts of the outstanding loads.  At the end group 1 hands its partial
// (max, sum, output) to group 0 through LDS and group 0 merges them in a
// fixed order.  The grid is one-dimensional, heaviest query blocks first
// over all heads, so the dispatcher hands out work longest-first.
//
// Per wavefront and key block: S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (lane: one query, the 16 keys 8I + 4h + J of its half), an online softmax
// whose reference maximum only moves (and O, l are rescaled) when a query's
// maximum grows by more than 2^8, which keeps P <= 256, and O^T += V^T P^T
// with V^T read from the V rows by the transposing LDS read and P entering
// as a two-term bf16 split (hi + lo), so its rounding stays near 2^-17
// relative even where V carries large values.
#include <type_traits>

#include "lh_mfma.h"

namespace lh {

constexpr int kFwdBQ = 128;        // queries per workgroup (32 per wavefront)
constexpr int kFwdThreads = 512;   // two groups of 4 wavefronts
constexpr int kFwdPairs = 3;       // LDS ring of key-block pairs

// Layer output under the causal hold (the scatter stage, done by the
// forward so that its writes overlap other workgroups' MFMA work): token t
// takes the output row of the LEADER with the largest anchor <= t, and the
// LEADER rows are exactly the rows whose anchor differs from the previous
// row's.  This workgroup's leaders cover the token range [T0, T1): T0 is the
// anchor of its first leader, T1 the end of its last leader's segment (the
// next row with another anchor, possibly in the next workgroup); the
// workgroup of row 0 also zero-fills the tokens before row 0's anchor.  The
// output rows are staged in LDS as the output type (the same rounding as
// the scatter stage), the token range is cut into one contiguous chunk per
// group of lanes (one 16-byte piece of a token row per lane), and a group
// walks its chunk with the row index, so each token is one LDS read and
// one coalesced store.
template <int D, int EPI>
__device__ __forceinline__ void scatter_hold(unsigned char *smraw, int32_t *ep,
                                             const f32x16 (&acc_o)[D / 32], int64_t R0,
                                             int nrows, bool has_row, int wg, int col, int h,
                                             int tid, int64_t bh, void *otok, int64_t N) {
  using OT = typename std::conditional<EPI == 1, bf16_t, float>::type;
  constexpr int DB = D / 32;
  constexpr int RB = D * (int)sizeof(OT);   // bytes per output row
  constexpr int CPT = RB / 16;              // lanes per token row
  constexpr int NG = kFwdThreads / CPT;     // token groups
  int32_t *ep_anc = ep, *ep_lead = ep + kFwdBQ;
  lds_barrier();   // every wavefront is past the merge's LDS reads
  unsigned char *orow = smraw;   // [kFwdBQ][RB]
  if (has_row) {
    const int r = wg * 32 + col;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int dd = b * 32 + 8 * I + 4 * h;
        if constexpr (EPI == 1) {
          *reinterpret_cast<uint2 *>(orow + r * RB + dd * 2) =
              make_uint2(pack2_bf16(acc_o[b][4 * I], acc_o[b][4 * I + 1]),
                         pack2_bf16(acc_o[b][4 * I + 2], acc_o[b][4 * I + 3]));
        } else {
          *reinterpret_cast<float4 *>(orow + r * RB + dd * 4) =
              make_float4(acc_o[b][4 * I], acc_o[b][4 * I + 1], acc_o[b][4 * I + 2],
                          acc_o[b][4 * I + 3]);
        }
      }
  }
  const int32_t a_prev = ep[2 * kFwdBQ + 1];
  // the leader of each local row (-1: its leader is in the previous
  // workgroup; such rows never hold the largest anchor <= t for t >= T0)
  if (tid < nrows) {
    int rr = tid;
    while (rr > 0 && ep_anc[rr - 1] == ep_anc[tid]) --rr;
    ep_lead[tid] = (rr == 0 && R0 > 0 && ep_anc[0] == a_prev) ? -1 : rr;
  }
  lds_barrier();
  const int64_t T1 = ep[2 * kFwdBQ];
  int r0 = 0;   // first local leader
  while (r0 < nrows && ep_lead[r0] != r0) ++r0;
  const int64_t T0 = r0 < nrows ? max((int64_t)0, min((int64_t)ep_anc[r0], N)) : T1;
  const int64_t Z0 = R0 == 0 ? 0 : T0;   // row 0's workgroup: zeros before row 0's anchor
  if (T1 <= Z0) return;
  const int gi = tid / CPT, c = tid % CPT;
  const int64_t chunk = (T1 - Z0 + NG - 1) / NG;
  int64_t t = Z0 + gi * chunk;
  const int64_t te = min(T1, t + chunk);
  if (t >= te) return;
  // last local row with anchor <= t (-1: none)
  int lo = 0, hi = nrows;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)ep_anc[mid] <= t) lo = mid + 1; else hi = mid;
  }
  // r, the anchor of row r + 1 (the next boundary) and the source row's
  // piece stay in registers: a token inside the current segment costs a
  // compare and a store.  r < 0 only before row 0's anchor (zeros); for
  // t >= T0 the row r is at or past the first leader, so its leader is local.
  int r = lo - 1;
  auto next_anchor = [&]() {
    return r + 1 < nrows ? (int64_t)ep_anc[r + 1] : INT64_MAX;
  };
  auto piece = [&]() {
    return r < 0 ? make_uint4(0, 0, 0, 0)
                 : *reinterpret_cast<const uint4 *>(orow + ep_lead[r] * RB + c * 16);
  };
  int64_t nb = next_anchor();
  uint4 val = piece();
  unsigned char *dst = reinterpret_cast<unsigned char *>(otok) + bh * N * RB + c * 16;
  for (; t < te; ++t) {
    if (t >= nb) {
      do {
        ++r;
        nb = next_anchor();
      } while (t >= nb);
      val = piece();
    }
    store16_nt(dst + t * RB, val);   // the layer output: streamed out
  }
}

// EPI: 0 = OS and lse only; 1 (bf16) or 2 (float32) = also the layer output
// under the causal hold, written from this workgroup's rows (see the end).
template <int D, int EPI>
__global__ __launch_bounds__(kFwdThreads) void attn_fwd_bf16_kernel(
    const bf16_t *__restrict__ qs, const bf16_t *__restrict__ ks, const bf16_t *__restrict__ vs,
    const uint8_t *__restrict__ flags, float *__restrict__ os, float *__restrict__ lse, int64_t S,
    int32_t BH, float sl2, const int32_t *__restrict__ anchor, void *__restrict__ otok,
    int64_t N) {
  static_assert(kFwdPairs == 3, "pair i + 2 is issued into the slots of pair i - 1");
  extern __shared__ __align__(16) unsigned char smraw[];
  KeyStage<D> *stg = reinterpret_cast<KeyStage<D> *>(smraw);
  // REDUNDANT bits of keys 0 .. kend-1, one 64-bit word per 64 keys
  uint64_t *fl_bits =
      reinterpret_cast<uint64_t *>(smraw + sizeof(KeyStage<D>) * 2 * kFwdPairs);
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  // the wavefronts that copy tiles: one 1 KB piece of each tile apiece
  constexpr int LOADERS = kKeyBlock * D / 8 < kFwdThreads ? kKeyBlock * D / 8 : kFwdThreads;
  using Map = TileMap<D, kKeyBlock, LOADERS>;
  constexpr int LP = 4 * Map::NP;   // tile loads per loading wavefront per pair

  const int nqb = (int)((S + kFwdBQ - 1) / kFwdBQ);
  const int item = (int)blockIdx.x;
  const int qb = nqb - 1 - item / BH;             // heaviest first
  const int64_t bh = item % BH;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar
  const int grp = wave >> 2, wg = wave & 3, gtid = tid & 255;
  const int col = lane & 31, h = lane >> 5;
  const int64_t q0w = (int64_t)qb * kFwdBQ + wg * 32;
  const int64_t q = q0w + col;
  const brsrc Kg = make_rsrc(ks + bh * S * D, (uint32_t)(S * D * 2)),
              Vg = make_rsrc(vs + bh * S * D, (uint32_t)(S * D * 2));

  const int64_t kend = min(S, (int64_t)(qb + 1) * kFwdBQ);
  const int nkb = (int)((kend + kKeyBlock - 1) / kKeyBlock);
  const int npair = (nkb + 1) / 2;
  stage_flag_bits<kFwdThreads>(fl_bits, flags + bh * S, kend, wave, lane);
  // output scatter: the anchors of this workgroup's rows (rows past S read
  // as +inf), and the end of the last leader's segment (the anchor of the
  // first later row with another anchor, or N) and the anchor of the row
  // before the workgroup, for after the loop (the loop's barriers publish
  // them)
  const int64_t R0 = (int64_t)qb * kFwdBQ;
  const int nrows = (int)min((int64_t)kFwdBQ, S - R0);
  int32_t *ep = reinterpret_cast<int32_t *>(smraw + sizeof(KeyStage<D>) * 2 * kFwdPairs +
                                            (S + 63) / 64 * 8);
  if constexpr (EPI != 0) {
    const int32_t *anc = anchor + bh * S;
    if (tid < kFwdBQ) ep[tid] = tid < nrows ? anc[R0 + tid] : INT32_MAX;
    if (tid == 0) {
      const int32_t alast = anc[R0 + nrows - 1];
      int64_t r = R0 + nrows;
      while (r < S && anc[r] == alast) ++r;
      const int64_t t1 = r < S ? (int64_t)anc[r] : N;
      ep[2 * kFwdBQ] = (int32_t)max((int64_t)0, min(t1, N));
      ep[2 * kFwdBQ + 1] = R0 > 0 ? anc[R0 - 1] : INT32_MIN;
    }
  }

  // this lane's query: the B operand of S^T = K Q^T
  bf16x8 qreg[KSTEPS];
  {
    const int64_t qc = (bh * S + min(q, S - 1)) * D + 8 * h;   // rows past S are never stored
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qreg[s] = ld_bf16x8(qs + qc + s * 16);
  }
  // a wait the compiler sees: the register loads above are complete before
  // the loop (otherwise it re-waits for them inside every iteration)
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  Map map;
  map.init(tid);
  // stage of block g of pair p: each group's ring slots are contiguous, so
  // that a slot fixed at compile time is an immediate offset (< 64 KB) from
  // the group's base
  auto stage = [&](int p, int g) { return &stg[g * kFwdPairs + p % kFwdPairs]; };
  // both blocks of pair p (a block past the range reads rows it never uses,
  // or zeros past S), so that every pair is the same number of loads
  auto issue = [&](int p) {
    if (p < npair && tid < LOADERS) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int64_t r0 = (int64_t)(2 * p + g) * kKeyBlock;
        map.load(stage(p, g)->k, Kg, r0);
        map.load(stage(p, g)->v, Vg, r0);
      }
    }
  };
  // the 64 keys of pair p: their bias, written by wavefront 0
  auto write_bias = [&](int p) {
    if (wave == 0 && p < npair)
      stage(p, lane >> 5)->bias[lane & 31] =
          key_bias(fl_bits, (int64_t)p * 2 * kKeyBlock + lane, kend);
  };
  // Iteration i (0 .. npair - 1) waits for pair i, has wavefront 0 write
  // pair i + 1's bias (read after the next barrier), and issues pair i + 2
  // into the slots of pair i - 1.
  auto sync = [&](int i) {
    if (i + 1 >= npair) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LP) : "memory");
    lds_barrier();
    write_bias(i + 1);
    issue(i + 2);
  };

  f32x16 acc_o[DB];   // O^T: lane = query, rows = head-dim 8I + 4h + J of block b
#pragma unroll
  for (int b = 0; b < DB; ++b) acc_o[b] = zero16();
  float m_ref = -INFINITY;   // reference maximum (log2 units), equal in both halves
  float l_half = 0.f;        // sum of P over this half's keys

  // one key block: S^T, masks, online softmax, O^T += V^T P^T.  On the
  // wavefront's diagonal block (a wave-uniform branch) keys past the query's
  // index qmax within the block are masked as well.
  auto block = [&](const KeyStage<D> *__restrict__ sb, bool diag, int qmax) {
    // all K-row operands in flight at once, then the first-step V^T operands
    bf16x8 kr[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) kr[s] = ld_rowop<D>(sb->k, col, s, h);
    bf16x8 a0[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) a0[b] = ld_colop<D>(sb->v, 0, 32 * b, lane);
    f32x16 sa = zero16();
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) sa = mfma32(kr[s], qreg[s], sa);
    float mloc = -INFINITY;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const f32x4 bj = *reinterpret_cast<const f32x4 *>(sb->bias + 8 * I + 4 * h);
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const int v = 4 * I + J;
        sa[v] = fmaf(sa[v], sl2, bj[J]);
      }
    }
    if (diag) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (8 * (v >> 2) + 4 * h + (v & 3) > qmax) sa[v] = -INFINITY;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, sa[v]);
    mloc = fmaxf(mloc, swap_halves(mloc));
    // move the reference maximum only when the maximum grew by > 2^8
    const bool grow = mloc > m_ref + 8.f;
    if (__any(grow)) {
      const float m_new = grow ? mloc : m_ref;
      const float alpha =
          grow ? (m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new)) : 1.f;
      m_ref = m_new;
      l_half *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[b][v] *= alpha;
    }
    const float mu = m_ref == -INFINITY ? 0.f : m_ref;
    float rs = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = __builtin_amdgcn_exp2f(sa[v] - mu);
      sa[v] = p;
      rs += p;
    }
    l_half += rs;
    // O^T += V^T P^T over two 16-key steps
    bf16x8 phi, plo;
    pack_split(sa, 0, phi, plo);
    bf16x8 a1[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) a1[b] = ld_colop<D>(sb->v, 1, 32 * b, lane);
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      acc_o[b] = mfma32(a0[b], phi, acc_o[b]);
      acc_o[b] = mfma32(a0[b], plo, acc_o[b]);
    }
    pack_split(sa, 8, phi, plo);
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      acc_o[b] = mfma32(a1[b], phi, acc_o[b]);
      acc_o[b] = mfma32(a1[b], plo, acc_o[b]);
    }
  };

  // last key block of this wavefront (its diagonal, or the last one of S)
  const int lw = q0w < S ? (int)min((int64_t)nkb - 1, (q0w + 31) / kKeyBlock) : -1;
  write_bias(0);   // keys 0..63: written and read by wavefront 0's own flag chunk
  issue(0);
  issue(1);
  // pair i of this group's ring slot i % 3; unrolled by the ring size so
  // that every slot is a constant offset from the group's base
  const KeyStage<D> *mine = stg + grp * kFwdPairs;
  auto step = [&](int i, const KeyStage<D> *sb) {
    sync(i);
    const int kb = 2 * i + grp;
    if (kb <= lw) block(sb, kb == lw, (int)(q - (int64_t)kb * kKeyBlock));
  };
  for (int i = 0; i < npair; i += kFwdPairs) {
    step(i, mine);
    if (i + 1 < npair) step(i + 1, mine + 1);
    if (i + 2 < npair) step(i + 2, mine + 2);
  }

  // merge: group 1 -> LDS -> group 0 (the ring is free once every
  // wavefront is past the barrier)
  lds_barrier();
  float *xo = reinterpret_cast<float *>(smraw);            // [DB*16][256 lanes]
  float *xm = xo + 256 * DB * 16, *xl = xm + 256;
  if (grp == 1) {
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) xo[(b * 16 + v) * 256 + gtid] = acc_o[b][v];
    xm[gtid] = m_ref;
    xl[gtid] = l_half;
  }
  lds_barrier();
  if (grp == 0 && lw >= 0) {
    const float m1 = xm[gtid], l1 = xl[gtid];
    const float m = fmaxf(m_ref, m1);
    const float mu = m == -INFINITY ? 0.f : m;
    const float a0 = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mu);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mu);
    const float lh = l_half * a0 + l1 * a1;
    const float l_tot = lh + swap_halves(lh);
    if (q < S) {
      const float inv = 1.f / l_tot;
      float *orow = os + (bh * S + q) * D;
      // lane: query; rows are head-dim 8I + 4h + J
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          float o4[4];
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            const int v = 4 * I + J;
            o4[J] = (acc_o[b][v] * a0 + xo[(b * 16 + v) * 256 + gtid] * a1) * inv;
            if constexpr (EPI != 0) acc_o[b][v] = o4[J];
          }
          *reinterpret_cast<float4 *>(orow + b * 32 + 8 * I + 4 * h) =
              make_float4(o4[0], o4[1], o4[2], o4[3]);
        }
      if (h == 0) lse[bh * S + q] = mu * 0.69314718055994531f + logf(l_tot);
    }
  }
  if constexpr (EPI != 0) scatter_hold<D, EPI>(smraw, ep, acc_o, R0, nrows, grp == 0 && q < S,
                                               wg, col, h, tid, bh, otok, N);
}

// LDS of one forward workgroup: the ring, then one REDUNDANT bit per key of
// the widest key range, then (output scatter) the workgroup's anchors,
// leaders and two bounds.  The merge reuses the ring (256 lanes x (16 DB +
// 2) floats), and so do the staged output rows.
static size_t fwd_lds(const Geo &g, bool epi) {
  const size_t ring = g.d == 128 ? sizeof(KeyStage<128>) * 2 * kFwdPairs
                                 : sizeof(KeyStage<64>) * 2 * kFwdPairs;
  const size_t flb = (size_t)((g.S + 63) / 64 * 8);
  const size_t epb = epi ? (2 * kFwdBQ + 2) * sizeof(int32_t) : 0;
  return ring + flb + epb;
}

// bf16 I/O: one head's rows fit a buffer resource, the grid's work-items
// fit 32 bits, and the LDS of the output-writing form (the larger) fits
lh_status check_attn_fwd_supported(const Geo &g) {
  if (g.io != LH_BF16) return LH_OK;
  if (!rsrc_fits(g)) return LH_ERR_UNSUPPORTED;
  if (!grid_fits((int64_t)cdiv(g.S, kFwdBQ) * g.BH(), kFwdThreads)) return LH_ERR_UNSUPPORTED;
  return fwd_lds(g, true) <= kMaxLds ? LH_OK : LH_ERR_UNSUPPORTED;
}

lh_status launch_attn_fwd_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                               const bf16_t *vs, const uint8_t *flags, float *os, float *lse,
                               hipStream_t st, const int32_t *sel_anchor, void *o) {
  if (check_attn_fwd_supported(g) != LH_OK) return LH_ERR_UNSUPPORTED;
  const unsigned items = cdiv(g.S, kFwdBQ) * (unsigned)g.BH();
  const float sl2 = g.scale * 1.4426950408889634f;
  const int epi = o ? (g.out == LH_BF16 ? 1 : 2) : 0;
#define LH_FWD(D, E)                                                                          \
  do {                                                                                        \
    static_assert(sizeof(KeyStage<D>) * 2 * kFwdPairs >= 256 * (16 * (D / 32) + 2) * 4,       \
                  "the merge fits in the ring");                                              \
    static_assert(sizeof(KeyStage<D>) * 2 * kFwdPairs >= kFwdBQ * D * 4,                      \
                  "the staged output rows fit in the ring");                                  \
    const size_t shm = fwd_lds(g, E != 0);                                                    \
    (void)hipFuncSetAttribute((const void *)attn_fwd_bf16_kernel<D, E>,                       \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);          \
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, E>), dim3(items), dim3(kFwdThreads), shm, st, \
                       qs, ks, vs, flags, os, lse, g.S, (int32_t)g.BH(), sl2, sel_anchor, o,  \
                       g.N);                                                                  \
  } while (0)
  if (g.d == 128) {
    if (epi == 0) LH_FWD(128, 0); else if (epi == 1) LH_FWD(128, 1); else LH_FWD(128, 2);
  } else {
    if (epi == 0) LH_FWD(64, 0); else if (epi == 1) LH_FWD(64, 1); else LH_FWD(64, 2);
  }
#undef LH_FWD
  return hip_status();
}

}  // namespace lh
