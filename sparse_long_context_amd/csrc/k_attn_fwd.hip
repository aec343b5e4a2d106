// Stage 3b forward for bf16 I/O: causal attention on the gathered
// subsequence on MFMA (gist.science explainer "Long Context Pre-Training with
// Lighthouse Attention", technical summary 2.C: standard attention on the
// dense, contiguous subsequence; edge.aivizor.me news item: the cost moves
// from O(N S d) to O(S^2 d)).  This is the layer's only dense contraction
// in the forward.
//
// Mask: query j sees keys j' <= j whose row is not REDUNDANT (a per-key -inf
// bias staged in LDS next to each key tile).
//
// Work decomposition.  A workgroup owns 128 queries of one (b, h) and has 8
// wavefronts in two groups of 4; group g takes the key blocks of 64 with
// index = g (mod 2), so two wavefronts share each SIMD and one's softmax
// overlaps the other's MFMAs.  At the end group 1 hands its partial (max,
// sum, output) to group 0 through LDS and group 0 merges them in a fixed
// order.  The grid is one-dimensional, heaviest query blocks first over all
// heads, so the dispatcher hands out work longest-first.
//
// Per wavefront (32 queries) and key block: S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16, the query being the MFMA column, so each lane
// holds one query's logits (two lanes per query, one per half of the keys).
// Those accumulator registers are the B operand of O^T += V^T P^T once P is
// formed; both operands use the same key permutation inside each 16-key step.
// P enters as a two-term bf16 split (hi + lo), so its rounding stays near
// 2^-17 relative even where V carries large values.  The reference maximum
// is only moved (and O, l rescaled) when a row's maximum grows by more than
// 2^8, which keeps P <= 256.
//
// Tiles reach LDS by direct buffer->LDS loads (buffer_load_dwordx4 ... lds),
// double-buffered, in an XOR-swizzled layout (no padding) that keeps the
// MFMA operand reads free of bank conflicts.
#include "lh_mfma.h"

namespace lh {

constexpr int kFwdBM = 128;   // queries per workgroup
constexpr int kFwdBN = 64;    // keys per block
constexpr int kFwdThreads = 512;

template <int D>
struct FwdSmem {
  bf16_t k[2][2][kFwdBN * D];   // [group][buffer] key rows, swizzled 16-byte chunks
  bf16_t vt[2][2][D * kFwdBN];  // [group][buffer] V^T rows (head dim), swizzled
  float bias[2][2][kFwdBN];     // [group][buffer] 0 or -inf per key
};

// swizzle of 16-byte chunk positions inside a K row (D/8 chunks per row) and
// inside a V^T row (8 chunks of keys per row)
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return (r / (128 / D)) % (D / 8);
}
__device__ __forceinline__ int swz_v(int dd) { return (dd >> 1) & 7; }

template <int D>
__global__ __launch_bounds__(kFwdThreads, 1) void attn_fwd_bf16_kernel(
    const bf16_t *__restrict__ qs, const bf16_t *__restrict__ ks,
    const bf16_t *__restrict__ vst, const uint8_t *__restrict__ flags, float *__restrict__ os,
    float *__restrict__ lse, int64_t S, int64_t Sp, int32_t BH, float scale_log2) {
  extern __shared__ __align__(16) unsigned char smraw[];
  FwdSmem<D> &sm = *reinterpret_cast<FwdSmem<D> *>(smraw);
  constexpr int KSTEPS = D / 16;          // k-steps of QK^T
  constexpr int DB = D / 32;              // 32-row blocks of O^T
  constexpr int KLOADS = kFwdBN * D / 8 / 64 / 4;   // 1 KB loads per wavefront, K tile
  constexpr int VLOADS = D * kFwdBN / 8 / 64 / 4;   // same for the V^T tile

  const int nqb = (int)((S + kFwdBM - 1) / kFwdBM);
  const int item = (int)blockIdx.x;
  const int qb = nqb - 1 - item / BH;     // heaviest first
  const int64_t bh = item % BH;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = wave >> 2, wg = wave & 3, gtid = tid & 255;
  const int col = lane & 31, h = lane >> 5;
  const int64_t q0w = (int64_t)qb * kFwdBM + wg * 32;
  const int64_t q = q0w + col;

  const bf16_t *Q = qs + bh * S * D;
  const brsrc Kg = make_rsrc(ks + bh * S * D, (uint32_t)(S * D * 2));
  const brsrc Vt = make_rsrc(vst + bh * (int64_t)D * Sp, (uint32_t)(D * Sp * 2));
  const uint8_t *fl = flags + bh * S;

  bf16x8 qreg[KSTEPS];
  {
    const int64_t qc = min(q, S - 1);     // rows past S are never stored
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qreg[s] = ld_bf16x8(Q + qc * D + s * 16 + 8 * h);
  }

  const int64_t kend = min(S, (int64_t)(qb + 1) * kFwdBM);
  const int nkb = (int)((kend + kFwdBN - 1) / kFwdBN);
  const int niter = (nkb + 1) / 2;

  // issue the async loads of key block kb into [grp][buf]
#define LH_FWD_ISSUE(kb_, buf_)                                                               \
  do {                                                                                        \
    const int64_t k0_ = (int64_t)(kb_) * kFwdBN;                                              \
    unsigned char *kdst = reinterpret_cast<unsigned char *>(sm.k[grp][buf_]);                 \
    unsigned char *vdst = reinterpret_cast<unsigned char *>(sm.vt[grp][buf_]);                \
    _Pragma("unroll") for (int i = 0; i < KLOADS; ++i) {                                     \
      const int j = wg * KLOADS + i;               /* 1 KB piece of the tile */               \
      const int chunk = j * 64 + lane;             /* 16-byte slot in LDS */                  \
      const int r = chunk / (D / 8), p = chunk % (D / 8);                                     \
      const int c = p ^ swz_k<D>(r);                                                          \
      const int64_t key = min(k0_ + r, S - 1);     /* rows past S: -inf bias */               \
      lds_dma<16>(Kg, kdst + j * 1024, (uint32_t)((key * D + c * 8) * 2));                    \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < VLOADS; ++i) {                                     \
      const int j = wg * VLOADS + i;                                                          \
      const int chunk = j * 64 + lane;                                                        \
      const int dd = chunk / 8, p = chunk % 8;                                                \
      const int c = p ^ swz_v(dd);                                                            \
      lds_dma<16>(Vt, vdst + j * 1024, (uint32_t)(((int64_t)dd * Sp + k0_ + c * 8) * 2));      \
    }                                                                                         \
  } while (0)
#define LH_FWD_BIAS(kb_)                                                                      \
  ([&]() -> float {                                                                           \
    const int64_t key_ = (int64_t)(kb_) * kFwdBN + (gtid & 63);                               \
    return (key_ < S && !(fl[key_] & LH_ROW_REDUNDANT)) ? 0.f : -INFINITY;                    \
  }())

  f32x16 acc_o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc_o[b] = zero16();
  float m_ref = -INFINITY, l_half = 0.f;

  if (grp < nkb) {
    LH_FWD_ISSUE(grp, 0);
    const float bv = LH_FWD_BIAS(grp);
    if (gtid < kFwdBN) sm.bias[grp][0][gtid] = bv;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int it = 0; it < niter; ++it) {
    const int kb = 2 * it + grp, kbn = kb + 2, buf = it & 1;
    float bnext = 0.f;
    if (kbn < nkb) {
      LH_FWD_ISSUE(kbn, buf ^ 1);
      bnext = LH_FWD_BIAS(kbn);
    }
    const int64_t k0 = (int64_t)kb * kFwdBN;
    if (kb < nkb && k0 <= q0w + 31) {   // wavefront-uniform
      const bf16_t *kt = sm.k[grp][buf];
      const bf16_t *vt = sm.vt[grp][buf];
      const float *bias = sm.bias[grp][buf];
      f32x16 acc_s[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        acc_s[kk] = zero16();
        const int r = kk * 32 + col;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const int c = (2 * s + h) ^ swz_k<D>(r);
          const bf16x8 a = ld_bf16x8(kt + (r * (D / 8) + c) * 8);
          acc_s[kk] = mfma32(a, qreg[s], acc_s[kk]);
        }
      }
      // scaled logits (log2 units) with masks; row maximum
      const bool diag = k0 + kFwdBN - 1 > q0w;
      float mloc = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          const int kl = kk * 32 + 8 * I + 4 * h;
          const float4 bv = *reinterpret_cast<const float4 *>(bias + kl);
          const float bj[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            float x = fmaf(acc_s[kk][4 * I + J], scale_log2, bj[J]);
            if (diag && k0 + kl + J > q) x = -INFINITY;
            acc_s[kk][4 * I + J] = x;
            mloc = fmaxf(mloc, x);
          }
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      // move the reference maximum only when the row maximum grew by > 2^8
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
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pv = __builtin_amdgcn_exp2f(acc_s[kk][v] - mu);
          acc_s[kk][v] = pv;
          rs += pv;
        }
      l_half += rs;
      // O^T += V^T P^T over four 16-key steps
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 phi, plo;
        pack_split(acc_s[s >> 1], 8 * (s & 1), phi, plo);
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const int dd = b * 32 + col;
          const bf16_t *row = vt + dd * kFwdBN;
          const int c0 = (2 * s) ^ swz_v(dd), c1 = (2 * s + 1) ^ swz_v(dd);
          const bf16x8 a = ld_bf16x4x2(row + c0 * 8 + 4 * h, row + c1 * 8 + 4 * h);
          acc_o[b] = mfma32(a, phi, acc_o[b]);
          acc_o[b] = mfma32(a, plo, acc_o[b]);
        }
      }
    }
    if (kbn < nkb && gtid < kFwdBN) sm.bias[grp][buf ^ 1][gtid] = bnext;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
#undef LH_FWD_ISSUE
#undef LH_FWD_BIAS

  // merge: group 1 -> LDS -> group 0 (the tile buffers are free now)
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
  __syncthreads();
  if (grp == 0) {
    const float m1 = xm[gtid], l1 = xl[gtid];
    const float m = fmaxf(m_ref, m1);
    const float mu = m == -INFINITY ? 0.f : m;
    const float a0 = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mu);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mu);
    const float lh = l_half * a0 + l1 * a1;
    const float l_tot = lh + __shfl_xor(lh, 32);
    if (q < S) {
      const float inv = 1.f / l_tot;
      float *orow = os + (bh * S + q) * D;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          float o4[4];
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            const int v = 4 * I + J;
            o4[J] = (acc_o[b][v] * a0 + xo[(b * 16 + v) * 256 + gtid] * a1) * inv;
          }
          const int dd = b * 32 + 8 * I + 4 * h;
          *reinterpret_cast<float4 *>(orow + dd) = make_float4(o4[0], o4[1], o4[2], o4[3]);
        }
      if (h == 0) lse[bh * S + q] = mu * 0.69314718055994531f + logf(l_tot);
    }
  }
}

lh_status launch_attn_fwd_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                               const bf16_t *vst, const uint8_t *flags, float *os, float *lse,
                               hipStream_t st) {
  if (!rsrc_fits(g)) return LH_ERR_UNSUPPORTED;
  const unsigned items = cdiv(g.S, kFwdBM) * (unsigned)g.BH();
  const float sl2 = g.scale * 1.4426950408889634f;
  if (g.d == 128) {
    const size_t shm = sizeof(FwdSmem<128>);
    (void)hipFuncSetAttribute((const void *)attn_fwd_bf16_kernel<128>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, dim3(items), dim3(kFwdThreads), shm, st, qs,
                       ks, vst, flags, os, lse, g.S, g.Sp, (int32_t)g.BH(), sl2);
  } else {
    const size_t shm = sizeof(FwdSmem<64>);
    (void)hipFuncSetAttribute((const void *)attn_fwd_bf16_kernel<64>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, dim3(items), dim3(kFwdThreads), shm, st, qs,
                       ks, vst, flags, os, lse, g.S, g.Sp, (int32_t)g.BH(), sl2);
  }
  return hip_status();
}

}  // namespace lh
