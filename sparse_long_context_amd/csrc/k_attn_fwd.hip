// Stage 3b forward for bf16 I/O: causal attention on the gathered
// subsequence on MFMA (gist.science explainer "Long Context Pre-Training with
// Lighthouse Attention", technical summary 2.C: standard attention on the
// dense, contiguous subsequence; edge.aivizor.me news item: the cost moves
// from O(N S d) to O(S^2 d)).  This is the layer's only dense contraction.
//
// Mask: query j sees keys j' <= j whose row is not REDUNDANT (a per-key -inf
// bias staged in LDS next to each key tile).
//
// Tiling.  A workgroup owns 128 queries (4 wavefronts x 32) of one (b, h) and
// walks the key blocks of 64 up to its diagonal, heaviest query blocks first.
// Each wavefront computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the
// query is the MFMA column, so each lane holds one query's 32 logits of the
// block (two lanes per query, one per half of the keys) and the online
// softmax needs one cross-half exchange.  The same accumulator registers,
// rounded to bf16, are the B operand of O^T += V^T P^T; V^T comes from the
// transposed copy of VS, staged in LDS.  Keys of both operands use the same
// permutation inside each 16-key step, so P never moves between lanes.
// The next key block is prefetched into registers while the current one is
// computed.  Accumulation is float32.  P enters the PV product as a two-term
// bf16 split (hi + lo, two MFMAs), so its rounding stays near 2^-17 relative
// even where V carries large values.
#include "lh_mfma.h"

namespace lh {

constexpr int kFwdBM = 128;   // queries per workgroup
constexpr int kFwdBN = 64;    // keys per step
constexpr int kPad = 8;       // LDS row padding (elements)

template <int D>
struct FwdSmem {
  bf16_t k[kFwdBN][D + kPad];        // key rows
  bf16_t vt[D][kFwdBN + kPad];       // V^T: head-dim rows, key columns
  float bias[kFwdBN];                // 0 or -inf per key
};

template <int D>
__global__ __launch_bounds__(256, 1) void attn_fwd_bf16_kernel(
    const bf16_t *__restrict__ qs, const bf16_t *__restrict__ ks,
    const bf16_t *__restrict__ vst, const uint8_t *__restrict__ flags, float *__restrict__ os,
    float *__restrict__ lse, int64_t S, int64_t Sp, float scale_log2) {
  __shared__ FwdSmem<D> sm;
  constexpr int KSTEPS = D / 16;          // k-steps of QK^T
  constexpr int DB = D / 32;              // 32-row blocks of O^T
  constexpr int KPASS = kFwdBN * D / 8 / 256;   // 16-byte chunks per thread, K tile
  constexpr int VPASS = D * kFwdBN / 8 / 256;   // same for the V^T tile

  const int nqb = (int)((S + kFwdBM - 1) / kFwdBM);
  const int qb = nqb - 1 - (int)blockIdx.x;     // heaviest first
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int col = lane & 31, h = lane >> 5;
  const int64_t q0w = (int64_t)qb * kFwdBM + w * 32;
  const int64_t q = q0w + col;

  const bf16_t *Q = qs + bh * S * D;
  const bf16_t *Kg = ks + bh * S * D;
  const bf16_t *Vt = vst + bh * (int64_t)D * Sp;
  const uint8_t *fl = flags + bh * S;

  // this lane's query slice as B operands (k = head dim)
  bf16x8 qreg[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    if (q < S) qreg[s] = ld_bf16x8(Q + q * D + s * 16 + 8 * h);
    else qreg[s] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }

  const int64_t kend = min(S, (int64_t)(qb + 1) * kFwdBM);
  const int nkb = (int)((kend + kFwdBN - 1) / kFwdBN);

  u32x4 kpre[KPASS], vpre[VPASS];
  float bpre = 0.f;
  // global -> registers for key block kb
#define LH_FWD_PREFETCH(kb)                                                                  \
  do {                                                                                       \
    _Pragma("unroll") for (int i = 0; i < KPASS; ++i) {                                     \
      const int idx = i * 256 + tid;                                                         \
      const int r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;                                 \
      /* rows past S repeat row S-1: their keys carry a -inf bias */                       \
      const int64_t key = min((int64_t)(kb) * kFwdBN + r, S - 1);                            \
      kpre[i] = *reinterpret_cast<const u32x4 *>(Kg + key * D + c8);                            \
    }                                                                                        \
    _Pragma("unroll") for (int i = 0; i < VPASS; ++i) {                                     \
      const int idx = i * 256 + tid;                                                         \
      const int r = idx / (kFwdBN / 8), c8 = (idx % (kFwdBN / 8)) * 8;                       \
      vpre[i] = *reinterpret_cast<const u32x4 *>(Vt + (int64_t)r * Sp +                      \
                                                 (int64_t)(kb) * kFwdBN + c8);               \
    }                                                                                        \
    if (tid < kFwdBN) {                                                                      \
      const int64_t key = (int64_t)(kb) * kFwdBN + tid;                                      \
      bpre = (key < S && !(fl[key] & LH_ROW_REDUNDANT)) ? 0.f : -INFINITY;                   \
    }                                                                                        \
  } while (0)
  // registers -> LDS
#define LH_FWD_COMMIT()                                                                      \
  do {                                                                                       \
    _Pragma("unroll") for (int i = 0; i < KPASS; ++i) {                                     \
      const int idx = i * 256 + tid;                                                         \
      const int r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;                                 \
      *reinterpret_cast<u32x4 *>(&sm.k[r][c8]) = kpre[i];                                    \
    }                                                                                        \
    _Pragma("unroll") for (int i = 0; i < VPASS; ++i) {                                     \
      const int idx = i * 256 + tid;                                                         \
      const int r = idx / (kFwdBN / 8), c8 = (idx % (kFwdBN / 8)) * 8;                       \
      *reinterpret_cast<u32x4 *>(&sm.vt[r][c8]) = vpre[i];                                   \
    }                                                                                        \
    if (tid < kFwdBN) sm.bias[tid] = bpre;                                                   \
  } while (0)

  f32x16 acc_o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc_o[b] = zero16();
  float m_run = -INFINITY, l_half = 0.f;

  LH_FWD_PREFETCH(0);
  LH_FWD_COMMIT();
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) LH_FWD_PREFETCH(kb + 1);
    const int64_t k0 = (int64_t)kb * kFwdBN;
    if (k0 <= q0w + 31) {          // some key of the block is visible to this wavefront
      f32x16 acc_s[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        acc_s[kk] = zero16();
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const bf16x8 a = ld_bf16x8(&sm.k[kk * 32 + col][s * 16 + 8 * h]);
          acc_s[kk] = mfma32(a, qreg[s], acc_s[kk]);
        }
      }
      // scaled logits (log2 units), masks, block max
      const bool diag = k0 + kFwdBN - 1 > q0w;
      float mloc = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kl = kk * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
          float x = acc_s[kk][v] * scale_log2 + sm.bias[kl];
          if (diag && k0 + kl > q) x = -INFINITY;
          acc_s[kk][v] = x;
          mloc = fmaxf(mloc, x);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float mu = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - mu);
      float rs = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pv = exp2f(acc_s[kk][v] - mu);
          acc_s[kk][v] = pv;
          rs += pv;
        }
      l_half = l_half * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[b][v] *= alpha;
      // O^T += V^T P^T over four 16-key steps
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 phi, plo;
        pack_split(acc_s[s >> 1], 8 * (s & 1), phi, plo);
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const bf16_t *row = &sm.vt[b * 32 + col][0];
          const bf16x8 a = ld_bf16x4x2(row + 16 * s + 4 * h, row + 16 * s + 8 + 4 * h);
          acc_o[b] = mfma32(a, phi, acc_o[b]);
          acc_o[b] = mfma32(a, plo, acc_o[b]);
        }
      }
    }
    __syncthreads();
    if (kb + 1 < nkb) {
      LH_FWD_COMMIT();
      __syncthreads();
    }
  }

#undef LH_FWD_PREFETCH
#undef LH_FWD_COMMIT
  const float l_tot = l_half + __shfl_xor(l_half, 32);
  if (q < S) {
    const float inv = 1.f / l_tot;
    float *orow = os + (bh * S + q) * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        float o4[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) o4[J] = acc_o[b][4 * I + J] * inv;
        const int dd = b * 32 + 8 * I + 4 * h;
        *reinterpret_cast<float4 *>(orow + dd) = make_float4(o4[0], o4[1], o4[2], o4[3]);
      }
    if (h == 0) lse[bh * S + q] = m_run * 0.69314718055994531f + logf(l_tot);
  }
}

lh_status launch_attn_fwd_bf16(const Geo &g, const bf16_t *qs, const bf16_t *ks,
                               const bf16_t *vst, const uint8_t *flags, float *os, float *lse,
                               hipStream_t st) {
  dim3 grid(cdiv(g.S, kFwdBM), (unsigned)g.BH());
  const float sl2 = g.scale * 1.4426950408889634f;
  if (g.d == 128)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, dim3(256), 0, st, qs, ks, vst, flags, os, lse, g.S, g.Sp, sl2);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, dim3(256), 0, st, qs, ks, vst, flags, os, lse, g.S, g.Sp, sl2);
  return hip_status();
}

}  // namespace lh
