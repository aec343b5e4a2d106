// Stage 3b for float32 I/O: causal attention on the gathered subsequence
// (gist.science explainer "Long Context Pre-Training with Lighthouse
// Attention", technical summary 2.C: ordinary SDPA on the dense
// subsequence), forward and backward, in float32 on the vector ALUs.
//
// Mask: query j sees keys j' <= j whose row is not REDUNDANT.
//
// Forward: one wavefront per query row.  Keys are visited in blocks of 64,
// one key per lane for the logit (a full dot product per lane), then an
// online softmax across the block; the block's probabilities go to LDS and
// each lane accumulates its own output columns.  Backward: the same shape,
// one wavefront per query row for dQ and one per key row for dK and dV, so
// no sum needs atomics.  Dot products and the sums over keys or queries are
// carried in float64 (the path serves float32 I/O, whose outputs are held to
// 1e-5), and results are rounded once to float32.
#include "lh_internal.h"

namespace lh {

template <int D>
__device__ __forceinline__ double dot_row(const float *a, const float *b) {
  double s = 0.0;
#pragma unroll 8
  for (int i = 0; i < D; i += 4) {
    const float4 x = *reinterpret_cast<const float4 *>(a + i);
    const float4 y = *reinterpret_cast<const float4 *>(b + i);
    s = fma((double)x.x, (double)y.x, s);
    s = fma((double)x.y, (double)y.y, s);
    s = fma((double)x.z, (double)y.z, s);
    s = fma((double)x.w, (double)y.w, s);
  }
  return s;
}

__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(const float *qs, const float *ks,
                                                           const float *vs,
                                                           const uint8_t *flags, float *os,
                                                           float *lse, int64_t S, float scale) {
  __shared__ double pbuf[4][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + w;
  const int64_t bh = blockIdx.y;
  if (j >= S) return;
  const float *q = qs + (bh * S + j) * D;
  const float *K = ks + bh * S * D, *V = vs + bh * S * D;
  const uint8_t *fl = flags + bh * S;
  constexpr int CPL = D / 64;   // output columns per lane
  double o[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) o[i] = 0.0;
  double m = -INFINITY, l = 0.0;
  for (int64_t k0 = 0; k0 <= j; k0 += 64) {
    const int64_t key = k0 + lane;
    double s = -INFINITY;
    if (key <= j && !(fl[key] & LH_ROW_REDUNDANT)) s = scale * dot_row<D>(q, K + key * D);
    const double mb = wave_max_d(s);
    const double mn = fmax(m, mb);
    const double mu = mn == -INFINITY ? 0.0 : mn;
    const double p = s == -INFINITY ? 0.0 : exp(s - mu);
    const double alpha = m == -INFINITY ? 0.0 : exp(m - mu);
    l = l * alpha + wave_sum_d(p);
    pbuf[w][lane] = p;
    __builtin_amdgcn_wave_barrier();
    const int nk = (int)min((int64_t)64, j + 1 - k0);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      double acc = o[i] * alpha;
      for (int u = 0; u < nk; ++u) acc = fma(pbuf[w][u], (double)V[(k0 + u) * D + lane + 64 * i], acc);
      o[i] = acc;
    }
    __builtin_amdgcn_wave_barrier();
    m = mn;
  }
  float *out = os + (bh * S + j) * D;
#pragma unroll
  for (int i = 0; i < CPL; ++i) out[lane + 64 * i] = (float)(o[i] / l);
  if (lane == 0) lse[bh * S + j] = (float)(m + log(l));
}

// dQ: one wavefront per query row j
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_f32_kernel(
    const float *qs, const float *ks, const float *vs, const float *lse, const float *drow,
    const uint8_t *flags, const float *dos, float *dqs, int64_t S, float scale) {
  __shared__ double pbuf[4][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + w;
  const int64_t bh = blockIdx.y;
  if (j >= S) return;
  const float *q = qs + (bh * S + j) * D, *dO = dos + (bh * S + j) * D;
  const float *K = ks + bh * S * D, *V = vs + bh * S * D;
  const uint8_t *fl = flags + bh * S;
  const double L = lse[bh * S + j], Dj = drow[bh * S + j];
  constexpr int CPL = D / 64;
  double dq[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) dq[i] = 0.0;
  for (int64_t k0 = 0; k0 <= j; k0 += 64) {
    const int64_t key = k0 + lane;
    double ds = 0.0;
    if (key <= j && !(fl[key] & LH_ROW_REDUNDANT)) {
      const double p = exp(scale * dot_row<D>(q, K + key * D) - L);
      const double dp = dot_row<D>(dO, V + key * D);
      ds = p * (dp - Dj);
    }
    pbuf[w][lane] = ds;
    __builtin_amdgcn_wave_barrier();
    const int nk = (int)min((int64_t)64, j + 1 - k0);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      double acc = dq[i];
      for (int u = 0; u < nk; ++u) acc = fma(pbuf[w][u], (double)K[(k0 + u) * D + lane + 64 * i], acc);
      dq[i] = acc;
    }
    __builtin_amdgcn_wave_barrier();
  }
  float *out = dqs + (bh * S + j) * D;
#pragma unroll
  for (int i = 0; i < CPL; ++i) out[lane + 64 * i] = (float)(dq[i] * scale);
}

// dK, dV: one wavefront per key row k (queries j >= k); a REDUNDANT key is
// attended by nobody and gets zero gradients
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dkv_f32_kernel(
    const float *qs, const float *ks, const float *vs, const float *lse, const float *drow,
    const uint8_t *flags, const float *dos, float *dks, float *dvs, int64_t S, float scale) {
  __shared__ double pbuf[4][64], dsbuf[4][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t kr = (int64_t)blockIdx.x * 4 + w;
  const int64_t bh = blockIdx.y;
  if (kr >= S) return;
  const float *k = ks + (bh * S + kr) * D, *v = vs + (bh * S + kr) * D;
  const float *Q = qs + bh * S * D, *dO = dos + bh * S * D;
  const float *LSE = lse + bh * S, *DR = drow + bh * S;
  const bool dead = (flags[bh * S + kr] & LH_ROW_REDUNDANT) != 0;
  constexpr int CPL = D / 64;
  double dk[CPL], dv[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) dk[i] = dv[i] = 0.0;
  if (!dead) {
    for (int64_t j0 = kr; j0 < S; j0 += 64) {
      const int64_t jq = j0 + lane;
      double p = 0.0, ds = 0.0;
      if (jq < S) {
        p = exp(scale * dot_row<D>(Q + jq * D, k) - (double)LSE[jq]);
        const double dp = dot_row<D>(dO + jq * D, v);
        ds = p * (dp - (double)DR[jq]);
      }
      pbuf[w][lane] = p;
      dsbuf[w][lane] = ds;
      __builtin_amdgcn_wave_barrier();
      const int nq = (int)min((int64_t)64, S - j0);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        double a1 = dv[i], a2 = dk[i];
        for (int u = 0; u < nq; ++u) {
          a1 = fma(pbuf[w][u], (double)dO[(j0 + u) * D + lane + 64 * i], a1);
          a2 = fma(dsbuf[w][u], (double)Q[(j0 + u) * D + lane + 64 * i], a2);
        }
        dv[i] = a1;
        dk[i] = a2;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    dks[(bh * S + kr) * D + lane + 64 * i] = (float)(dk[i] * scale);
    dvs[(bh * S + kr) * D + lane + 64 * i] = (float)dv[i];
  }
}

// one workgroup of 256 per 4 rows of every head along x
lh_status check_attn_f32_supported(const Geo &g) {
  return grid_fits(cdiv(g.S, 4), 256) ? LH_OK : LH_ERR_UNSUPPORTED;
}

lh_status launch_attn_fwd_f32(const Geo &g, const float *qs, const float *ks, const float *vs,
                              const uint8_t *flags, float *os, float *lse, hipStream_t st) {
  dim3 grid(cdiv(g.S, 4), (unsigned)g.BH());
  if (g.d == 128)
    hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, grid, dim3(256), 0, st, qs, ks, vs, flags, os, lse, g.S, g.scale);
  else
    hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, grid, dim3(256), 0, st, qs, ks, vs, flags, os, lse, g.S, g.scale);
  return hip_status();
}

lh_status launch_attn_bwd_f32(const Geo &g, const float *qs, const float *ks, const float *vs,
                              const float *os, const float *lse, const uint8_t *flags,
                              const float *dos, float *drow, float *dqs, float *dks, float *dvs,
                              hipStream_t st) {
  (void)os;
  dim3 grid(cdiv(g.S, 4), (unsigned)g.BH());
  if (g.d == 128) {
    hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<128>, grid, dim3(256), 0, st, qs, ks, vs, lse, drow, flags, dos, dqs, g.S, g.scale);
    hipLaunchKernelGGL(attn_bwd_dkv_f32_kernel<128>, grid, dim3(256), 0, st, qs, ks, vs, lse, drow, flags, dos, dks, dvs, g.S, g.scale);
  } else {
    hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<64>, grid, dim3(256), 0, st, qs, ks, vs, lse, drow, flags, dos, dqs, g.S, g.scale);
    hipLaunchKernelGGL(attn_bwd_dkv_f32_kernel<64>, grid, dim3(256), 0, st, qs, ks, vs, lse, drow, flags, dos, dks, dvs, g.S, g.scale);
  }
  return hip_status();
}

}  // namespace lh
