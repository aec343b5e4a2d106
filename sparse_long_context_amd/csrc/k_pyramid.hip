// Stage 1 + 2a: symmetric average-pooled pyramid and l2 scores with max-pool
// inheritance, in one pass over Q, K, V.
//
// Method (gist.science explainer "Long Context Pre-Training with Lighthouse
// Attention", technical summary 2.A and 2.B; edge.aivizor.me news item,
// four-stages paragraph): level l entry i is the mean of p consecutive
// level-(l-1) entries, for Q, K and V alike; every entry carries two scores,
// the l2 norms of its level-0 q and k rows, and coarse entries take the max
// of their children.
//
// Work decomposition.  One workgroup covers `spw` whole coarsest cells
// (strata) of one (b, h) and one tensor.  A thread owns an 8-column slice
// (CPR = d/8 threads per row) of one level-g subtree (G = p^g consecutive
// tokens) and streams its tokens once, keeping the running sums of levels
// 1..g in registers (a carry chain: when a level-l entry completes, its sum
// moves into level l+1).  The level-g sums of the workgroup's subtrees go to
// LDS, where levels g+1..L-1 of each stratum are formed.  Every input byte is
// read once and every output byte written once; the kernel is HBM-bound.
//
// Rounding: sums are float64, which holds the sum of a cell's bf16 or
// float32 inputs exactly unless their magnitudes span tens of binades; the
// mean sum / p^l is formed in float64 (exact whenever the mean is
// representable, as every rounding tie is) and then rounded once to the I/O
// type.  A float32 sum would round twice (the sum, then the mean) and, for p
// not a power of two, move some means across a bf16 rounding boundary.
// Squares of a row are summed in float64 and the square root is rounded once
// to float32.
#include "lh_internal.h"

namespace lh {

constexpr int kPyrMaxG = 6;       // deepest per-thread carry chain
constexpr int kPyrThreads = 256;  // workgroup size cap

struct PyrArgs {
  const void *in[3];
  void *pyr[3];
  float *score[3];   // sq for tensor 0, sk for tensor 1, none for V
  int64_t N, E, Bc;
  int32_t d, p, L, g, R, spw;
  int64_t lsize[kMaxLevels], loff[kMaxLevels], pw[kMaxLevels + 1];
  int64_t per[kMaxLevels];   // entries of level l per stratum (Bc / p^l)
  double rp[kMaxLevels];     // 1 / p^l
  double pwd[kMaxLevels];    // p^l
  int32_t pow2;              // p is a power of two: 1 / p^l is exact
  int32_t zbase;             // tensor of blockIdx.z = 0 (tensors before it are skipped)
};

// float64 -> float32 rounding to odd: truncate toward zero and set the last
// bit when anything was dropped.  Rounding that result to a format with at
// least two fewer significant bits (bf16 keeps 8 of float32's 24) gives the
// same value as rounding the float64 directly, so the float32 -> bf16
// convert of the store is the only rounding that counts.
__device__ __forceinline__ float f64_to_f32_odd(double x) {
  const float f = (float)x;
  uint32_t b = __float_as_uint(f);
  const double back = (double)f;
  const bool inexact = back != x;
  b -= (inexact && fabs(back) > fabs(x)) ? 1u : 0u;   // rounded away: step back
  b |= inexact ? 1u : 0u;
  return __uint_as_float(b);
}

// the mean sum / p^l of a level-l entry, as the float32 that the store
// rounds to T: float32 I/O rounds the float64 mean to nearest once; bf16 I/O
// rounds it to odd here and to nearest-even in the store.  The mean is a
// multiply by the exact reciprocal when p is a power of two, else a
// correctly rounded division.
template <typename T>
__device__ __forceinline__ float level_mean(const PyrArgs &a, double sum, int l) {
  const double m = a.pow2 ? sum * a.rp[l] : sum / a.pwd[l];
  if constexpr (sizeof(T) == 2) {
    return f64_to_f32_odd(m);
  } else {
    return (float)m;
  }
}

// a float64 moved across lanes by one DPP pattern (both halves)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}

// sum over the CPR (8 or 16) lanes of a row group, left in every lane of the
// group: swap neighbours, swap pairs, mirror halves of 8 (and halves of 16);
// each step adds two equal-sized partial sums, so all lanes end bit-equal
template <int CPR>
__device__ __forceinline__ double rowsum_f64(double v) {
  v += dpp_f64<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);   // row_half_mirror
  if constexpr (CPR == 16) v += dpp_f64<0x140>(v);   // row_mirror
  return v;
}

// lane u (or 8 + u) of each row group of CPR lanes, broadcast to the group
template <int CPR>
__device__ __forceinline__ float group_bcast(float v, int u) {
  const int x = __float_as_int(v);
  int r;
  switch (u) {
#define LH_BC(U)                                                                        \
  case U:                                                                               \
    if constexpr (CPR == 16) {                                                          \
      r = __builtin_amdgcn_update_dpp(0, x, 0x150 + U, 0xf, 0xf, false);                \
    } else {                                                                            \
      r = __builtin_amdgcn_update_dpp(0, x, 0x150 + U, 0xf, 0x3, false);                \
      r = __builtin_amdgcn_update_dpp(r, x, 0x158 + U, 0xf, 0xc, false);                \
    }                                                                                   \
    break;
    LH_BC(0) LH_BC(1) LH_BC(2) LH_BC(3) LH_BC(4) LH_BC(5) LH_BC(6) LH_BC(7)
#undef LH_BC
    default: r = x;
  }
  return __int_as_float(r);
}

// U token rows of 8 columns held in their I/O encoding until used: bf16
// rows stay packed (4 registers a row instead of 8), float rows as they are
template <typename T, int U> struct RowBuf;
template <int U> struct RowBuf<bf16_t, U> {
  uint32_t w[U][4];
  __device__ __forceinline__ void load(int u, const bf16_t *p) {
    const uint4 a = *reinterpret_cast<const uint4 *>(p);
    w[u][0] = a.x; w[u][1] = a.y; w[u][2] = a.z; w[u][3] = a.w;
  }
  __device__ __forceinline__ void zero(int u) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[u][i] = 0u;
  }
  __device__ __forceinline__ float get(int u, int i) const {
    const uint32_t v = w[u][i >> 1];
    return __uint_as_float((i & 1) ? (v & 0xffff0000u) : (v << 16));
  }
};
template <int U> struct RowBuf<float, U> {
  float x[U][8];
  __device__ __forceinline__ void load(int u, const float *p) { load8(p, x[u]); }
  __device__ __forceinline__ void zero(int u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[u][i] = 0.f;
  }
  __device__ __forceinline__ float get(int u, int i) const { return x[u][i]; }
};

template <typename T, int CPR, int G>
__global__ __launch_bounds__(kPyrThreads) void pyr_score_kernel(PyrArgs a) {
  extern __shared__ double lds[];                // [spw*R][d] sums, then [spw*R] maxima
  constexpr int U = 8;                           // token rows in flight per thread
  const int z = blockIdx.z + a.zbase;
  const T *X = (const T *)a.in[z];
  if (!X) return;
  const int64_t bh = blockIdx.y;
  const int d = a.d;
  X += bh * a.N * d;
  T *P = a.pyr[z] ? (T *)a.pyr[z] + bh * (a.E - a.N) * d : nullptr;
  float *Sc = a.score[z] ? a.score[z] + bh * a.E : nullptr;
  const bool do_pyr = P != nullptr, do_sc = Sc != nullptr;

  const int tid = threadIdx.x;
  const int c = tid % CPR;                 // column slice
  const int rs = tid / CPR;                // row slot in workgroup
  const int sub = rs / a.R, r = rs % a.R;  // stratum within workgroup, subtree
  const int64_t m = (int64_t)blockIdx.x * a.spw + sub;
  const int Gt = (int)a.pw[G];             // tokens of the subtree
  const int64_t base = m * a.Bc + (int64_t)r * Gt;
  const int rows = a.spw * a.R;
  double *lsum = lds;                                  // [rows][d]
  float *lmax = reinterpret_cast<float *>(lds + (size_t)rows * d);   // [rows]

  // running sums / maxima of the levels 1..G entries being completed, the
  // children each has taken so far, and the index (within its level) of the
  // entry it will complete next
  double acc[G + 1][8];
  float smx[G + 1];
  int cnt[G + 1];
  int64_t idx[G + 1];
#pragma unroll
  for (int l = 0; l <= G; ++l) {
    smx[l] = 0.f;
    cnt[l] = 0;
    idx[l] = m * a.per[l] + (int64_t)r * a.pw[G - l];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[l][i] = 0.0;
  }

  for (int t0 = 0; t0 < Gt; t0 += U) {
    RowBuf<T, U> x;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t0 + u < Gt) {
        x.load(u, X + (base + t0 + u) * d + c * 8);
      } else {
        x.zero(u);
      }
    }
    // l2 norms of the U rows: float64 sums of squares over the row group;
    // lane c takes the square root of row c % U only, then every lane
    // receives all U norms
    float s_all[U];
    if (do_sc) {
      const int own = c & (U - 1);
      double mine = 0.0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        double t = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double v = (double)x.get(u, i);
          t += v * v;
        }
        t = rowsum_f64<CPR>(t);
        mine = own == u ? t : mine;
      }
      const float s_own = (float)sqrt(mine);
      if (c < U && t0 + c < Gt) Sc[base + t0 + c] = s_own;
#pragma unroll
      for (int u = 0; u < U; ++u) s_all[u] = group_bcast<CPR>(s_own, u);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) s_all[u] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t0 + u >= Gt) break;
      const float s = s_all[u];
      if constexpr (G == 0) {
        // the subtree is a single token: it goes straight to LDS
#pragma unroll
        for (int i = 0; i < 8; ++i) lsum[(size_t)rs * d + c * 8 + i] = x.get(u, i);
        if (c == 0) lmax[rs] = s;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[1][i] += (double)x.get(u, i);
        smx[1] = fmaxf(smx[1], s);
#pragma unroll
        for (int l = 1; l <= G; ++l) {
          if (++cnt[l] < a.p) break;
          cnt[l] = 0;
          if (do_pyr) {
            float mean[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) mean[i] = level_mean<T>(a, acc[l][i], l);
            store8(P + (a.loff[l] - a.N + idx[l]) * d + c * 8, mean);
          }
          if (do_sc && c == 0) Sc[a.loff[l] + idx[l]] = smx[l];
          ++idx[l];
          if (l == G) {
#pragma unroll
            for (int i = 0; i < 8; ++i) lsum[(size_t)rs * d + c * 8 + i] = acc[l][i];
            if (c == 0) lmax[rs] = smx[l];
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[l + 1][i] += acc[l][i];
            smx[l + 1] = fmaxf(smx[l + 1], smx[l]);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[l][i] = 0.0;
          smx[l] = 0.f;
        }
      }
    }
  }
  __syncthreads();

  // levels G+1 .. L-1 of each stratum from the LDS sums (compacted in place:
  // entry e of the current level lives in row sub*R + e)
  int n = a.R;
  for (int l = G + 1; l < a.L; ++l) {
    n /= a.p;
    const bool act = rs < a.spw * n;
    const int s2 = act ? rs / n : 0, e = act ? rs % n : 0;
    double sum[8];
    float mx = 0.f;
    if (act) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sum[i] = 0.0;
      for (int k = 0; k < a.p; ++k) {
        const int row = s2 * a.R + e * a.p + k;
#pragma unroll
        for (int i = 0; i < 8; ++i) sum[i] += lsum[(size_t)row * d + c * 8 + i];
        mx = fmaxf(mx, lmax[row]);
      }
    }
    __syncthreads();
    if (act) {
      const int row = s2 * a.R + e;
#pragma unroll
      for (int i = 0; i < 8; ++i) lsum[(size_t)row * d + c * 8 + i] = sum[i];
      if (c == 0) lmax[row] = mx;
      const int64_t mm = (int64_t)blockIdx.x * a.spw + s2;
      const int64_t idx = mm * n + e;
      if (do_pyr) {
        float mean[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) mean[i] = level_mean<T>(a, sum[i], l);
        store8(P + (a.loff[l] - a.N + idx) * d + c * 8, mean);
      }
      if (do_sc && c == 0) Sc[a.loff[l] + idx] = mx;
    }
    __syncthreads();
  }
}

// chain depth g, subtrees per stratum R, strata per workgroup spw
static bool pyr_plan(const Geo &g, int *gd, int *R, int *spw) {
  const int cpr = g.d / 8;
  for (int gg = 0; gg <= kPyrMaxG && gg < g.L; ++gg) {
    const int64_t r = g.Bc / g.pw[gg];
    if (r * cpr <= kPyrThreads) {
      int s = (int)(kPyrThreads / (r * cpr));
      while (s > 1 && g.n_c % s) --s;
      *gd = gg;
      *R = (int)r;
      *spw = s;
      return true;
    }
  }
  return false;
}

lh_status check_pyramid_supported(const Geo &g) {
  int a, b, c;
  return pyr_plan(g, &a, &b, &c) ? LH_OK : LH_ERR_UNSUPPORTED;
}

lh_status launch_pyramid_score(const Geo &g, const void *q, const void *k, const void *v,
                               void *pq, void *pk, void *pv, float *sq, float *sk,
                               hipStream_t st) {
  PyrArgs a;
  a.in[0] = q; a.in[1] = k; a.in[2] = v;
  a.pyr[0] = pq; a.pyr[1] = pk; a.pyr[2] = pv;
  if (g.L == 1) a.pyr[0] = a.pyr[1] = a.pyr[2] = nullptr;   // no coarse levels
  a.score[0] = sq; a.score[1] = sk; a.score[2] = nullptr;
  // a tensor with neither pyramid nor score output is skipped
  for (int z = 0; z < 3; ++z)
    if (!a.pyr[z] && !a.score[z]) a.in[z] = nullptr;
  a.N = g.N; a.E = g.E; a.Bc = g.Bc; a.d = g.d; a.p = g.p; a.L = g.L;
  for (int l = 0; l < kMaxLevels; ++l) { a.lsize[l] = g.lsize[l]; a.loff[l] = g.loff[l]; }
  for (int l = 0; l <= kMaxLevels; ++l) a.pw[l] = g.pw[l];
  for (int l = 0; l < kMaxLevels; ++l) {
    a.per[l] = l < g.L ? g.Bc / g.pw[l] : 0;
    a.rp[l] = l < g.L ? 1.0 / (double)g.pw[l] : 0.0;
    a.pwd[l] = l < g.L ? (double)g.pw[l] : 1.0;
  }
  a.pow2 = (g.p & (g.p - 1)) == 0;
  if (!pyr_plan(g, &a.g, &a.R, &a.spw)) return LH_ERR_UNSUPPORTED;
  int nz = 0;
  for (int z = 0; z < 3; ++z) nz = a.in[z] ? z + 1 : nz;
  if (nz == 0) return LH_OK;
  a.zbase = 0;
  while (!a.in[a.zbase]) ++a.zbase;
  nz -= a.zbase;
  const int cpr = g.d / 8;
  dim3 grid((unsigned)(g.n_c / a.spw), (unsigned)g.BH(), (unsigned)nz);
  dim3 block((unsigned)(a.spw * a.R * cpr));
  const size_t shm = (size_t)a.spw * a.R * ((size_t)g.d * sizeof(double) + sizeof(float));
#define LH_PYR_G(T, C, GG) \
  case GG: hipLaunchKernelGGL((pyr_score_kernel<T, C, GG>), grid, block, shm, st, a); break;
#define LH_PYR(T, C)                                                                          \
  switch (a.g) {                                                                              \
    LH_PYR_G(T, C, 0) LH_PYR_G(T, C, 1) LH_PYR_G(T, C, 2) LH_PYR_G(T, C, 3)                   \
    LH_PYR_G(T, C, 4) LH_PYR_G(T, C, 5) LH_PYR_G(T, C, 6)                                     \
    default: return LH_ERR_UNSUPPORTED;                                                       \
  }
  if (g.io == LH_BF16) {
    if (g.d == 128) { LH_PYR(bf16_t, 16) } else { LH_PYR(bf16_t, 8) }
  } else {
    if (g.d == 128) { LH_PYR(float, 16) } else { LH_PYR(float, 8) }
  }
#undef LH_PYR
#undef LH_PYR_G
  return hip_status();
}

}  // namespace lh
