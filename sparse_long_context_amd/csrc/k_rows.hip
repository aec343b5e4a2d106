// Row-movement stages: gather (3a), transposed copies for the MFMA operands,
// scatter-back (4) and its adjoint, the gather+pooling adjoint (unpool) and
// the prologue of the attention backward.  All are HBM-bound copies or
// segmented sums, with no atomics: every output element has one writer and
// every sum runs in a fixed order.
//
// Method (gist.science explainer "Long Context Pre-Training with Lighthouse
// Attention", technical summary 2.B and 2.C): the selected entries are
// gathered into one dense subsequence, attention outputs are put back at
// their positions by a deterministic scatter, and gradients reach Q, K, V
// through scatter, attention, gather and the pooling only.
//
// Scatter reading (design notes, causal hold): token t takes the output of
// the LEADER row with the largest anchor <= t; tokens before the first anchor
// take 0.  A leader's hold segment is [its anchor, next leader's anchor).
#include "lh_internal.h"

namespace lh {

// ---------------------------------------------------------------- gather
struct GatherArgs {
  const void *src[3], *psrc[3];
  void *dst[3];
  const int32_t *sel_idx;
  int64_t N, E, S;
  int32_t d;
};

template <typename T, int CPR>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int z = blockIdx.z;
  const int64_t bh = blockIdx.y;
  const int c = threadIdx.x % CPR;
  const int64_t j = (int64_t)blockIdx.x * (256 / CPR) + threadIdx.x / CPR;
  if (j >= a.S) return;
  const int d = a.d;
  const int64_t f = a.sel_idx[bh * a.S + j];
  T *o = (T *)a.dst[z] + (bh * a.S + j) * d;
  float x[8];
  if (f >= 0 && f < a.E) {
    const T *s = f < a.N ? (const T *)a.src[z] + (bh * a.N + f) * d
                         : (const T *)a.psrc[z] + (bh * (a.E - a.N) + f - a.N) * d;
    load8(s + c * 8, x);
  } else {   // not a flat index of this geometry: the row is left zero
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.f;
  }
  store8(o + c * 8, x);
}

lh_status launch_gather(const Geo &g, const void *const src[3], const void *const psrc[3],
                        const int32_t *sel_idx, void *const dst[3], hipStream_t st) {
  GatherArgs a;
  for (int i = 0; i < 3; ++i) { a.src[i] = src[i]; a.psrc[i] = psrc[i]; a.dst[i] = dst[i]; }
  a.sel_idx = sel_idx; a.N = g.N; a.E = g.E; a.S = g.S; a.d = g.d;
  const int cpr = g.d / 8;
  dim3 grid(cdiv(g.S, 256 / cpr), (unsigned)g.BH(), 3);
  if (g.io == LH_BF16) {
    if (g.d == 128) hipLaunchKernelGGL((gather_kernel<bf16_t, 16>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((gather_kernel<bf16_t, 8>), grid, dim3(256), 0, st, a);
  } else {
    if (g.d == 128) hipLaunchKernelGGL((gather_kernel<float, 16>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((gather_kernel<float, 8>), grid, dim3(256), 0, st, a);
  }
  return hip_status();
}

// ---------------------------------------------------------------- transpose
// [BH, S, d] bf16 rows -> [BH, d, Sp] bf16, 64x64 tiles through LDS; columns
// S..Sp-1 are written as zeros.
__global__ __launch_bounds__(256) void transpose_kernel(const bf16_t *in, bf16_t *out, int64_t S,
                                                        int64_t Sp, int32_t d) {
  __shared__ bf16_t tile[64][64 + 2];
  const int64_t bh = blockIdx.z;
  const int64_t j0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const bf16_t *src = in + bh * S * d;
  bf16_t *dst = out + bh * d * Sp;
  const int tid = threadIdx.x;
  // load: 64 rows x 64 cols, 8 elements per thread per pass, 2 passes
  for (int pass = 0; pass < 2; ++pass) {
    const int idx = pass * 256 + tid;
    const int rr = idx / 8, cc = (idx % 8) * 8;
    const int64_t j = j0 + rr;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < S) v = *reinterpret_cast<const uint4 *>(src + j * d + c0 + cc);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[rr][cc + 2 * i] = (bf16_t)(w[i] & 0xffff);
      tile[rr][cc + 2 * i + 1] = (bf16_t)(w[i] >> 16);
    }
  }
  __syncthreads();
  for (int pass = 0; pass < 2; ++pass) {
    const int idx = pass * 256 + tid;
    const int cr = idx / 8, jj = (idx % 8) * 8;   // output row (column of input), 8 j's
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)tile[jj + 2 * i][cr] | ((uint32_t)tile[jj + 2 * i + 1][cr] << 16);
    *reinterpret_cast<uint4 *>(dst + (int64_t)(c0 + cr) * Sp + j0 + jj) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

lh_status launch_transpose(const Geo &g, const void *rows, void *tr, hipStream_t st) {
  dim3 grid((unsigned)(g.Sp / 64), (unsigned)(g.d / 64), (unsigned)g.BH());
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, (const bf16_t *)rows,
                     (bf16_t *)tr, g.S, g.Sp, g.d);
  return hip_status();
}

// ---------------------------------------------------------------- scatter
// One workgroup per (token chunk of one stratum, b*h).  The stratum's rows are
// staged in LDS; each token finds its row by binary search on the anchors,
// then its leader (first row at that anchor).  Tokens before the stratum's
// first anchor take the last leader of the previous stratum.
constexpr int kScatChunk = 1024;

struct ScatArgs {
  const float *os;
  const int32_t *anchor;
  const uint8_t *flags;
  void *o;
  int64_t N, S, Bc, k_s;
  int32_t d, chunks;
};

template <typename T, int CPR>
__global__ __launch_bounds__(256) void scatter_kernel(ScatArgs a) {
  extern __shared__ int32_t sanc[];        // [k_s+1] anchors, then [k_s+1] leader rows
  __shared__ int32_t prev_leader;
  const int64_t bh = blockIdx.y;
  const int64_t m = blockIdx.x / a.chunks;
  const int64_t t_begin = m * a.Bc + (int64_t)(blockIdx.x % a.chunks) * kScatChunk;
  const int64_t t_end = min(m * a.Bc + a.Bc, t_begin + kScatChunk);
  const int nr = (int)(a.k_s + 1);
  const int64_t row0 = m * nr;
  const int32_t *anc = a.anchor + bh * a.S;
  int32_t *lead = sanc + nr;
  for (int r = threadIdx.x; r < nr; r += 256) sanc[r] = anc[row0 + r];
  if (threadIdx.x == 0) {
    int32_t pl = -1;
    if (m > 0) {
      // last leader of stratum m-1: first row holding that stratum's last anchor
      int64_t r = row0 - 1;
      const int32_t last = anc[r];
      while (r - 1 >= (m - 1) * nr && anc[r - 1] == last) --r;
      pl = (int32_t)r;
    }
    prev_leader = pl;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < nr; r += 256) {
    int rr = r;
    while (rr > 0 && sanc[rr - 1] == sanc[r]) --rr;
    lead[r] = (int32_t)(row0 + rr);
  }
  __syncthreads();
  const int c = threadIdx.x % CPR;
  const int d = a.d;
  const float *os = a.os + bh * a.S * d;
  T *o = (T *)a.o + bh * a.N * d;
  constexpr int TW = 256 / CPR;   // token lanes
  for (int64_t tb = t_begin + threadIdx.x / CPR; tb < t_end; tb += 4 * TW) {
    float x[4][8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t t = tb + k * TW;
      // last row with anchor <= t
      int lo = 0, hi = nr;          // answer in [lo-1, hi-1]
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sanc[mid] <= t) lo = mid + 1; else hi = mid;
      }
      const int32_t src = lo == 0 ? prev_leader : lead[lo - 1];
      if (t < t_end && src >= 0 && src < a.S) {
        load8(os + (int64_t)src * d + c * 8, x[k]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[k][i] = 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (tb + k * TW < t_end) store8(o + (tb + k * TW) * d + c * 8, x[k]);
  }
}

lh_status launch_scatter(const Geo &g, const float *os, const int32_t *sel_anchor,
                         const uint8_t *sel_flags, void *o, hipStream_t st) {
  ScatArgs a;
  a.os = os; a.anchor = sel_anchor; a.flags = sel_flags; a.o = o;
  a.N = g.N; a.S = g.S; a.Bc = g.Bc; a.k_s = g.k_s; a.d = g.d;
  a.chunks = (int)cdiv(g.Bc, kScatChunk);
  dim3 grid((unsigned)(g.n_c * a.chunks), (unsigned)g.BH());
  const size_t shm = (size_t)(g.k_s + 1) * 2 * sizeof(int32_t);
  if (g.out == LH_BF16) {
    if (g.d == 128) hipLaunchKernelGGL((scatter_kernel<bf16_t, 16>), grid, dim3(256), shm, st, a);
    else hipLaunchKernelGGL((scatter_kernel<bf16_t, 8>), grid, dim3(256), shm, st, a);
  } else {
    if (g.d == 128) hipLaunchKernelGGL((scatter_kernel<float, 16>), grid, dim3(256), shm, st, a);
    else hipLaunchKernelGGL((scatter_kernel<float, 8>), grid, dim3(256), shm, st, a);
  }
  return hip_status();
}

// ---------------------------------------------------------------- scatter adjoint
// One wavefront per subsequence row.  A leader sums dO over its hold segment:
// 64/CPR token lanes take every (64/CPR)-th token, then the lanes are folded
// in a fixed order.  Optionally writes the float32 sums, their two-term bf16
// split (the MFMA operands of the attention backward) and
// drow = <dOS_j, OS_j>.
struct ScatBwdArgs {
  const void *dout;
  const int32_t *anchor;
  const uint8_t *flags;
  float *dos;
  bf16_t *dos_hi, *dos_lo;
  const float *os;
  float *drow;
  int64_t N, S;
  int32_t d;
};

template <typename T, int CPR>
__global__ __launch_bounds__(256) void scatter_bwd_kernel(ScatBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t bh = blockIdx.y;
  if (j >= a.S) return;
  const int d = a.d;
  const int c = lane % CPR, u = lane / CPR;
  constexpr int TL = 64 / CPR;
  const int32_t *anc = a.anchor + bh * a.S;
  const bool leader = (a.flags[bh * a.S + j] & LH_ROW_LEADER) != 0;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (leader) {
    const int64_t t0 = max((int64_t)0, min((int64_t)anc[j], a.N));
    int64_t nx = j + 1;
    while (nx < a.S && anc[nx] == anc[j]) ++nx;
    const int64_t t1 = max(t0, min(nx < a.S ? (int64_t)anc[nx] : a.N, a.N));
    const T *dO = (const T *)a.dout + bh * a.N * d;
    // four rows in flight per lane; each lane still adds its tokens in order
    for (int64_t t = t0 + u; t < t1; t += 4 * TL) {
      float x[4][8];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (t + k * TL < t1) load8(dO + (t + k * TL) * d + c * 8, x[k]);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (t + k * TL < t1) {
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += x[k][i];
        }
    }
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], off);
  }
  const int64_t row = (bh * a.S + j) * d + c * 8;
  if (u == 0) {
    if (a.dos) store8(a.dos + row, acc);
    if (a.dos_hi) store8_split(a.dos_hi + row, a.dos_lo + row, acc);
  }
  if (a.drow) {
    float o[8];
    load8(a.os + row, o);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += acc[i] * o[i];
#pragma unroll
    for (int off = 1; off < CPR; off <<= 1) s += __shfl_xor(s, off);
    if (lane == 0) a.drow[bh * a.S + j] = s;
  }
}

lh_status launch_scatter_bwd(const Geo &g, const void *dout, const int32_t *sel_anchor,
                             const uint8_t *sel_flags, float *dos, bf16_t *dos_hi,
                             bf16_t *dos_lo, const float *os, float *drow, hipStream_t st) {
  ScatBwdArgs a;
  a.dout = dout; a.anchor = sel_anchor; a.flags = sel_flags; a.dos = dos;
  a.dos_hi = dos_lo ? dos_hi : nullptr; a.dos_lo = dos_lo;
  a.os = os; a.drow = os ? drow : nullptr; a.N = g.N; a.S = g.S; a.d = g.d;
  dim3 grid(cdiv(g.S, 4), (unsigned)g.BH());
  // dO and OS both have the output type
  if (g.out == LH_BF16) {
    if (g.d == 128) hipLaunchKernelGGL((scatter_bwd_kernel<bf16_t, 16>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((scatter_bwd_kernel<bf16_t, 8>), grid, dim3(256), 0, st, a);
  } else {
    if (g.d == 128) hipLaunchKernelGGL((scatter_bwd_kernel<float, 16>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((scatter_bwd_kernel<float, 8>), grid, dim3(256), 0, st, a);
  }
  return hip_status();
}

// ---------------------------------------------------------------- dOS prologue
// float32 dOS -> optional bf16 split (hi, lo) and drow = <dOS_j, OS_j>; one
// wavefront per row.
template <int CPR>
__global__ __launch_bounds__(256) void dos_prep_kernel(const float *dos, const float *os_,
                                                       bf16_t *hi, bf16_t *lo, float *drow,
                                                       int64_t rows, int32_t d) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= rows) return;
  float s = 0.f;
  if (lane < CPR) {
    float x[8], o[8];
    load8(dos + j * d + lane * 8, x);
    load8(os_ + j * d + lane * 8, o);
    if (hi) store8_split(hi + j * d + lane * 8, lo + j * d + lane * 8, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) s += x[i] * o[i];
  }
#pragma unroll
  for (int off = 1; off < CPR; off <<= 1) s += __shfl_xor(s, off);
  if (lane == 0) drow[j] = s;
}

lh_status launch_dos_prep(const Geo &g, const float *dos, const float *os, bf16_t *dos_hi,
                          bf16_t *dos_lo, float *drow, hipStream_t st) {
  const int64_t rows = g.BH() * g.S;
  dim3 grid(cdiv(rows, 4));
  if (!dos_lo) dos_hi = nullptr;
  if (g.d == 128)
    hipLaunchKernelGGL(dos_prep_kernel<16>, grid, dim3(256), 0, st, dos, os, dos_hi, dos_lo, drow, rows, g.d);
  else
    hipLaunchKernelGGL(dos_prep_kernel<8>, grid, dim3(256), 0, st, dos, os, dos_hi, dos_lo, drow, rows, g.d);
  return hip_status();
}

// ---------------------------------------------------------------- unpool
// dx[t] = sum_l dxs[row_of(l, t / p^l)] / p^l over the selected ancestors of
// t.  One workgroup covers `spw` whole strata of one (b, h) and one tensor:
// the strata's row_of entries (their subtrees) are staged in LDS, so lookups
// are LDS reads.  A thread walks level-1 entries (CPR lanes per row): the
// levels L-1..1 part, shared by the entry's p tokens, is summed once
// (coarsest first), then each token adds its own level-0 row when selected.
// The summation order is fixed, so results are reproducible.
constexpr int kUnpoolThreads = 256;
constexpr int kUnpoolLdsEntries = 8192;   // row_of entries staged per workgroup

struct UnpoolArgs {
  const float *dxs[3];
  void *dx[3];
  const int32_t *row_of;
  int64_t N, E, S, Bc;
  int32_t d, L, p, spw, lgp;    // lgp = log2(p) when p is a power of two, else -1
  int32_t T;                 // subtree entries per stratum
  int64_t loff[kMaxLevels], pw[kMaxLevels];
  int32_t cstart[kMaxLevels];   // first entry of level l inside a stratum's subtree
  float inv[kMaxLevels];
};

template <typename TO, int CPR>
__global__ __launch_bounds__(kUnpoolThreads) void unpool_kernel(UnpoolArgs a) {
  __shared__ int32_t ro[kUnpoolLdsEntries];
  const int z = blockIdx.z;
  const int64_t bh = blockIdx.y;
  const int64_t m0 = (int64_t)blockIdx.x * a.spw;   // first stratum of the workgroup
  const int tid = threadIdx.x;
  const int32_t *rog = a.row_of + bh * a.E;
  // stage row_of of the spw subtrees: entry (s, l, j) at s*T + cstart[l] + j
  for (int i = tid; i < a.spw * a.T; i += kUnpoolThreads) {
    const int sidx = i / a.T, e = i % a.T;
    int l = 0;
    while (l + 1 < a.L && e >= a.cstart[l + 1]) ++l;
    const int64_t per = a.Bc / a.pw[l];
    const int32_t r = rog[a.loff[l] + (m0 + sidx) * per + (e - a.cstart[l])];
    ro[i] = (r >= 0 && r < a.S) ? r : -1;
  }
  __syncthreads();
  const int c = tid % CPR;
  constexpr int LANES = kUnpoolThreads / CPR;   // lanes along the tokens
  const int d = a.d;
  const float *dxs = a.dxs[z] + bh * a.S * d;
  TO *out = (TO *)a.dx[z] + bh * a.N * d;
  const int64_t t0 = m0 * a.Bc;
  const int ntok = a.spw * (int)a.Bc;
  // work unit: one level-1 entry (p tokens; a single token when L == 1),
  // whose tokens share every ancestor above level 0
  const int P1 = a.L >= 2 ? a.p : 1;
  const int nent = ntok / P1;
  const int per = (nent + LANES - 1) / LANES;
  const int e_begin = (tid / CPR) * per, e_end = min(nent, e_begin + per);
  for (int e = e_begin; e < e_end; ++e) {
    const int u0 = e * P1;
    const int sidx = u0 / (int)a.Bc, ul = u0 - sidx * (int)a.Bc;
    const int base = sidx * a.T;
    // coarse part: levels L-1 .. 1, coarsest first
    float A[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) A[i] = 0.f;
    for (int l = a.L - 1; l >= 1; --l) {
      const int j = a.lgp >= 0 ? (ul >> (a.lgp * l)) : (int)(ul / a.pw[l]);
      const int32_t r = ro[base + a.cstart[l] + j];
      if (r >= 0) {
        float x[8];
        load8(dxs + (int64_t)r * d + c * 8, x);
        const float w = a.inv[l];
#pragma unroll
        for (int i = 0; i < 8; ++i) A[i] += x[i] * w;
      }
    }
    // the entry's tokens: A plus their own level-0 row when selected
    for (int k0 = 0; k0 < P1; k0 += 4) {
      float x[4][8];
      int32_t r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        r[k] = k0 + k < P1 ? ro[base + ul + k0 + k] : -1;   // level 0 starts at entry 0
        if (r[k] >= 0) load8(dxs + (int64_t)r[k] * d + c * 8, x[k]);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k0 + k >= P1) break;
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = r[k] >= 0 ? A[i] + x[k][i] : A[i];
        store8(out + (t0 + u0 + k0 + k) * d + c * 8, o);
      }
    }
  }
}

static int unpool_spw(const Geo &g) {
  int spw = (int)(1024 / g.Bc);
  if (spw < 1) spw = 1;
  while (spw > 1 && (spw * g.T > kUnpoolLdsEntries || g.n_c % spw)) --spw;
  return spw;
}

lh_status launch_unpool(const Geo &g, const float *const dxs[3], const int32_t *row_of,
                        void *const dx[3], hipStream_t st) {
  if (g.T > kUnpoolLdsEntries) return LH_ERR_UNSUPPORTED;
  UnpoolArgs a;
  for (int i = 0; i < 3; ++i) { a.dxs[i] = dxs[i]; a.dx[i] = dx[i]; }
  a.row_of = row_of; a.N = g.N; a.E = g.E; a.S = g.S; a.Bc = g.Bc; a.d = g.d; a.L = g.L;
  a.p = g.p; a.T = (int32_t)g.T;
  a.spw = unpool_spw(g);
  a.lgp = -1;
  for (int k = 0; k < 31; ++k)
    if ((1 << k) == g.p) a.lgp = k;
  int cs = 0;
  for (int l = 0; l < kMaxLevels; ++l) {
    a.loff[l] = g.loff[l];
    a.pw[l] = g.pw[l];
    a.inv[l] = (float)(1.0 / (double)g.pw[l]);
    a.cstart[l] = cs;
    if (l < g.L) cs += (int)(g.Bc / g.pw[l]);
  }
  dim3 grid((unsigned)(g.n_c / a.spw), (unsigned)g.BH(), 3);
  if (g.out == LH_BF16) {
    if (g.d == 128) hipLaunchKernelGGL((unpool_kernel<bf16_t, 16>), grid, dim3(kUnpoolThreads), 0, st, a);
    else hipLaunchKernelGGL((unpool_kernel<bf16_t, 8>), grid, dim3(kUnpoolThreads), 0, st, a);
  } else {
    if (g.d == 128) hipLaunchKernelGGL((unpool_kernel<float, 16>), grid, dim3(kUnpoolThreads), 0, st, a);
    else hipLaunchKernelGGL((unpool_kernel<float, 8>), grid, dim3(kUnpoolThreads), 0, st, a);
  }
  return hip_status();
}

}  // namespace lh
