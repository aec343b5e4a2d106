// Stage 2b: stratified top-K with the coarsest level always kept, the
// subsequence order, redundancy and leader flags, and the row_of map.
//
// Method (gist.science explainer "Long Context Pre-Training with Lighthouse
// Attention", technical summary 2.B and 2.C; edge.aivizor.me news item,
// four-stages paragraph and the paragraph after it): entries are ranked
// jointly across levels; the top-K is stratified so it cannot collapse onto a
// narrow range, and the coarsest level is always kept so every position is
// covered; the selection is ordered topologically and causally.
//
// Readings (stated in the design notes): a stratum is one coarsest cell with
// its subtree; its root is always kept and k_s = K/n_c further entries are
// taken by sigma descending, ties to the lower flat index (or, by
// strata_mode, a quota per level ranked within the level), with sigma =
// float32(sq + sk) (or, by sigma_mode, max(sq, sk) or float32(sq * sk));
// rows follow (anchor, level) ascending; an entry is REDUNDANT when all its
// children are selected or redundant; a LEADER is the first row at its anchor.
//
// One workgroup per (stratum, b*h).  Candidates are enumerated level by level
// (level 0 first, positions ascending), which is also ascending flat index.
//  1. sigma bit patterns -> LDS (sigma >= 0, so unsigned order = value order)
//  2. radix select (4 passes of 8 bits, LDS histograms) finds the k_s-th
//     largest sigma `thr` and how many entries equal to it are still needed;
//     the first `need` of those in candidate order are taken (exact ties go
//     to the lower flat index)
//  3. redundancy bottom-up over the levels
//  4. post-order position of every entry (children before parent, left to
//     right), which equals (anchor, level) order; an exclusive scan over the
//     post-order gives each selected entry its row
//  5. rows, anchors, flags and row_of (every entry of the subtree written).
#include "lh_internal.h"

namespace lh {

// threads per workgroup: 256, or 512 where the whole grid is resident in one
// round at that size (see launch_select); at least one thread per radix digit
constexpr int kSelThreads = 256, kSelThreadsWide = 512;
constexpr int kSelMaxT = 7936;     // LDS holds 8 bytes per subtree entry
constexpr int kSelLoads = 8;       // score loads a thread keeps in flight

struct SelArgs {
  const float *sq, *sk;
  int32_t *sel_idx, *sel_anchor, *row_of;
  uint8_t *sel_flags;
  int64_t N, E, S, Bc, k_s;
  int32_t p, L, T, sigma, strata;
  int64_t quota[kMaxLevels];        // per-level quotas (LH_STRATA_PER_LEVEL)
  int64_t lsize[kMaxLevels], loff[kMaxLevels], pw[kMaxLevels + 1];
  int32_t cstart[kMaxLevels + 1];   // first candidate index of each level
  int32_t tsub[kMaxLevels];         // subtree size of a level-l entry
  int32_t lgp;                      // log2(p) when p is a power of two, else -1
};

// block-wide exclusive scan of one int per thread; returns the total too
template <int NT>
__device__ int block_excl_scan(int v, int *total, int *wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int i = 0; i < NT / 64; ++i) {
    if (i < w) pre += wsum[i];
    tot += wsum[i];
  }
  __syncthreads();
  *total = tot;
  return pre + x - v;
}

__device__ __forceinline__ int level_of_cand(const SelArgs &a, int ci) {
  int l = 0;
  while (l + 1 < a.L && ci >= a.cstart[l + 1]) ++l;
  return l;
}

// flat index of entry j of level l in stratum m (a level-l stratum holds
// cstart[l+1] - cstart[l] entries)
__device__ __forceinline__ int64_t entry_of(const SelArgs &a, int64_t m, int l, int j) {
  return a.loff[l] + m * (int64_t)(a.cstart[l + 1] - a.cstart[l]) + j;
}

template <int NT>
__global__ __launch_bounds__(NT) void select_kernel(SelArgs a) {
  static_assert(NT >= 256 && NT % 64 == 0, "one thread per radix digit");
  extern __shared__ uint32_t sm[];
  const int T = a.T;
  uint32_t *key = sm;                                    // [T]   sigma bits / row anchors
  uint16_t *post2c = (uint16_t *)(key + T);              // [T]
  uint8_t *st = (uint8_t *)(post2c + T);                 // [T]   bit0 selected, bit1 redundant
  uint8_t *rowred = st + T;                              // [T]   redundant bit of each row
  __shared__ int wsum[NT / 64];
  __shared__ int sh_digit, sh_need;
  __shared__ int hist[256];

  const int64_t m = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  const float *sq = a.sq + bh * a.E, *sk = a.sk + bh * a.E;
  const int ncand = T - 1;
  const int64_t k_s = a.k_s;

  // 1. keys and post-order map.  A thread's score loads are all issued
  // before any is used (one memory round trip per kSelLoads candidates),
  // and index math stays in 32 bits (j < entries per stratum).
  for (int c0 = 0; c0 < T; c0 += NT * kSelLoads) {
    float s1[kSelLoads], s2[kSelLoads];
#pragma unroll
    for (int u = 0; u < kSelLoads; ++u) {
      const int ci = c0 + u * NT + tid;
      s1[u] = s2[u] = 0.f;
      if (ci < T) {
        const int l = level_of_cand(a, ci);
        const int64_t f = entry_of(a, m, l, ci - a.cstart[l]);
        s1[u] = sq[f];
        s2[u] = sk[f];
      }
    }
#pragma unroll
    for (int u = 0; u < kSelLoads; ++u) {
      const int ci = c0 + u * NT + tid;
      if (ci >= T) break;
      const int l = level_of_cand(a, ci);
      const float sg = a.sigma == LH_SIGMA_SUM   ? __fadd_rn(s1[u], s2[u])
                       : a.sigma == LH_SIGMA_MAX ? fmaxf(s1[u], s2[u])
                                                 : __fmul_rn(s1[u], s2[u]);
      key[ci] = __float_as_uint(sg);
      st[ci] = 0;
      // post-order position: the subtree of each ancestor's earlier
      // siblings precedes this entry
      int post = a.tsub[l] - 1;
      int jj = ci - a.cstart[l];
      for (int lam = l; lam <= a.L - 2; ++lam) {
        int q, r;
        if (a.lgp >= 0) {
          q = jj >> a.lgp;
          r = jj - (q << a.lgp);
        } else {
          q = jj / a.p;
          r = jj - q * a.p;
        }
        post += r * a.tsub[lam];
        jj = q;
      }
      post2c[post] = (uint16_t)ci;
    }
  }
  __syncthreads();

  // 2. selection among candidates 0..T-2 (the root T-1 is always kept):
  // the k largest keys of candidates [c0, c1), exact ties to the lower
  // candidate index; one range of k_s (joint ranking) or one per level
  auto select_range = [&](int c0r, int c1r, int k) {
    const int nr = c1r - c0r;
    if (k >= nr) {
      for (int ci = c0r + tid; ci < c1r; ci += NT) st[ci] = 1;
      return;
    }
    if (k <= 0) return;
    uint32_t prefix = 0, pmask = 0;
    int remaining = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int ci = c0r + tid; ci < c1r; ci += NT) {
        const uint32_t kk = key[ci];
        if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 255], 1);
      }
      __syncthreads();
      // descending digit order: thread t < 256 looks at digit 255 - t
      const int cnt = tid < 256 ? hist[255 - tid] : 0;
      int tot;
      const int before = block_excl_scan<NT>(cnt, &tot, wsum);   // keys with larger digits
      if (before < remaining && before + cnt >= remaining) {
        sh_digit = 255 - tid;
        sh_need = remaining - before;
      }
      __syncthreads();
      prefix |= (uint32_t)sh_digit << shift;
      pmask |= 255u << shift;
      remaining = sh_need;
      __syncthreads();
    }
    const uint32_t thr = prefix;
    const int need = remaining;
    // first `need` candidates (in candidate order) with key == thr
    const int chunk = (nr + NT - 1) / NT;
    const int q0 = c0r + tid * chunk, q1 = min(c1r, q0 + chunk);
    int eq = 0;
    for (int ci = q0; ci < q1; ++ci) eq += key[ci] == thr;
    int tot;
    int rank = block_excl_scan<NT>(eq, &tot, wsum);
    for (int ci = q0; ci < q1; ++ci) {
      const uint32_t kk = key[ci];
      bool s = kk > thr;
      if (kk == thr) s = rank++ < need;
      st[ci] = s ? 1 : 0;
    }
  };
  if (a.strata == LH_STRATA_PER_LEVEL) {
    for (int l = 0; l + 1 < a.L; ++l) select_range(a.cstart[l], a.cstart[l + 1], (int)a.quota[l]);
  } else {
    select_range(0, ncand, (int)k_s);
  }
  if (tid == 0) st[ncand] = 1;   // root
  __syncthreads();

  // 3. redundancy, bottom-up
  for (int l = 1; l < a.L; ++l) {
    const int n = a.cstart[l + 1] - a.cstart[l];
    for (int j = tid; j < n; j += NT) {
      bool red = true;
      const int ch = a.cstart[l - 1] + j * a.p;
      for (int k = 0; k < a.p; ++k) red = red && (st[ch + k] != 0);
      if (red) st[a.cstart[l] + j] |= 2;
    }
    __syncthreads();
  }

  // 4. rows in post-order
  const int chunk = (T + NT - 1) / NT;
  const int q0 = tid * chunk, q1 = min(T, q0 + chunk);
  int nsel = 0;
  for (int q = q0; q < q1; ++q) nsel += st[post2c[q]] & 1;
  int tot;
  int r = block_excl_scan<NT>(nsel, &tot, wsum);
  __syncthreads();                     // key[] is reused for row anchors below
  const int64_t row0 = m * (k_s + 1);
  int32_t *sel_idx = a.sel_idx + bh * a.S, *sel_anchor = a.sel_anchor + bh * a.S;
  int32_t *row_of = a.row_of + bh * a.E;
  for (int q = q0; q < q1; ++q) {
    const int ci = post2c[q];
    const int l = level_of_cand(a, ci);
    const int j = ci - a.cstart[l];
    const int64_t f = entry_of(a, m, l, j);
    if ((st[ci] & 1) && r <= k_s) {
      const int64_t anchor = m * a.Bc + (int64_t)(j + 1) * a.pw[l] - 1;
      sel_idx[row0 + r] = (int32_t)f;
      sel_anchor[row0 + r] = (int32_t)anchor;
      key[r] = (uint32_t)anchor;
      rowred[r] = (st[ci] >> 1) & 1;
      row_of[f] = (int32_t)(row0 + r);
      ++r;
    } else {
      row_of[f] = -1;
    }
  }
  __syncthreads();

  // 5. flags
  uint8_t *flags = a.sel_flags + bh * a.S;
  for (int rr = tid; rr <= k_s; rr += NT) {
    const bool lead = rr == 0 || key[rr] != key[rr - 1];
    flags[row0 + rr] = (uint8_t)((rowred[rr] ? LH_ROW_REDUNDANT : 0u) | (lead ? LH_ROW_LEADER : 0u));
  }
}

lh_status check_select_supported(const Geo &g) {
  return g.T <= kSelMaxT ? LH_OK : LH_ERR_UNSUPPORTED;
}

lh_status launch_select(const Geo &g, const float *sq, const float *sk, int32_t *sel_idx,
                        int32_t *sel_anchor, uint8_t *sel_flags, int32_t *row_of,
                        hipStream_t st) {
  if (g.T > kSelMaxT) return LH_ERR_UNSUPPORTED;
  SelArgs a;
  a.sq = sq; a.sk = sk; a.sel_idx = sel_idx; a.sel_anchor = sel_anchor; a.row_of = row_of;
  a.sel_flags = sel_flags;
  a.N = g.N; a.E = g.E; a.S = g.S; a.Bc = g.Bc; a.k_s = g.k_s;
  a.p = g.p; a.L = g.L; a.T = (int32_t)g.T; a.sigma = g.sigma; a.strata = g.strata;
  for (int l = 0; l < kMaxLevels; ++l) a.quota[l] = g.quota[l];
  for (int l = 0; l < kMaxLevels; ++l) { a.lsize[l] = g.lsize[l]; a.loff[l] = g.loff[l]; }
  for (int l = 0; l <= kMaxLevels; ++l) a.pw[l] = g.pw[l];
  int cs = 0;
  for (int l = 0; l < g.L; ++l) {
    a.cstart[l] = cs;
    cs += (int)(g.Bc / g.pw[l]);
    a.tsub[l] = (int32_t)((g.pw[l + 1] - 1) / (g.p - 1));
  }
  a.cstart[g.L] = cs;
  a.lgp = -1;
  for (int k = 0; k < 31; ++k)
    if ((1 << k) == g.p) a.lgp = k;
  const size_t shm = (size_t)g.T * 8;
  dim3 grid((unsigned)g.n_c, (unsigned)g.BH());
  // 512 threads where every workgroup of the grid is resident at once on the
  // 256 compute units (four per unit: 8 wavefronts each, and four times the
  // LDS fits) and the subtrees are large enough to keep them busy; measured
  // on MI355X: 91 -> 65 us at the 1M-token workload, 30.3 -> 28.8 us at
  // 128K, while grids of two rounds or more ran slower (19.7 -> 29 us,
  // 35 -> 42 us)
  const bool wide = (int64_t)g.n_c * g.BH() <= 1024 && g.T >= 1024 && shm * 4 <= 150 * 1024;
  if (wide)
    hipLaunchKernelGGL(select_kernel<kSelThreadsWide>, grid, dim3(kSelThreadsWide), shm, st, a);
  else
    hipLaunchKernelGGL(select_kernel<kSelThreads>, grid, dim3(kSelThreads), shm, st, a);
  return hip_status();
}

}  // namespace lh
