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
#include "lh_unpool.h"

namespace lh {

// ---------------------------------------------------------------- gather
struct GatherArgs {
  const void *src[3], *psrc[3];
  void *dst[3];
  const int32_t *sel_idx;
  int64_t N, E, S;
  int32_t d;
  int32_t z0;   // first tensor of blockIdx.z = 0
};

template <typename T, int CPR>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int z = a.z0 + blockIdx.z;
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
                        const int32_t *sel_idx, void *const dst[3], hipStream_t st, int z0,
                        int nz) {
  if (z0 < 0 || nz < 1 || z0 + nz > 3) return LH_ERR_INVALID_ARG;
  GatherArgs a;
  for (int i = 0; i < 3; ++i) { a.src[i] = src[i]; a.psrc[i] = psrc[i]; a.dst[i] = dst[i]; }
  a.sel_idx = sel_idx; a.N = g.N; a.E = g.E; a.S = g.S; a.d = g.d; a.z0 = z0;
  const int cpr = g.d / 8;
  dim3 grid(cdiv(g.S, 256 / cpr), (unsigned)g.BH(), (unsigned)nz);
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
// One workgroup per (chunk of kScatChunk tokens of one stratum, b*h).  The
// stratum's anchors are staged in LDS; each thread resolves one token's hold
// source (the leader of the last row with anchor <= t, found by binary
// search; tokens before the stratum's first anchor take the last leader of
// the previous stratum) into an LDS map, then the workgroup streams the
// source rows out, CPR lanes per row, NF rows in flight per lane.
constexpr int kScatChunk = 256;
constexpr size_t kMaxLdsRows = 160 * 1024;   // LDS of one CU

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
  __shared__ int32_t srcmap[kScatChunk];
  const int64_t bh = blockIdx.y;
  const int64_t m = blockIdx.x / a.chunks;
  const int64_t t_begin = m * a.Bc + (int64_t)(blockIdx.x % a.chunks) * kScatChunk;
  const int ntok = (int)min((int64_t)kScatChunk, m * a.Bc + a.Bc - t_begin);
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
  for (int i = threadIdx.x; i < ntok; i += 256) {
    const int64_t t = t_begin + i;
    int lo = 0, hi = nr;          // last row with anchor <= t is lo - 1
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sanc[mid] <= t) lo = mid + 1; else hi = mid;
    }
    const int32_t src = lo == 0 ? prev_leader : lead[lo - 1];
    srcmap[i] = (src >= 0 && src < a.S) ? src : -1;
  }
  __syncthreads();
  const int c = threadIdx.x % CPR;
  const int d = a.d;
  const float *os = a.os + bh * a.S * d + c * 8;
  T *o = (T *)a.o + (bh * a.N + t_begin) * d + c * 8;
  constexpr int TW = 256 / CPR;   // token lanes
  constexpr int NF = 8;
  for (int tb = threadIdx.x / CPR; tb < ntok; tb += NF * TW) {
    float x[NF][8];
#pragma unroll
    for (int k = 0; k < NF; ++k) {
      const int i = tb + k * TW;
      const int32_t src = i < ntok ? srcmap[i] : -1;
      if (src >= 0) {
        load8(os + (int64_t)src * d, x[k]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[k][e] = 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < NF; ++k)
      if (tb + k * TW < ntok) store8_nt(o + (int64_t)(tb + k * TW) * d, x[k]);
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
// 8 consecutive elements held as loaded (bf16 stays packed: 4 registers)
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  uint4 w;
  __device__ void load(const bf16_t *p) { w = *reinterpret_cast<const uint4 *>(p); }
  __device__ void add_to(float *acc) const {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(v[i] << 16);
      acc[2 * i + 1] += __uint_as_float(v[i] & 0xffff0000u);
    }
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ void load(const float *p) {
    a = *reinterpret_cast<const float4 *>(p);
    b = *reinterpret_cast<const float4 *>(p + 4);
  }
  __device__ void add_to(float *acc) const {
    acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
    acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
  }
};

struct ScatBwdArgs {
  const void *dout;
  const int32_t *anchor;
  const uint8_t *flags;
  float *dos;
  bf16_t *dos_hi, *dos_lo;
  const float *os;
  float *drow;
  float *dsum;   // float32 dOS rows kept for drow (dos itself, or scratch rows)
  int64_t N, S, n_c, k_s;
  int32_t d;
};

// One workgroup per (stratum m, b*h).  The segments of stratum m's leaders
// tile the tokens [T0, T1): T0 is the stratum's first anchor (its first row
// is always a leader) and T1 the next stratum's first anchor (N after the
// last stratum), since the last leader of a stratum holds up to there.  The
// range is cut into one contiguous chunk per group of CPR lanes (a group
// reads one token row per instruction, NF rows in flight per lane) and each
// group sums its chunk in token order, segment by segment.  A segment that
// starts and ends inside one chunk is finished by its group; a piece at a
// chunk's start (segment begun in an earlier chunk) or end (continuing into
// the next) goes to LDS, and the group where a segment starts adds the later
// chunks' pieces in chunk order.  Every dO row is read once, the work is
// balanced however long the segments are, and the sums run in a fixed order.
// Tokens before the first anchor belong to no segment.  Rows that are not
// leaders get zeros.
constexpr int kScatBwdThreads = 256;

template <int CPR>
struct ScatBwdSmem {
  static constexpr int G = kScatBwdThreads / CPR;   // groups of CPR lanes
  float piece[2][G][CPR * 8];   // [0]: piece at a chunk's start, [1]: at its end
  int32_t tag[2][G];            // leader index of each piece, -1: none
  int32_t span[G];              // 1: the chunk lies inside one segment begun earlier
  int32_t nl;                   // leaders of the stratum
};

template <typename T, int CPR>
__global__ __launch_bounds__(kScatBwdThreads) void scatter_bwd_kernel(ScatBwdArgs a) {
  using Smem = ScatBwdSmem<CPR>;
  constexpr int G = Smem::G;
  extern __shared__ __align__(16) unsigned char sraw[];
  Smem &sm = *reinterpret_cast<Smem *>(sraw);
  const int nr = (int)(a.k_s + 1);
  int32_t *la = reinterpret_cast<int32_t *>(sraw + sizeof(Smem));   // leader anchors
  int32_t *lr = la + nr;                                             // leader rows
  int32_t *wtot = lr + nr;                          // [kScatBwdThreads / 64] wave counts
  uint8_t *lead = reinterpret_cast<uint8_t *>(wtot + kScatBwdThreads / 64);   // [nr]
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.x, bh = blockIdx.y;
  const int64_t row0 = m * nr;
  const int32_t *anc = a.anchor + bh * a.S;
  const uint8_t *flg = a.flags + bh * a.S;
  const int d = a.d;

  // leaders of the stratum in row order, rows taken one per thread: a
  // ballot per wavefront and the wavefronts' counts place them.  Each row's
  // flag and anchor are read once (their loads together) and the leader bit
  // is kept in LDS for the zero rows at the end.
  {
    const int lane = tid & 63, wv = tid >> 6;
    int nl_run = 0;   // leaders of the earlier batches (the same in every thread)
    for (int b0 = 0; b0 < nr; b0 += kScatBwdThreads) {
      const int r = b0 + tid;
      const bool in = r < nr;
      const uint8_t f = in ? flg[row0 + r] : (uint8_t)0;
      const int32_t an = in ? anc[row0 + r] : 0;
      const bool isl = (f & LH_ROW_LEADER) != 0;
      if (in) lead[r] = isl ? 1 : 0;
      const uint64_t bal = __ballot(isl);
      if (lane == 0) wtot[wv] = __popcll(bal);
      __syncthreads();
      int before = nl_run, tot = 0;
#pragma unroll
      for (int i = 0; i < kScatBwdThreads / 64; ++i) {
        before += i < wv ? wtot[i] : 0;
        tot += wtot[i];
      }
      if (isl) {
        const int pos = before + __popcll(bal & ((1ull << lane) - 1ull));
        la[pos] = an;
        lr[pos] = (int32_t)(row0 + r);
      }
      nl_run += tot;
      __syncthreads();   // wtot is rewritten by the next batch
    }
    if (tid == 0) sm.nl = nl_run;
  }
  if (tid < G) {
    sm.tag[0][tid] = sm.tag[1][tid] = -1;
    sm.span[tid] = 0;
  }
  __syncthreads();
  const int nl = sm.nl;
  const int64_t T0 = nl > 0 ? max((int64_t)0, min((int64_t)la[0], a.N)) : a.N;
  const int64_t T1 = m + 1 < a.n_c ? max(T0, min((int64_t)anc[row0 + nr], a.N)) : a.N;

  const int g = tid / CPR, c = tid % CPR;
  const T *dO = (const T *)a.dout + bh * a.N * d + c * 8;
  // final value of leader k: dOS (and its split); its float32 row is kept
  // for drow = <dOS, OS>, which the last phase forms for all leaders at once
  // (a load of OS here, waited for at once, would leave the wavefront with
  // no loads in flight at every segment's end)
  auto finish = [&](int k, const float *acc) {
    const int64_t row = (bh * a.S + lr[k]) * d + c * 8;
    if (a.dos) store8(a.dos + row, acc);
    if (a.dos_hi) store8_split(a.dos_hi + row, a.dos_lo + row, acc);
    if (a.drow && a.dsum != a.dos) store8(a.dsum + row, acc);
  };

  const int64_t n = nl > 0 ? T1 - T0 : 0;   // a valid selection has a leader per stratum
  const int64_t C = (n + G - 1) / G;
  const int64_t cb = T0 + g * C, ce = min(T1, cb + C);
  if (cb < ce) {
    // segment open at the chunk's start: the last leader with anchor <= cb
    int lo = 0, hi = nl;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)la[mid] <= cb) lo = mid + 1; else hi = mid;
    }
    int k = lo - 1;                                   // >= 0: la[0] = T0 <= cb
    int64_t nb = k + 1 < nl ? (int64_t)la[k + 1] : T1;   // end of segment k
    bool begun_here = (int64_t)la[k] == cb;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    auto close = [&]() {   // segment k ends at nb <= ce
      if (begun_here) {
        finish(k, acc);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) sm.piece[0][g][c * 8 + i] = acc[i];
        if (c == 0) sm.tag[0][g] = k;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
      ++k;
      nb = k + 1 < nl ? (int64_t)la[k + 1] : T1;
      begun_here = true;
    };
    constexpr int NF = 8;
    for (int64_t t0 = cb; t0 < ce; t0 += NF) {
      Raw8<T> x[NF];
#pragma unroll
      for (int j = 0; j < NF; ++j)
        if (t0 + j < ce) x[j].load(dO + (t0 + j) * d);
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int64_t t = t0 + j;
        if (t < ce) {
          while (t >= nb) close();
          x[j].add_to(acc);
        }
      }
    }
    if (nb <= ce) {
      close();   // the segment ends exactly at the chunk's end
    } else if (begun_here) {
      // begun in this chunk, continues: the piece at the chunk's end
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.piece[1][g][c * 8 + i] = acc[i];
      if (c == 0) sm.tag[1][g] = k;
    } else {
      // the whole chunk lies inside a segment begun earlier that goes on
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.piece[0][g][c * 8 + i] = acc[i];
      if (c == 0) {
        sm.tag[0][g] = k;
        sm.span[g] = 1;
      }
    }
  }
  __syncthreads();
  // segments that cross chunks: the group where one begins adds the pieces
  // of the following chunks in order, up to the chunk where it ends
  if (sm.tag[1][g] >= 0) {
    const int k = sm.tag[1][g];
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = sm.piece[1][g][c * 8 + i];
    for (int h = g + 1; h < G && sm.tag[0][h] == k; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += sm.piece[0][h][c * 8 + i];
      if (!sm.span[h]) break;
    }
    finish(k, acc);
  }
  // drow of every leader: its float32 dOS row (stored above by this
  // workgroup) and its OS row, up to 4 leaders per group in flight
  if (a.drow) {
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    constexpr int B = 4;
    for (int k0 = g; k0 < nl; k0 += B * G) {
      float xs[B][8], o[B][8];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int k = k0 + b * G;
        if (k < nl) {
          const int64_t row = (bh * a.S + lr[k]) * d + c * 8;
          load8(a.dsum + row, xs[b]);
          load8(a.os + row, o[b]);
        }
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int k = k0 + b * G;
        if (k < nl) {
          float s = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) s += xs[b][i] * o[b][i];
#pragma unroll
          for (int off = 1; off < CPR; off <<= 1) s += __shfl_xor(s, off);
          if (c == 0) a.drow[bh * a.S + lr[k]] = s;
        }
      }
    }
  }
  // rows that are not leaders: zeros
  const float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = g; r < nr; r += G) {
    if (lead[r]) continue;
    const int64_t row = (bh * a.S + row0 + r) * d + c * 8;
    if (a.dos) store8(a.dos + row, zero);
    if (a.dos_hi) {
      store8(a.dos_hi + row, zero);
      store8(a.dos_lo + row, zero);
    }
    if (a.drow && c == 0) a.drow[bh * a.S + row0 + r] = 0.f;
  }
}

static size_t scatter_bwd_lds(const Geo &g) {
  const size_t fixed = g.d == 128 ? sizeof(ScatBwdSmem<16>) : sizeof(ScatBwdSmem<8>);
  const size_t nr = (size_t)(g.k_s + 1);
  return fixed + (2 * nr + kScatBwdThreads / 64) * sizeof(int32_t) + nr;   // + leader bytes
}

lh_status launch_scatter_bwd(const Geo &g, const void *dout, const int32_t *sel_anchor,
                             const uint8_t *sel_flags, float *dos, bf16_t *dos_hi,
                             bf16_t *dos_lo, const float *os, float *drow, float *scratch,
                             hipStream_t st) {
  ScatBwdArgs a;
  a.dout = dout; a.anchor = sel_anchor; a.flags = sel_flags; a.dos = dos;
  a.dos_hi = dos_lo ? dos_hi : nullptr; a.dos_lo = dos_lo;
  a.os = os; a.drow = os ? drow : nullptr; a.N = g.N; a.S = g.S; a.n_c = g.n_c; a.k_s = g.k_s;
  a.dsum = dos ? dos : scratch;
  if (a.drow && !a.dsum) return LH_ERR_INVALID_ARG;
  a.d = g.d;
  const size_t shm = scatter_bwd_lds(g);
  if (shm > kMaxLdsRows) return LH_ERR_UNSUPPORTED;
  dim3 grid((unsigned)g.n_c, (unsigned)g.BH());
#define LH_SBWD(T, C)                                                                         \
  do {                                                                                        \
    (void)hipFuncSetAttribute((const void *)scatter_bwd_kernel<T, C>,                         \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);          \
    hipLaunchKernelGGL((scatter_bwd_kernel<T, C>), grid, dim3(kScatBwdThreads), shm, st, a);  \
  } while (0)
  // dO and OS both have the output type
  if (g.out == LH_BF16) {
    if (g.d == 128) LH_SBWD(bf16_t, 16); else LH_SBWD(bf16_t, 8);
  } else {
    if (g.d == 128) LH_SBWD(float, 16); else LH_SBWD(float, 8);
  }
#undef LH_SBWD
  return hip_status();
}

// ---------------------------------------------------------------- row copies
// Pads a [BH, rows_src, *] tensor with zero rows to rows_dst rows, or keeps
// its first rows_dst rows; 16 bytes per thread.
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint4 *src, uint4 *dst,
                                                        int64_t rows_src, int64_t rows_dst,
                                                        int64_t row_vec) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // vector within the head
  const int64_t bh = blockIdx.y;
  if (i >= rows_dst * row_vec) return;
  const int64_t r = i / row_vec;
  dst[bh * rows_dst * row_vec + i] =
      r < rows_src ? src[bh * rows_src * row_vec + i] : make_uint4(0u, 0u, 0u, 0u);
}

lh_status launch_copy_rows(const Geo &g, const void *src, void *dst, int64_t rows_src,
                           int64_t rows_dst, int64_t row_bytes, hipStream_t st) {
  const int64_t row_vec = row_bytes / 16;
  dim3 grid(cdiv(rows_dst * row_vec, 256), (unsigned)g.BH());
  hipLaunchKernelGGL(copy_rows_kernel, grid, dim3(256), 0, st, (const uint4 *)src, (uint4 *)dst,
                     rows_src, rows_dst, row_vec);
  return hip_status();
}

// ---------------------------------------------------------------- span broadcast
// The other reading of the scatter-back: every token takes the output of the
// finest selected entry whose span holds it (its owner); the stratum root is
// always selected, so every token has one, and redundant rows own nothing.
//
// owner_kernel: owner[t] = row_of(l, t / p^l) for the smallest l at which it
// is selected; one thread per token, levels walked finest first.
struct OwnerArgs {
  const int32_t *row_of;
  int32_t *owner;
  int64_t N, E, S;
  int32_t L, lgp;   // lgp = log2(p) when p is a power of two, else -1
  int64_t loff[kMaxLevels], pw[kMaxLevels];
};

__global__ __launch_bounds__(256) void owner_kernel(OwnerArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t bh = blockIdx.y;
  if (t >= a.N) return;
  const int32_t *ro = a.row_of + bh * a.E;
  int32_t own = -1;
  for (int l = 0; l < a.L && own < 0; ++l) {
    const int64_t i = a.lgp >= 0 ? (t >> (a.lgp * l)) : t / a.pw[l];
    const int32_t r = ro[a.loff[l] + i];
    if (r >= 0 && r < a.S) own = r;
  }
  a.owner[bh * a.N + t] = own;
}

lh_status launch_owner(const Geo &g, const int32_t *row_of, int32_t *owner, hipStream_t st) {
  OwnerArgs a;
  a.row_of = row_of; a.owner = owner; a.N = g.N; a.E = g.E; a.S = g.S; a.L = g.L;
  a.lgp = -1;
  for (int k = 0; k < 31; ++k)
    if ((1 << k) == g.p) a.lgp = k;
  for (int l = 0; l < kMaxLevels; ++l) {
    a.loff[l] = g.loff[l];
    a.pw[l] = l < g.L ? g.pw[l] : 1;
  }
  hipLaunchKernelGGL(owner_kernel, dim3(cdiv(g.N, 256), (unsigned)g.BH()), dim3(256), 0, st, a);
  return hip_status();
}

// scatter_span_kernel: O[t] = OS[owner[t]], CPR lanes per token row, eight
// rows in flight per lane.
template <typename T, int CPR>
__global__ __launch_bounds__(256) void scatter_span_kernel(const float *os, const int32_t *owner,
                                                           void *o_, int64_t N, int64_t S,
                                                           int32_t d) {
  constexpr int TW = 256 / CPR;   // token lanes
  constexpr int NF = 8;
  const int64_t bh = blockIdx.y;
  const int c = threadIdx.x % CPR;
  const int64_t t0 = (int64_t)blockIdx.x * (TW * NF) + threadIdx.x / CPR;
  const float *src = os + bh * S * d + c * 8;
  T *o = (T *)o_ + bh * N * d + c * 8;
  const int32_t *own = owner + bh * N;
  float x[NF][8];
#pragma unroll
  for (int k = 0; k < NF; ++k) {
    const int64_t t = t0 + k * TW;
    const int32_t r = t < N ? own[t] : -1;
    if (r >= 0 && r < S) {
      load8(src + (int64_t)r * d, x[k]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[k][e] = 0.f;
    }
  }
#pragma unroll
  for (int k = 0; k < NF; ++k)
    if (t0 + k * TW < N) store8_nt(o + (t0 + k * TW) * d, x[k]);
}

lh_status launch_scatter_span(const Geo &g, const float *os, const int32_t *owner, void *o,
                              hipStream_t st) {
  const int cpr = g.d / 8;
  dim3 grid(cdiv(g.N, (256 / cpr) * 8), (unsigned)g.BH());
  if (g.out == LH_BF16) {
    if (g.d == 128) hipLaunchKernelGGL((scatter_span_kernel<bf16_t, 16>), grid, dim3(256), 0, st, os, owner, o, g.N, g.S, g.d);
    else hipLaunchKernelGGL((scatter_span_kernel<bf16_t, 8>), grid, dim3(256), 0, st, os, owner, o, g.N, g.S, g.d);
  } else {
    if (g.d == 128) hipLaunchKernelGGL((scatter_span_kernel<float, 16>), grid, dim3(256), 0, st, os, owner, o, g.N, g.S, g.d);
    else hipLaunchKernelGGL((scatter_span_kernel<float, 8>), grid, dim3(256), 0, st, os, owner, o, g.N, g.S, g.d);
  }
  return hip_status();
}

// scatter_span_bwd_kernel: dOS[j] = sum of dO[t] over the tokens t of row j's
// span that it owns.  One wavefront per row; the span's tokens are taken by
// 64/CPR token lanes in increasing order, NF rows in flight per lane, and the
// lanes folded in a fixed order.  Writes the same outputs as the hold adjoint.
struct SpanBwdArgs {
  const void *dout;
  const int32_t *sel_idx, *owner;
  const uint8_t *flags;
  float *dos;
  bf16_t *dos_hi, *dos_lo;
  const float *os;
  float *drow;
  int64_t N, S, E;
  int32_t d, L;
  int64_t loff[kMaxLevels], pw[kMaxLevels];
};

template <typename T, int CPR>
__global__ __launch_bounds__(256) void scatter_span_bwd_kernel(SpanBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t bh = blockIdx.y;
  if (j >= a.S) return;
  const int d = a.d;
  const int c = lane % CPR, u = lane / CPR;
  constexpr int TL = 64 / CPR;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (!(a.flags[bh * a.S + j] & LH_ROW_REDUNDANT)) {
    const int64_t f = a.sel_idx[bh * a.S + j];
    int l = 0;
    while (l + 1 < a.L && f >= a.loff[l + 1]) ++l;
    const int64_t span = a.pw[l];
    const int64_t t0 = min(max((int64_t)0, (f - a.loff[l]) * span), a.N);
    const int64_t t1 = min(t0 + span, a.N);
    const T *dO = (const T *)a.dout + bh * a.N * d + c * 8;
    const int32_t *own = a.owner + bh * a.N;
    constexpr int NF = sizeof(T) == 2 ? 16 : 8;
    for (int64_t t = t0 + u; t < t1; t += NF * TL) {
      Raw8<T> x[NF];
      bool mine[NF];
#pragma unroll
      for (int k = 0; k < NF; ++k) {
        const int64_t tk = t + k * TL;
        mine[k] = tk < t1 && own[tk] == (int32_t)j;
        if (mine[k]) x[k].load(dO + tk * d);
      }
#pragma unroll
      for (int k = 0; k < NF; ++k)
        if (mine[k]) x[k].add_to(acc);
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

lh_status launch_scatter_span_bwd(const Geo &g, const void *dout, const int32_t *sel_idx,
                                  const uint8_t *sel_flags, const int32_t *owner, float *dos,
                                  bf16_t *dos_hi, bf16_t *dos_lo, const float *os, float *drow,
                                  hipStream_t st) {
  SpanBwdArgs a;
  a.dout = dout; a.sel_idx = sel_idx; a.owner = owner; a.flags = sel_flags; a.dos = dos;
  a.dos_hi = dos_lo ? dos_hi : nullptr; a.dos_lo = dos_lo;
  a.os = os; a.drow = os ? drow : nullptr; a.N = g.N; a.S = g.S; a.E = g.E; a.d = g.d;
  a.L = g.L;
  for (int l = 0; l < kMaxLevels; ++l) {
    a.loff[l] = l < g.L ? g.loff[l] : g.E;
    a.pw[l] = l < g.L ? g.pw[l] : 1;
  }
  dim3 grid(cdiv(g.S, 4), (unsigned)g.BH());
  if (g.out == LH_BF16) {
    if (g.d == 128) hipLaunchKernelGGL((scatter_span_bwd_kernel<bf16_t, 16>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((scatter_span_bwd_kernel<bf16_t, 8>), grid, dim3(256), 0, st, a);
  } else {
    if (g.d == 128) hipLaunchKernelGGL((scatter_span_bwd_kernel<float, 16>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((scatter_span_bwd_kernel<float, 8>), grid, dim3(256), 0, st, a);
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
// One workgroup per group of `spw` whole strata of one (b, h) and one tensor
// (the summation itself is unpool_strata in lh_unpool.h).
template <typename TO, int CPR>
__global__ __launch_bounds__(kUnpoolThreads) void unpool_kernel(UnpoolArgs a) {
  extern __shared__ int32_t ro[];
  const int z = blockIdx.z;
  const int64_t bh = blockIdx.y;
  const int part = (int)(blockIdx.x % (unsigned)a.parts);
  const int64_t m0 = (int64_t)(blockIdx.x / (unsigned)a.parts) * a.spw;   // first stratum
  const int tid = threadIdx.x;
  unpool_stage_ro<kUnpoolThreads>(a, ro, a.row_of + bh * a.E, m0, a.spw, 0, a.S, tid);
  __syncthreads();
  const float *dxs = a.dxs[z] + bh * a.S * a.d + (tid % CPR) * 4;
  const int half = a.d / 2;
  auto rows = [&](int32_t r, float *x) {   // columns c*4 .. +3 and d/2 + c*4 .. +3
    const float *p = dxs + (int64_t)r * a.d;
    const float4 u = *reinterpret_cast<const float4 *>(p);
    const float4 v = *reinterpret_cast<const float4 *>(p + half);
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
  };
  unpool_strata<TO, CPR, kUnpoolThreads, true>(
      a, ro, rows, (TO *)a.dx[z] + (bh * a.N + m0 * a.Bc) * a.d, a.spw, tid, part, a.parts);
}

static int unpool_spw(const Geo &g) {
  int spw = (int)(1024 / g.Bc);
  if (spw < 1) spw = 1;
  while (spw > 1 && (spw * g.T > kUnpoolLdsEntries || g.n_c % spw)) --spw;
  return spw;
}

// every launch of this file fits its grid limits for the geometry (grid x in
// work-items within 32 bits; y = B*H and z <= 3 are checked by make_geo) and
// the unpool kernel's LDS staging holds one stratum's row_of entries
lh_status check_rows_supported(const Geo &g) {
  const int64_t S = g.S, N = g.N, BH = g.BH();
  const int cpr = g.d / 8;
  const int64_t row_vec = (int64_t)g.d * 4 / 16;   // widest token row (float32) in 16 B
  const bool ok = grid_fits(cdiv(S, 256 / cpr), 256) &&            // gather
                  grid_fits(g.Sp / 64, 256) &&                      // transpose
                  grid_fits(g.n_c * (int64_t)cdiv(g.Bc, kScatChunk), 256) &&   // scatter
                  grid_fits(g.n_c, kScatBwdThreads) &&              // scatter adjoint
                  scatter_bwd_lds(g) <= kMaxLdsRows &&
                  grid_fits(cdiv(S, 4), 256) &&                     // span adjoint
                  grid_fits(cdiv(N * row_vec, 256), 256) &&         // copy_rows
                  grid_fits(cdiv(N, 256), 256) &&                   // owner
                  grid_fits(cdiv(N, (256 / cpr) * 8), 256) &&       // span scatter
                  grid_fits(cdiv(BH * S, 4), 256) &&                // dos_prep (all heads)
                  grid_fits(2 * g.n_c, kUnpoolThreads);              // unpool (up to 2 parts)
  if (!ok) return LH_ERR_UNSUPPORTED;
  return g.T <= kUnpoolLdsEntries ? LH_OK : LH_ERR_UNSUPPORTED;
}

UnpoolArgs make_unpool_args(const Geo &g, int spw) {
  UnpoolArgs a;
  for (int i = 0; i < 3; ++i) {
    a.dxs[i] = nullptr;
    a.dx[i] = nullptr;
  }
  a.row_of = nullptr;
  a.N = g.N; a.E = g.E; a.S = g.S; a.Bc = g.Bc; a.d = g.d; a.L = g.L; a.p = g.p;
  a.spw = spw;
  a.parts = 1;
  a.lgp = -1;
  for (int k = 0; k < 31; ++k)
    if ((1 << k) == g.p) a.lgp = k;
  int lb = 0;
  for (int l = 0; l < kMaxLevels; ++l) {
    a.loff[l] = g.loff[l];
    a.pw[l] = l < g.L ? (int32_t)g.pw[l] : 0;
    a.per[l] = l < g.L ? (int32_t)(g.Bc / g.pw[l]) : 0;
    a.inv[l] = l < g.L ? (float)(1.0 / (double)g.pw[l]) : 0.f;
    a.lb[l] = lb;
    lb += spw * a.per[l];
  }
  return a;
}

lh_status launch_unpool(const Geo &g, const float *const dxs[], const int32_t *row_of,
                        void *const dx[], int nt, hipStream_t st) {
  if (g.T > kUnpoolLdsEntries) return LH_ERR_UNSUPPORTED;
  if (nt < 1 || nt > 3) return LH_ERR_INVALID_ARG;
  UnpoolArgs a = make_unpool_args(g, unpool_spw(g));
  for (int i = 0; i < nt; ++i) {
    a.dxs[i] = dxs[i];
    a.dx[i] = dx[i];
  }
  a.row_of = row_of;
  // one tensor alone (the layer's dQ at d = 128, after the dQ kernel): two
  // workgroups per group of strata, so the launch keeps as many loads in
  // flight as the three-tensor one
  a.parts = nt == 1 ? 2 : 1;
  const size_t smem = (size_t)a.spw * g.T * sizeof(int32_t);
  dim3 grid((unsigned)(g.n_c / a.spw * a.parts), (unsigned)g.BH(), (unsigned)nt);
  if (g.out == LH_BF16) {
    if (g.d == 128) hipLaunchKernelGGL((unpool_kernel<bf16_t, 16>), grid, dim3(kUnpoolThreads), smem, st, a);
    else hipLaunchKernelGGL((unpool_kernel<bf16_t, 8>), grid, dim3(kUnpoolThreads), smem, st, a);
  } else {
    if (g.d == 128) hipLaunchKernelGGL((unpool_kernel<float, 16>), grid, dim3(kUnpoolThreads), smem, st, a);
    else hipLaunchKernelGGL((unpool_kernel<float, 8>), grid, dim3(kUnpoolThreads), smem, st, a);
  }
  return hip_status();
}

}  // namespace lh
