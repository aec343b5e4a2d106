// Public C ABI of liblighthouse: validation, sizes, and the stage / layer
// entry points declared in include/lighthouse.h.  Host code only; the
// kernels live in the k_*.hip sources.
#include <math.h>
#include <string.h>

#include <mutex>

#include "lh_internal.h"

namespace lh {

static bool mul_ok(int64_t a, int64_t b, int64_t lim, int64_t *out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > lim / a) return false;
  *out = a * b;
  return true;
}

lh_status make_geo(const lh_dims *dm, Geo *g) {
  if (!dm || !g) return LH_ERR_INVALID_ARG;
  memset(g, 0, sizeof(*g));
  if (dm->B < 1 || dm->H < 1 || dm->N < 1 || dm->p < 2 || dm->L < 1 || dm->d < 1)
    return LH_ERR_INVALID_ARG;
  if (dm->scatter_mode != LH_SCATTER_HOLD && dm->scatter_mode != LH_SCATTER_SPAN)
    return LH_ERR_INVALID_ARG;
  if (dm->sigma_mode != LH_SIGMA_SUM && dm->sigma_mode != LH_SIGMA_MAX &&
      dm->sigma_mode != LH_SIGMA_PRODUCT)
    return LH_ERR_INVALID_ARG;
  if (dm->strata_mode != LH_STRATA_JOINT && dm->strata_mode != LH_STRATA_PER_LEVEL)
    return LH_ERR_INVALID_ARG;
  if (dm->L >= kMaxLevels) return LH_ERR_UNSUPPORTED;
  if (!(dm->scale >= 0.0f) || !isfinite(dm->scale)) return LH_ERR_INVALID_ARG;
  if ((dm->io_dtype != LH_F32 && dm->io_dtype != LH_BF16) ||
      (dm->out_dtype != LH_F32 && dm->out_dtype != LH_BF16))
    return LH_ERR_INVALID_ARG;
  const int64_t lim = (int64_t)1 << 40;
  g->B = dm->B; g->N = dm->N; g->H = dm->H; g->d = dm->d; g->p = dm->p; g->L = dm->L;
  g->K = dm->K; g->S = dm->S; g->io = dm->io_dtype; g->out = dm->out_dtype;
  g->mode = dm->scatter_mode;
  g->sigma = dm->sigma_mode;
  g->strata = dm->strata_mode;
  g->pw[0] = 1;
  for (int l = 1; l <= g->L; ++l)
    if (!mul_ok(g->pw[l - 1], g->p, lim, &g->pw[l])) return LH_ERR_INVALID_ARG;
  g->Bc = g->pw[g->L - 1];
  // a length that is not whole coarsest cells: the layer calls run on the
  // sequence extended with zero rows to the next multiple (stage calls that
  // take token tensors need whole cells)
  g->Nreal = dm->N;
  g->N = (dm->N + g->Bc - 1) / g->Bc * g->Bc;
  g->n_c = g->N / g->Bc;
  g->T = (g->pw[g->L] - 1) / (g->p - 1);
  int64_t off = 0;
  for (int l = 0; l < g->L; ++l) {
    g->lsize[l] = g->N / g->pw[l];
    g->loff[l] = off;
    off += g->lsize[l];
  }
  g->E = off;
  if (g->K < 0 || g->K % g->n_c) return LH_ERR_INVALID_ARG;
  g->k_s = g->K / g->n_c;
  if (g->k_s > g->T - 1) return LH_ERR_INVALID_ARG;
  if (g->strata == LH_STRATA_PER_LEVEL && g->L >= 2) {
    // levels L-2 .. 1 in turn take min(their size, remaining / levels left);
    // level 0 takes what remains, which must fit in it
    int64_t rem = g->k_s;
    for (int l = g->L - 2; l >= 1; --l) {
      const int64_t n = g->Bc / g->pw[l];
      const int64_t share = rem / (l + 1);
      g->quota[l] = share < n ? share : n;
      rem -= g->quota[l];
    }
    if (rem > g->Bc) return LH_ERR_INVALID_ARG;
    g->quota[0] = rem;
  }
  if (g->S != g->K + g->n_c) return LH_ERR_INVALID_ARG;
  if (g->E >= ((int64_t)1 << 31) || g->S >= ((int64_t)1 << 31)) return LH_ERR_UNSUPPORTED;
  if (g->BH() > 65535) return LH_ERR_UNSUPPORTED;
  if (g->d != 64 && g->d != 128) return LH_ERR_UNSUPPORTED;
  if (g->io == LH_F32 && g->out != LH_F32) return LH_ERR_UNSUPPORTED;
  g->Sp = (g->S + 63) / 64 * 64;
  g->scale = dm->scale == 0.0f ? (float)(1.0 / sqrt((double)g->d)) : dm->scale;
  // every kernel family's launch limits, so that a call that passes
  // validation launches nothing it would later have to refuse
  lh_status (*const checks[])(const Geo &) = {
      check_pyramid_supported, check_select_supported,    check_rows_supported,
      check_attn_f32_supported, check_attn_fwd_supported, check_attn_dkv_supported,
      check_attn_dq_supported};
  for (auto chk : checks) {
    const lh_status s = chk(*g);
    if (s != LH_OK) return s;
  }
  return LH_OK;
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Sizes {
  size_t subseq, rowf32, subseq_f32, drow;
};

static Sizes sizes_of(const Geo &g) {
  Sizes z;
  const size_t bh = (size_t)g.BH();
  z.subseq = bh * g.S * g.d * el_size(g.io);
  z.subseq_f32 = bh * g.S * g.d * 4;
  z.drow = bh * g.S * 4;
  return z;
}

static size_t ws_attn_fwd(const Geo &) { return 0; }
static size_t rows_bf16(const Geo &g) { return (size_t)g.BH() * g.S * g.d * 2; }
static size_t ws_attn_bwd(const Geo &g) {
  Sizes z = sizes_of(g);
  if (g.io == LH_F32) return al256(z.drow);
  return 2 * al256(rows_bf16(g)) + al256(z.drow);        // dos split (hi, lo), drow
}
static size_t owner_bytes(const Geo &g) { return (size_t)g.BH() * g.N * 4; }
static bool ragged(const Geo &g) { return g.N != g.Nreal; }
// one padded token tensor [B,H,N,d] of element type t
static size_t padded_bytes(const Geo &g, int32_t t) {
  return (size_t)g.BH() * g.N * g.d * el_size(t);
}
static size_t ws_layer_fwd(const Geo &g) {
  size_t b = g.mode == LH_SCATTER_SPAN ? al256(owner_bytes(g)) : 0;   // span owner map
  if (ragged(g)) b += 3 * al256(padded_bytes(g, g.io)) + al256(padded_bytes(g, g.out));
  return b;
}
static size_t ws_layer_bwd(const Geo &g) {
  Sizes z = sizes_of(g);
  size_t b = 3 * al256(z.subseq_f32) + al256(z.drow);   // dqs, dks, dvs, drow
  if (g.io == LH_BF16) b += 2 * al256(rows_bf16(g));     // dos split
  else b += al256(z.subseq_f32);                          // float32 dos
  if (g.mode == LH_SCATTER_SPAN) b += al256(owner_bytes(g));
  if (ragged(g)) b += 4 * al256(padded_bytes(g, g.out));  // dO, dQ, dK, dV padded
  return b;
}
// stage calls that read or write token tensors [B,H,N,d] need whole cells
static lh_status need_whole(const Geo &g) { return ragged(g) ? LH_ERR_INVALID_ARG : LH_OK; }

// carve consecutive 256-aligned sub-buffers out of a workspace
struct Carver {
  char *base;
  size_t off, cap;
  void *take(size_t n) {
    void *p = base + off;
    off += al256(n);
    return p;
  }
  bool ok() const { return off <= cap; }
};

// A second stream of each device (default priority, non-blocking) and two
// events, created on first use and kept until the process ends: the layer
// backward forks the pooling adjoint of dK and dV onto it (beside the dQ
// kernel) and joins it back.  The mutex keeps each fork/join sequence whole
// when several host threads call on one device.
constexpr int kMaxDevices = 64;
static std::mutex g_side_mu;
static hipStream_t g_side[kMaxDevices];
static hipEvent_t g_fork[kMaxDevices], g_join[kMaxDevices];
static bool g_side_ok[kMaxDevices];

// call with g_side_mu held
static lh_status side_stream(hipStream_t *s, hipEvent_t *fork, hipEvent_t *join) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LH_ERR_HIP;
  if (!g_side_ok[dev]) {
    if (hipStreamCreateWithFlags(&g_side[dev], hipStreamNonBlocking) != hipSuccess)
      return LH_ERR_HIP;
    // The events order kernels of this device only: each kernel's own
    // completion already releases its writes at device scope, so the events
    // skip the system-scope fence (a cache write-back on every record, which
    // cost the caller's stream 7-11 us per fork or join).  The host never
    // waits on them.
    const unsigned ev = hipEventDisableTiming | hipEventDisableSystemFence;
    if (hipEventCreateWithFlags(&g_fork[dev], ev) != hipSuccess ||
        hipEventCreateWithFlags(&g_join[dev], ev) != hipSuccess)
      return LH_ERR_HIP;
    g_side_ok[dev] = true;
  }
  *s = g_side[dev];
  *fork = g_fork[dev];
  *join = g_join[dev];
  return LH_OK;
}

// Joins the side stream back to the caller's stream when it goes out of
// scope (after a fork, on every return path): the side stream's work so far
// is then complete whenever the caller's is, also when a launch on either
// stream failed in between.  join() does it at a chosen point.
struct SideJoin {
  hipStream_t st, side;
  hipEvent_t ev;
  bool armed;
  lh_status join() {
    if (!armed) return LH_OK;
    armed = false;
    if (hipEventRecord(ev, side) != hipSuccess || hipStreamWaitEvent(st, ev, 0) != hipSuccess)
      return LH_ERR_HIP;
    return LH_OK;
  }
  ~SideJoin() { (void)join(); }
};

// Clears an error an earlier HIP call of this host thread left pending, so
// that the status after this call's launches reports its own launches only.
static void clear_pending_error() { (void)hipGetLastError(); }

static bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }
static bool aligned4(const void *p) { return ((uintptr_t)p & 3) == 0; }

}  // namespace lh

using namespace lh;

#define LH_TRY(expr)                   \
  do {                                 \
    lh_status _s = (expr);             \
    if (_s != LH_OK) return _s;        \
  } while (0)
#define LH_REQ(cond)                              \
  do {                                            \
    if (!(cond)) return LH_ERR_INVALID_ARG;       \
  } while (0)

extern "C" {

lh_status lh_validate(const lh_dims *dims) {
  Geo g;
  return make_geo(dims, &g);
}

lh_status lh_get_sizes(const lh_dims *dims, lh_sizes *out) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_REQ(out);
  memset(out, 0, sizeof(*out));
  const size_t bh = (size_t)g.BH();
  out->E = g.E; out->n_c = g.n_c; out->T = g.T; out->k_s = g.k_s; out->Bc = g.Bc; out->Sp = g.Sp;
  out->pyramid_bytes = bh * (g.E - g.N) * g.d * el_size(g.io);
  out->score_bytes = bh * g.E * 4;
  out->row_i32_bytes = bh * g.S * 4;
  out->row_u8_bytes = bh * g.S;
  out->row_of_bytes = bh * g.E * 4;
  out->subseq_bytes = g.io == LH_BF16 ? bh * g.d * g.Sp * 2 : bh * g.S * g.d * 4;
  if (g.io == LH_BF16 && bh * g.S * g.d * 2 > out->subseq_bytes) out->subseq_bytes = bh * g.S * g.d * 2;
  out->os_bytes = bh * g.S * g.d * 4;
  out->lse_bytes = bh * g.S * 4;
  out->token_io_bytes = bh * g.Nreal * g.d * el_size(g.io);
  out->token_out_bytes = bh * g.Nreal * g.d * el_size(g.out);
  out->ws_attn_fwd = ws_attn_fwd(g);
  out->ws_attn_bwd = ws_attn_bwd(g);
  out->ws_layer_fwd = ws_layer_fwd(g);
  out->ws_layer_bwd = ws_layer_bwd(g);
  out->owner_bytes = owner_bytes(g);
  return LH_OK;
}

const char *lh_status_string(lh_status s) {
  switch (s) {
    case LH_OK: return "ok";
    case LH_ERR_INVALID_ARG: return "invalid argument (geometry, null or misaligned pointer)";
    case LH_ERR_UNSUPPORTED: return "unsupported configuration";
    case LH_ERR_WORKSPACE: return "workspace missing or too small";
    case LH_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

const char *lh_version(void) { return "0.1.0"; }

lh_status lh_pyramid_build(const lh_dims *dims, const void *q, const void *k, const void *v,
                           void *pq, void *pk, void *pv, lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_TRY(need_whole(g));
  const void *in[3] = {q, k, v};
  void *out[3] = {pq, pk, pv};
  int any = 0;
  for (int i = 0; i < 3; ++i) {
    LH_REQ(g.L == 1 || (in[i] == nullptr) == (out[i] == nullptr));
    LH_REQ(aligned16(in[i]) && aligned16(out[i]));
    any += in[i] != nullptr;
  }
  LH_REQ(any > 0);
  clear_pending_error();
  return launch_pyramid_score(g, q, k, v, pq, pk, pv, nullptr, nullptr, (hipStream_t)stream);
}

lh_status lh_score(const lh_dims *dims, const void *q, const void *k, float *sq, float *sk,
                   lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_TRY(need_whole(g));
  LH_REQ(q && k && sq && sk && aligned16(q) && aligned16(k) && aligned4(sq) && aligned4(sk));
  clear_pending_error();
  return launch_pyramid_score(g, q, k, nullptr, nullptr, nullptr, nullptr, sq, sk,
                              (hipStream_t)stream);
}

lh_status lh_pyramid_score(const lh_dims *dims, const void *q, const void *k, const void *v,
                           void *pq, void *pk, void *pv, float *sq, float *sk,
                           lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_TRY(need_whole(g));
  LH_REQ(q && k && v && sq && sk);
  LH_REQ(g.L == 1 || (pq && pk && pv));
  LH_REQ(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(pq) && aligned16(pk) &&
         aligned16(pv) && aligned4(sq) && aligned4(sk));
  clear_pending_error();
  return launch_pyramid_score(g, q, k, v, pq, pk, pv, sq, sk, (hipStream_t)stream);
}

lh_status lh_topk_select(const lh_dims *dims, const float *sq, const float *sk,
                         int32_t *sel_idx, int32_t *sel_anchor, uint8_t *sel_flags,
                         int32_t *row_of, lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_REQ(sq && sk && sel_idx && sel_anchor && sel_flags && row_of);
  LH_REQ(aligned4(sq) && aligned4(sk) && aligned4(sel_idx) && aligned4(sel_anchor) &&
         aligned4(row_of));
  clear_pending_error();
  return launch_select(g, sq, sk, sel_idx, sel_anchor, sel_flags, row_of, (hipStream_t)stream);
}

static lh_status gather_impl(const Geo &g, const void *q, const void *k, const void *v,
                             const void *pq, const void *pk, const void *pv,
                             const int32_t *sel_idx, void *qs, void *ks, void *vs, void *qst,
                             void *kst, void *vst, hipStream_t st) {
  const void *src[3] = {q, k, v};
  const void *psrc[3] = {pq, pk, pv};
  void *dst[3] = {qs, ks, vs};
  LH_TRY(launch_gather(g, src, psrc, sel_idx, dst, st));
  void *tr[3] = {qst, kst, vst};
  for (int i = 0; i < 3; ++i)
    if (tr[i]) LH_TRY(launch_transpose(g, dst[i], tr[i], st));
  return LH_OK;
}

lh_status lh_gather(const lh_dims *dims, const void *q, const void *k, const void *v,
                    const void *pq, const void *pk, const void *pv, const int32_t *sel_idx,
                    void *qs, void *ks, void *vs, void *qst, void *kst, void *vst,
                    lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_TRY(need_whole(g));
  LH_REQ(q && k && v && sel_idx && qs && ks && vs);
  LH_REQ(g.L == 1 || (pq && pk && pv));
  LH_REQ(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(pq) && aligned16(pk) &&
         aligned16(pv) && aligned16(qs) && aligned16(ks) && aligned16(vs) && aligned4(sel_idx));
  LH_REQ(aligned16(qst) && aligned16(kst) && aligned16(vst));
  if (g.io == LH_F32) LH_REQ(!qst && !kst && !vst);
  clear_pending_error();
  return gather_impl(g, q, k, v, pq, pk, pv, sel_idx, qs, ks, vs, qst, kst, vst,
                     (hipStream_t)stream);
}

lh_status lh_subseq_attn_fwd(const lh_dims *dims, const void *qs, const void *ks,
                             const void *vs, const uint8_t *sel_flags, void *os, float *lse,
                             void *ws, size_t ws_bytes, lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_REQ(qs && ks && vs && sel_flags && os && lse);
  LH_REQ(aligned16(qs) && aligned16(ks) && aligned16(vs) && aligned16(os) && aligned4(lse));
  hipStream_t st = (hipStream_t)stream;
  clear_pending_error();
  if (g.io == LH_F32)
    return launch_attn_fwd_f32(g, (const float *)qs, (const float *)ks, (const float *)vs,
                               sel_flags, (float *)os, lse, st);
  (void)ws;
  (void)ws_bytes;
  return launch_attn_fwd_bf16(g, (const bf16_t *)qs, (const bf16_t *)ks, (const bf16_t *)vs,
                              sel_flags, (float *)os, lse, st);
}

// the attention backward after validation: the dO split and drow go to the
// workspace `ws` of at least ws_attn_bwd(g) bytes
static lh_status attn_bwd_impl(const Geo &g, const void *qs, const void *ks, const void *vs,
                               const void *os, const float *lse, const uint8_t *sel_flags,
                               const float *dos, float *dqs, float *dks, float *dvs, void *ws,
                               size_t ws_bytes, hipStream_t st) {
  Carver c{(char *)ws, 0, ws_bytes};
  Sizes z = sizes_of(g);
  clear_pending_error();
  if (g.io == LH_F32) {
    float *drow = (float *)c.take(z.drow);
    LH_TRY(launch_dos_prep(g, dos, (const float *)os, nullptr, nullptr, drow, st));
    return launch_attn_bwd_f32(g, (const float *)qs, (const float *)ks, (const float *)vs,
                               (const float *)os, lse, sel_flags, dos, drow, dqs, dks, dvs, st);
  }
  bf16_t *dhi = (bf16_t *)c.take(rows_bf16(g));
  bf16_t *dlo = (bf16_t *)c.take(rows_bf16(g));
  float *drow = (float *)c.take(z.drow);
  if (!c.ok()) return LH_ERR_WORKSPACE;
  LH_TRY(launch_dos_prep(g, dos, (const float *)os, dhi, dlo, drow, st));
  return launch_attn_bwd_bf16(g, (const bf16_t *)qs, (const bf16_t *)ks, (const bf16_t *)vs,
                              dhi, dlo, lse, drow, sel_flags, dqs, dks, dvs, st);
}

static lh_status attn_bwd_args(const Geo &g, const void *qs, const void *ks, const void *vs,
                               const void *os, const float *lse, const uint8_t *sel_flags,
                               const float *dos, const float *dqs, const float *dks,
                               const float *dvs) {
  (void)g;
  LH_REQ(qs && ks && vs && os && lse && sel_flags && dos && dqs && dks && dvs);
  LH_REQ(aligned16(qs) && aligned16(ks) && aligned16(vs) && aligned16(os) && aligned4(lse) &&
         aligned16(dos) && aligned16(dqs) && aligned16(dks) && aligned16(dvs));
  return LH_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- no-alloc form
// Scratch memory of lh_subseq_attn_bwd_noalloc: a fixed device array (each
// device that loads the library holds its own copy until the process ends).
// In host code `scratch` names a host-side stand-in, not device memory; the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is handed to kernels.
namespace lh {
constexpr size_t kNoAllocScratch = (size_t)LH_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratch];
static std::mutex g_scratch_mu;
static void *g_scratch[kMaxDevices];

static lh_status scratch_ptr(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LH_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LH_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return LH_OK;
}
}  // namespace lh

extern "C" {

lh_status lh_subseq_attn_bwd(const lh_dims *dims, const void *qs, const void *ks,
                             const void *vs, const void *os, const float *lse,
                             const uint8_t *sel_flags, const float *dos, float *dqs, float *dks,
                             float *dvs, void *ws, size_t ws_bytes, lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_TRY(attn_bwd_args(g, qs, ks, vs, os, lse, sel_flags, dos, dqs, dks, dvs));
  if (ws_bytes < ws_attn_bwd(g) || !ws || !aligned16(ws)) return LH_ERR_WORKSPACE;
  return attn_bwd_impl(g, qs, ks, vs, os, lse, sel_flags, dos, dqs, dks, dvs, ws, ws_bytes,
                       (hipStream_t)stream);
}

lh_status lh_subseq_attn_bwd_noalloc(const lh_dims *dims, const void *qs, const void *ks,
                                     const void *vs, const void *os, const float *lse,
                                     const uint8_t *sel_flags, const float *dos, float *dqs,
                                     float *dks, float *dvs, lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_TRY(attn_bwd_args(g, qs, ks, vs, os, lse, sel_flags, dos, dqs, dks, dvs));
  const size_t need = ws_attn_bwd(g);
  if (need > kNoAllocScratch) return LH_ERR_UNSUPPORTED;
  void *ws = nullptr;
  LH_TRY(scratch_ptr(&ws));
  return attn_bwd_impl(g, qs, ks, vs, os, lse, sel_flags, dos, dqs, dks, dvs, ws,
                       kNoAllocScratch, (hipStream_t)stream);
}

lh_status lh_attn_bwd_prep(const lh_dims *dims, const float *dos, const float *os, void *dos_hi,
                           void *dos_lo, float *drow, lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  if (g.io != LH_BF16) return LH_ERR_UNSUPPORTED;
  LH_REQ(dos && os && dos_hi && dos_lo && drow);
  LH_REQ(aligned16(dos) && aligned16(os) && aligned16(dos_hi) && aligned16(dos_lo) &&
         aligned4(drow));
  clear_pending_error();
  return launch_dos_prep(g, dos, os, (bf16_t *)dos_hi, (bf16_t *)dos_lo, drow,
                         (hipStream_t)stream);
}

lh_status lh_attn_fwd_mfma(const lh_dims *dims, const void *qs, const void *ks, const void *vs,
                           const uint8_t *sel_flags, float *os, float *lse, lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  if (g.io != LH_BF16) return LH_ERR_UNSUPPORTED;
  LH_REQ(qs && ks && vs && sel_flags && os && lse);
  LH_REQ(aligned16(qs) && aligned16(ks) && aligned16(vs) && aligned16(os) && aligned4(lse));
  clear_pending_error();
  return launch_attn_fwd_bf16(g, (const bf16_t *)qs, (const bf16_t *)ks, (const bf16_t *)vs,
                              sel_flags, os, lse, (hipStream_t)stream);
}

lh_status lh_attn_bwd_dkv_mfma(const lh_dims *dims, const void *qs, const void *ks,
                               const void *vs, const void *dos_hi, const void *dos_lo,
                               const float *lse, const float *drow, const uint8_t *sel_flags,
                               float *dks, float *dvs, lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  if (g.io != LH_BF16) return LH_ERR_UNSUPPORTED;
  LH_REQ(qs && ks && vs && dos_hi && dos_lo && lse && drow && sel_flags && dks && dvs);
  LH_REQ(aligned16(qs) && aligned16(ks) && aligned16(vs) && aligned16(dos_hi) &&
         aligned16(dos_lo) && aligned4(lse) && aligned4(drow) && aligned16(dks) &&
         aligned16(dvs));
  clear_pending_error();
  return launch_attn_bwd_dkv_bf16(g, (const bf16_t *)qs, (const bf16_t *)ks, (const bf16_t *)vs,
                                  (const bf16_t *)dos_hi, (const bf16_t *)dos_lo, lse, drow,
                                  sel_flags, dks, dvs, (hipStream_t)stream);
}

lh_status lh_attn_bwd_dq_mfma(const lh_dims *dims, const void *qs, const void *ks,
                              const void *vs, const void *dos_hi, const void *dos_lo,
                              const float *lse, const float *drow, const uint8_t *sel_flags,
                              float *dqs, lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  if (g.io != LH_BF16) return LH_ERR_UNSUPPORTED;
  LH_REQ(qs && ks && vs && dos_hi && dos_lo && lse && drow && sel_flags && dqs);
  LH_REQ(aligned16(qs) && aligned16(ks) && aligned16(vs) && aligned16(dos_hi) &&
         aligned16(dos_lo) && aligned4(lse) && aligned4(drow) && aligned16(dqs));
  clear_pending_error();
  return launch_attn_bwd_dq_bf16(g, (const bf16_t *)qs, (const bf16_t *)ks, (const bf16_t *)vs,
                                 (const bf16_t *)dos_hi, (const bf16_t *)dos_lo, lse, drow,
                                 sel_flags, dqs, (hipStream_t)stream);
}

lh_status lh_scatter(const lh_dims *dims, const void *os, const int32_t *sel_anchor,
                     const uint8_t *sel_flags, void *o, lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_TRY(need_whole(g));
  LH_REQ(os && sel_anchor && sel_flags && o);
  LH_REQ(aligned16(os) && aligned16(o) && aligned4(sel_anchor));
  clear_pending_error();
  return launch_scatter(g, (const float *)os, sel_anchor, sel_flags, o, (hipStream_t)stream);
}

lh_status lh_scatter_bwd(const lh_dims *dims, const void *dout, const int32_t *sel_anchor,
                         const uint8_t *sel_flags, float *dos, lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_TRY(need_whole(g));
  LH_REQ(dout && sel_anchor && sel_flags && dos);
  LH_REQ(aligned16(dout) && aligned16(dos) && aligned4(sel_anchor));
  clear_pending_error();
  return launch_scatter_bwd(g, dout, sel_anchor, sel_flags, dos, nullptr, nullptr, nullptr,
                            nullptr, nullptr, (hipStream_t)stream);
}

lh_status lh_span_owner(const lh_dims *dims, const int32_t *row_of, int32_t *owner,
                        lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_TRY(need_whole(g));
  LH_REQ(row_of && owner);
  LH_REQ(aligned4(row_of) && aligned4(owner));
  clear_pending_error();
  return launch_owner(g, row_of, owner, (hipStream_t)stream);
}

lh_status lh_scatter_span(const lh_dims *dims, const float *os, const int32_t *owner, void *o,
                          lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_TRY(need_whole(g));
  LH_REQ(os && owner && o);
  LH_REQ(aligned16(os) && aligned4(owner) && aligned16(o));
  clear_pending_error();
  return launch_scatter_span(g, os, owner, o, (hipStream_t)stream);
}

lh_status lh_scatter_span_bwd(const lh_dims *dims, const void *dout, const int32_t *sel_idx,
                              const uint8_t *sel_flags, const int32_t *owner, float *dos,
                              lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_TRY(need_whole(g));
  LH_REQ(dout && sel_idx && sel_flags && owner && dos);
  LH_REQ(aligned16(dout) && aligned4(sel_idx) && aligned4(owner) && aligned16(dos));
  clear_pending_error();
  return launch_scatter_span_bwd(g, dout, sel_idx, sel_flags, owner, dos, nullptr, nullptr,
                                 nullptr, nullptr, (hipStream_t)stream);
}

lh_status lh_gather_bwd(const lh_dims *dims, const float *dqs, const float *dks,
                        const float *dvs, const int32_t *row_of, void *dq, void *dk, void *dv,
                        lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_TRY(need_whole(g));
  LH_REQ(dqs && dks && dvs && row_of && dq && dk && dv);
  LH_REQ(aligned16(dqs) && aligned16(dks) && aligned16(dvs) && aligned4(row_of) &&
         aligned16(dq) && aligned16(dk) && aligned16(dv));
  const float *in[3] = {dqs, dks, dvs};
  void *out[3] = {dq, dk, dv};
  clear_pending_error();
  return launch_unpool(g, in, row_of, out, 3, (hipStream_t)stream);
}

static lh_status check_saved(const Geo &g, const lh_saved *s) {
  LH_REQ(s);
  LH_REQ(s->sq && s->sk && s->sel_idx && s->sel_anchor && s->sel_flags && s->row_of);
  LH_REQ(s->qs && s->ks && s->vs && s->os && s->lse);
  LH_REQ(g.L == 1 || (s->pq && s->pk && s->pv));
  LH_REQ(aligned16(s->pq) && aligned16(s->pk) && aligned16(s->pv) && aligned4(s->sq) &&
         aligned4(s->sk) && aligned4(s->sel_idx) && aligned4(s->sel_anchor) &&
         aligned4(s->row_of) && aligned16(s->qs) && aligned16(s->ks) && aligned16(s->vs) &&
         aligned16(s->os) && aligned4(s->lse));
  return LH_OK;
}

lh_status lh_layer_fwd(const lh_dims *dims, const void *q, const void *k, const void *v,
                       void *o, const lh_saved *s, void *ws, size_t ws_bytes,
                       lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_REQ(q && k && v && o);
  LH_REQ(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o));
  LH_TRY(check_saved(g, s));
  const size_t need = ws_layer_fwd(g);
  if (need && (ws_bytes < need || !ws || !aligned16(ws))) return LH_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  clear_pending_error();
  Carver c{(char *)ws, 0, ws_bytes};
  int32_t *owner = g.mode == LH_SCATTER_SPAN ? (int32_t *)c.take(owner_bytes(g)) : nullptr;
  void *o_run = o;
  if (ragged(g)) {
    // whole coarsest cells: the inputs extended with zero rows, the output
    // written to a padded buffer and its real rows copied out at the end
    const size_t tin = padded_bytes(g, g.io);
    void *qp = c.take(tin), *kp = c.take(tin), *vp = c.take(tin);
    o_run = c.take(padded_bytes(g, g.out));
    const int64_t rb = (int64_t)g.d * el_size(g.io);
    LH_TRY(launch_copy_rows(g, q, qp, g.Nreal, g.N, rb, st));
    LH_TRY(launch_copy_rows(g, k, kp, g.Nreal, g.N, rb, st));
    LH_TRY(launch_copy_rows(g, v, vp, g.Nreal, g.N, rb, st));
    q = qp;
    k = kp;
    v = vp;
  }
  if (!c.ok()) return LH_ERR_WORKSPACE;
  // the three pyramids and the scores in one launch, the selection, then
  // the three gathers in one launch, all on the caller's stream (measured
  // as fast as or faster than forking V's pyramid and gather onto the
  // second stream beside the selection, on every workload)
  LH_TRY(launch_pyramid_score(g, q, k, v, s->pq, s->pk, s->pv, s->sq, s->sk, st));
  LH_TRY(launch_select(g, s->sq, s->sk, s->sel_idx, s->sel_anchor, s->sel_flags, s->row_of, st));
  {
    const void *src[3] = {q, k, v}, *psrc[3] = {s->pq, s->pk, s->pv};
    void *dst[3] = {s->qs, s->ks, s->vs};
    LH_TRY(launch_gather(g, src, psrc, s->sel_idx, dst, st, 0, 3));
  }
  const bool bf = g.io == LH_BF16;
  // bf16 I/O in hold mode: the attention kernel also writes the output
  // under the causal hold (the scatter stage fused into its epilogue)
  const bool fused = bf && g.mode != LH_SCATTER_SPAN;
  if (bf)
    LH_TRY(launch_attn_fwd_bf16(g, (const bf16_t *)s->qs, (const bf16_t *)s->ks,
                                (const bf16_t *)s->vs, s->sel_flags, (float *)s->os, s->lse,
                                st, fused ? s->sel_anchor : nullptr, fused ? o_run : nullptr));
  else
    LH_TRY(launch_attn_fwd_f32(g, (const float *)s->qs, (const float *)s->ks,
                               (const float *)s->vs, s->sel_flags, (float *)s->os, s->lse, st));
  if (g.mode == LH_SCATTER_SPAN) {
    LH_TRY(launch_owner(g, s->row_of, owner, st));
    LH_TRY(launch_scatter_span(g, (const float *)s->os, owner, o_run, st));
  } else if (!fused) {
    LH_TRY(launch_scatter(g, (const float *)s->os, s->sel_anchor, s->sel_flags, o_run, st));
  }
  if (ragged(g))
    return launch_copy_rows(g, o_run, o, g.N, g.Nreal, (int64_t)g.d * el_size(g.out), st);
  return LH_OK;
}

lh_status lh_layer_bwd(const lh_dims *dims, const lh_saved *s, const void *dout, void *dq,
                       void *dk, void *dv, void *ws, size_t ws_bytes, lh_stream stream) {
  Geo g;
  LH_TRY(make_geo(dims, &g));
  LH_REQ(dout && dq && dk && dv);
  LH_REQ(aligned16(dout) && aligned16(dq) && aligned16(dk) && aligned16(dv));
  LH_TRY(check_saved(g, s));
  const size_t need = ws_layer_bwd(g);
  if (ws_bytes < need || !ws || !aligned16(ws)) return LH_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  clear_pending_error();
  Sizes z = sizes_of(g);
  Carver c{(char *)ws, 0, ws_bytes};
  float *dqs = (float *)c.take(z.subseq_f32);
  float *dks = (float *)c.take(z.subseq_f32);
  float *dvs = (float *)c.take(z.subseq_f32);
  float *drow = (float *)c.take(z.drow);
  int32_t *owner = g.mode == LH_SCATTER_SPAN ? (int32_t *)c.take(owner_bytes(g)) : nullptr;
  void *grad[3] = {dq, dk, dv};
  if (ragged(g)) {
    // dO extended with zero rows; the gradients go to padded buffers whose
    // real rows are copied out at the end
    const size_t tout = padded_bytes(g, g.out);
    void *dop = c.take(tout);
    for (int i = 0; i < 3; ++i) grad[i] = c.take(tout);
    if (!c.ok()) return LH_ERR_WORKSPACE;
    LH_TRY(launch_copy_rows(g, dout, dop, g.Nreal, g.N, (int64_t)g.d * el_size(g.out), st));
    dout = dop;
  }
  // scatter adjoint in the layer's mode (dos float32 and/or its bf16 split);
  // the hold adjoint keeps float32 dOS rows for drow in dqs, which nothing
  // uses before the dQ kernel
  auto scatter_adj = [&](float *dos, bf16_t *hi, bf16_t *lo) -> lh_status {
    if (g.mode == LH_SCATTER_SPAN) {
      LH_TRY(launch_owner(g, s->row_of, owner, st));
      return launch_scatter_span_bwd(g, dout, s->sel_idx, s->sel_flags, owner, dos, hi, lo,
                                     (const float *)s->os, drow, st);
    }
    return launch_scatter_bwd(g, dout, s->sel_anchor, s->sel_flags, dos, hi, lo,
                              (const float *)s->os, drow, dqs, st);
  };
  if (g.io == LH_BF16) {
    bf16_t *dhi = (bf16_t *)c.take(rows_bf16(g));
    bf16_t *dlo = (bf16_t *)c.take(rows_bf16(g));
    if (!c.ok()) return LH_ERR_WORKSPACE;
    LH_TRY(scatter_adj(nullptr, dhi, dlo));
    LH_TRY(launch_attn_bwd_dkv_bf16(g, (const bf16_t *)s->qs, (const bf16_t *)s->ks,
                                    (const bf16_t *)s->vs, dhi, dlo, s->lse, drow, s->sel_flags,
                                    dks, dvs, st));
    // dK, dV are final: their pooling adjoint runs on the side stream beside
    // the dQ kernel (MFMA-bound; one wavefront per SIMD leaves room for it)
    std::lock_guard<std::mutex> lock(g_side_mu);
    hipStream_t side;
    hipEvent_t fork, join;
    LH_TRY(side_stream(&side, &fork, &join));
    if (hipEventRecord(fork, st) != hipSuccess || hipStreamWaitEvent(side, fork, 0) != hipSuccess)
      return LH_ERR_HIP;
    SideJoin sj{st, side, join, true};
    const float *in_kv[2] = {dks, dvs};
    void *out_kv[2] = {grad[1], grad[2]};
    LH_TRY(launch_unpool(g, in_kv, s->row_of, out_kv, 2, side));
    if (dq_can_unpool(g)) {
      // d = 64 and every dQ workgroup's 128 rows are whole strata: it runs
      // the gather + pooling adjoint of its own rows in its epilogue (no dQS
      // round trip, and dQ's token writes overlap the MFMA work of the other
      // workgroup on its CU); otherwise dQS, then dQ's own unpool launch
      LH_TRY(launch_attn_bwd_dq_unpool(g, (const bf16_t *)s->qs, (const bf16_t *)s->ks,
                                       (const bf16_t *)s->vs, dhi, dlo, s->lse, drow,
                                       s->sel_flags, s->row_of, grad[0], st));
    } else {
      LH_TRY(launch_attn_bwd_dq_bf16(g, (const bf16_t *)s->qs, (const bf16_t *)s->ks,
                                     (const bf16_t *)s->vs, dhi, dlo, s->lse, drow, s->sel_flags,
                                     dqs, st));
      const float *in_q[1] = {dqs};
      void *out_q[1] = {grad[0]};
      LH_TRY(launch_unpool(g, in_q, s->row_of, out_q, 1, st));
    }
    LH_TRY(sj.join());
  } else {
    float *dos = (float *)c.take(z.subseq_f32);
    if (!c.ok()) return LH_ERR_WORKSPACE;
    LH_TRY(scatter_adj(dos, nullptr, nullptr));
    LH_TRY(launch_attn_bwd_f32(g, (const float *)s->qs, (const float *)s->ks,
                               (const float *)s->vs, (const float *)s->os, s->lse, s->sel_flags,
                               dos, drow, dqs, dks, dvs, st));
    const float *in[3] = {dqs, dks, dvs};
    LH_TRY(launch_unpool(g, in, s->row_of, grad, 3, st));
  }
  if (ragged(g)) {
    void *out[3] = {dq, dk, dv};
    for (int i = 0; i < 3; ++i)
      LH_TRY(launch_copy_rows(g, grad[i], out[i], g.N, g.Nreal, (int64_t)g.d * el_size(g.out),
                              st));
  }
  return LH_OK;
}

}  // extern "C"
