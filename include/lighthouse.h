/*
 * lighthouse.h -- C ABI of the MI355X (gfx950) Lighthouse Attention layer.
 *
 * The layer (gist.science explainer "Long Context Pre-Training with
 * Lighthouse Attention", technical summary section 2; edge.aivizor.me news
 * item on the same paper, four-stages paragraph) wraps ordinary causal
 * attention in four stages: a symmetric average-pooled Q/K/V pyramid, a
 * parameter-free per-head l2 scorer with max-pool inheritance and a
 * stratified top-K that always keeps the coarsest level, dense causal
 * attention on the gathered subsequence, and a deterministic scatter back to
 * token positions.  Every stage is a hand-written HIP kernel.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers: device pointers to caller-owned memory unless stated.  The
 *    library never allocates, frees or retains them; scratch memory comes
 *    only through an explicit workspace argument (ws, ws_bytes).  Vector
 *    pointers must be 16-byte aligned.
 *  - Layouts: row-major and contiguous with the head dimension fastest:
 *      token tensors         [B, H, N, d]
 *      coarse pyramid rows   [B, H, E - N, d]   (levels 1..L-1, finest first)
 *      score planes          [B, H, E]          float32
 *      subsequence rows      [B, H, S, d]
 *      per-row vectors       [B, H, S]
 *      transposed copies     [B, H, d, Sp]      ("...t" buffers; Sp = S
 *                                                rounded up to a multiple of
 *                                                64, padding columns zero)
 *    with N_l = N / p^l entries at level l, E = sum_l N_l, and the flat index
 *    of entry (l, i) equal to off_l + i, off_l = sum_{m<l} N_m (level 0 uses
 *    the input's own row numbers).  Flat indices are int32 per (b, h).
 *  - Geometry: B_c = p^(L-1) tokens per coarsest cell, n_c = N / B_c strata,
 *    T = (p^L - 1)/(p - 1) entries per stratum, k_s = K / n_c ranked entries
 *    per stratum, S = K + n_c subsequence rows.
 *  - Streams: all work is ordered on `stream` (a hipStream_t; NULL is the
 *    null stream) and is asynchronous.  The layer backward also runs the
 *    pooling adjoint of dK and dV on a second stream of the device that the
 *    library keeps (default priority), forked from `stream` and joined back
 *    to it by events, so that it is complete whenever `stream`'s work is.
 *    No call synchronises or reads device memory back to the host.
 *  - Outputs are overwritten, never accumulated.  Token-length outputs that
 *    no later kernel of the layer reads (the layer output, the input
 *    gradients, the scatter stages' outputs) are written with nontemporal
 *    stores: they go to HBM rather than staying dirty in the caches, so a
 *    consumer reads them from HBM.
 *  - Errors: every call validates its dims and pointers first and returns a
 *    negative lh_status without launching anything if they are invalid.
 *    lh_validate applies every limit a launch has (grid sizes, LDS budgets,
 *    buffer-resource ranges), so a call whose dims it accepts is never
 *    refused part-way.  A call that launches first clears any HIP error an
 *    earlier call of the same host thread left pending, so that LH_ERR_HIP
 *    reports a failure of its own launches.  After a fork onto the second
 *    stream (below) the join back to `stream` is made on every return path,
 *    error paths included.  No C++ exception crosses the ABI.
 *  - Concurrency: calls are reentrant; the library has no mutable global
 *    state apart from a per-device second stream with two events and the
 *    per-device address of the no-alloc entry point's scratch array, each
 *    set once under a lock and kept until the process ends.
 *  - Determinism: every kernel is free of atomics on floating-point data;
 *    results are bitwise reproducible run to run.
 */
#ifndef LIGHTHOUSE_H
#define LIGHTHOUSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lh_status;
#define LH_OK               0
#define LH_ERR_INVALID_ARG (-1)   /* bad geometry, null or misaligned pointer */
#define LH_ERR_UNSUPPORTED (-2)   /* valid geometry this library does not cover */
#define LH_ERR_WORKSPACE   (-3)   /* workspace missing or too small           */
#define LH_ERR_HIP         (-4)   /* a HIP launch or runtime call failed      */

/* element types of Q/K/V/dO (io_dtype) and of O/dQ/dK/dV (out_dtype) */
#define LH_F32  0
#define LH_BF16 1

/* sel_flags bits of a subsequence row */
#define LH_ROW_REDUNDANT 1u  /* every token of its span is covered by selected
                                finer entries: masked as a key              */
#define LH_ROW_LEADER    2u  /* finest row at its anchor: owns the outputs of
                                tokens [anchor, next leader's anchor)       */

/* lh_dims.scatter_mode: how subsequence outputs go back to token positions
 * (explainer 2.C: a deterministic scatter puts each output back at its
 * positions; the pages leave open which positions a coarse output covers) */
#define LH_SCATTER_HOLD 0    /* causal hold: token t takes the leader with the
                                largest anchor <= t (0 before the first)    */
#define LH_SCATTER_SPAN 1    /* span broadcast: token t takes the finest
                                selected entry whose span holds t (acausal
                                inside a span, causal across coarsest cells) */

/* lh_dims.sigma_mode: how an entry's two scores combine into the one score
 * the stratified top-K ranks (the pages give two scores per cell and leave
 * their combination open).  Every mode keeps a parent's score at least its
 * children's, since both planes are max-pooled and non-negative. */
#define LH_SIGMA_SUM     0   /* float32(sq + sk), the default reading       */
#define LH_SIGMA_MAX     1   /* max(sq, sk)                                 */
#define LH_SIGMA_PRODUCT 2   /* float32(sq * sk)                            */

/* lh_dims.strata_mode: how a stratum's k_s ranked entries are shared out
 * (the pages stratify the top-K against collapse and also call it joint
 * across levels; which of the two governs the levels is open).  Either way a
 * stratum is one coarsest cell with its subtree and its root is kept. */
#define LH_STRATA_JOINT     0   /* one ranking over levels 0..L-2, the default */
#define LH_STRATA_PER_LEVEL 1   /* a quota per level, ranked within the level:
                                   levels L-2 down to 1 in turn take
                                   min(their entries in the stratum,
                                   remaining / levels left),
                                   level 0 takes the rest (lh_validate
                                   rejects a budget where that would not fit
                                   in level 0; none with k_s <= T-1 was found
                                   for p <= 8, L <= 7)                      */

typedef void *lh_stream;     /* a hipStream_t */

/* Problem statement of one layer call (explainer section 2.A-2.C: sequence
 * length N, pooling factor p, L levels, top-K budget K, subsequence length
 * S).  Constraints checked by lh_validate:
 *   B >= 1, H >= 1, N >= 1, p >= 2, L >= 1,
 *   K >= 0, K % n_c == 0, K / n_c <= T - 1, S == K + n_c,
 *   E < 2^31, d in {64, 128}, io_dtype/out_dtype in {LH_F32, LH_BF16},
 *   out_dtype == LH_F32 when io_dtype == LH_F32, scale >= 0 and finite,
 *   scatter_mode in {LH_SCATTER_HOLD, LH_SCATTER_SPAN},
 *   sigma_mode in {LH_SIGMA_SUM, LH_SIGMA_MAX, LH_SIGMA_PRODUCT},
 *   strata_mode in {LH_STRATA_JOINT, LH_STRATA_PER_LEVEL};
 * and the launch limits of this library (LH_ERR_UNSUPPORTED otherwise):
 *   B*H <= 65535, S < 2^31, T <= 7936 (one stratum's subtree in LDS), a
 *   pyramid plan with B_c / p^g <= 256 / (d/8) rows for some g <= 6,
 *   every grid's work-items along x within 2^32 - 1 (e.g. 64*B*H*S),
 *   and for bf16 I/O: S*d*2 < 2^31 bytes per head (buffer-resource range)
 *   and the forward's and the dQ kernel's LDS (their ring plus one REDUNDANT
 *   bit per key, S/8 bytes) within 160 KiB, i.e. S up to about 490,000 at
 *   d = 128.
 * The geometry (levels, strata, E, n_c, ...) is that of N rounded up to
 * whole coarsest cells of B_c = p^(L-1) tokens: n_c = ceil(N / B_c).  When N
 * is not a multiple of B_c (the pages assume whole cells; the reading taken
 * is zero padding), lh_layer_fwd / lh_layer_bwd extend q, k, v and dO with
 * zero rows to n_c * B_c tokens in their workspace, run the layer on the
 * extended sequence and return the outputs and gradients of the N real
 * tokens; stage calls that take token tensors return LH_ERR_INVALID_ARG. */
typedef struct lh_dims {
  int64_t B;
  int64_t N;
  int32_t H;
  int32_t d;
  int32_t p;
  int32_t L;
  int64_t K;          /* ranked entries (the kept coarsest rows come on top) */
  int64_t S;          /* subsequence rows = K + n_c                          */
  int32_t io_dtype;   /* Q, K, V, dO, pyramid and subsequence rows           */
  int32_t out_dtype;  /* O, OS, dQ, dK, dV                                   */
  float scale;        /* softmax scale; 0 selects 1/sqrt(d)                  */
  int32_t scatter_mode; /* LH_SCATTER_HOLD (0) or LH_SCATTER_SPAN (1)        */
  int32_t sigma_mode;   /* LH_SIGMA_SUM (0), LH_SIGMA_MAX (1), LH_SIGMA_PRODUCT */
  int32_t strata_mode;  /* LH_STRATA_JOINT (0) or LH_STRATA_PER_LEVEL (1)     */
} lh_dims;

/* Buffers the forward fills and the backward reads (all caller-owned).
 *   pq, pk, pv   [B,H,E-N,d] io_dtype  coarse pyramid levels
 *   sq, sk       [B,H,E]     float32   score planes
 *   sel_idx      [B,H,S]     int32     flat index of each subsequence row
 *   sel_anchor   [B,H,S]     int32     last token of the row's span
 *   sel_flags    [B,H,S]     uint8     LH_ROW_* bits
 *   row_of       [B,H,E]     int32     subsequence row of each entry, -1 if
 *                                      unselected
 *   qs, ks, vs   [B,H,S,d]   io_dtype  gathered subsequence
 *   qst, kst, vst                      unused by the layer calls (may be
 *                                      NULL); kept so callers can hold the
 *                                      transposed copies lh_gather writes
 *   os           [B,H,S,d]   float32   subsequence attention output (kept
 *                                      in float32: the backward's
 *                                      rowsum(dOS * OS) needs it unrounded)
 *   lse          [B,H,S]     float32   natural-log softmax denominator of
 *                                      each row's scaled logits            */
typedef struct lh_saved {
  void *pq, *pk, *pv;
  float *sq, *sk;
  int32_t *sel_idx, *sel_anchor;
  uint8_t *sel_flags;
  int32_t *row_of;
  void *qs, *ks, *vs;
  void *qst, *kst, *vst;
  void *os;
  float *lse;
} lh_saved;

/* Derived sizes of one call.  Byte counts cover all B*H heads; token
 * tensors have the caller's N rows, everything else the padded geometry. */
typedef struct lh_sizes {
  int64_t E, n_c, T, k_s, Bc, Sp;
  size_t pyramid_bytes;     /* one of pq/pk/pv        */
  size_t score_bytes;       /* one of sq/sk           */
  size_t row_i32_bytes;     /* sel_idx / sel_anchor   */
  size_t row_u8_bytes;      /* sel_flags              */
  size_t row_of_bytes;      /* row_of                 */
  size_t subseq_bytes;      /* one of qs/ks/vs (and the transposed copies) */
  size_t os_bytes;          /* os (float32)           */
  size_t lse_bytes;         /* lse                    */
  size_t token_io_bytes;    /* one of q/k/v/dO        */
  size_t token_out_bytes;   /* one of o/dq/dk/dv      */
  size_t ws_attn_fwd;       /* workspace of lh_subseq_attn_fwd */
  size_t ws_attn_bwd;       /* workspace of lh_subseq_attn_bwd */
  size_t ws_layer_fwd;      /* workspace of lh_layer_fwd       */
  size_t ws_layer_bwd;      /* workspace of lh_layer_bwd       */
  size_t owner_bytes;       /* span owner map [B,H,N] int32    */
} lh_sizes;

/* Host only (no HIP call).  LH_OK if `dims` satisfies every constraint
 * above, else LH_ERR_INVALID_ARG (malformed) or LH_ERR_UNSUPPORTED. */
lh_status lh_validate(const lh_dims *dims);

/* Host only.  Fills *out for a valid `dims`; errors as lh_validate. */
lh_status lh_get_sizes(const lh_dims *dims, lh_sizes *out);

/* Host only.  Static text of a status code. */
const char *lh_status_string(lh_status s);

/* Library version, "MAJOR.MINOR.PATCH". */
const char *lh_version(void);

/* ---- stage 1: symmetric pyramid (explainer 2.A; news item: Theta(N)) ----
 * pq/pk/pv[b,h, off_l - N + i] = mean of the p children of entry (l-1, .),
 * i.e. the mean of tokens [i p^l, (i+1) p^l), for l = 1..L-1: the block's
 * tokens are summed in float64 (exact for bf16 and float32 inputs), divided
 * by p^l and rounded once to io_dtype.  Q, K and V are pooled alike.
 * In: q, k, v [B,H,N,d] io_dtype.  Out: pq, pk, pv.  Any of the three pairs
 * may be skipped by passing NULL for both its input and output. */
lh_status lh_pyramid_build(const lh_dims *dims, const void *q, const void *k,
                           const void *v, void *pq, void *pk, void *pv,
                           lh_stream stream);

/* ---- stage 2a: parameter-free scores (explainer 2.B; news item: two scalar
 * scores per cell, max-pooled to coarser levels) ----
 * sq[b,h,t] = float32(||q_t||_2) and sk likewise for level-0 rows (squares
 * summed in float64, one rounding); coarse entries take the max of their p
 * children, exactly.  In: q, k [B,H,N,d].  Out: sq, sk [B,H,E] float32. */
lh_status lh_score(const lh_dims *dims, const void *q, const void *k,
                   float *sq, float *sk, lh_stream stream);

/* Stages 1 and 2a in one pass over the inputs (what the layer uses). */
lh_status lh_pyramid_score(const lh_dims *dims, const void *q, const void *k,
                           const void *v, void *pq, void *pk, void *pv,
                           float *sq, float *sk, lh_stream stream);

/* ---- stage 2b: stratified top-K (explainer 2.B: joint selection across
 * levels; news item: stratified against collapse, coarsest level kept) ----
 * Per (b, h) and stratum m (coarsest entry (L-1, m) with its subtree): keep
 * the root and the k_s entries of levels 0..L-2 with the largest
 * sigma = float32(sq + sk), ties to the lower flat index (finer level first,
 * then lower position); with LH_STRATA_PER_LEVEL, level l's quota of them
 * is ranked among level l's entries only (same key).  Rows of stratum m are [m (k_s+1), (m+1)(k_s+1)),
 * ordered by (anchor, level) ascending.  Out:
 *   sel_idx, sel_anchor [B,H,S] int32; sel_flags [B,H,S] uint8 (REDUNDANT:
 *   all p children selected or redundant; LEADER: first row or anchor
 *   differs from the previous row's); row_of [B,H,E] int32 (every entry
 *   written: its row or -1). */
lh_status lh_topk_select(const lh_dims *dims, const float *sq, const float *sk,
                         int32_t *sel_idx, int32_t *sel_anchor,
                         uint8_t *sel_flags, int32_t *row_of, lh_stream stream);

/* ---- stage 3a: gather (explainer 2.C: selected triplets form one dense,
 * causally consistent sequence) ----
 * xs[b,h,j] = row sel_idx[j] of the pyramid of x: q[...] when the flat index
 * is < N, else pq[... flat - N].  Same for k and v.  qst/kst/vst, when not
 * NULL, receive the transposed copies [B,H,d,Sp] with zeroed padding
 * (LH_BF16 only). */
lh_status lh_gather(const lh_dims *dims, const void *q, const void *k,
                    const void *v, const void *pq, const void *pk,
                    const void *pv, const int32_t *sel_idx, void *qs, void *ks,
                    void *vs, void *qst, void *kst, void *vst,
                    lh_stream stream);

/* ---- stage 3b: dense causal attention on the subsequence (explainer 2.C:
 * ordinary SDPA on the dense subsequence) ----
 * os[j] = sum_{j'} softmax_j'(scale <qs_j, ks_j'>) vs_j' over the keys
 * j' <= j whose row is not REDUNDANT; lse[j] = log of that softmax's
 * denominator (natural log, scaled logits).  os is float32 [B,H,S,d].
 * bf16 I/O runs on MFMA with float32 accumulation; f32 I/O runs on the
 * vector ALUs with float64 sums.
 * Workspace: sizes.ws_attn_fwd bytes (0: ws may be NULL). */
lh_status lh_subseq_attn_fwd(const lh_dims *dims, const void *qs,
                             const void *ks, const void *vs,
                             const uint8_t *sel_flags, void *os, float *lse,
                             void *ws, size_t ws_bytes, lh_stream stream);

/* ---- stage 3b backward: standard SDPA backward on the same mask ----
 * In: qs, ks, vs, os (float32), lse, sel_flags, dos [B,H,S,d] float32.
 * Out: dqs, dks, dvs [B,H,S,d] float32.  Workspace: sizes.ws_attn_bwd. */
lh_status lh_subseq_attn_bwd(const lh_dims *dims, const void *qs,
                             const void *ks, const void *vs, const void *os,
                             const float *lse, const uint8_t *sel_flags,
                             const float *dos, float *dqs, float *dks,
                             float *dvs, void *ws, size_t ws_bytes,
                             lh_stream stream);

/* ---- stage 3b backward without a workspace argument ----
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The same
 * operation, arguments and kernels as lh_subseq_attn_bwd, but the scratch
 * it needs (the dO split and drow, sizes.ws_attn_bwd bytes) lives in a
 * fixed device array inside the library, LH_NOALLOC_SCRATCH_BYTES per
 * device, held from the library's first use on a device until the process
 * ends.  Nothing is allocated or freed by the call.  Every call on one
 * device shares that device's array (no part of it needs to start at zero:
 * each call overwrites what it reads), so calls that overlap in time on one
 * device race and must be ordered by the caller (e.g. one stream).
 * Errors: as lh_subseq_attn_bwd, and LH_ERR_UNSUPPORTED when
 * sizes.ws_attn_bwd exceeds LH_NOALLOC_SCRATCH_BYTES (nothing launched). */
#define LH_NOALLOC_SCRATCH_BYTES (80u << 20)
lh_status lh_subseq_attn_bwd_noalloc(const lh_dims *dims, const void *qs,
                                     const void *ks, const void *vs,
                                     const void *os, const float *lse,
                                     const uint8_t *sel_flags, const float *dos,
                                     float *dqs, float *dks, float *dvs,
                                     lh_stream stream);

/* ---- stage 3b, operand-prepared forms: each of the three MFMA calls
 * launches exactly one kernel (LH_BF16 I/O only; LH_ERR_UNSUPPORTED
 * otherwise).  They take the operand layouts the kernels read directly, for
 * callers that keep those buffers themselves, and for per-kernel timing.
 *   dos_hi, dos_lo        [B,H,S,d]  bf16 two-term split of dOS (hi + lo)
 *   drow                  [B,H,S]    float32 rowsum(dOS * OS)
 * lh_attn_bwd_prep:     dos (float32 [B,H,S,d]) and os (float32) -> dos_hi,
 *                       dos_lo, drow
 * lh_attn_fwd_mfma:     qs, ks, vs rows -> os [B,H,S,d] float32, lse [B,H,S]
 *                       (as lh_subseq_attn_fwd)
 * lh_attn_bwd_dkv_mfma: dks, dvs [B,H,S,d] float32
 * lh_attn_bwd_dq_mfma:  dqs [B,H,S,d] float32 */
lh_status lh_attn_bwd_prep(const lh_dims *dims, const float *dos, const float *os,
                           void *dos_hi, void *dos_lo, float *drow, lh_stream stream);
lh_status lh_attn_fwd_mfma(const lh_dims *dims, const void *qs, const void *ks,
                           const void *vs, const uint8_t *sel_flags, float *os,
                           float *lse, lh_stream stream);
lh_status lh_attn_bwd_dkv_mfma(const lh_dims *dims, const void *qs, const void *ks,
                               const void *vs, const void *dos_hi, const void *dos_lo,
                               const float *lse, const float *drow,
                               const uint8_t *sel_flags, float *dks, float *dvs,
                               lh_stream stream);
lh_status lh_attn_bwd_dq_mfma(const lh_dims *dims, const void *qs, const void *ks,
                              const void *vs, const void *dos_hi, const void *dos_lo,
                              const float *lse, const float *drow,
                              const uint8_t *sel_flags, float *dqs, lh_stream stream);

/* ---- stage 4: scatter-back (explainer 2.C: a deterministic kernel puts the
 * outputs back at their positions) ----
 * Causal hold: token t takes os[j] of the LEADER row j with the largest
 * anchor <= t; tokens before the first anchor get 0.  Every token has one
 * source (no atomics).  In: os [B,H,S,d] float32.  Out: o [B,H,N,d]
 * out_dtype (one rounding when out_dtype is LH_BF16). */
lh_status lh_scatter(const lh_dims *dims, const void *os,
                     const int32_t *sel_anchor, const uint8_t *sel_flags,
                     void *o, lh_stream stream);

/* Adjoint of lh_scatter: dos[j] = sum of dout[t] over the tokens whose
 * source is row j, in token order, float32; 0 for non-leader rows.
 * In: dout [B,H,N,d] out_dtype.  Out: dos [B,H,S,d] float32. */
lh_status lh_scatter_bwd(const lh_dims *dims, const void *dout,
                         const int32_t *sel_anchor, const uint8_t *sel_flags,
                         float *dos, lh_stream stream);

/* ---- stage 4, span broadcast (lh_dims.scatter_mode == LH_SCATTER_SPAN) ----
 * lh_span_owner: owner[b,h,t] = the row of the finest selected entry whose
 * span holds token t, from row_of [B,H,E]; out: owner [B,H,N] int32.
 * lh_scatter_span: o[t] = os[owner[t]]; os [B,H,S,d] float32, o [B,H,N,d]
 * out_dtype.
 * lh_scatter_span_bwd: adjoint: dos[j] = sum of dout[t] over the tokens t
 * of row j's span with owner[t] == j, in token order (zero for REDUNDANT
 * rows, which own nothing); dout [B,H,N,d] out_dtype, sel_idx and
 * sel_flags as the selection wrote them; out: dos [B,H,S,d] float32.
 * These three ignore dims->scatter_mode. */
lh_status lh_span_owner(const lh_dims *dims, const int32_t *row_of, int32_t *owner,
                        lh_stream stream);
lh_status lh_scatter_span(const lh_dims *dims, const float *os, const int32_t *owner,
                          void *o, lh_stream stream);
lh_status lh_scatter_span_bwd(const lh_dims *dims, const void *dout,
                              const int32_t *sel_idx, const uint8_t *sel_flags,
                              const int32_t *owner, float *dos, lh_stream stream);

/* Adjoint of gather and pooling (explainer 2.B: gradients reach W_Q, W_K,
 * W_V through gather, attention and scatter only; the selection carries
 * none):  dx[t] = sum_l dxs[row_of(l, t / p^l)] / p^l over the selected
 * ancestors of t, in level order.  In: dqs, dks, dvs [B,H,S,d] float32,
 * row_of.  Out: dq, dk, dv [B,H,N,d] out_dtype. */
lh_status lh_gather_bwd(const lh_dims *dims, const float *dqs,
                        const float *dks, const float *dvs,
                        const int32_t *row_of, void *dq, void *dk, void *dv,
                        lh_stream stream);

/* ---- whole layer ----
 * Forward: pyramid+score, select, gather, attention,
 * scatter (causal hold, or span broadcast per dims->scatter_mode).  Fills
 * every buffer of *saved and o [B,H,N,d] out_dtype.
 * Workspace: sizes.ws_layer_fwd bytes (may be 0 / NULL when that is 0; the
 * span owner map in span mode, the zero-padded q, k, v and o when N is not
 * whole coarsest cells). */
lh_status lh_layer_fwd(const lh_dims *dims, const void *q, const void *k,
                       const void *v, void *o, const lh_saved *saved,
                       void *ws, size_t ws_bytes, lh_stream stream);

/* Backward from the buffers a forward filled: scatter adjoint, attention
 * backward, gather and pooling adjoints.  dout [B,H,N,d] out_dtype;
 * out: dq, dk, dv [B,H,N,d] out_dtype.  Workspace: sizes.ws_layer_bwd. */
lh_status lh_layer_bwd(const lh_dims *dims, const lh_saved *saved,
                       const void *dout, void *dq, void *dk, void *dv,
                       void *ws, size_t ws_bytes, lh_stream stream);

/* ---- measurement helper (not part of the layer) ----
 * Runs `blocks` workgroups of 256 threads, each wavefront issuing `iters`
 * rounds of 8 independent v_mfma_f32_32x32x16_bf16 (the MFMA the attention
 * kernels use), so one launch performs blocks * 4 * 8 * iters * 32768 flops
 * with no memory traffic.  Timing a launch gives the bf16 MFMA rate the
 * device sustains, the achievable ceiling beside the published peak.
 * out: device float32 [blocks * 256], caller-owned, overwritten with a
 * checksum.  Errors: LH_ERR_INVALID_ARG for blocks outside 1 .. 2^24-1
 * (the launch's work-items must fit 32 bits), iters <= 0 or a NULL out
 * (nothing launched); LH_ERR_HIP after a failed launch.  Asynchronous on
 * `stream`. */
lh_status lh_probe_mfma_bf16(int64_t blocks, int32_t iters, float *out,
                             lh_stream stream);

/* ---- measurement helper (not part of the layer) ----
 * Streams `bytes` bytes through HBM with 16-byte accesses, four in flight
 * per lane, over `blocks` workgroups of 256 threads (grid-stride), so that
 * timing a launch gives the bandwidth this device sustains for the kind of
 * traffic the memory-bound stages make:
 *   mode 0: copy src -> dst (reads and writes `bytes` each);
 *   mode 1: read src only; dst receives one uint32 checksum per thread
 *           (blocks * 256 * 4 bytes);
 *   mode 2: write dst only (a fixed pattern).
 * Pointers are device pointers, 16-byte aligned, caller-owned; bytes must be
 * a positive multiple of 16.  Errors: LH_ERR_INVALID_ARG for a bad mode,
 * size, pointer or blocks outside 1 .. 2^24-1 (nothing launched);
 * LH_ERR_HIP after a failed launch.  Asynchronous on `stream`. */
lh_status lh_probe_stream(int32_t mode, const void *src, void *dst, size_t bytes,
                          int64_t blocks, lh_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTHOUSE_H */
