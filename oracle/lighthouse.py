"""CPU oracle for the Lighthouse Attention layer -- TEST INFRASTRUCTURE ONLY.

This module is the plain, slow, obviously-correct statement of what the layer
computes, in NumPy float64.  It exists to check the HIP path.  Only the test
suite, the package's smoke check and the benchmark's CPU-baseline leg may
import it; the product path never does, and this module imports nothing from
the product package (they share no code).

Sources (cited by short tag below):
  [EXP-2A] "Long Context Pre-Training with Lighthouse Attention" -- gist.science
           explainer (zh and ko editions), technical summary, section 2.A
           (symmetric pyramid).
  [EXP-2B] same page, section 2.B (parameter-free scoring and selection; no
           gradient through the selection).
  [EXP-2C] same page, section 2.C (gather into a dense, causally consistent
           subsequence; standard SDPA on it; deterministic scatter-back).
  [NEWS]   edge.aivizor.me news item on the same paper, the paragraph that
           lists the four stages (Theta(N) pyramid, two scalar scores per
           cell, max-pool inheritance, stratified top-K keeping the coarsest
           level, indices carry no gradient) and the paragraph after it
           (coarsest level kept to cover every position; stratification
           against selection collapse).

Where the pages leave a step open, the reading taken is stated at the step
(tag R-n); every reading is listed in the design notes of the repository.

Notation (one batch element b, one head h):
  N tokens, head dim d, pooling factor p, L levels (l = 0..L-1),
  N_l = N / p**l entries at level l, E = sum_l N_l.
  flat index f(l, i) = off_l + i with off_l = sum_{m<l} N_m (finest first,
  so level 0 uses the input's own row numbers).
  Entry (l, i) spans tokens [i*p**l, (i+1)*p**l - 1]; its anchor is the span's
  last token a(l, i) = (i+1)*p**l - 1.
  Coarsest span B_c = p**(L-1); n_c = N / B_c strata; subtree size
  T = (p**L - 1)/(p - 1); per-stratum ranked quota k_s = K / n_c;
  subsequence length S = K + n_c.

Parity pins for every function live in tests/test_oracle_*.py.  Conventions
R-5, R-7, R-7', R-9, R-11, R-12, R-14 and R-14' are readings of open points: they are
pinned by invariants and special cases, not by a value the pages print
("parity unpinned" by the pages themselves).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# sel_flags bits (same meaning as the C header's, restated independently)
FLAG_REDUNDANT = 1
FLAG_LEADER = 2


# --------------------------------------------------------------------------
# shapes
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Geometry:
    N: int
    p: int
    L: int
    K: int

    @property
    def level_sizes(self):
        return [self.N // self.p ** l for l in range(self.L)]

    @property
    def level_offsets(self):
        offs, o = [], 0
        for n in self.level_sizes:
            offs.append(o)
            o += n
        return offs

    @property
    def E(self):
        return sum(self.level_sizes)

    @property
    def Bc(self):
        return self.p ** (self.L - 1)

    @property
    def n_c(self):
        return self.N // self.Bc

    @property
    def T(self):
        return sum(self.p ** l for l in range(self.L))

    @property
    def k_s(self):
        return self.K // self.n_c

    @property
    def S(self):
        return self.K + self.n_c

    def check(self):
        """R-1: levels l = 0..L-1 with level 0 counted; N must be a multiple
        of p**(L-1); K a multiple of n_c with k_s <= T-1 (R-8)."""
        if self.p < 2 or self.L < 1 or self.N < 1:
            raise ValueError("need p >= 2, L >= 1, N >= 1")
        if self.N % self.Bc:
            raise ValueError("N must be a multiple of p**(L-1)")
        if self.K < 0 or self.K % self.n_c:
            raise ValueError("K must be a non-negative multiple of N/p**(L-1)")
        if self.k_s > self.T - 1:
            raise ValueError("K/n_c must not exceed the T-1 candidates of a stratum")
        return self


def level_of_flat(g: Geometry, f):
    f = np.asarray(f)
    lev = np.zeros(f.shape, dtype=np.int64)
    for l, o in enumerate(g.level_offsets):
        lev[f >= o] = l
    return lev


def entry_of_flat(g: Geometry, f):
    """(level, index-in-level) of flat indices."""
    f = np.asarray(f, dtype=np.int64)
    lev = level_of_flat(g, f)
    offs = np.asarray(g.level_offsets, dtype=np.int64)
    return lev, f - offs[lev]


def anchor_of(g: Geometry, lev, idx):
    """Last token of the span of entry (l, i)."""
    lev = np.asarray(lev, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    return (idx + 1) * (g.p ** lev) - 1


# --------------------------------------------------------------------------
# rounding of stored intermediates to bfloat16 (R-2)
# --------------------------------------------------------------------------
def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value (ties to even),
    returned as float64.  bfloat16 keeps 8 significant bits (7 stored plus
    the implicit one) and float32's exponent range; only normal values
    arise in this use (means of normal values), so the mantissa is rounded
    at 8 bits with round-half-even and the exponent kept."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                        # x = m * 2**e, 0.5 <= |m| < 1
    r = np.round(m * 256.0) / 256.0           # numpy rounds halves to even
    return np.ldexp(r, e)


# --------------------------------------------------------------------------
# O1  pyramid  [EXP-2A], [NEWS]
# --------------------------------------------------------------------------
def pyramid(X, g: Geometry, store: str | None = None):
    """Levels 0..L-1 of one head's [N, d] tensor.

    Level 0 is X itself; level l averages p consecutive entries of level l-1
    (non-overlapping, stride p) [EXP-2A].  The same pooling applies to Q, K
    and V alike (the pyramid is symmetric).  The recursion is exact in
    float64.

    R-2: the pooled levels are tensors of the layer's I/O dtype.  With
    store='bf16' (or 'f32') each coarse level is rounded once, from the
    exact mean, to bfloat16 (float32); the rounding does not feed the next
    level's mean.  The exact mean of a level-l entry is the mean of the p^l
    tokens it covers (the recursion unrolled); it is formed here as that
    block's float64 sum divided by p^l.  For bf16 or float32 inputs the
    sum is exact (unless one block's magnitudes span some thirty binades or
    more) and the division rounds at most once, and not at all when the
    mean is representable, as every bf16 rounding tie is.  The recursive
    float64 means above carry a rounding per level when p is not a power
    of two, which can move a tie by one float64 step and flip its rounding.
    """
    X = np.asarray(X, dtype=np.float64)
    levels = [X]
    for _ in range(1, g.L):
        prev = levels[-1]
        levels.append(prev.reshape(prev.shape[0] // g.p, g.p, -1).mean(axis=1))
    if store is None:
        return levels
    if store not in ("bf16", "f32"):
        raise ValueError(store)
    out = [X]
    for l in range(1, g.L):
        w = g.p ** l
        exact = X.reshape(X.shape[0] // w, w, -1).sum(axis=1) / w
        out.append(round_bf16(exact) if store == "bf16"
                   else exact.astype(np.float32).astype(np.float64))
    return out


def flat_rows(levels):
    """Concatenate levels finest-first: row f of the result is entry f."""
    return np.concatenate(levels, axis=0)


# --------------------------------------------------------------------------
# O2  scores  [EXP-2B], [NEWS]
# --------------------------------------------------------------------------
def scores(Q, K_, g: Geometry):
    """Two score planes sQ, sK over all E entries (float32 values).

    Level 0: the l2 norm of each projected q (resp. k) row, so every cell
    carries two scalar scores [NEWS]; computed in float64 and rounded once
    to float32 (R-3: norms of the level-0 inputs, not of pooled rows).
    Level l >= 1: max over its p children (coarse spans keep their strongest
    token's score [EXP-2B]).  Max is exact, so parent == max(children).
    """
    planes = []
    for X in (Q, K_):
        X = np.asarray(X, dtype=np.float64)
        s0 = np.sqrt(np.sum(X * X, axis=1)).astype(np.float32)
        lev = [s0]
        for _ in range(1, g.L):
            lev.append(lev[-1].reshape(-1, g.p).max(axis=1))
        planes.append(np.concatenate(lev))
    return planes[0], planes[1]


SIGMA_MODES = ("sum", "max", "product")


def sigma(sQ, sK, mode="sum"):
    """R-5 (the pages are silent on how the two scores combine): one ranking
    score per entry, sigma = float32(sQ + sK), added in float32.  The other
    combinations, kept as options: the larger of the two, and their product
    rounded once to float32.  Each keeps a parent's score at least its
    children's (both planes are max-pooled and non-negative)."""
    sQ = np.asarray(sQ, dtype=np.float32)
    sK = np.asarray(sK, dtype=np.float32)
    if mode == "sum":
        return (sQ + sK).astype(np.float32)
    if mode == "max":
        return np.maximum(sQ, sK).astype(np.float32)
    if mode == "product":
        return (sQ * sK).astype(np.float32)
    raise ValueError(mode)


# --------------------------------------------------------------------------
# O3-O5  stratified top-K, order, redundancy, leaders  [EXP-2B], [EXP-2C], [NEWS]
# --------------------------------------------------------------------------
@dataclass
class Selection:
    sel_idx: np.ndarray      # [S] int64 flat index of row j
    sel_anchor: np.ndarray   # [S] int64 anchor (span end) of row j
    sel_level: np.ndarray    # [S] int64 level of row j
    sel_flags: np.ndarray    # [S] uint8 (bit0 REDUNDANT, bit1 LEADER)
    row_of: np.ndarray       # [E] int64, -1 if unselected
    near_tie: np.ndarray = field(default=None)  # [n_c] bool, per stratum


def stratum_members(g: Geometry, m: int):
    """Flat indices of stratum m: the coarsest entry (L-1, m) and its whole
    subtree (R-7: strata are the coarsest-level cells)."""
    out = []
    for l, o in enumerate(g.level_offsets):
        per = g.Bc // g.p ** l
        out.append(o + m * per + np.arange(per))
    return np.concatenate(out)


def level_quotas(g: Geometry):
    """R-7' (the per-level reading of "stratified", an ablation of R-7): the
    k_s ranked entries of a stratum are shared out as quotas over levels
    0..L-2.  Going from the coarsest ranked level L-2 down to level 1, each
    level takes an equal share of what is left, floor(left / levels left),
    but no more than the p**(L-1-l) entries it has in the stratum; level 0
    takes the remainder, which must fit in its B_c entries.  Returns the
    list of quotas indexed by level (length L-1)."""
    q = [0] * max(g.L - 1, 0)
    left = g.k_s
    for l in range(g.L - 2, 0, -1):
        have = g.Bc // g.p ** l
        q[l] = min(have, left // (l + 1))
        left -= q[l]
    if g.L >= 2:
        if left > g.Bc:
            raise ValueError("per-level quotas: level 0 cannot hold the remainder")
        q[0] = left
    return q


def select(sig, g: Geometry, near_tie_rel: float = 1e-6, strata="joint"):
    """Stratified joint top-K with the coarsest level always kept.

    [EXP-2B]: a top-K chosen jointly across all levels.  [NEWS]: the top-K is
    stratified so the selection cannot collapse onto a narrow range, and
    the coarsest level is always kept so every position is covered.

    R-7: stratum m is coarsest cell m with its subtree; its root is always
         kept and k_s = K/n_c further entries are ranked jointly across the
         stratum's levels 0..L-2.
    R-8: S = K + n_c rows (the kept coarsest rows come on top of K).
    R-9: ranking key (-sigma, f) ascending: larger sigma first; on equal
         sigma the lower flat index, i.e. the finer level, then the lower
         position.
    R-11: within a stratum the rows are ordered by (anchor, level)
         ascending -- a child precedes its parent (topological) and a row
         precedes every row whose span ends later (causal) [EXP-2C].
         Strata follow each other in order, stratum m owning rows
         [m*(k_s+1), (m+1)*(k_s+1)).
    R-12 / O5: entry (l, i), l >= 1, is REDUNDANT when each of its p
         children is selected or itself redundant, i.e. every token of its
         span is covered by selected strictly finer entries.
    LEADER: row j is a leader when j == 0 or its anchor differs from row
         j-1's -- the finest row at its anchor.
    near_tie (R-10): the last selected and first unselected candidate of a
         stratum differ by at most near_tie_rel * (largest sigma of the
         stratum); index mismatches are only excusable in such strata.
    strata: "joint" (R-7) or "per_level" (R-7', level_quotas): the same key
         ranks each level's entries of the stratum for that level's quota.
    """
    g.check()
    sig = np.asarray(sig, dtype=np.float32)
    k_s = g.k_s
    E = g.E
    sel_mask = np.zeros(E, dtype=bool)
    near = np.zeros(g.n_c, dtype=bool)
    root0 = g.level_offsets[-1]
    if strata not in ("joint", "per_level"):
        raise ValueError(f"strata {strata!r}")
    quotas = level_quotas(g) if strata == "per_level" else None
    for m in range(g.n_c):
        members = stratum_members(g, m)
        root = root0 + m
        sel_mask[root] = True
        smax = float(sig[members].max())
        if quotas is None:
            groups = [(members[members != root], k_s)]
        else:
            groups = []
            for l in range(g.L - 1):
                per = g.Bc // g.p ** l
                groups.append((g.level_offsets[l] + m * per + np.arange(per), quotas[l]))
        for cand, k in groups:
            # ranking: sigma descending, then flat index ascending
            order = np.lexsort((cand, -sig[cand].astype(np.float64)))
            sel_mask[cand[order[:k]]] = True
            if 0 < k < len(cand):
                s_last = float(sig[cand[order[k - 1]]])
                s_next = float(sig[cand[order[k]]])
                near[m] |= (s_last - s_next) <= near_tie_rel * smax

    # redundancy, bottom-up over levels
    sizes, offs = g.level_sizes, g.level_offsets
    red = np.zeros(E, dtype=bool)
    for l in range(1, g.L):
        o_c, o_p = offs[l - 1], offs[l]
        child_cov = sel_mask[o_c:o_c + sizes[l - 1]] | red[o_c:o_c + sizes[l - 1]]
        red[o_p:o_p + sizes[l]] = child_cov.reshape(-1, g.p).all(axis=1)

    # rows: strata in order, each ordered by (anchor, level)
    rows = []
    for m in range(g.n_c):
        members = stratum_members(g, m)
        chosen = members[sel_mask[members]]
        lev, idx = entry_of_flat(g, chosen)
        anc = anchor_of(g, lev, idx)
        o = np.lexsort((lev, anc))
        rows.append(chosen[o])
    sel_idx = np.concatenate(rows).astype(np.int64)
    lev, idx = entry_of_flat(g, sel_idx)
    anc = anchor_of(g, lev, idx)
    flags = np.zeros(len(sel_idx), dtype=np.uint8)
    flags[red[sel_idx]] |= FLAG_REDUNDANT
    lead = np.ones(len(sel_idx), dtype=bool)
    lead[1:] = anc[1:] != anc[:-1]
    flags[lead] |= FLAG_LEADER
    row_of = -np.ones(E, dtype=np.int64)
    row_of[sel_idx] = np.arange(len(sel_idx))
    return Selection(sel_idx, anc, lev, flags, row_of, near)


# --------------------------------------------------------------------------
# O6  gather  [EXP-2C]
# --------------------------------------------------------------------------
def gather(levels, sel_idx):
    """Row j of the subsequence is pyramid entry sel_idx[j]."""
    return flat_rows(levels)[np.asarray(sel_idx, dtype=np.int64)]


# --------------------------------------------------------------------------
# O7  subsequence attention  [EXP-2C]
# --------------------------------------------------------------------------
def attention_fwd(QS, KS, VS, flags, scale, row_block=2048):
    """Standard scaled-dot-product attention on the subsequence.  Query j
    sees key j' when j' <= j and row j' is not REDUNDANT (R-12; R-11 makes
    index order the span-causal order).  R-13: scale 1/sqrt(d) by default,
    no other bias.
    Returns OS [S, d] and LSE [S] (natural log of the softmax denominator of
    the scaled logits).  Rows are processed in chunks only to bound memory;
    each row's softmax is taken over its whole key set at once."""
    QS = np.asarray(QS, np.float64)
    KS = np.asarray(KS, np.float64)
    VS = np.asarray(VS, np.float64)
    S = QS.shape[0]
    red = (np.asarray(flags) & FLAG_REDUNDANT) != 0
    OS = np.empty((S, VS.shape[1]))
    LSE = np.empty(S)
    keys = np.arange(S)
    for r0 in range(0, S, row_block):
        r1 = min(S, r0 + row_block)
        s = scale * (QS[r0:r1] @ KS.T)
        ok = (keys[None, :] <= np.arange(r0, r1)[:, None]) & (~red)[None, :]
        s = np.where(ok, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        z = e.sum(axis=1, keepdims=True)
        OS[r0:r1] = (e / z) @ VS
        LSE[r0:r1] = (mx + np.log(z))[:, 0]
    return OS, LSE


def attention_bwd(QS, KS, VS, flags, scale, dOS, row_block=2048):
    """Standard SDPA backward on the same mask.  With P the softmax weights:
    dVS = P^T dOS; dP = dOS VS^T; Drow = rowsum(P * dP) = rowsum(dOS * OS);
    dS = P * (dP - Drow); dQS = scale dS KS; dKS = scale dS^T QS."""
    QS = np.asarray(QS, np.float64)
    KS = np.asarray(KS, np.float64)
    VS = np.asarray(VS, np.float64)
    dOS = np.asarray(dOS, np.float64)
    S = QS.shape[0]
    red = (np.asarray(flags) & FLAG_REDUNDANT) != 0
    dQS = np.zeros_like(QS)
    dKS = np.zeros_like(KS)
    dVS = np.zeros_like(VS)
    keys = np.arange(S)
    for r0 in range(0, S, row_block):
        r1 = min(S, r0 + row_block)
        s = scale * (QS[r0:r1] @ KS.T)
        ok = (keys[None, :] <= np.arange(r0, r1)[:, None]) & (~red)[None, :]
        s = np.where(ok, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        P = e / e.sum(axis=1, keepdims=True)
        dP = dOS[r0:r1] @ VS.T
        Drow = np.sum(P * dP, axis=1, keepdims=True)
        dS = P * (dP - Drow)
        dVS += P.T @ dOS[r0:r1]
        dQS[r0:r1] = scale * (dS @ KS)
        dKS += scale * (dS.T @ QS[r0:r1])
    return dQS, dKS, dVS


# --------------------------------------------------------------------------
# O8, O9  scatter-back and its adjoint  [EXP-2C]
# --------------------------------------------------------------------------
def hold_source(sel: Selection, N: int):
    """R-14 (causal hold): for each token t the subsequence row whose output
    lands on t -- the leader with the largest anchor <= t; -1 before the
    first anchor.  Each token has exactly one source (the scatter is a
    deterministic, atomic-free copy)."""
    lead = np.nonzero(sel.sel_flags & FLAG_LEADER)[0]
    anc = sel.sel_anchor[lead]
    pos = np.searchsorted(anc, np.arange(N), side="right") - 1
    src = np.where(pos >= 0, lead[np.maximum(pos, 0)], -1)
    return src


def scatter(OS, sel: Selection, N: int):
    """O[t] = OS[hold_source(t)], zero where there is no source."""
    OS = np.asarray(OS, np.float64)
    src = hold_source(sel, N)
    O = np.zeros((N, OS.shape[1]))
    ok = src >= 0
    O[ok] = OS[src[ok]]
    return O


def scatter_adjoint(dO, sel: Selection, N: int):
    """dOS[j] = sum of dO[t] over the tokens t whose source is row j (the
    leader's hold segment), in token order; zero for non-leaders."""
    dO = np.asarray(dO, np.float64)
    S = len(sel.sel_idx)
    dOS = np.zeros((S, dO.shape[1]))
    lead = np.nonzero(sel.sel_flags & FLAG_LEADER)[0]
    starts = sel.sel_anchor[lead]
    ends = np.append(starts[1:], N)          # hold segment [a_j, a_next)
    for j, t0, t1 in zip(lead, starts, ends):
        dOS[j] = dO[t0:t1].sum(axis=0)
    return dOS


# --------------------------------------------------------------------------
# O8'  span-broadcast scatter: the other reading of [EXP-2C]'s scatter-back,
#      where an output is put back over the whole span of its entry
# --------------------------------------------------------------------------
def span_owner(sel: Selection, g: Geometry):
    """R-14' (span broadcast): for each token t the row of the finest
    selected entry whose span [i*p**l, (i+1)*p**l) contains t.  The stratum
    root is always selected, so every token has one; a REDUNDANT entry never
    owns a token, since finer selected entries cover its whole span.  Inside
    a span this is acausal (a token sees the summary of later tokens), which
    is the pages' own caveat about decoding; across coarsest cells it is
    causal."""
    t = np.arange(g.N)
    own = np.full(g.N, -1)
    for l in range(g.L - 1, -1, -1):          # coarse to fine: finer entries win
        r = sel.row_of[g.level_offsets[l] + t // g.p ** l]
        own = np.where(r >= 0, r, own)
    return own


def scatter_span(OS, sel: Selection, g: Geometry):
    """O[t] = OS[span_owner(t)]."""
    OS = np.asarray(OS, np.float64)
    return OS[span_owner(sel, g)]


def scatter_span_adjoint(dO, sel: Selection, g: Geometry):
    """dOS[j] = sum of dO[t] over the tokens t that row j owns, in token
    order; zero for rows that own no token."""
    dO = np.asarray(dO, np.float64)
    dOS = np.zeros((len(sel.sel_idx), dO.shape[1]))
    own = span_owner(sel, g)
    for t in range(g.N):
        dOS[own[t]] += dO[t]
    return dOS


# --------------------------------------------------------------------------
# O11, O12  gather adjoint and pooling adjoint
# --------------------------------------------------------------------------
def gather_adjoint(dXS, sel: Selection, g: Geometry):
    """Per level: dX^(l)_i = dXS[row_of(l, i)] if entry (l, i) is selected,
    else zero."""
    dXS = np.asarray(dXS, np.float64)
    out = []
    for l, o in enumerate(g.level_offsets):
        n = g.level_sizes[l]
        r = sel.row_of[o:o + n]
        dl = np.zeros((n, dXS.shape[1]))
        dl[r >= 0] = dXS[r[r >= 0]]
        out.append(dl)
    return out


def pool_adjoint(dlevels, g: Geometry):
    """dX_t = sum_l dX^(l)_{floor(t / p**l)} / p**l (each level-l entry is the
    mean of its p**l tokens)."""
    d = dlevels[0].shape[1]
    dX = np.zeros((g.N, d))
    for l, dl in enumerate(dlevels):
        dX += np.repeat(dl, g.p ** l, axis=0) / float(g.p ** l)
    return dX


# --------------------------------------------------------------------------
# whole layer, one head, forward and backward
# --------------------------------------------------------------------------
@dataclass
class HeadForward:
    g: Geometry
    scale: float
    sQ: np.ndarray
    sK: np.ndarray
    sig: np.ndarray
    sel: Selection
    Ql: list
    Kl: list
    Vl: list
    QS: np.ndarray
    KS: np.ndarray
    VS: np.ndarray
    OS: np.ndarray
    LSE: np.ndarray
    O: np.ndarray
    scatter_mode: str = "hold"


def head_forward(Q, K_, V, g: Geometry, scale=None, store=None, selection=None,
                 scatter_mode="hold", sigma_mode="sum", strata_mode="joint"):
    """One head of the layer: pyramid -> scores -> selection -> gather ->
    attention -> scatter.  `selection` (a Selection) replaces the computed
    one, so downstream stages can be checked on a given selection.
    scatter_mode: "hold" (R-14, causal hold) or "span" (R-14', span
    broadcast).  sigma_mode: how the two scores combine (R-5).  strata_mode:
    "joint" (R-7) or "per_level" (R-7')."""
    g.check()
    d = np.asarray(Q).shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    sQ, sK = scores(Q, K_, g)
    sig = sigma(sQ, sK, sigma_mode)
    sel = select(sig, g, strata=strata_mode) if selection is None else selection
    Ql, Kl, Vl = (pyramid(X, g, store) for X in (Q, K_, V))
    QS, KS, VS = gather(Ql, sel.sel_idx), gather(Kl, sel.sel_idx), gather(Vl, sel.sel_idx)
    OS, LSE = attention_fwd(QS, KS, VS, sel.sel_flags, scale)
    if scatter_mode == "hold":
        O = scatter(OS, sel, g.N)
    elif scatter_mode == "span":
        O = scatter_span(OS, sel, g)
    else:
        raise ValueError(f"scatter_mode {scatter_mode!r}")
    return HeadForward(g, scale, sQ, sK, sig, sel, Ql, Kl, Vl, QS, KS, VS, OS, LSE, O,
                       scatter_mode)


def head_backward(fw: HeadForward, dO):
    """Gradients of one head with respect to Q, K, V: scatter adjoint ->
    attention backward -> gather adjoint -> pooling adjoint.  Nothing flows
    through the scores or the selection [EXP-2B], [NEWS]."""
    g = fw.g
    if fw.scatter_mode == "span":
        dOS = scatter_span_adjoint(dO, fw.sel, g)
    else:
        dOS = scatter_adjoint(dO, fw.sel, g.N)
    dQS, dKS, dVS = attention_bwd(fw.QS, fw.KS, fw.VS, fw.sel.sel_flags, fw.scale, dOS)
    out = []
    for dXS in (dQS, dKS, dVS):
        out.append(pool_adjoint(gather_adjoint(dXS, fw.sel, g), g))
    return tuple(out) + (dOS, dQS, dKS, dVS)


# --------------------------------------------------------------------------
# R-19  lengths that are not a multiple of the coarsest span
# --------------------------------------------------------------------------
def padded_length(N, p, L):
    """R-19 (the pages assume whole coarsest cells): a length N that is not
    a multiple of B_c = p**(L-1) is extended to the next multiple."""
    Bc = p ** (L - 1)
    return -(-N // Bc) * Bc


def _pad_rows(X, n):
    X = np.asarray(X, dtype=np.float64)
    return np.concatenate([X, np.zeros((n - X.shape[0], X.shape[1]))])


def ragged_forward(Q, K_, V, p, L, K, **kw):
    """R-19: one head on a sequence of any length N.  The sequence is
    extended with zero rows (q = k = v = 0) to the next multiple of B_c,
    the layer runs on the extended sequence (K counts ranked entries of the
    extended geometry), and the outputs of the N real tokens are kept.
    Causality keeps the real tokens' outputs free of the padding except
    through the last stratum's selection.  Returns (HeadForward of the
    extended sequence, O of the real tokens)."""
    N = np.asarray(Q).shape[0]
    Np = padded_length(N, p, L)
    g = Geometry(Np, p, L, K).check()
    fw = head_forward(_pad_rows(Q, Np), _pad_rows(K_, Np), _pad_rows(V, Np), g, **kw)
    return fw, fw.O[:N]


def ragged_backward(fw: HeadForward, dO):
    """R-19: gradients of the real tokens: dO extended with zero rows."""
    N = np.asarray(dO).shape[0]
    dQ, dK, dV = head_backward(fw, _pad_rows(dO, fw.g.N))[:3]
    return dQ[:N], dK[:N], dV[:N]
