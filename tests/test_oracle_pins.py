"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a closed
form, a brute-force restatement, a library routine (torch SDPA, torch's
bfloat16 conversion, autograd), an invariant, or the hand-worked fixture in
tests/golden/.  CPU only.
"""
import json
import os

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import lighthouse as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- geometry
@pytest.mark.parametrize("N,p,L,S,E,n_c,T,k_s", [
    (4096, 4, 3, 512, 5376, 256, 21, 1),
    (32768, 4, 5, 4096, 43648, 128, 341, 31),
    (98304, 4, 6, 6144, 131040, 96, 1365, 63),
    (131072, 4, 6, 8192, 174720, 128, 1365, 63),
    (1048576, 8, 5, 16384, 1198336, 256, 4681, 63),
])
def test_geometry_table(N, p, L, S, E, n_c, T, k_s):
    """Level counts of the five workloads, summed by brute force."""
    g = orc.Geometry(N, p, L, S - n_c).check()
    assert g.E == sum(len(range(0, N, p ** l)) for l in range(L)) == E
    assert (g.n_c, g.T, g.k_s, g.S) == (n_c, T, k_s, S)


def test_geometry_rejects():
    with pytest.raises(ValueError):
        orc.Geometry(100, 4, 3, 0).check()          # N not multiple of 16
    with pytest.raises(ValueError):
        orc.Geometry(64, 4, 3, 3).check()           # K not multiple of n_c
    with pytest.raises(ValueError):
        orc.Geometry(64, 4, 3, 4 * 21).check()      # k_s > T-1


# ---------------------------------------------------------------- bf16 rounding
def test_round_bf16_matches_torch_on_float32_values():
    x = np.concatenate([rnd(20000, 1), rnd(2000, 2) * 1e-30, rnd(2000, 3) * 1e30]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.round_bf16(x.astype(np.float64)), want)


def test_round_bf16_ties_to_even():
    one = 1.0
    assert orc.round_bf16(one + 2.0 ** -8) == 1.0                   # halfway -> even (1.0)
    assert orc.round_bf16(one + 3 * 2.0 ** -8) == one + 2.0 ** -6    # halfway -> even
    assert orc.round_bf16(one + 2.0 ** -8 + 2.0 ** -30) == one + 2.0 ** -7
    assert orc.round_bf16(-(one + 2.0 ** -8)) == -1.0


# ---------------------------------------------------------------- O1 pyramid
@pytest.mark.parametrize("N,p,L", [(64, 2, 4), (256, 4, 4), (512, 8, 3), (16, 4, 1)])
def test_pyramid_is_brute_force_mean(N, p, L):
    g = orc.Geometry(N, p, L, 0)
    X = rnd((N, 5), 7)
    lv = orc.pyramid(X, g)
    assert len(lv) == L and lv[0] is not None
    for l in range(L):
        w = p ** l
        brute = np.array([X[i * w:(i + 1) * w].sum(axis=0) / w for i in range(N // w)])
        np.testing.assert_allclose(lv[l], brute, rtol=0, atol=1e-14)


def _round_exact(q, bits):
    """Round the rational q to the nearest binary float with `bits`
    significant bits, ties to even, in exact rational arithmetic (normal
    range only)."""
    if q == 0:
        return q
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    unit = Fraction(2) ** (e - bits + 1)
    n, rem = divmod(a, unit)
    if rem > unit / 2 or (rem == unit / 2 and n % 2 == 1):
        n += 1
    return (n * unit) if q > 0 else -(n * unit)


@pytest.mark.parametrize("store,bits,N,p,L", [("bf16", 8, 486, 3, 4), ("bf16", 8, 256, 4, 4),
                                             ("f32", 24, 243, 3, 4), ("bf16", 8, 250, 5, 3)])
def test_pyramid_store_rounds_exact_mean_once(store, bits, N, p, L):
    # R-2: a stored coarse entry is the exact mean of the p^l tokens it
    # covers, rounded once (ties to even).  Means of bf16 values land
    # exactly on a bf16 rounding tie often enough (dozens of times here)
    # to catch a chain of rounded float64 means, which moves some ties when
    # p is not a power of two.  Exact rational arithmetic throughout.
    g = orc.Geometry(N, p, L, 0)
    X = torch.from_numpy(rnd((N, 8), 41))
    X = (X.to(torch.bfloat16) if store == "bf16" else X.float()).double().numpy()
    st = orc.pyramid(X, g, store=store)
    assert np.array_equal(st[0], X)
    ties = 0
    for l in range(1, L):
        w = p ** l
        for i in range(N // w):
            for j in range(X.shape[1]):
                q = sum(Fraction(float(v)) for v in X[i * w:(i + 1) * w, j]) / w
                want = _round_exact(q, bits)
                assert Fraction(float(st[l][i, j])) == want, (l, i, j)
                ties += _round_exact(q, bits + 1) == q and _round_exact(q, bits) != q
    if store == "bf16":
        assert ties >= 10      # the input really exercises the tie rule


# ---------------------------------------------------------------- O2 scores
def test_scores_level0_is_l2_norm_and_coarse_is_span_max():
    N, p, L = 128, 2, 5
    g = orc.Geometry(N, p, L, 0)
    Q, K = rnd((N, 16), 11), rnd((N, 16), 12)
    sQ, sK = orc.scores(Q, K, g)
    assert sQ.dtype == np.float32 and len(sQ) == g.E
    np.testing.assert_array_equal(sQ[:N], np.linalg.norm(Q, axis=1).astype(np.float32))
    np.testing.assert_array_equal(sK[:N], np.linalg.norm(K, axis=1).astype(np.float32))
    for l, o in enumerate(g.level_offsets):
        w = p ** l
        for i in range(N // w):
            assert sQ[o + i] == sQ[i * w:(i + 1) * w].max()
            assert sK[o + i] == sK[i * w:(i + 1) * w].max()


def test_sigma_modes_closed_form():
    # exact in float32; the sum and the product rank the first two entries
    # in opposite orders
    sQ = np.array([1.0, 2.0, 0.5, 3.0], np.float32)
    sK = np.array([4.0, 2.5, 0.25, 0.0], np.float32)
    assert list(orc.sigma(sQ, sK)) == [5.0, 4.5, 0.75, 3.0]
    assert list(orc.sigma(sQ, sK, "max")) == [4.0, 2.5, 0.5, 3.0]
    assert list(orc.sigma(sQ, sK, "product")) == [4.0, 5.0, 0.125, 0.0]
    assert orc.sigma(sQ, sK, "product").dtype == np.float32
    # one rounding of the exact product: 1 + 2^-12 squared needs 25 bits
    a = np.float32(1 + 2.0 ** -12)
    assert orc.sigma([a], [a], "product")[0] == np.float32(1 + 2.0 ** -11)
    with pytest.raises(ValueError):
        orc.sigma(sQ, sK, "min")


@pytest.mark.parametrize("mode", orc.SIGMA_MODES)
def test_sigma_reduces_to_one_plane(mode):
    # max with a zero plane, product with a plane of ones and sum with a zero
    # plane all rank by sQ alone: the selection equals the one made on sQ
    g = orc.Geometry(1024, 4, 4, 16 * 10)
    sQ, _ = orc.scores(rnd((1024, 8), 5), rnd((1024, 8), 6), g)
    other = np.ones_like(sQ) if mode == "product" else np.zeros_like(sQ)
    a = orc.select(orc.sigma(sQ, other, mode), g)
    b = orc.select(np.asarray(sQ, np.float32), g)
    assert np.array_equal(a.sel_idx, b.sel_idx) and np.array_equal(a.sel_flags, b.sel_flags)


@pytest.mark.parametrize("mode", orc.SIGMA_MODES)
def test_sigma_parent_dominates_children(mode):
    g = orc.Geometry(256, 4, 4, 0)
    sQ, sK = orc.scores(rnd((256, 8), 1), rnd((256, 8), 2), g)
    s = orc.sigma(sQ, sK, mode)
    for l in range(1, g.L):
        par = s[g.level_offsets[l]:g.level_offsets[l] + g.level_sizes[l]]
        ch = s[g.level_offsets[l - 1]:g.level_offsets[l - 1] + g.level_sizes[l - 1]].reshape(-1, 4)
        assert np.all(par[:, None] >= ch)


# ---------------------------------------------------------------- golden
def _sel_from_golden(K):
    gd = json.load(open(os.path.join(GOLD, "selection_hand_N8_p2_L3.json")))
    g = orc.Geometry(gd["N"], gd["p"], gd["L"], K)
    Q = np.stack([np.array(gd["sQ"], float), np.zeros(8)], axis=1)
    Kk = np.stack([np.zeros(8), np.array(gd["sK"], float)], axis=1)
    sQ, sK = orc.scores(Q, Kk, g)
    return gd, g, orc.sigma(sQ, sK)


def test_golden_hand_selection():
    gd, g, s = _sel_from_golden(6)
    assert list(s) == gd["expect_sigma"]
    sel = orc.select(s, g)
    assert list(sel.sel_idx) == gd["expect_sel_idx"]
    assert list(sel.sel_anchor) == gd["expect_sel_anchor"]
    assert list(sel.sel_flags) == gd["expect_sel_flags"]
    assert list(orc.hold_source(sel, 8)) == gd["expect_hold_source"]
    assert list(sel.near_tie) == gd["expect_near_tie"]
    for j, f in enumerate(gd["expect_sel_idx"]):
        assert sel.row_of[f] == j
    assert (sel.row_of >= 0).sum() == len(gd["expect_sel_idx"])


def test_golden_hand_selection_tie():
    gd, g, s = _sel_from_golden(4)
    sel = orc.select(s, g)
    assert list(sel.sel_idx) == gd["expect_sel_idx_K_tie"]
    assert list(sel.near_tie) == gd["expect_near_tie_K_tie"]


def test_golden_hand_span_owner():
    for K, key in ((6, "expect_span_owner"), (4, "expect_span_owner_K_tie")):
        gd, g, s = _sel_from_golden(K)
        assert list(orc.span_owner(orc.select(s, g), g)) == gd[key]


# ---------------------------------------------------------------- O3-O5 selection
def _selection_case(N, p, L, ks, seed, ties=False):
    g = orc.Geometry(N, p, L, ks * (N // p ** (L - 1))).check()
    Q, K = rnd((N, 4), seed), rnd((N, 4), seed + 1)
    if ties:   # quantise norms so exact sigma ties are frequent
        Q = np.round(Q * 2) / 2
        K = np.round(K * 2) / 2
    sQ, sK = orc.scores(Q, K, g)
    s = orc.sigma(sQ, sK)
    return g, s, orc.select(s, g)


@pytest.mark.parametrize("N,p,L,ks,ties", [
    (256, 2, 4, 5, False), (256, 4, 3, 7, True), (512, 8, 3, 20, True),
    (64, 2, 6, 30, True), (4096, 4, 3, 1, False), (256, 4, 4, 0, False)])
def test_selection_brute_force_sort(N, p, L, ks, ties):
    """Selected set == brute-force Python sort of each stratum by
    (-sigma, level, position); exactly k_s+1 rows per stratum, root kept."""
    g, s, sel = _selection_case(N, p, L, ks, 5, ties)
    assert len(sel.sel_idx) == g.S
    for m in range(g.n_c):
        ents = []
        for l in range(L - 1):
            w = p ** l
            for i in range(m * g.Bc // w, (m + 1) * g.Bc // w):
                f = g.level_offsets[l] + i
                ents.append((-float(s[f]), l, i, f))
        best = sorted(ents)[:ks]
        root = g.level_offsets[L - 1] + m
        want = {e[3] for e in best} | {root}
        rows = sel.sel_idx[m * (ks + 1):(m + 1) * (ks + 1)]
        assert set(rows.tolist()) == want


@pytest.mark.parametrize("N,p,L,ks", [(256, 2, 4, 5), (512, 8, 3, 20), (1024, 4, 4, 30)])
def test_selection_dominance_and_order(N, p, L, ks):
    g, s, sel = _selection_case(N, p, L, ks, 9, ties=True)
    chosen = set(sel.sel_idx.tolist())
    for m in range(g.n_c):
        mem = orc.stratum_members(g, m)
        root = g.level_offsets[-1] + m
        assert root in chosen
        cand = [f for f in mem if f != root]
        a = [f for f in cand if f in chosen]
        b = [f for f in cand if f not in chosen]
        for x in a:
            for y in b:
                assert (-s[x], x) < (-s[y], y)
    # rows strictly increasing in (anchor, level); anchors non-decreasing
    lev, idx = orc.entry_of_flat(g, sel.sel_idx)
    anc = (idx + 1) * p ** lev - 1
    key = anc * 64 + lev
    assert np.all(np.diff(key) > 0)
    assert np.array_equal(anc, sel.sel_anchor)
    # stratum m owns rows [m(k_s+1), (m+1)(k_s+1))
    assert np.array_equal(anc // g.Bc, np.repeat(np.arange(g.n_c), ks + 1))


# ---------------------------------------------------------------- R-7' per-level quotas
def test_level_quotas_closed_form():
    # 128K tokens, p = 4, L = 6, k_s = 63: levels 4, 3, 2, 1 take
    # min(size, left // levels left) = 4, 14, 15, 15; level 0 the rest, 15
    assert orc.level_quotas(orc.Geometry(131072, 4, 6, 8064)) == [15, 15, 15, 14, 4]
    # every budget of small trees: quotas sum to k_s and fit their levels;
    # a full budget takes every entry
    for p in (2, 3, 4, 8):
        for L in (1, 2, 3, 4):
            Bc = p ** (L - 1)
            T = sum(p ** l for l in range(L))
            for ks in range(T):
                q = orc.level_quotas(orc.Geometry(Bc, p, L, ks))
                assert len(q) == L - 1 and sum(q) == ks
                assert all(0 <= q[l] <= Bc // p ** l for l in range(L - 1))
            full = orc.level_quotas(orc.Geometry(Bc, p, L, T - 1))
            assert full == [Bc // p ** l for l in range(L - 1)]


@pytest.mark.parametrize("N,p,L,ks,ties", [
    (256, 2, 4, 5, False), (256, 4, 3, 7, True), (512, 8, 3, 20, True),
    (64, 2, 6, 30, True), (1024, 4, 4, 30, True)])
def test_per_level_selection_brute_force(N, p, L, ks, ties):
    """Each level of each stratum holds exactly its quota, and the chosen
    entries of a level are its first ones in a Python sort by
    (-sigma, position); root kept; rows ordered as in the joint reading."""
    g, s, _ = _selection_case(N, p, L, ks, 7, ties)
    sel = orc.select(s, g, strata="per_level")
    q = orc.level_quotas(g)
    chosen = set(sel.sel_idx.tolist())
    assert len(sel.sel_idx) == g.S and len(chosen) == g.S
    for m in range(g.n_c):
        for l in range(L - 1):
            w = p ** l
            ents = sorted((-float(s[g.level_offsets[l] + i]), i)
                          for i in range(m * g.Bc // w, (m + 1) * g.Bc // w))
            want = {g.level_offsets[l] + i for _, i in ents[:q[l]]}
            got = {f for f in chosen
                   if g.level_offsets[l] <= f - m * g.Bc // w < g.level_offsets[l] + g.Bc // w}
            assert got == want, (m, l)
        assert g.level_offsets[-1] + m in chosen
    lev, idx = orc.entry_of_flat(g, sel.sel_idx)
    anc = (idx + 1) * p ** lev - 1
    assert np.all(np.diff(anc * 64 + lev) > 0)


def test_per_level_is_joint_with_one_ranked_level():
    # L = 2: level 0 is the only ranked level, so the two readings agree
    g, s, joint = _selection_case(512, 8, 2, 5, 3, ties=True)
    per = orc.select(s, g, strata="per_level")
    for a, b in ((joint.sel_idx, per.sel_idx), (joint.sel_flags, per.sel_flags),
                 (joint.row_of, per.row_of)):
        assert np.array_equal(a, b)


def test_per_level_differs_from_joint():
    # N = 4, p = 2, L = 3, k_s = 2: quotas [1, 1].  Tokens 0 and 2 carry the
    # largest norm 3, so both level-1 entries inherit 3 too; the joint
    # ranking breaks the four-way tie by flat index and takes the two
    # tokens, while the per-level quotas take one token and one level-1
    # entry.  Flat layout: tokens 0-3, level-1 entries 4-5, root 6.
    g = orc.Geometry(4, 2, 3, 2).check()
    assert orc.level_quotas(g) == [1, 1]
    Q = np.array([[3.0], [1.0], [3.0], [1.0]])
    s = orc.sigma(*orc.scores(Q, np.zeros((4, 1)), g))
    assert list(s) == [3.0, 1.0, 3.0, 1.0, 3.0, 3.0, 3.0]
    assert list(orc.select(s, g).sel_idx) == [0, 2, 6]
    assert list(orc.select(s, g, strata="per_level").sel_idx) == [0, 4, 6]
    with pytest.raises(ValueError):
        orc.select(s, g, strata="per_cell")


@pytest.mark.parametrize("N,p,L,ks", [(256, 2, 4, 9), (512, 4, 4, 40), (512, 8, 3, 50)])
def test_redundancy_is_token_coverage(N, p, L, ks):
    """Recursive rule == 'every token of the span is covered by a selected
    strictly finer entry', checked with an explicit token bitmap."""
    g, s, sel = _selection_case(N, p, L, ks, 21, ties=True)
    lev, idx = orc.entry_of_flat(g, sel.sel_idx)
    for j in range(len(sel.sel_idx)):
        l0, i0 = lev[j], idx[j]
        lo, hi = i0 * p ** l0, (i0 + 1) * p ** l0
        cov = np.zeros(hi - lo, bool)
        for k in range(len(sel.sel_idx)):
            if lev[k] < l0:
                a, b = idx[k] * p ** lev[k], (idx[k] + 1) * p ** lev[k]
                if a >= lo and b <= hi:
                    cov[a - lo:b - lo] = True
        want = bool(l0 > 0 and cov.all())
        assert bool(sel.sel_flags[j] & orc.FLAG_REDUNDANT) == want
        # a leader is never redundant
        if sel.sel_flags[j] & orc.FLAG_LEADER:
            assert not sel.sel_flags[j] & orc.FLAG_REDUNDANT


def test_hold_source_brute_force():
    g, s, sel = _selection_case(1024, 4, 4, 13, 33, ties=True)
    src = orc.hold_source(sel, g.N)
    lead = [j for j in range(g.S) if sel.sel_flags[j] & orc.FLAG_LEADER]
    for t in range(g.N):
        c = [j for j in lead if sel.sel_anchor[j] <= t]
        assert src[t] == (max(c, key=lambda j: sel.sel_anchor[j]) if c else -1)


@pytest.mark.parametrize("N,p,L,ks", [(1024, 4, 4, 13), (512, 2, 5, 9), (512, 8, 3, 30)])
def test_span_owner_brute_force(N, p, L, ks):
    """Every token's owner is the finest selected entry whose span holds it,
    found by scanning every selected row's span; the owners are exactly the
    non-redundant rows (a non-redundant row keeps an uncovered token)."""
    g, s, sel = _selection_case(N, p, L, ks, 35, ties=True)
    own = orc.span_owner(sel, g)
    best = np.full(g.N, -1)
    best_lev = np.full(g.N, 99)
    for j, f in enumerate(sel.sel_idx):
        lev, i = orc.entry_of_flat(g, f)
        lo, hi = i * p ** lev, (i + 1) * p ** lev
        for t in range(lo, hi):
            if lev < best_lev[t]:
                best[t], best_lev[t] = j, lev
    assert np.array_equal(own, best)
    nonred = {j for j in range(g.S) if not sel.sel_flags[j] & orc.FLAG_REDUNDANT}
    assert set(own.tolist()) == nonred


# ---------------------------------------------------------------- O6-O8 special cases
def torch_causal_sdpa(Q, K, V):
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x))[None, None] for x in (Q, K, V))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)[0, 0].numpy()


@pytest.mark.parametrize("N,p,L,ks", [
    (64, 2, 3, 6),       # k_s = T-1: everything selected
    (128, 4, 2, 4),      # L = 2, k_s = p
    (96, 3, 1, 0),       # L = 1: every token is its own coarsest entry
    (256, 4, 3, 20)])
@pytest.mark.parametrize("mode", ["hold", "span"])
def test_full_selection_is_dense_causal_sdpa(N, p, L, ks, mode):
    g = orc.Geometry(N, p, L, ks * (N // p ** (L - 1))).check()
    Q, K, V = rnd((N, 8), 1), rnd((N, 8), 2), rnd((N, 8), 3)
    fw = orc.head_forward(Q, K, V, g, scatter_mode=mode)
    np.testing.assert_allclose(fw.O, torch_causal_sdpa(Q, K, V), rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,p,L", [(256, 4, 3), (512, 2, 5)])
def test_coarsest_only_closed_form(N, p, L):
    """K = 0: attention runs on the coarsest pooled triplets and token t
    takes row floor((t+1)/B_c) - 1 (zero before the first anchor)."""
    g = orc.Geometry(N, p, L, 0).check()
    Q, K, V = rnd((N, 8), 4), rnd((N, 8), 5), rnd((N, 8), 6)
    fw = orc.head_forward(Q, K, V, g)
    Bc = g.Bc
    blk = lambda X: X.reshape(N // Bc, Bc, -1).mean(axis=1)
    OS = torch_causal_sdpa(blk(Q), blk(K), blk(V))
    want = np.zeros((N, 8))
    for t in range(Bc - 1, N):
        want[t] = OS[(t + 1) // Bc - 1]
    np.testing.assert_allclose(fw.O, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,p,L", [(256, 4, 3), (512, 2, 5)])
def test_coarsest_only_closed_form_span(N, p, L):
    """K = 0, span broadcast: every token of coarsest cell m takes row m."""
    g = orc.Geometry(N, p, L, 0).check()
    Q, K, V = rnd((N, 8), 4), rnd((N, 8), 5), rnd((N, 8), 6)
    fw = orc.head_forward(Q, K, V, g, scatter_mode="span")
    Bc = g.Bc
    blk = lambda X: X.reshape(N // Bc, Bc, -1).mean(axis=1)
    OS = torch_causal_sdpa(blk(Q), blk(K), blk(V))
    np.testing.assert_allclose(fw.O, np.repeat(OS, Bc, axis=0), rtol=0, atol=1e-12)


def test_softmax_rows_nonempty_and_normalised():
    g, s, sel = _selection_case(1024, 4, 4, 40, 3, ties=True)
    S = g.S
    QS, KS = rnd((S, 8), 1), rnd((S, 8), 2)
    VS = np.ones((S, 3))
    OS, LSE = orc.attention_fwd(QS, KS, VS, sel.sel_flags, 0.3)
    assert np.all(np.isfinite(LSE))
    np.testing.assert_allclose(OS, 1.0, atol=1e-12)   # weights sum to one


# ---------------------------------------------------------------- causality
def test_token_causality_with_selection_fixed():
    N, p, L, ks = 512, 4, 4, 20
    g = orc.Geometry(N, p, L, ks * (N // 64)).check()
    Q, K, V = rnd((N, 8), 1), rnd((N, 8), 2), rnd((N, 8), 3)
    base = orc.head_forward(Q, K, V, g)
    rng = np.random.default_rng(0)
    for t in (0, 37, 63, 64, 200, 511):
        Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
        sgn = lambda shape: np.where(rng.random(shape) < 0.5, -1.0, 1.0)
        Q2[t + 1:] *= sgn(Q2[t + 1:].shape)      # sign flips keep every norm
        K2[t + 1:] *= sgn(K2[t + 1:].shape)
        V2[t + 1:] = rng.standard_normal(V2[t + 1:].shape) * 5
        pert = orc.head_forward(Q2, K2, V2, g)
        assert np.array_equal(pert.sel.sel_idx, base.sel.sel_idx)
        assert np.array_equal(pert.O[:t + 1], base.O[:t + 1])


@pytest.mark.parametrize("mode", ["hold", "span"])
def test_block_causality_unconditional(mode):
    N, p, L, ks = 512, 4, 4, 20
    g = orc.Geometry(N, p, L, ks * (N // 64)).check()
    Q, K, V = rnd((N, 8), 1), rnd((N, 8), 2), rnd((N, 8), 3)
    base = orc.head_forward(Q, K, V, g, scatter_mode=mode)
    for m in (1, 3, 7):
        b = m * g.Bc
        Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
        Q2[b:] = rnd(Q2[b:].shape, 50 + m) * 9
        K2[b:] = rnd(K2[b:].shape, 60 + m) * 9
        V2[b:] = rnd(V2[b:].shape, 70 + m)
        pert = orc.head_forward(Q2, K2, V2, g, scatter_mode=mode)
        r = m * (ks + 1)
        assert np.array_equal(pert.sel.sel_idx[:r], base.sel.sel_idx[:r])
        assert np.array_equal(pert.O[:b], base.O[:b])


# ---------------------------------------------------------------- R-19 ragged lengths
def test_padded_length():
    assert orc.padded_length(257, 2, 5) == 272
    assert orc.padded_length(256, 2, 5) == 256
    assert orc.padded_length(1, 4, 3) == 16
    assert orc.padded_length(1000, 4, 1) == 1000


@pytest.mark.parametrize("mode", ["hold", "span"])
@pytest.mark.parametrize("N,p,L,ks", [(257, 2, 5, 6), (1000, 4, 3, 5), (1090, 3, 4, 9)])
def test_ragged_length_prefix(N, p, L, ks, mode):
    # the strata before the last one are complete; causality and stratum-local
    # selection make their tokens' outputs those of the layer run on those
    # strata alone (the BF1-style partial-last-block gate at N = 257)
    Bc = p ** (L - 1)
    Np = orc.padded_length(N, p, L)
    m = N // Bc
    Q, K, V = rnd((N, 8), 21), rnd((N, 8), 22), rnd((N, 8), 23)
    fw, O = orc.ragged_forward(Q, K, V, p, L, ks * (Np // Bc), scatter_mode=mode)
    assert O.shape == (N, 8) and np.all(np.isfinite(O))
    g = orc.Geometry(m * Bc, p, L, ks * m).check()
    ref = orc.head_forward(Q[:m * Bc], K[:m * Bc], V[:m * Bc], g, scatter_mode=mode)
    np.testing.assert_allclose(O[:m * Bc], ref.O, rtol=0, atol=1e-12)
    r = m * (ks + 1)   # the rows of the complete strata (flat indices differ by geometry)
    assert np.array_equal(fw.sel.sel_anchor[:r], ref.sel.sel_anchor)
    assert np.array_equal(fw.sel.sel_level[:r], ref.sel.sel_level)
    assert np.array_equal(fw.sel.sel_flags[:r], ref.sel.sel_flags)


def test_ragged_length_pads_with_zero_rows():
    # N = 1000, p = 4, L = 3: the last coarsest cell (tokens 992..1007) holds
    # 8 real tokens, so its entry is their sum over 16, and the padded
    # tokens score zero
    N, p, L = 1000, 4, 3
    X = rnd((N, 8), 31)
    fw, _ = orc.ragged_forward(X, X, X, p, L, 0)
    np.testing.assert_allclose(fw.Ql[2][-1], X[992:1000].sum(axis=0) / 16, rtol=0, atol=1e-15)
    np.testing.assert_allclose(fw.Ql[1][249], X[996:1000].mean(axis=0), rtol=0, atol=1e-15)
    assert np.all(fw.Ql[1][250:] == 0) and np.all(fw.sQ[N:1008] == 0)


def test_ragged_length_whole_cells_is_the_layer():
    N, p, L, K = 256, 4, 3, 16 * 4
    Q, K_, V = rnd((N, 8), 1), rnd((N, 8), 2), rnd((N, 8), 3)
    fw, O = orc.ragged_forward(Q, K_, V, p, L, K)
    ref = orc.head_forward(Q, K_, V, orc.Geometry(N, p, L, K))
    assert np.array_equal(O, ref.O)


# ---------------------------------------------------------------- adjoints
def test_scatter_adjoint_dot_product():
    g, s, sel = _selection_case(1024, 4, 4, 13, 41, ties=True)
    x, y = rnd((g.S, 6), 1), rnd((g.N, 6), 2)
    lhs = np.sum(orc.scatter(x, sel, g.N) * y)
    rhs = np.sum(x * orc.scatter_adjoint(y, sel, g.N))
    assert abs(lhs - rhs) < 1e-10 * (1 + abs(lhs))


def test_scatter_span_adjoint_dot_product():
    g, s, sel = _selection_case(1024, 4, 4, 13, 42, ties=True)
    x, y = rnd((g.S, 6), 3), rnd((g.N, 6), 4)
    lhs = np.sum(orc.scatter_span(x, sel, g) * y)
    rhs = np.sum(x * orc.scatter_span_adjoint(y, sel, g))
    assert abs(lhs - rhs) < 1e-10 * (1 + abs(lhs))


def test_pool_gather_adjoint_dot_product():
    g, s, sel = _selection_case(512, 2, 5, 11, 43, ties=True)
    X, Y = rnd((g.N, 6), 1), rnd((g.S, 6), 2)
    lhs = np.sum(orc.gather(orc.pyramid(X, g), sel.sel_idx) * Y)
    rhs = np.sum(X * orc.pool_adjoint(orc.gather_adjoint(Y, sel, g), g))
    assert abs(lhs - rhs) < 1e-10 * (1 + abs(lhs))
