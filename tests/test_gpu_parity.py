"""GPU parity of every stage and of the whole layer against the CPU oracle.

Stage tests feed each kernel the GPU's own upstream outputs, so that a
difference is located in the stage under test; the layer tests run
lh_layer_fwd / lh_layer_bwd end to end from the inputs.  Integer outputs
(scores' max inheritance, selection, indices, flags, row_of, gathers and
scatters) must be bit-exact; floating point within the stated tolerance.
"""
import numpy as np
import pytest
import torch

from oracle import lighthouse as orc
from tests.gpu_cases import (CASES, Case, bh_pairs, f64, geometry, inputs, selection_from_gpu,
                             store_of, tol_for)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_long_context_amd import ops


def _ctx(case, q, scatter_mode="hold", sigma_mode="sum", strata_mode="joint"):
    out = torch.float32 if case.out == "f32" else torch.bfloat16
    if case.dtype == "f32":
        out = torch.float32
    return ops.Ctx(ops.make_dims(q, case.p, case.L, case.S, out_dtype=out,
                                 scatter_mode=scatter_mode, sigma_mode=sigma_mode,
                                 strata_mode=strata_mode))


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _run_stages(case, dev):
    Q, K, V, dO = (t.to(dev) for t in inputs(case))
    c = _ctx(case, Q)
    r = {"c": c, "Q": Q, "K": K, "V": V}
    r["pq"], r["pk"], r["pv"], r["sq"], r["sk"] = ops.pyramid_score(c, Q, K, V)
    r["sel_idx"], r["anchor"], r["flags"], r["row_of"] = ops.topk_select(c, r["sq"], r["sk"])
    bf = case.dtype == "bf16"
    g = ops.gather(c, Q, K, V, r["pq"], r["pk"], r["pv"], r["sel_idx"], transposed=bf)
    r["qs"], r["ks"], r["vs"] = g[:3]
    if bf:
        r["qst"], r["kst"], r["vst"] = g[3:]
    r["os"], r["lse"] = ops.subseq_attn_fwd(c, r["qs"], r["ks"], r["vs"], r["flags"])
    r["o"] = ops.scatter(c, r["os"], r["anchor"], r["flags"])
    r["dO"] = dO.to(dev, c.out)
    r["dos"] = ops.scatter_bwd(c, r["dO"], r["anchor"], r["flags"])
    r["dqs"], r["dks"], r["dvs"] = ops.subseq_attn_bwd(c, r["qs"], r["ks"], r["vs"], r["os"],
                                                       r["lse"], r["flags"], r["dos"])
    r["dq"], r["dk"], r["dv"] = ops.gather_bwd(c, r["dqs"], r["dks"], r["dvs"], r["row_of"])
    torch.cuda.synchronize()
    return r


_cache = {}


def stages(case, dev):
    if case.name not in _cache:
        print(f"[gpu] stages {case.name}", flush=True)
        _cache[case.name] = _run_stages(case, dev)
    return _cache[case.name]


ids = [c.name for c in CASES]


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_pyramid_and_scores(case, dev):
    r = stages(case, dev)
    g = geometry(case)
    for b, h in bh_pairs(case):
        Qh, Kh, Vh = (f64(r[n][b, h]) for n in ("Q", "K", "V"))
        sQ, sK = orc.scores(Qh, Kh, g)
        assert np.array_equal(r["sq"][b, h].cpu().numpy(), sQ), "sq differs"
        assert np.array_equal(r["sk"][b, h].cpu().numpy(), sK), "sk differs"
        if case.L == 1:
            continue
        for X, P in ((Qh, "pq"), (Kh, "pk"), (Vh, "pv")):
            want = np.concatenate(orc.pyramid(X, g, store=store_of(case))[1:])
            got = f64(r[P][b, h])
            # both sides round each block's exact mean once: bit-exact
            bad = np.argwhere(got != want)
            assert len(bad) == 0, (P, b, h, len(bad), [(got[i, j], want[i, j]) for i, j in bad[:3]])


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_selection_bit_exact(case, dev):
    r = stages(case, dev)
    g = geometry(case)
    for b, h in bh_pairs(case):
        sig = orc.sigma(r["sq"][b, h].cpu().numpy(), r["sk"][b, h].cpu().numpy())
        sel = orc.select(sig, g)
        assert np.array_equal(r["sel_idx"][b, h].cpu().numpy(), sel.sel_idx)
        assert np.array_equal(r["anchor"][b, h].cpu().numpy(), sel.sel_anchor)
        assert np.array_equal(r["flags"][b, h].cpu().numpy(), sel.sel_flags)
        assert np.array_equal(r["row_of"][b, h].cpu().numpy(), sel.row_of)


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_gather_and_transposes(case, dev):
    r = stages(case, dev)
    S = case.S
    for b, h in bh_pairs(case):
        for X, P, XS in (("Q", "pq", "qs"), ("K", "pk", "ks"), ("V", "pv", "vs")):
            rows = r[X][b, h] if case.L == 1 else torch.cat([r[X][b, h], r[P][b, h]])
            want = rows[r["sel_idx"][b, h].long()]
            assert torch.equal(r[XS][b, h], want)
        if case.dtype == "bf16":
            for XS, XT in (("qs", "qst"), ("ks", "kst"), ("vs", "vst")):
                t = r[XT][b, h]
                assert torch.equal(t[:, :S], r[XS][b, h].t())
                assert torch.all(t[:, S:] == 0)


def _close(got, want, tol, what):
    err = np.abs(got - want)
    worst = float(np.max(err - tol)) if err.size else -1.0
    print(f"[parity] {what}: max|err| {float(err.max()) if err.size else 0:.3e}", flush=True)
    assert worst <= 0, f"{what}: exceeds tolerance by {worst:.3e}"


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_attention_fwd(case, dev):
    r = stages(case, dev)
    c = r["c"]
    for b, h in bh_pairs(case):
        OS, LSE = orc.attention_fwd(f64(r["qs"][b, h]), f64(r["ks"][b, h]), f64(r["vs"][b, h]),
                                    r["flags"][b, h].cpu().numpy(), c.dims.scale or 1 / np.sqrt(case.d))
        _close(f64(r["os"][b, h]), OS, tol_for(case, OS, case.out), f"{case.name} h{h} OS")
        _close(f64(r["lse"][b, h]), LSE, 1e-4 if case.dtype == "f32" else 2e-3, f"{case.name} h{h} LSE")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_scatter_and_adjoint(case, dev):
    r = stages(case, dev)
    g = geometry(case)
    for b, h in bh_pairs(case):
        sel = selection_from_gpu(g, *(r[n][b, h].cpu().numpy() for n in ("sel_idx", "anchor", "flags", "row_of")))
        src = orc.hold_source(sel, case.N)
        os_ = r["os"][b, h]
        want = torch.zeros_like(r["o"][b, h])
        ok = torch.from_numpy(src >= 0)
        want[ok.to(dev)] = os_[torch.from_numpy(src[src >= 0]).to(dev)].to(want.dtype)
        assert torch.equal(r["o"][b, h], want), "scatter is a pure copy"
        dOS = orc.scatter_adjoint(f64(r["dO"][b, h]), sel, case.N)
        got = f64(r["dos"][b, h])
        scale = 1e-5 * (1 + np.abs(dOS))
        assert np.all(np.abs(got - dOS) <= scale), float(np.max(np.abs(got - dOS)))


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_attention_bwd(case, dev):
    r = stages(case, dev)
    c = r["c"]
    scale = c.dims.scale or 1 / np.sqrt(case.d)
    for b, h in bh_pairs(case):
        dQS, dKS, dVS = orc.attention_bwd(f64(r["qs"][b, h]), f64(r["ks"][b, h]), f64(r["vs"][b, h]),
                                          r["flags"][b, h].cpu().numpy(), scale, f64(r["dos"][b, h]))
        for n, want in (("dqs", dQS), ("dks", dKS), ("dvs", dVS)):
            _close(f64(r[n][b, h]), want, tol_for(case, want, "f32"), f"{case.name} h{h} {n}")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_unpool(case, dev):
    r = stages(case, dev)
    g = geometry(case)
    for b, h in bh_pairs(case):
        sel = selection_from_gpu(g, *(r[n][b, h].cpu().numpy() for n in ("sel_idx", "anchor", "flags", "row_of")))
        for n, o in (("dqs", "dq"), ("dks", "dk"), ("dvs", "dv")):
            want = orc.pool_adjoint(orc.gather_adjoint(f64(r[n][b, h]), sel, g), g)
            got = f64(r[o][b, h])
            if case.out == "bf16" and case.dtype == "bf16":
                tol = 1e-5 * (1 + np.abs(want)) + np.abs(want) * 2.0 ** -8
            else:
                tol = 1e-5 * (1 + np.abs(want))
            assert np.all(np.abs(got - want) <= tol), float(np.max(np.abs(got - want)))


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_layer_vs_oracle(case, dev):
    """lh_layer_fwd/bwd end to end against the oracle run from the inputs."""
    Q, K, V, dO = (t.to(dev) for t in inputs(case))
    c = _ctx(case, Q)
    o, saved = ops.layer_fwd(c, Q, K, V)
    dOc = dO.to(c.out)
    dq, dk, dv = ops.layer_bwd(c, saved, dOc)
    torch.cuda.synchronize()
    g = geometry(case)
    for b, h in bh_pairs(case):
        fw = orc.head_forward(f64(Q[b, h]), f64(K[b, h]), f64(V[b, h]), g, store=store_of(case))
        assert np.array_equal(saved["sel_idx"][b, h].cpu().numpy(), fw.sel.sel_idx)
        _close(f64(o[b, h]), fw.O, tol_for(case, fw.O, case.out), f"{case.name} h{h} O")
        gq, gk, gv = orc.head_backward(fw, f64(dOc[b, h]))[:3]
        for got, want, n in ((dq, gq, "dQ"), (dk, gk, "dK"), (dv, gv, "dV")):
            _close(f64(got[b, h]), want, tol_for(case, want, case.out), f"{case.name} h{h} {n}")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_layer_matches_stages_and_is_deterministic(case, dev):
    r = stages(case, dev)
    c = r["c"]
    o1, s1 = ops.layer_fwd(c, r["Q"], r["K"], r["V"])
    o2, s2 = ops.layer_fwd(c, r["Q"], r["K"], r["V"])
    g1 = ops.layer_bwd(c, s1, r["dO"])
    g2 = ops.layer_bwd(c, s2, r["dO"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and all(torch.equal(a, b) for a, b in zip(g1, g2))
    assert torch.equal(o1, r["o"])
    for a, n in zip(g1, ("dq", "dk", "dv")):
        assert torch.equal(a, r[n]), n
    # everything the layer forward saves for the backward (pyramids, scores,
    # selection, gathered rows) equals the separate stages' outputs, bitwise
    for n, m in (("sq", "sq"), ("sk", "sk"), ("pq", "pq"), ("pk", "pk"), ("pv", "pv"),
                 ("sel_idx", "sel_idx"), ("sel_anchor", "anchor"), ("sel_flags", "flags"),
                 ("row_of", "row_of"), ("qs", "qs"), ("ks", "ks"), ("vs", "vs")):
        for sv in (s1, s2):
            if sv[n] is None:
                assert r[m] is None or r[m].numel() == 0, n
            else:
                assert torch.equal(sv[n], r[m]), n


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_span_scatter_and_adjoint(case, dev):
    """Span broadcast: the owner map bit-exact, the scatter a pure copy, its
    adjoint within float32 summation error of the oracle."""
    r = stages(case, dev)
    c = r["c"]
    g = geometry(case)
    owner = ops.span_owner(c, r["row_of"])
    o = ops.scatter_span(c, r["os"], owner)
    dos = ops.scatter_span_bwd(c, r["dO"], r["sel_idx"], r["flags"], owner)
    torch.cuda.synchronize()
    for b, h in bh_pairs(case):
        sel = selection_from_gpu(g, *(r[n][b, h].cpu().numpy() for n in ("sel_idx", "anchor", "flags", "row_of")))
        own = orc.span_owner(sel, g)
        assert np.array_equal(owner[b, h].cpu().numpy(), own), f"owner head {h}"
        want = r["os"][b, h][torch.from_numpy(own).to(dev)].to(o.dtype)
        assert torch.equal(o[b, h], want), "span scatter is a pure copy"
        dOS = orc.scatter_span_adjoint(f64(r["dO"][b, h]), sel, g)
        got = f64(dos[b, h])
        assert np.all(np.abs(got - dOS) <= 1e-5 * (1 + np.abs(dOS))), float(np.max(np.abs(got - dOS)))


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_layer_span_mode_vs_oracle(case, dev):
    """lh_layer_fwd/bwd in span-broadcast mode against the oracle; the layer
    equals its stages bitwise and two runs are identical."""
    Q, K, V, dO = (t.to(dev) for t in inputs(case))
    c = _ctx(case, Q, scatter_mode="span")
    o, saved = ops.layer_fwd(c, Q, K, V)
    dOc = dO.to(c.out)
    dq, dk, dv = ops.layer_bwd(c, saved, dOc)
    o2, saved2 = ops.layer_fwd(c, Q, K, V)
    g2 = ops.layer_bwd(c, saved2, dOc)
    owner = ops.span_owner(c, saved["row_of"])
    dos = ops.scatter_span_bwd(c, dOc, saved["sel_idx"], saved["sel_flags"], owner)
    sq = ops.subseq_attn_bwd(c, saved["qs"], saved["ks"], saved["vs"], saved["os"], saved["lse"],
                             saved["sel_flags"], dos)
    stage_grads = ops.gather_bwd(c, *sq, saved["row_of"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and all(torch.equal(a, b) for a, b in zip((dq, dk, dv), g2))
    assert torch.equal(o, ops.scatter_span(c, saved["os"], owner))
    for a, b, n in zip((dq, dk, dv), stage_grads, ("dq", "dk", "dv")):
        assert torch.equal(a, b), n
    g = geometry(case)
    for b, h in bh_pairs(case):
        fw = orc.head_forward(f64(Q[b, h]), f64(K[b, h]), f64(V[b, h]), g, store=store_of(case),
                              scatter_mode="span")
        assert np.array_equal(saved["sel_idx"][b, h].cpu().numpy(), fw.sel.sel_idx)
        _close(f64(o[b, h]), fw.O, tol_for(case, fw.O, case.out), f"{case.name} h{h} span O")
        gq, gk, gv = orc.head_backward(fw, f64(dOc[b, h]))[:3]
        for got, want, n in ((dq, gq, "dQ"), (dk, gk, "dK"), (dv, gv, "dV")):
            _close(f64(got[b, h]), want, tol_for(case, want, case.out), f"{case.name} h{h} span {n}")


def test_full_selection_is_dense_sdpa(dev):
    """With every entry selected the layer is dense causal SDPA (float32
    reference on the CPU)."""
    case = [c for c in CASES if c.name == "bf16-full-selection"][0]
    Q, K, V, _ = inputs(case)
    c = _ctx(case, Q.to(dev))
    o, _ = ops.layer_fwd(c, Q.to(dev), K.to(dev), V.to(dev))
    ref = torch.nn.functional.scaled_dot_product_attention(Q.double(), K.double(), V.double(),
                                                           is_causal=True)
    err = (o.double().cpu() - ref).abs().max().item()
    print(f"[parity] full selection vs SDPA: {err:.3e}", flush=True)
    assert err < 2e-2


SIGMA_CASES = [c for c in CASES if c.name in ("tiny-f32", "bf16-d128-ragged", "bf16-p3",
                                              "bf16-p2-L3-k1536")]


@pytest.mark.parametrize("mode", ["max", "product"])
@pytest.mark.parametrize("case", SIGMA_CASES, ids=lambda c: c.name)
def test_selection_sigma_modes(case, mode, dev):
    """The other combinations of the two scores (R-5 options): the whole
    selection bit-exact against the oracle's on the same score planes."""
    r = stages(case, dev)
    c = _ctx(case, r["Q"], sigma_mode=mode)
    sel_idx, anchor, flags, row_of = ops.topk_select(c, r["sq"], r["sk"])
    torch.cuda.synchronize()
    g = geometry(case)
    for b, h in bh_pairs(case):
        sig = orc.sigma(r["sq"][b, h].cpu().numpy(), r["sk"][b, h].cpu().numpy(), mode)
        sel = orc.select(sig, g)
        assert np.array_equal(sel_idx[b, h].cpu().numpy(), sel.sel_idx)
        assert np.array_equal(anchor[b, h].cpu().numpy(), sel.sel_anchor)
        assert np.array_equal(flags[b, h].cpu().numpy(), sel.sel_flags)
        assert np.array_equal(row_of[b, h].cpu().numpy(), sel.row_of)


@pytest.mark.parametrize("case", SIGMA_CASES[1:3], ids=lambda c: c.name)
def test_layer_product_sigma_vs_oracle(case, dev):
    """lh_layer_fwd/bwd with sigma_mode = product against the oracle."""
    Q, K, V, dO = (t.to(dev) for t in inputs(case))
    c = _ctx(case, Q, sigma_mode="product")
    o, saved = ops.layer_fwd(c, Q, K, V)
    dOc = dO.to(c.out)
    dq, dk, dv = ops.layer_bwd(c, saved, dOc)
    torch.cuda.synchronize()
    g = geometry(case)
    for b, h in bh_pairs(case):
        fw = orc.head_forward(f64(Q[b, h]), f64(K[b, h]), f64(V[b, h]), g, store=store_of(case),
                              sigma_mode="product")
        assert np.array_equal(saved["sel_idx"][b, h].cpu().numpy(), fw.sel.sel_idx)
        _close(f64(o[b, h]), fw.O, tol_for(case, fw.O, case.out), f"{case.name} h{h} O")
        gq, gk, gv = orc.head_backward(fw, f64(dOc[b, h]))[:3]
        for got, want, n in ((dq, gq, "dQ"), (dk, gk, "dK"), (dv, gv, "dV")):
            _close(f64(got[b, h]), want, tol_for(case, want, case.out), f"{case.name} h{h} {n}")


STRATA_CASES = [c for c in CASES if c.name in (
    "tiny-f32", "bf16-d128-ragged", "bf16-d64-p8-ragged", "bf16-full-selection",
    "bf16-coarsest-only", "bf16-batch2-p2", "bf16-p3", "bf16-one-stratum")]


@pytest.mark.parametrize("case", STRATA_CASES, ids=lambda c: c.name)
def test_selection_per_level_strata(case, dev):
    """Per-level quotas (reading R-7', the strata option): the whole
    selection bit-exact against the oracle's on the same score planes."""
    r = stages(case, dev)
    c = _ctx(case, r["Q"], strata_mode="per_level")
    sel_idx, anchor, flags, row_of = ops.topk_select(c, r["sq"], r["sk"])
    torch.cuda.synchronize()
    g = geometry(case)
    for b, h in bh_pairs(case):
        sig = orc.sigma(r["sq"][b, h].cpu().numpy(), r["sk"][b, h].cpu().numpy())
        sel = orc.select(sig, g, strata="per_level")
        assert np.array_equal(sel_idx[b, h].cpu().numpy(), sel.sel_idx)
        assert np.array_equal(anchor[b, h].cpu().numpy(), sel.sel_anchor)
        assert np.array_equal(flags[b, h].cpu().numpy(), sel.sel_flags)
        assert np.array_equal(row_of[b, h].cpu().numpy(), sel.row_of)


@pytest.mark.parametrize("case", [c for c in STRATA_CASES if c.name in ("bf16-d128-ragged",
                                                                      "bf16-p3")],
                         ids=lambda c: c.name)
def test_layer_per_level_strata_vs_oracle(case, dev):
    """lh_layer_fwd/bwd with strata_mode = per level against the oracle."""
    Q, K, V, dO = (t.to(dev) for t in inputs(case))
    c = _ctx(case, Q, strata_mode="per_level")
    o, saved = ops.layer_fwd(c, Q, K, V)
    dOc = dO.to(c.out)
    dq, dk, dv = ops.layer_bwd(c, saved, dOc)
    torch.cuda.synchronize()
    g = geometry(case)
    for b, h in bh_pairs(case):
        fw = orc.head_forward(f64(Q[b, h]), f64(K[b, h]), f64(V[b, h]), g, store=store_of(case),
                              strata_mode="per_level")
        assert np.array_equal(saved["sel_idx"][b, h].cpu().numpy(), fw.sel.sel_idx)
        _close(f64(o[b, h]), fw.O, tol_for(case, fw.O, case.out), f"{case.name} h{h} O")
        gq, gk, gv = orc.head_backward(fw, f64(dOc[b, h]))[:3]
        for got, want, n in ((dq, gq, "dQ"), (dk, gk, "dK"), (dv, gv, "dV")):
            _close(f64(got[b, h]), want, tol_for(case, want, case.out), f"{case.name} h{h} {n}")


# Lengths that are not whole coarsest cells (reading R-19): the layer pads
# with zero rows in its workspace and returns the real tokens' outputs.
RAGGED = [
    # the partial-last-block gate length 257: 16 full cells of 16 and one token
    Case("ragged-257", 257, 2, 64, 2, 5, 6),
    # 62 full cells of 16 and a cell of 8 tokens, spiky rows, d = 128
    Case("ragged-1000", 1000, 2, 128, 4, 3, 5, structure="spikes"),
    # float32 I/O, one real token in the last cell
    Case("ragged-f32-4001", 4001, 2, 64, 4, 3, 1, dtype="f32"),
]


@pytest.mark.parametrize("mode", ["hold", "span"])
@pytest.mark.parametrize("case", RAGGED, ids=lambda c: c.name)
def test_layer_ragged_length_vs_oracle(case, mode, dev):
    Q, K, V, dO = (t.to(dev) for t in inputs(case))
    c = _ctx(case, Q, scatter_mode=mode)
    assert c.Np % case.p ** (case.L - 1) == 0 and c.Np > case.N
    o, saved = ops.layer_fwd(c, Q, K, V)
    dOc = dO.to(c.out)
    dq, dk, dv = ops.layer_bwd(c, saved, dOc)
    o2, saved2 = ops.layer_fwd(c, Q, K, V)
    g2 = ops.layer_bwd(c, saved2, dOc)
    torch.cuda.synchronize()
    assert o.shape[2] == case.N and dq.shape[2] == case.N
    assert torch.equal(o, o2) and all(torch.equal(a, b) for a, b in zip((dq, dk, dv), g2))
    Kp = c.dims.K
    for b, h in bh_pairs(case):
        fw, O = orc.ragged_forward(f64(Q[b, h]), f64(K[b, h]), f64(V[b, h]), case.p, case.L, Kp,
                                   store=store_of(case), scatter_mode=mode)
        assert np.array_equal(saved["sel_idx"][b, h].cpu().numpy(), fw.sel.sel_idx)
        _close(f64(o[b, h]), O, tol_for(case, O, case.out), f"{case.name} h{h} O")
        gq, gk, gv = orc.ragged_backward(fw, f64(dOc[b, h]))
        for got, want, n in ((dq, gq, "dQ"), (dk, gk, "dK"), (dv, gv, "dV")):
            _close(f64(got[b, h]), want, tol_for(case, want, case.out), f"{case.name} h{h} {n}")


@pytest.mark.parametrize("mode", ["hold", "span"])
@pytest.mark.parametrize("name", ["bf16-d128-ragged", "bf16-bursts-bf16out"])
def test_autograd_wrapper_matches_layer_calls(name, mode, dev):
    """torch.autograd through lighthouse_attention gives the outputs and
    gradients of the direct lh_layer_fwd / lh_layer_bwd calls, bitwise, and
    the gradient of a weighted sum of O is dO through the layer backward."""
    from sparse_long_context_amd.layer import lighthouse_attention
    case = [c for c in CASES if c.name == name][0]
    Q, K, V, dO = (t.to(dev) for t in inputs(case))
    c = _ctx(case, Q, scatter_mode=mode)
    out = c.out
    o_ref, saved = ops.layer_fwd(c, Q, K, V)
    g_ref = ops.layer_bwd(c, saved, dO.to(out))
    q, k, v = (t.clone().requires_grad_(True) for t in (Q, K, V))
    o = lighthouse_attention(q, k, v, case.p, case.L, case.S, out_dtype=out, scatter_mode=mode)
    o.backward(dO.to(out))
    torch.cuda.synchronize()
    assert o.dtype == out and torch.equal(o.detach(), o_ref)
    # autograd hands each gradient back in its input's dtype
    for got, want, n in zip((q.grad, k.grad, v.grad), g_ref, ("dq", "dk", "dv")):
        assert got is not None and got.dtype == Q.dtype, n
        assert torch.equal(got, want.to(Q.dtype)), n


def test_layer_from_two_threads_on_two_streams(dev):
    """Two host threads run lh_layer_fwd + lh_layer_bwd at the same time on
    two streams of one device (the calls share the library's second stream
    and its events); each result equals the sequential one, bitwise."""
    import threading
    case = [c for c in CASES if c.name == "bf16-bursts-bf16out"][0]
    Q, K, V, dO = (t.to(dev) for t in inputs(case))
    c = _ctx(case, Q)
    ref_o, s = ops.layer_fwd(c, Q, K, V)
    ref_g = ops.layer_bwd(c, s, dO.to(c.out))
    torch.cuda.synchronize()
    results, errors = [None, None], []

    def run(i):
        try:
            st = torch.cuda.Stream(device=dev)   # default priority
            with torch.cuda.stream(st):
                outs = []
                for _ in range(3):
                    o, sv = ops.layer_fwd(c, Q, K, V)
                    g = ops.layer_bwd(c, sv, dO.to(c.out))
                    outs.append((o, g))
            st.synchronize()
            results[i] = outs
        except Exception as e:   # reported below
            errors.append(repr(e))

    ts = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for outs in results:
        for o, g in outs:
            assert torch.equal(o, ref_o)
            for a, b in zip(g, ref_g):
                assert torch.equal(a, b)
