"""Pins of the oracle's hand-written backward.

(1) central finite differences in float64 on tiny inputs, with the
    selection checked unchanged at +-h (both scatter modes);
(2) autograd through an independent plain-torch float64 forward of the
    layer on the same selection (pooling by avg_pool1d over whole spans,
    index_select gathers, a masked softmax, and a hold map built with a
    cumulative max), general case;
(3) the full-selection case against torch's SDPA autograd.
"""
import numpy as np
import pytest
import torch

from oracle import lighthouse as orc


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("mode", ["hold", "span"])
def test_finite_differences(mode):
    N, p, L, d, ks = 32, 2, 3, 4, 3
    g = orc.Geometry(N, p, L, ks * (N // 4)).check()
    Q, K, V, dO = (rnd((N, d), s) for s in (1, 2, 3, 4))
    fw = orc.head_forward(Q, K, V, g, scatter_mode=mode)
    dQ, dK, dV = orc.head_backward(fw, dO)[:3]
    h = 1e-6
    X = [Q, K, V]
    for which, grad in enumerate((dQ, dK, dV)):
        for t in range(N):
            for c in range(d):
                outs = []
                for sgn in (1, -1):
                    Xs = [x.copy() for x in X]
                    Xs[which][t, c] += sgn * h
                    f2 = orc.head_forward(*Xs, g, scatter_mode=mode)
                    assert np.array_equal(f2.sel.sel_idx, fw.sel.sel_idx)
                    outs.append(np.sum(f2.O * dO))
                fd = (outs[0] - outs[1]) / (2 * h)
                assert abs(fd - grad[t, c]) < 1e-6 * (1 + abs(fd)), (which, t, c, fd, grad[t, c])


@pytest.mark.parametrize("mode", ["hold", "span"])
def test_finite_differences_ragged_length(mode):
    # R-19: N = 27 with B_c = 4 runs on 28 tokens; the gradients of the 27
    # real tokens against central differences of sum(O_real * dO)
    N, p, L, d = 27, 2, 3, 3
    Np = orc.padded_length(N, p, L)
    K = 2 * (Np // 4)
    Q, K_, V, dO = (rnd((N, d), s) for s in (11, 12, 13, 14))
    fw, O = orc.ragged_forward(Q, K_, V, p, L, K, scatter_mode=mode)
    grads = orc.ragged_backward(fw, dO)
    h = 1e-6
    X = [Q, K_, V]
    for which, grad in enumerate(grads):
        assert grad.shape == (N, d)
        for t in range(N):
            for c in range(d):
                outs = []
                for sgn in (1, -1):
                    Xs = [x.copy() for x in X]
                    Xs[which][t, c] += sgn * h
                    f2, O2 = orc.ragged_forward(*Xs, p, L, K, scatter_mode=mode)
                    assert np.array_equal(f2.sel.sel_idx, fw.sel.sel_idx)
                    outs.append(np.sum(O2 * dO))
                fd = (outs[0] - outs[1]) / (2 * h)
                assert abs(fd - grad[t, c]) < 1e-6 * (1 + abs(fd)), (which, t, c, fd, grad[t, c])


def torch_layer(Q, K, V, g, sel_idx, flags, scale):
    """Independent float64 torch forward for a fixed selection."""
    N, d = Q.shape
    red = torch.from_numpy((flags & orc.FLAG_REDUNDANT) != 0)
    lead = torch.from_numpy((flags & orc.FLAG_LEADER) != 0)

    def pyr(X):
        rows = [X]
        for l in range(1, g.L):
            w = g.p ** l
            rows.append(torch.nn.functional.avg_pool1d(X.T[None], w, w)[0].T)
        return torch.cat(rows, 0)

    idx = torch.from_numpy(np.asarray(sel_idx, np.int64))
    QS, KS, VS = (pyr(X).index_select(0, idx) for X in (Q, K, V))
    S = QS.shape[0]
    s = scale * QS @ KS.T
    jj = torch.arange(S)
    ok = (jj[None, :] <= jj[:, None]) & ~red[None, :]
    P = torch.softmax(s.masked_fill(~ok, float("-inf")), dim=1)
    OS = P @ VS
    # anchors from levels/positions, then the hold map by a running max
    lev = np.zeros(S, np.int64)
    for l, o in enumerate(g.level_offsets):
        lev[np.asarray(sel_idx) >= o] = l
    pos = np.asarray(sel_idx) - np.asarray(g.level_offsets)[lev]
    anc = (pos + 1) * g.p ** lev - 1
    mark = torch.full((N,), -1, dtype=torch.int64)
    for j in range(S):
        if lead[j]:
            mark[anc[j]] = j
    src = torch.cummax(mark, 0).values
    O = torch.where((src >= 0)[:, None], OS[src.clamp(min=0)], torch.zeros(1, dtype=OS.dtype))
    return O


@pytest.mark.parametrize("N,p,L,ks,d", [(256, 4, 4, 9, 8), (128, 2, 5, 7, 4), (512, 8, 3, 17, 6)])
def test_backward_vs_independent_torch_autograd(N, p, L, ks, d):
    g = orc.Geometry(N, p, L, ks * (N // p ** (L - 1))).check()
    Q, K, V, dO = (rnd((N, d), s) for s in (5, 6, 7, 8))
    Q[::17] *= 4                           # some larger-norm rows
    fw = orc.head_forward(Q, K, V, g)
    dQ, dK, dV = orc.head_backward(fw, dO)[:3]
    tQ, tK, tV = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    O = torch_layer(tQ, tK, tV, g, fw.sel.sel_idx, fw.sel.sel_flags, fw.scale)
    np.testing.assert_allclose(O.detach().numpy(), fw.O, rtol=0, atol=1e-12)
    (O * torch.from_numpy(dO)).sum().backward()
    for a, b in ((tQ.grad, dQ), (tK.grad, dK), (tV.grad, dV)):
        np.testing.assert_allclose(a.numpy(), b, rtol=0, atol=1e-11)


def test_full_selection_backward_is_sdpa_backward():
    N, p, L, d = 64, 2, 3, 8
    g = orc.Geometry(N, p, L, (g_T := 6) * (N // 4)).check()
    Q, K, V, dO = (rnd((N, d), s) for s in (9, 10, 11, 12))
    fw = orc.head_forward(Q, K, V, g)
    dQ, dK, dV = orc.head_backward(fw, dO)[:3]
    tQ, tK, tV = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    O = torch.nn.functional.scaled_dot_product_attention(tQ[None], tK[None], tV[None], is_causal=True)[0]
    (O * torch.from_numpy(dO)).sum().backward()
    for a, b in ((tQ.grad, dQ), (tK.grad, dK), (tV.grad, dV)):
        np.testing.assert_allclose(a.numpy(), b, rtol=0, atol=1e-12)
