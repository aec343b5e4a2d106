"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, and its host-side validation returns the documented codes without
launching anything (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

from sparse_long_context_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lighthouse.h")


def header_symbols():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lh_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("liblighthouse.so not built (python -m sparse_long_context_amd.build)")
    return L.lib()


def test_exports_every_declared_symbol(lib):
    syms = header_symbols()
    assert len(syms) >= 16
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(L.EXPORTS)
    assert lib.lh_version().decode().count(".") == 2


def dims(**kw):
    base = dict(B=1, N=4096, H=2, d=64, p=4, L=3, K=256, S=512, io_dtype=L.LH_F32,
                out_dtype=L.LH_F32, scale=0.0)
    base.update(kw)
    return L.Dims(base["B"], base["N"], base["H"], base["d"], base["p"], base["L"], base["K"],
                  base["S"], base["io_dtype"], base["out_dtype"], base["scale"], 0)


@pytest.mark.parametrize("kw,code", [
    ({}, L.LH_OK),
    (dict(io_dtype=L.LH_BF16, out_dtype=L.LH_BF16), L.LH_OK),
    (dict(io_dtype=L.LH_BF16, out_dtype=L.LH_F32), L.LH_OK),
    (dict(N=4100, K=257, S=514), L.LH_OK),            # N % p^(L-1): padded to 4112
    (dict(N=4100), L.LH_ERR_INVALID_ARG),             # K % n_c with n_c = 257
    (dict(K=255, S=511), L.LH_ERR_INVALID_ARG),       # K % n_c
    (dict(K=256, S=513), L.LH_ERR_INVALID_ARG),       # S != K + n_c
    (dict(K=21 * 256, S=22 * 256), L.LH_ERR_INVALID_ARG),   # k_s > T-1
    (dict(K=20 * 256, S=21 * 256), L.LH_OK),          # k_s = T-1: everything selected
    (dict(K=0, S=256), L.LH_OK),                      # coarsest only
    (dict(p=1), L.LH_ERR_INVALID_ARG),
    (dict(L=0), L.LH_ERR_INVALID_ARG),
    (dict(B=0), L.LH_ERR_INVALID_ARG),
    (dict(d=96), L.LH_ERR_UNSUPPORTED),
    (dict(d=0), L.LH_ERR_INVALID_ARG),
    (dict(io_dtype=7), L.LH_ERR_INVALID_ARG),
    (dict(out_dtype=L.LH_BF16), L.LH_ERR_UNSUPPORTED),  # f32 in, bf16 out
    (dict(scale=-1.0), L.LH_ERR_INVALID_ARG),
    (dict(scale=float("nan")), L.LH_ERR_INVALID_ARG),
    (dict(N=2 ** 31, K=0, S=2 ** 27), L.LH_ERR_UNSUPPORTED),   # E >= 2^31
    (dict(p=2, L=14, N=2 ** 14, K=0, S=2), L.LH_ERR_UNSUPPORTED),  # subtree too large
])
def test_validate(lib, kw, code):
    assert lib.lh_validate(C.byref(dims(**kw))) == code


def test_validate_null_and_scatter_mode(lib):
    assert lib.lh_validate(None) == L.LH_ERR_INVALID_ARG
    d = dims()
    for mode, code in ((L.LH_SCATTER_HOLD, L.LH_OK), (L.LH_SCATTER_SPAN, L.LH_OK), (2, L.LH_ERR_INVALID_ARG),
                       (-1, L.LH_ERR_INVALID_ARG)):
        d.scatter_mode = mode
        assert lib.lh_validate(C.byref(d)) == code, mode


def test_validate_sigma_mode(lib):
    d = dims()
    for mode, code in ((L.LH_SIGMA_SUM, L.LH_OK), (L.LH_SIGMA_MAX, L.LH_OK),
                       (L.LH_SIGMA_PRODUCT, L.LH_OK), (3, L.LH_ERR_INVALID_ARG),
                       (-1, L.LH_ERR_INVALID_ARG)):
        d.sigma_mode = mode
        assert lib.lh_validate(C.byref(d)) == code, mode


def test_validate_strata_mode(lib):
    d = dims()
    for mode, code in ((L.LH_STRATA_JOINT, L.LH_OK), (L.LH_STRATA_PER_LEVEL, L.LH_OK),
                       (2, L.LH_ERR_INVALID_ARG), (-1, L.LH_ERR_INVALID_ARG)):
        d.strata_mode = mode
        assert lib.lh_validate(C.byref(d)) == code, mode
    # the largest budget of the 128K workload's trees is feasible per level
    d = dims(N=131072, H=8, d=128, p=4, L=6, K=1365 * 128 - 128, S=1365 * 128,
             io_dtype=L.LH_BF16, out_dtype=L.LH_BF16)
    d.strata_mode = L.LH_STRATA_PER_LEVEL
    assert lib.lh_validate(C.byref(d)) == L.LH_OK


def test_span_mode_workspace_holds_the_owner_map(lib):
    d = dims(N=131072, H=8, d=128, p=4, L=6, K=8064, S=8192, io_dtype=L.LH_BF16,
             out_dtype=L.LH_BF16)
    hold, span = L.Sizes(), L.Sizes()
    assert lib.lh_get_sizes(C.byref(d), C.byref(hold)) == L.LH_OK
    d.scatter_mode = L.LH_SCATTER_SPAN
    assert lib.lh_get_sizes(C.byref(d), C.byref(span)) == L.LH_OK
    owner = 8 * 131072 * 4
    assert hold.owner_bytes == span.owner_bytes == owner
    assert hold.ws_layer_fwd == 0 and span.ws_layer_fwd >= owner
    assert span.ws_layer_bwd >= hold.ws_layer_bwd + owner


def test_forward_attention_needs_no_workspace(lib):
    # the MFMA forward reads the gathered V rows directly (no transposed copy)
    for io in (L.LH_F32, L.LH_BF16):
        z = L.Sizes()
        assert lib.lh_get_sizes(C.byref(dims(io_dtype=io, out_dtype=io)), C.byref(z)) == L.LH_OK
        assert z.ws_attn_fwd == 0


def test_sizes_c4_shape(lib):
    d = dims(N=131072, H=8, d=128, p=4, L=6, K=8064, S=8192, io_dtype=L.LH_BF16,
             out_dtype=L.LH_BF16)
    z = L.Sizes()
    assert lib.lh_get_sizes(C.byref(d), C.byref(z)) == L.LH_OK
    assert (z.E, z.n_c, z.T, z.k_s, z.Bc, z.Sp) == (174720, 128, 1365, 63, 1024, 8192)
    assert z.pyramid_bytes == 8 * (174720 - 131072) * 128 * 2
    assert z.score_bytes == 8 * 174720 * 4
    assert z.token_io_bytes == 8 * 131072 * 128 * 2
    assert z.ws_layer_fwd == 0 and z.ws_layer_bwd > 4 * 8 * 8192 * 128 * 4


def test_sizes_of_a_partial_last_cell(lib):
    # N = 4100 with B_c = 16: the geometry is that of 4112 tokens (257 cells);
    # token tensors keep 4100 rows; the layer workspaces hold the padded
    # copies (q, k, v, o forward; dO, dQ, dK, dV backward)
    whole, rag = L.Sizes(), L.Sizes()
    assert lib.lh_get_sizes(C.byref(dims(N=4112, K=257, S=514)), C.byref(whole)) == L.LH_OK
    assert lib.lh_get_sizes(C.byref(dims(N=4100, K=257, S=514)), C.byref(rag)) == L.LH_OK
    assert (rag.E, rag.n_c, rag.T, rag.k_s, rag.Sp) == (whole.E, whole.n_c, whole.T, whole.k_s,
                                                       whole.Sp)
    assert rag.pyramid_bytes == whole.pyramid_bytes and rag.row_of_bytes == whole.row_of_bytes
    assert rag.token_io_bytes == 2 * 4100 * 64 * 4
    padded = 2 * 4112 * 64 * 4
    assert rag.ws_layer_fwd == whole.ws_layer_fwd + 4 * padded
    assert rag.ws_layer_bwd == whole.ws_layer_bwd + 4 * padded


def test_ragged_sp(lib):
    d = dims(N=2560, p=8, L=3, K=40 * 12, S=40 * 13, io_dtype=L.LH_BF16, out_dtype=L.LH_BF16)
    z = L.Sizes()
    assert lib.lh_get_sizes(C.byref(d), C.byref(z)) == L.LH_OK
    assert z.Sp == 576


def test_stage_calls_reject_bad_args_without_launch(lib):
    d = dims()
    P = C.c_void_p
    # null pointers: rejected by host validation, nothing is launched
    assert lib.lh_pyramid_score(C.byref(d), *([None] * 8), None) == L.LH_ERR_INVALID_ARG
    assert lib.lh_topk_select(C.byref(d), *([None] * 6), None) == L.LH_ERR_INVALID_ARG
    assert lib.lh_scatter(C.byref(d), *([None] * 4), None) == L.LH_ERR_INVALID_ARG
    assert lib.lh_layer_fwd(C.byref(d), None, None, None, None, None, None, 0, None) == \
        L.LH_ERR_INVALID_ARG
    # misaligned pointer
    bad = P(0x1003)
    assert lib.lh_scatter(C.byref(d), bad, bad, bad, bad, None) == L.LH_ERR_INVALID_ARG
    # invalid dims come first
    dd = dims(N=4100)
    assert lib.lh_scatter(C.byref(dd), P(0x1000), P(0x1000), P(0x1000), P(0x1000), None) == \
        L.LH_ERR_INVALID_ARG
    # missing workspace
    d2 = dims(io_dtype=L.LH_BF16, out_dtype=L.LH_BF16)
    p = P(0x10000)
    assert lib.lh_subseq_attn_bwd(C.byref(d2), *([p] * 10), None, 0, None) == \
        L.LH_ERR_WORKSPACE
    s = L.Saved(*([0x10000] * 17))
    assert lib.lh_layer_bwd(C.byref(d2), C.byref(s), p, p, p, p, None, 0, None) == \
        L.LH_ERR_WORKSPACE
    # span mode: the forward needs a workspace for the owner map
    d3 = dims(io_dtype=L.LH_BF16, out_dtype=L.LH_BF16)
    d3.scatter_mode = L.LH_SCATTER_SPAN
    assert lib.lh_layer_fwd(C.byref(d3), p, p, p, p, C.byref(s), None, 0, None) == \
        L.LH_ERR_WORKSPACE
    # span-mode stage calls
    assert lib.lh_span_owner(C.byref(d), None, p, None) == L.LH_ERR_INVALID_ARG
    assert lib.lh_span_owner(C.byref(d), p, bad, None) == L.LH_ERR_INVALID_ARG
    assert lib.lh_scatter_span(C.byref(d), p, p, None, None) == L.LH_ERR_INVALID_ARG
    assert lib.lh_scatter_span(C.byref(d), bad, p, p, None) == L.LH_ERR_INVALID_ARG
    assert lib.lh_scatter_span_bwd(C.byref(d), p, p, p, None, p, None) == L.LH_ERR_INVALID_ARG
    assert lib.lh_scatter_span_bwd(C.byref(dd), p, p, p, p, p, None) == L.LH_ERR_INVALID_ARG


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -99):
        assert len(lib.lh_status_string(s)) > 0


def test_mfma_probe_rejects_bad_args_without_launch(lib):
    buf = C.c_void_p(0x1000)   # never dereferenced: every case fails validation first
    for blocks, iters, out in ((0, 10, buf), (-1, 10, buf), (1 << 31, 10, buf), (8, 0, buf),
                               (8, 10, None)):
        st = lib.lh_probe_mfma_bf16(blocks, iters, out, None)
        assert st == L.LH_ERR_INVALID_ARG, (blocks, iters, out, st)


@pytest.mark.parametrize("d,S", [(128, 524288), (128, 1048576), (64, 1048576)])
def test_validate_rejects_what_the_attention_kernels_cannot_launch(lib, d, S):
    """L = 1 (dense, S = N) with bf16 I/O: the forward and dQ kernels keep one
    REDUNDANT bit per key in LDS beside their rings, so past about 490,000
    keys at d = 128 (more at d = 64) they do not fit; lh_validate must say so,
    and the layer calls must return the same code before launching anything
    (every pointer below is a fake address that is never dereferenced)."""
    dd = dims(N=S, H=1, d=d, p=2, L=1, K=0, S=S, io_dtype=L.LH_BF16, out_dtype=L.LH_BF16)
    assert lib.lh_validate(C.byref(dd)) == L.LH_ERR_UNSUPPORTED
    p = C.c_void_p(0x10000)
    s = L.Saved(*([0x10000] * 17))
    assert lib.lh_layer_fwd(C.byref(dd), p, p, p, p, C.byref(s), None, 0, None) == \
        L.LH_ERR_UNSUPPORTED
    assert lib.lh_layer_bwd(C.byref(dd), C.byref(s), p, p, p, p, p, 1 << 40, None) == \
        L.LH_ERR_UNSUPPORTED
    assert lib.lh_attn_fwd_mfma(C.byref(dd), p, p, p, p, p, p, None) == L.LH_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(N=262144, H=1, d=128, p=2, L=1, K=0, S=262144),   # forward and dQ LDS fit
    dict(N=131072, H=8, d=128, p=4, L=6, K=8064, S=8192),  # the 128K workload
    dict(N=1048576, H=4, d=128, p=8, L=5, K=16128, S=16384),
])
def test_validate_accepts_the_workload_shapes(lib, kw):
    dd = dims(io_dtype=L.LH_BF16, out_dtype=L.LH_BF16, **kw)
    assert lib.lh_validate(C.byref(dd)) == L.LH_OK


def test_validate_rejects_grids_past_32_bits(lib):
    """64 work-items per subsequence row of every head in one dimension (the
    dO split of the attention backward) must fit 32 bits."""
    dd = dims(B=1, N=2 ** 20, H=1024, d=64, p=4, L=3, K=3 * 2 ** 16, S=2 ** 18,
              io_dtype=L.LH_BF16, out_dtype=L.LH_BF16)
    assert lib.lh_validate(C.byref(dd)) == L.LH_ERR_UNSUPPORTED
    dd.H = 256   # 64 * 256 * 2^18 = 2^32: one past the limit
    assert lib.lh_validate(C.byref(dd)) == L.LH_ERR_UNSUPPORTED
    dd.H = 128
    assert lib.lh_validate(C.byref(dd)) == L.LH_OK


def test_stream_probe_rejects_bad_args_without_launch(lib):
    p = C.c_void_p(0x1000)   # never dereferenced: every case fails validation first
    for mode, src, dst, nbytes, blocks in ((3, p, p, 4096, 8), (0, None, p, 4096, 8),
                                           (0, p, None, 4096, 8), (1, p, p, 4100, 8),
                                           (2, None, p, 0, 8), (0, p, p, 4096, 0),
                                           (0, p, p, 4096, 1 << 24), (0, C.c_void_p(0x1008), p, 4096, 8)):
        st = lib.lh_probe_stream(mode, src, dst, nbytes, blocks, None)
        assert st == L.LH_ERR_INVALID_ARG, (mode, nbytes, blocks, st)
