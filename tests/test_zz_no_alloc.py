"""lh_subseq_attn_bwd_noalloc (the attention backward whose scratch is the
library's fixed device array, for callers that cannot allocate) against
lh_subseq_attn_bwd (the same kernels with a caller workspace), through the C
ABI: the results must be identical, on two calls in a row whose second input
is smaller (the array keeps the first call's contents), and a call whose
scratch would exceed the array must be refused without a launch."""
import ctypes as C

import pytest
import torch

from sparse_long_context_amd import _lib as L
from tests.gpu_cases import inputs, Case

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_long_context_amd import ops

BIG = Case("noalloc-big", 8192, 3, 128, 4, 4, 20, structure="spikes", seed=77)
SMALL = Case("noalloc-small", 2048, 2, 64, 4, 3, 7, structure="bursts", seed=78)


def _operands(case, dev):
    Q, K, V, dO = (t.to(dev) for t in inputs(case))
    c = ops.Ctx(ops.make_dims(Q, case.p, case.L, case.S, out_dtype=torch.float32))
    pq, pk, pv, sq, sk = ops.pyramid_score(c, Q, K, V)
    idx, anc, fl, _ = ops.topk_select(c, sq, sk)
    qs, ks, vs = ops.gather(c, Q, K, V, pq, pk, pv, idx)[:3]
    os_, lse = ops.subseq_attn_fwd(c, qs, ks, vs, fl)
    dos = ops.scatter_bwd(c, dO.to(torch.float32), anc, fl)
    return c, (qs, ks, vs, os_, lse, fl, dos)


def test_noalloc_matches_workspace_form_twice_shrinking():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    for case in (BIG, SMALL):
        print(f"[noalloc] {case.name}", flush=True)
        c, args = _operands(case, dev)
        assert c.z.ws_attn_bwd <= L.LH_NOALLOC_SCRATCH_BYTES
        want = ops.subseq_attn_bwd(c, *args)
        got = ops.subseq_attn_bwd_noalloc(c, *args)
        torch.cuda.synchronize()
        for n, a, b in zip(("dqs", "dks", "dvs"), got, want):
            assert torch.equal(a, b), f"{case.name} {n}: max diff {(a - b).abs().max().item()}"


def test_noalloc_rejects_scratch_beyond_the_array():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    # bf16 I/O: the dO split and drow take 4 S d + 4 S bytes per head
    S = 262144
    dims = L.make_dims(1, S, 1, 128, 2, 1, 0, S, L.LH_BF16, L.LH_F32)
    assert L.sizes(dims).ws_attn_bwd > L.LH_NOALLOC_SCRATCH_BYTES
    p = C.c_void_p(0x10000)   # never dereferenced: refused before any launch
    st = L.lib().lh_subseq_attn_bwd_noalloc(C.byref(dims), *([p] * 10), None)
    assert st == L.LH_ERR_UNSUPPORTED
