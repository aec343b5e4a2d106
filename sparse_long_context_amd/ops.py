"""Torch-facing calls of the C ABI, one per entry point of include/lighthouse.h.

Argument marshalling only: each function checks shapes and dtypes, allocates
its outputs with torch on the inputs' device, and calls the library on the
current stream.  Every stage runs in the library's HIP kernels; there is no
CPU or torch fallback.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib as L

TDT = {L.LH_F32: torch.float32, L.LH_BF16: torch.bfloat16}
LHDT = {torch.float32: L.LH_F32, torch.bfloat16: L.LH_BF16}


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


SCATTER_MODES = {"hold": L.LH_SCATTER_HOLD, "span": L.LH_SCATTER_SPAN}
SIGMA_MODES = {"sum": L.LH_SIGMA_SUM, "max": L.LH_SIGMA_MAX, "product": L.LH_SIGMA_PRODUCT}
STRATA_MODES = {"joint": L.LH_STRATA_JOINT, "per_level": L.LH_STRATA_PER_LEVEL}


def make_dims(q: torch.Tensor, p: int, L_: int, S: int, out_dtype=None, scale: float = 0.0,
              scatter_mode: str = "hold", sigma_mode: str = "sum", strata_mode: str = "joint"):
    """Dims of a call on q [B, H, N, d]; K is S minus the n_c kept roots."""
    B, H, N, d = q.shape
    Bc = p ** (L_ - 1)
    n_c = -(-N // Bc)   # a partial last cell counts (the layer pads it with zero rows)
    io = LHDT[q.dtype]
    out = io if out_dtype is None else LHDT[out_dtype]
    return L.make_dims(B, N, H, d, p, L_, S - n_c, S, io, out, scale, SCATTER_MODES[scatter_mode],
                       SIGMA_MODES[sigma_mode], STRATA_MODES[strata_mode])


class Ctx:
    """Dims plus the derived sizes and dtypes of one call."""

    def __init__(self, dims):
        self.dims = dims
        st = L.validate(dims)
        L.check(st, "lh_validate")
        self.z = L.sizes(dims)
        self.B, self.H, self.N, self.d = dims.B, dims.H, dims.N, dims.d
        self.Np = self.z.n_c * self.z.Bc   # N rounded up to whole coarsest cells
        self.S, self.E, self.Sp = dims.S, self.z.E, self.z.Sp
        self.io, self.out = TDT[dims.io_dtype], TDT[dims.out_dtype]

    def empty(self, *shape, dtype, device):
        return torch.empty(shape, dtype=dtype, device=device)

    def call(self, name, *args):
        L.check(getattr(L.lib(), name)(C.byref(self.dims), *args), name)


def _bh(c: Ctx):
    return (c.B, c.H)


def pyramid_score(c: Ctx, q, k, v):
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need(t, _bh(c) + (c.N, c.d), c.io, n)
    pq, pk, pv = (c.empty(*_bh(c), c.E - c.Np, c.d, dtype=c.io, device=dev) for _ in range(3))
    sq, sk = (c.empty(*_bh(c), c.E, dtype=torch.float32, device=dev) for _ in range(2))
    c.call("lh_pyramid_score", _ptr(q), _ptr(k), _ptr(v), _ptr(pq), _ptr(pk), _ptr(pv),
           _ptr(sq), _ptr(sk), _stream())
    return pq, pk, pv, sq, sk


def pyramid_build(c: Ctx, q=None, k=None, v=None):
    outs = []
    for n, t in (("q", q), ("k", k), ("v", v)):
        if t is not None:
            _need(t, _bh(c) + (c.N, c.d), c.io, n)
            outs.append(c.empty(*_bh(c), c.E - c.Np, c.d, dtype=c.io, device=t.device))
        else:
            outs.append(None)
    c.call("lh_pyramid_build", _ptr(q), _ptr(k), _ptr(v), *(_ptr(o) for o in outs), _stream())
    return tuple(outs)


def score(c: Ctx, q, k):
    _need(q, _bh(c) + (c.N, c.d), c.io, "q")
    _need(k, _bh(c) + (c.N, c.d), c.io, "k")
    sq, sk = (c.empty(*_bh(c), c.E, dtype=torch.float32, device=q.device) for _ in range(2))
    c.call("lh_score", _ptr(q), _ptr(k), _ptr(sq), _ptr(sk), _stream())
    return sq, sk


def topk_select(c: Ctx, sq, sk):
    _need(sq, _bh(c) + (c.E,), torch.float32, "sq")
    _need(sk, _bh(c) + (c.E,), torch.float32, "sk")
    dev = sq.device
    idx = c.empty(*_bh(c), c.S, dtype=torch.int32, device=dev)
    anc = c.empty(*_bh(c), c.S, dtype=torch.int32, device=dev)
    flags = c.empty(*_bh(c), c.S, dtype=torch.uint8, device=dev)
    row_of = c.empty(*_bh(c), c.E, dtype=torch.int32, device=dev)
    c.call("lh_topk_select", _ptr(sq), _ptr(sk), _ptr(idx), _ptr(anc), _ptr(flags), _ptr(row_of),
           _stream())
    return idx, anc, flags, row_of


def gather(c: Ctx, q, k, v, pq, pk, pv, sel_idx, transposed=False):
    dev = q.device
    _need(sel_idx, _bh(c) + (c.S,), torch.int32, "sel_idx")
    qs, ks, vs = (c.empty(*_bh(c), c.S, c.d, dtype=c.io, device=dev) for _ in range(3))
    tr = [None, None, None]
    if transposed:
        tr = [torch.empty(*_bh(c), c.d, c.Sp, dtype=c.io, device=dev) for _ in range(3)]
    c.call("lh_gather", _ptr(q), _ptr(k), _ptr(v), _ptr(pq), _ptr(pk), _ptr(pv), _ptr(sel_idx),
           _ptr(qs), _ptr(ks), _ptr(vs), *(_ptr(t) for t in tr), _stream())
    return (qs, ks, vs) + (tuple(tr) if transposed else ())


def subseq_attn_fwd(c: Ctx, qs, ks, vs, flags):
    dev = qs.device
    for n, t in (("qs", qs), ("ks", ks), ("vs", vs)):
        _need(t, _bh(c) + (c.S, c.d), c.io, n)
    _need(flags, _bh(c) + (c.S,), torch.uint8, "sel_flags")
    os_ = c.empty(*_bh(c), c.S, c.d, dtype=torch.float32, device=dev)
    lse = c.empty(*_bh(c), c.S, dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, c.z.ws_attn_fwd), dtype=torch.uint8, device=dev)
    c.call("lh_subseq_attn_fwd", _ptr(qs), _ptr(ks), _ptr(vs), _ptr(flags), _ptr(os_), _ptr(lse),
           _ptr(ws), C.c_size_t(c.z.ws_attn_fwd), _stream())
    return os_, lse


def subseq_attn_bwd(c: Ctx, qs, ks, vs, os_, lse, flags, dos):
    dev = qs.device
    _need(dos, _bh(c) + (c.S, c.d), torch.float32, "dos")
    _need(os_, _bh(c) + (c.S, c.d), torch.float32, "os")
    dqs, dks, dvs = (c.empty(*_bh(c), c.S, c.d, dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(max(1, c.z.ws_attn_bwd), dtype=torch.uint8, device=dev)
    c.call("lh_subseq_attn_bwd", _ptr(qs), _ptr(ks), _ptr(vs), _ptr(os_), _ptr(lse), _ptr(flags),
           _ptr(dos), _ptr(dqs), _ptr(dks), _ptr(dvs), _ptr(ws), C.c_size_t(c.z.ws_attn_bwd),
           _stream())
    return dqs, dks, dvs


def subseq_attn_bwd_noalloc(c: Ctx, qs, ks, vs, os_, lse, flags, dos, outs=None):
    """lh_subseq_attn_bwd_noalloc: the same backward with the library's fixed
    scratch array instead of a workspace (outputs may be passed in)."""
    dev = qs.device
    _need(dos, _bh(c) + (c.S, c.d), torch.float32, "dos")
    _need(os_, _bh(c) + (c.S, c.d), torch.float32, "os")
    if outs is None:
        outs = [c.empty(*_bh(c), c.S, c.d, dtype=torch.float32, device=dev) for _ in range(3)]
    for n, t in zip(("dqs", "dks", "dvs"), outs):
        _need(t, _bh(c) + (c.S, c.d), torch.float32, n)
    dqs, dks, dvs = outs
    c.call("lh_subseq_attn_bwd_noalloc", _ptr(qs), _ptr(ks), _ptr(vs), _ptr(os_), _ptr(lse),
           _ptr(flags), _ptr(dos), _ptr(dqs), _ptr(dks), _ptr(dvs), _stream())
    return dqs, dks, dvs


def attn_bwd_prep(c: Ctx, dos, os_):
    """Operands of the two backward MFMA kernels (bf16 I/O only): the
    two-term bf16 split of dOS and drow = rowsum(dOS * OS)."""
    dev = dos.device
    hi, lo = (c.empty(*_bh(c), c.S, c.d, dtype=torch.bfloat16, device=dev) for _ in range(2))
    drow = c.empty(*_bh(c), c.S, dtype=torch.float32, device=dev)
    c.call("lh_attn_bwd_prep", _ptr(dos), _ptr(os_), _ptr(hi), _ptr(lo), _ptr(drow), _stream())
    return hi, lo, drow


def attn_fwd_mfma(c: Ctx, qs, ks, vs, flags, os_=None, lse=None):
    dev = qs.device
    os_ = c.empty(*_bh(c), c.S, c.d, dtype=torch.float32, device=dev) if os_ is None else os_
    lse = c.empty(*_bh(c), c.S, dtype=torch.float32, device=dev) if lse is None else lse
    c.call("lh_attn_fwd_mfma", _ptr(qs), _ptr(ks), _ptr(vs), _ptr(flags), _ptr(os_), _ptr(lse),
           _stream())
    return os_, lse


def attn_bwd_dkv_mfma(c: Ctx, qs, ks, vs, hi, lo, lse, drow, flags, dks=None, dvs=None):
    dev = qs.device
    dks = c.empty(*_bh(c), c.S, c.d, dtype=torch.float32, device=dev) if dks is None else dks
    dvs = c.empty(*_bh(c), c.S, c.d, dtype=torch.float32, device=dev) if dvs is None else dvs
    c.call("lh_attn_bwd_dkv_mfma", _ptr(qs), _ptr(ks), _ptr(vs), _ptr(hi), _ptr(lo), _ptr(lse),
           _ptr(drow), _ptr(flags), _ptr(dks), _ptr(dvs), _stream())
    return dks, dvs


def attn_bwd_dq_mfma(c: Ctx, qs, ks, vs, hi, lo, lse, drow, flags, dqs=None):
    dev = qs.device
    dqs = c.empty(*_bh(c), c.S, c.d, dtype=torch.float32, device=dev) if dqs is None else dqs
    c.call("lh_attn_bwd_dq_mfma", _ptr(qs), _ptr(ks), _ptr(vs), _ptr(hi), _ptr(lo), _ptr(lse),
           _ptr(drow), _ptr(flags), _ptr(dqs), _stream())
    return dqs


def scatter(c: Ctx, os_, sel_anchor, sel_flags):
    _need(os_, _bh(c) + (c.S, c.d), torch.float32, "os")
    o = c.empty(*_bh(c), c.N, c.d, dtype=c.out, device=os_.device)
    c.call("lh_scatter", _ptr(os_), _ptr(sel_anchor), _ptr(sel_flags), _ptr(o), _stream())
    return o


def scatter_bwd(c: Ctx, dout, sel_anchor, sel_flags):
    _need(dout, _bh(c) + (c.N, c.d), c.out, "dout")
    dos = c.empty(*_bh(c), c.S, c.d, dtype=torch.float32, device=dout.device)
    c.call("lh_scatter_bwd", _ptr(dout), _ptr(sel_anchor), _ptr(sel_flags), _ptr(dos), _stream())
    return dos


def gather_bwd(c: Ctx, dqs, dks, dvs, row_of):
    dev = dqs.device
    outs = [c.empty(*_bh(c), c.N, c.d, dtype=c.out, device=dev) for _ in range(3)]
    c.call("lh_gather_bwd", _ptr(dqs), _ptr(dks), _ptr(dvs), _ptr(row_of),
           *(_ptr(o) for o in outs), _stream())
    return tuple(outs)


SAVED_FIELDS = [f for f, _ in L.Saved._fields_]


def alloc_saved(c: Ctx, device):
    """Buffers a forward fills and the backward reads."""
    bh = _bh(c)
    s = {
        "pq": None, "pk": None, "pv": None,
        "sq": torch.empty(*bh, c.E, dtype=torch.float32, device=device),
        "sk": torch.empty(*bh, c.E, dtype=torch.float32, device=device),
        "sel_idx": torch.empty(*bh, c.S, dtype=torch.int32, device=device),
        "sel_anchor": torch.empty(*bh, c.S, dtype=torch.int32, device=device),
        "sel_flags": torch.empty(*bh, c.S, dtype=torch.uint8, device=device),
        "row_of": torch.empty(*bh, c.E, dtype=torch.int32, device=device),
        "os": torch.empty(*bh, c.S, c.d, dtype=torch.float32, device=device),
        "lse": torch.empty(*bh, c.S, dtype=torch.float32, device=device),
        "qst": None, "kst": None, "vst": None,
    }
    if c.E > c.Np:
        for n in ("pq", "pk", "pv"):
            s[n] = torch.empty(*bh, c.E - c.Np, c.d, dtype=c.io, device=device)
    for n in ("qs", "ks", "vs"):
        s[n] = torch.empty(*bh, c.S, c.d, dtype=c.io, device=device)
    return s


def _saved_struct(s):
    return L.Saved(*[None if s[f] is None else s[f].data_ptr() for f in SAVED_FIELDS])


def span_owner(c: Ctx, row_of):
    owner = c.empty(*_bh(c), c.N, dtype=torch.int32, device=row_of.device)
    c.call("lh_span_owner", _ptr(row_of), _ptr(owner), _stream())
    return owner


def scatter_span(c: Ctx, os_, owner):
    _need(os_, _bh(c) + (c.S, c.d), torch.float32, "os")
    o = c.empty(*_bh(c), c.N, c.d, dtype=c.out, device=os_.device)
    c.call("lh_scatter_span", _ptr(os_), _ptr(owner), _ptr(o), _stream())
    return o


def scatter_span_bwd(c: Ctx, dout, sel_idx, sel_flags, owner):
    _need(dout, _bh(c) + (c.N, c.d), c.out, "dout")
    dos = c.empty(*_bh(c), c.S, c.d, dtype=torch.float32, device=dout.device)
    c.call("lh_scatter_span_bwd", _ptr(dout), _ptr(sel_idx), _ptr(sel_flags), _ptr(owner),
           _ptr(dos), _stream())
    return dos


def layer_fwd(c: Ctx, q, k, v, saved=None, o=None):
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need(t, _bh(c) + (c.N, c.d), c.io, n)
    saved = alloc_saved(c, dev) if saved is None else saved
    o = c.empty(*_bh(c), c.N, c.d, dtype=c.out, device=dev) if o is None else o
    st = _saved_struct(saved)
    nws = c.z.ws_layer_fwd
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    c.call("lh_layer_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), C.byref(st),
           None if ws is None else _ptr(ws), C.c_size_t(nws), _stream())
    return o, saved


def layer_bwd(c: Ctx, saved, dout, ws=None, outs=None):
    dev = dout.device
    _need(dout, _bh(c) + (c.N, c.d), c.out, "dout")
    if ws is None:
        ws = torch.empty(max(1, c.z.ws_layer_bwd), dtype=torch.uint8, device=dev)
    if outs is None:
        outs = [c.empty(*_bh(c), c.N, c.d, dtype=c.out, device=dev) for _ in range(3)]
    st = _saved_struct(saved)
    c.call("lh_layer_bwd", C.byref(st), _ptr(dout), *(_ptr(o) for o in outs), _ptr(ws),
           C.c_size_t(ws.numel()), _stream())
    return tuple(outs)
