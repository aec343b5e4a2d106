"""ctypes binding of liblighthouse.so (include/lighthouse.h).

Argument marshalling only: structs and prototypes mirroring the header, and
a loader that raises when the library is missing.  There is no fallback
path: every stage runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblighthouse.so")

LH_OK, LH_ERR_INVALID_ARG, LH_ERR_UNSUPPORTED, LH_ERR_WORKSPACE, LH_ERR_HIP = 0, -1, -2, -3, -4
LH_F32, LH_BF16 = 0, 1
LH_ROW_REDUNDANT, LH_ROW_LEADER = 1, 2
LH_SCATTER_HOLD, LH_SCATTER_SPAN = 0, 1
LH_SIGMA_SUM, LH_SIGMA_MAX, LH_SIGMA_PRODUCT = 0, 1, 2
LH_STRATA_JOINT, LH_STRATA_PER_LEVEL = 0, 1
LH_NOALLOC_SCRATCH_BYTES = 80 << 20


class LighthouseError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


class Dims(C.Structure):
    _fields_ = [("B", C.c_int64), ("N", C.c_int64), ("H", C.c_int32), ("d", C.c_int32),
                ("p", C.c_int32), ("L", C.c_int32), ("K", C.c_int64), ("S", C.c_int64),
                ("io_dtype", C.c_int32), ("out_dtype", C.c_int32), ("scale", C.c_float),
                ("scatter_mode", C.c_int32), ("sigma_mode", C.c_int32),
                ("strata_mode", C.c_int32)]


class Saved(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "pq", "pk", "pv", "sq", "sk", "sel_idx", "sel_anchor", "sel_flags", "row_of",
        "qs", "ks", "vs", "qst", "kst", "vst", "os", "lse")]


class Sizes(C.Structure):
    _fields_ = [("E", C.c_int64), ("n_c", C.c_int64), ("T", C.c_int64), ("k_s", C.c_int64),
                ("Bc", C.c_int64), ("Sp", C.c_int64)] + [(n, C.c_size_t) for n in (
                    "pyramid_bytes", "score_bytes", "row_i32_bytes", "row_u8_bytes",
                    "row_of_bytes", "subseq_bytes", "os_bytes", "lse_bytes", "token_io_bytes",
                    "token_out_bytes", "ws_attn_fwd", "ws_attn_bwd", "ws_layer_fwd",
                    "ws_layer_bwd", "owner_bytes")]


_P = C.c_void_p
_PD = C.POINTER(Dims)
# name -> argument types after the dims pointer (all return lh_status)
_PROTOS = {
    "lh_pyramid_build": [_P] * 6 + [_P],
    "lh_score": [_P] * 4 + [_P],
    "lh_pyramid_score": [_P] * 8 + [_P],
    "lh_topk_select": [_P] * 6 + [_P],
    "lh_gather": [_P] * 13 + [_P],
    "lh_subseq_attn_fwd": [_P] * 6 + [_P, C.c_size_t, _P],
    "lh_subseq_attn_bwd": [_P] * 10 + [_P, C.c_size_t, _P],
    "lh_subseq_attn_bwd_noalloc": [_P] * 10 + [_P],
    "lh_attn_bwd_prep": [_P] * 5 + [_P],
    "lh_attn_fwd_mfma": [_P] * 6 + [_P],
    "lh_attn_bwd_dkv_mfma": [_P] * 10 + [_P],
    "lh_attn_bwd_dq_mfma": [_P] * 9 + [_P],
    "lh_scatter": [_P] * 4 + [_P],
    "lh_scatter_bwd": [_P] * 4 + [_P],
    "lh_gather_bwd": [_P] * 7 + [_P],
    "lh_span_owner": [_P] * 2 + [_P],
    "lh_scatter_span": [_P] * 3 + [_P],
    "lh_scatter_span_bwd": [_P] * 5 + [_P],
    "lh_layer_fwd": [_P] * 4 + [C.POINTER(Saved), _P, C.c_size_t, _P],
    "lh_layer_bwd": [C.POINTER(Saved)] + [_P] * 4 + [_P, C.c_size_t, _P],
}
EXPORTS = ["lh_validate", "lh_get_sizes", "lh_status_string", "lh_version", "lh_probe_mfma_bf16",
           "lh_probe_stream", *_PROTOS]

_lib = None
_lock = threading.Lock()


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise LighthouseError(LH_ERR_HIP, f"{LIB_PATH} is missing; run "
                                      "python -m sparse_long_context_amd.build")
            L = C.CDLL(LIB_PATH)
            L.lh_validate.argtypes = [_PD]
            L.lh_validate.restype = C.c_int32
            L.lh_get_sizes.argtypes = [_PD, C.POINTER(Sizes)]
            L.lh_get_sizes.restype = C.c_int32
            L.lh_status_string.argtypes = [C.c_int32]
            L.lh_status_string.restype = C.c_char_p
            L.lh_version.argtypes = []
            L.lh_version.restype = C.c_char_p
            L.lh_probe_mfma_bf16.argtypes = [C.c_int64, C.c_int32, _P, _P]
            L.lh_probe_mfma_bf16.restype = C.c_int32
            L.lh_probe_stream.argtypes = [C.c_int32, _P, _P, C.c_size_t, C.c_int64, _P]
            L.lh_probe_stream.restype = C.c_int32
            for name, args in _PROTOS.items():
                fn = getattr(L, name)
                fn.argtypes = [_PD] + args
                fn.restype = C.c_int32
            _lib = L
        return _lib


def status_string(s: int) -> str:
    try:
        return lib().lh_status_string(s).decode()
    except Exception:  # library missing: plain text
        return str(s)


def check(status: int, what: str):
    if status != LH_OK:
        raise LighthouseError(status, what)


def make_dims(B, N, H, d, p, L, K, S, io_dtype=LH_BF16, out_dtype=None, scale=0.0,
              scatter_mode=LH_SCATTER_HOLD, sigma_mode=LH_SIGMA_SUM,
              strata_mode=LH_STRATA_JOINT) -> Dims:
    return Dims(B, N, H, d, p, L, K, S, io_dtype, io_dtype if out_dtype is None else out_dtype,
                float(scale), int(scatter_mode), int(sigma_mode), int(strata_mode))


def sizes(dims: Dims) -> Sizes:
    z = Sizes()
    check(lib().lh_get_sizes(C.byref(dims), C.byref(z)), "lh_get_sizes")
    return z


def validate(dims: Dims) -> int:
    return lib().lh_validate(C.byref(dims))
