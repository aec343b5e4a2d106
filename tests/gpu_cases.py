"""Shared helpers of the GPU parity tests (not collected as tests).

Each case is a seeded synthetic workload small enough for the float64 oracle
to finish in seconds, spanning several kernel tiles and a ragged tail.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from oracle import lighthouse as orc
from sparse_long_context_amd import synth


@dataclass(frozen=True)
class Case:
    name: str
    N: int
    H: int
    d: int
    p: int
    L: int
    k_s: int
    dtype: str = "bf16"
    structure: str = "none"
    out: str = "f32"          # output dtype of the parity run
    seed: int = 1234
    B: int = 1                # batch; heads of the generator are split into batches

    @property
    def n_c(self):
        return -(-self.N // self.p ** (self.L - 1))   # a partial last cell counts

    @property
    def S(self):
        return self.n_c * (self.k_s + 1)

    @property
    def K(self):
        return self.n_c * self.k_s


CASES = [
    # the tiny float32 workload itself: N=4096, H=2, d=64, p=4, L=3, S=512
    Case("tiny-f32", 4096, 2, 64, 4, 3, 1, dtype="f32", seed=synth.SEED_BASE + 1),
    # d=128, S=1056: 8.25 query tiles of 128, ragged tail; spiky rows
    Case("bf16-d128-ragged", 6144, 2, 128, 4, 4, 10, structure="spikes"),
    # d=64, p=8, S=520 (ragged at 64); log-normal row scales
    Case("bf16-d64-p8-ragged", 2560, 3, 64, 8, 3, 12, structure="lognormal"),
    # every entry selected: the layer must equal dense causal SDPA
    Case("bf16-full-selection", 1024, 2, 64, 4, 3, 20),
    # K = 0: only the coarsest level
    Case("bf16-coarsest-only", 4096, 2, 128, 4, 4, 0),
    # L = 1: no pyramid, S = N
    Case("bf16-L1-dense", 768, 1, 64, 2, 1, 0),
    # bursts of high-norm tokens, d=128, bf16 outputs
    Case("bf16-bursts-bf16out", 8192, 2, 128, 4, 5, 15, structure="bursts", out="bf16"),
    # batch 2 (flattened (b, h) indexing), p = 2 with six levels: B_c = 32, S = 384
    Case("bf16-batch2-p2", 2048, 3, 64, 2, 6, 5, B=2),
    # p = 3, not a power of two (division instead of shifts): B_c = 27, S = 440
    Case("bf16-p3", 1080, 2, 64, 3, 4, 10, structure="spikes"),
    # a single coarsest cell: n_c = 1, S = 101 (less than one tile)
    Case("bf16-one-stratum", 1024, 2, 128, 4, 6, 100),
    # the pages' ablation point p = 2, L = 3, k = 1536, in the one form the
    # stratification admits: 1536 coarsest cells of 4 tokens, one ranked
    # entry each (K = 1536, S = 3072)
    Case("bf16-p2-L3-k1536", 6144, 2, 64, 2, 3, 1, structure="lognormal"),
]


def inputs(case: Case):
    """Q, K, V, dO [B, H, N, d]: the generator's B*H heads, split into batches."""
    w = synth.Workload(0, case.name, case.N, case.B * case.H, case.d, case.p, case.L, case.S,
                       case.dtype, case.structure)
    return tuple(t.reshape(case.B, case.H, case.N, case.d)
                 for t in synth.make_inputs(w, seed=case.seed))


def bh_pairs(case: Case):
    return [(b, h) for b in range(case.B) for h in range(case.H)]


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def store_of(case: Case):
    return "bf16" if case.dtype == "bf16" else "f32"


def geometry(case: Case) -> orc.Geometry:
    return orc.Geometry(case.N, case.p, case.L, case.K).check()


def selection_from_gpu(g: orc.Geometry, sel_idx, anchor, flags, row_of) -> orc.Selection:
    lev, _ = orc.entry_of_flat(g, sel_idx)
    return orc.Selection(np.asarray(sel_idx, np.int64), np.asarray(anchor, np.int64), lev,
                         np.asarray(flags, np.uint8), np.asarray(row_of, np.int64))


def ulp_bf16(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def tol_for(case: Case, ref, out_dtype: str):
    """Stated tolerance: max-abs 1e-5 for float32 I/O; 2e-2 for bf16 I/O
    (plus half a bf16 step of the reference when the output is stored in
    bf16)."""
    if case.dtype == "f32":
        return 1e-5
    t = 2e-2
    if out_dtype == "bf16":
        return t + 0.5 * ulp_bf16(ref)
    return t
