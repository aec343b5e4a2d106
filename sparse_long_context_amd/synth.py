"""Seeded synthetic inputs for the Lighthouse layer workloads.

This module is shared by the tests, the benchmark and the CPU oracle's
callers.  It holds the workload shapes and the random-number recipe only --
none of the layer's arithmetic -- so the oracle and the HIP path stay
independent.

The pages measure on activations of a 530M Llama-3-style decoder trained on
C4 at 98,304 tokens of context (gist.science explainer, technical summary
section 4).  That model and dataset are not available, so these seeded
inputs stand in for them, with the pages' shapes (98,304-token context, the
128K-1M range of the problem statement) and value structure chosen to stress
the selection: norm spikes, per-head log-normal row scales and high-norm
bursts.

Recipe (per workload c = 1..5):
  seed_c = 260506554 + c
  values: numpy default_rng([seed_c, tensor_id, h]).standard_normal((N, d),
          float32) with tensor_id Q=0, K=1, V=2, dO=3, one stream per head so
          a head can be generated alone;
  structure: default_rng([seed_c, 99]);
  bf16 workloads round the float32 values to bfloat16 (round to nearest
  even, torch CPU conversion); the rounded values are the inputs of both
  sides.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from dataclasses import dataclass

import numpy as np
import torch

SEED_BASE = 260506554


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    N: int
    H: int
    d: int
    p: int
    L: int
    S: int
    dtype: str           # "f32" or "bf16" (Q, K, V and dO)
    structure: str       # none | spikes | lognormal | bursts
    B: int = 1

    @property
    def n_c(self):
        return self.N // self.p ** (self.L - 1)

    @property
    def K(self):
        """Ranked entries: the subsequence length minus the always-kept
        coarsest entries."""
        return self.S - self.n_c


WORKLOADS = {
    1: Workload(1, "tiny-f32 N=4096 H=2 d=64 p=4 L=3 S=512", 4096, 2, 64, 4, 3, 512, "f32", "none"),
    2: Workload(2, "spikes N=32768 H=16 d=64 p=4 L=5 S=4096", 32768, 16, 64, 4, 5, 4096, "bf16", "spikes"),
    3: Workload(3, "llama530m-shape N=98304 H=16 d=64 p=4 L=6 S=6144", 98304, 16, 64, 4, 6, 6144, "bf16", "lognormal"),
    4: Workload(4, "bursts N=131072 H=8 d=128 p=4 L=6 S=8192", 131072, 8, 128, 4, 6, 8192, "bf16", "bursts"),
    5: Workload(5, "extreme N=1048576 H=4 d=128 p=8 L=5 S=16384", 1048576, 4, 128, 8, 5, 16384, "bf16", "none"),
}


def _row_multipliers(w: Workload, seed: int, heads):
    """Per-(head, token) float32 row multipliers of the workload's structure,
    or None."""
    rng = np.random.default_rng([seed, 99])
    if w.structure == "none":
        return None
    if w.structure == "spikes":
        # 2% of token positions, all heads, rows x8 (exact in bf16)
        n = int(round(0.02 * w.N))
        pos = rng.choice(w.N, size=n, replace=False)
        m = np.ones(w.N, np.float32)
        m[pos] = 8.0
        return {h: m for h in heads}
    if w.structure == "lognormal":
        z = rng.standard_normal((w.H, w.N), dtype=np.float32)
        m = np.exp(0.5 * z.astype(np.float64)).astype(np.float32)
        return {h: m[h] for h in heads}
    if w.structure == "bursts":
        # floor(0.01 N / 64) runs of 64 tokens, x6; slots drawn without
        # replacement among the even 64-token slots, start offset 0..63, so
        # runs never overlap and straddle pyramid cells
        runs = int(0.01 * w.N / 64)
        slots = rng.choice(np.arange(0, w.N // 64, 2), size=runs, replace=False)
        delta = rng.integers(0, 64, size=runs)
        m = np.ones(w.N, np.float32)
        for s, dl in zip(slots, delta):
            t0 = 64 * int(s) + int(dl)
            m[t0:t0 + 64] = 6.0
        return {h: m for h in heads}
    raise ValueError(w.structure)


def head_tensor(w: Workload, tensor_id: int, h: int, mult=None, seed=None):
    """One head's [N, d] float32 values (before any bf16 rounding)."""
    seed = SEED_BASE + w.cid if seed is None else seed
    x = np.random.default_rng([seed, tensor_id, h]).standard_normal((w.N, w.d), dtype=np.float32)
    if mult is not None and tensor_id < 3:
        x *= mult[:, None]
    return x


def make_inputs(w: Workload, heads=None, seed=None):
    """Q, K, V, dO as CPU torch tensors [B, len(heads), N, d] in the
    workload dtype (B = 1).  Every (tensor, head) has its own generator, so
    they are drawn in parallel threads; the values do not depend on the
    thread count."""
    seed = SEED_BASE + w.cid if seed is None else seed
    heads = list(range(w.H)) if heads is None else list(heads)
    mults = _row_multipliers(w, seed, heads)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    out = [torch.empty((1, len(heads), w.N, w.d), dtype=tdt) for _ in range(4)]

    def fill(job):
        tid, k = job
        h = heads[k]
        x = head_tensor(w, tid, h, None if mults is None else mults[h], seed)
        out[tid][0, k] = torch.from_numpy(x).to(tdt)

    jobs = [(tid, k) for tid in range(4) for k in range(len(heads))]
    workers = max(1, min(16, os.cpu_count() or 1, len(jobs)))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, jobs))
    return tuple(out)


def small(N, H, d, p, L, S, dtype="f32", structure="none", seed=1234):
    """An ad-hoc workload for tests (cid is only used for the seed)."""
    w = Workload(0, f"adhoc N={N} H={H} d={d} p={p} L={L} S={S}", N, H, d, p, L, S, dtype, structure)
    return w, make_inputs(w, seed=seed)
