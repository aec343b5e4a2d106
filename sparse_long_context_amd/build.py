"""Build liblighthouse.so (the C-ABI library) for gfx950 with hipcc.

Usage: python -m sparse_long_context_amd.build   (or build() from Python).
Every call recompiles; objects go to sparse_long_context_amd/_build/.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "liblighthouse.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(os.path.dirname(PKG), "include"),
]


# per-file flags: the dQ kernel keeps MFMA results in VGPRs (its softmax
# reads them there); the dK/dV kernel, with twice the accumulators, does not
EXTRA = {"k_attn_bwd_dq.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def _compile(src: str, obj: str) -> tuple[str, int, str]:
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    return src, p.returncode, (p.stdout + p.stderr)


def build(verbose: bool = False) -> str:
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(bdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        res = list(ex.map(_compile, srcs, objs))
    failed = False
    for src, rc, log in res:
        noise = [ln for ln in log.splitlines() if "packed-fp32-ops" not in ln]
        if rc != 0 or (verbose and noise):
            print(f"== {os.path.basename(src)} (rc={rc})\n" + "\n".join(noise), file=sys.stderr)
        failed |= rc != 0
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        print(p.stdout + p.stderr, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
