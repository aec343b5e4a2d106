"""CPU tests of the layer calls' host code: lh_layer_fwd and lh_layer_bwd run
against a stub HIP runtime (tests/stub_hip/stub_hip.c) that records every
kernel launch instead of running it.  For each geometry below (the five
workloads, the GPU parity cases' shapes, both scatter modes, both strata
modes, lengths that are not whole coarsest cells) both calls must return
LH_OK and every launch must fit the device limits: at most 1024 threads and
160 KiB of LDS per workgroup, grid y and z below 65536 and the grid's
work-items within 32 bits.  Device pointers are stand-in addresses: the host
code only carves and offsets them, so no device memory is needed."""
import json
import os
import shutil
import subprocess
import sys

import pytest

from sparse_long_context_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STUB = os.path.join(ROOT, "tests", "stub_hip")

BF, F32 = L.LH_BF16, L.LH_F32
# name, (B, N, H, d, p, L, S, io, out, scatter, strata)
GEOMETRIES = [
    ("tiny f32", (1, 4096, 2, 64, 4, 3, 512, F32, F32, 0, 0)),
    ("spikes", (1, 32768, 16, 64, 4, 5, 4096, BF, BF, 0, 0)),
    ("530M shape", (1, 98304, 16, 64, 4, 6, 6144, BF, BF, 0, 0)),
    ("128K bursts", (1, 131072, 8, 128, 4, 6, 8192, BF, BF, 0, 0)),
    ("1M tokens", (1, 1048576, 4, 128, 8, 5, 16384, BF, BF, 0, 0)),
    ("128K float32 out", (1, 131072, 8, 128, 4, 6, 8192, BF, F32, 0, 0)),
    ("small d=64 float32 out", (1, 2048, 2, 64, 4, 3, 512, BF, F32, 0, 0)),
    ("d=128, S past whole tiles", (1, 6144, 2, 128, 4, 4, 1056, BF, F32, 0, 0)),
    ("ragged N=1000", (1, 1000, 2, 64, 4, 3, 252, BF, F32, 0, 0)),
    ("p=8 ragged", (1, 2560, 3, 64, 8, 3, 520, BF, F32, 0, 0)),
    ("dense L=1", (1, 768, 1, 64, 2, 1, 768, BF, F32, 0, 0)),
    ("batch 2, p=2, L=6", (2, 2048, 3, 64, 2, 6, 384, BF, F32, 0, 0)),
    ("p=3", (1, 1080, 2, 64, 3, 4, 440, BF, F32, 0, 0)),
    ("one stratum", (1, 1024, 2, 128, 4, 6, 101, BF, F32, 0, 0)),
    ("p=2, L=3, k=1536", (1, 6144, 2, 64, 2, 3, 3072, BF, F32, 0, 0)),
    ("span mode", (1, 8192, 2, 128, 4, 5, 480, BF, BF, 1, 0)),
    ("per-level strata", (1, 131072, 8, 128, 4, 6, 8192, BF, BF, 0, 1)),
]

# run in a child process with the stub runtime first on the library path;
# prints one JSON line per geometry with the two statuses
DRIVER = r"""
import ctypes as C, json, sys
sys.path.insert(0, sys.argv[1])
from sparse_long_context_amd import _lib as L
geoms = json.loads(sys.argv[2])
lib = L.lib()
for name, (B, N, H, d, p, Lv, S, io, out, scat, strata) in geoms:
    Bc = p ** (Lv - 1)
    n_c = -(-N // Bc)
    dims = L.make_dims(B, N, H, d, p, Lv, S - n_c, S, io, out, 0.0, scat, 0, strata)
    v = lib.lh_validate(C.byref(dims))
    z = L.sizes(dims)
    nxt = [1 << 40]
    def addr():
        nxt[0] += 1 << 36
        return nxt[0]
    s = L.Saved(*[None] * len(L.Saved._fields_))
    for f, _ in L.Saved._fields_:
        if f not in ("qst", "kst", "vst") and not (f in ("pq", "pk", "pv") and Lv == 1):
            setattr(s, f, addr())
    print(f"[call] {name}", file=sys.stderr, flush=True)
    fw = lib.lh_layer_fwd(C.byref(dims), C.c_void_p(addr()), C.c_void_p(addr()),
                          C.c_void_p(addr()), C.c_void_p(addr()), C.byref(s),
                          C.c_void_p(addr()) if z.ws_layer_fwd else None,
                          C.c_size_t(z.ws_layer_fwd), None)
    bw = lib.lh_layer_bwd(C.byref(dims), C.byref(s), C.c_void_p(addr()), C.c_void_p(addr()),
                          C.c_void_p(addr()), C.c_void_p(addr()), C.c_void_p(addr()),
                          C.c_size_t(z.ws_layer_bwd), None)
    print(json.dumps({"name": name, "validate": v, "fwd": fw, "bwd": bw}), flush=True)
"""


@pytest.fixture(scope="module")
def launches(tmp_path_factory):
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("liblighthouse.so not built (python -m sparse_long_context_amd.build)")
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc is needed to build the stub runtime")
    d = tmp_path_factory.mktemp("stub_hip")
    so = d / "libamdhip64.so.7"
    subprocess.run([cc, "-shared", "-fPIC", "-O1", "-o", str(so), "-Wl,-soname,libamdhip64.so.7",
                    "-Wl,--version-script=" + os.path.join(STUB, "hip_4.2.map"),
                    os.path.join(STUB, "stub_hip.c")], check=True)
    env = dict(os.environ, LD_LIBRARY_PATH=str(d) + os.pathsep + os.environ.get("LD_LIBRARY_PATH", ""))
    geoms = [[n, list(g)] for n, g in GEOMETRIES]
    p = subprocess.run([sys.executable, "-c", DRIVER, ROOT, json.dumps(geoms)], env=env,
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stderr[-2000:]
    results = {r["name"]: r for r in map(json.loads, p.stdout.splitlines())}
    per_call, cur = {}, None
    for line in p.stderr.splitlines():
        if line.startswith("[call] "):
            cur = line[len("[call] "):]
            per_call[cur] = []
        elif line.startswith("[launch] "):
            per_call[cur].append(line)
    return results, per_call


def test_the_stub_runtime_is_the_one_loaded(launches):
    results, per_call = launches
    assert set(results) == {n for n, _ in GEOMETRIES}
    assert all(per_call[n] for n, _ in GEOMETRIES), "no launch was recorded"


@pytest.mark.parametrize("name", [n for n, _ in GEOMETRIES])
def test_layer_calls_launch_within_device_limits(launches, name):
    results, per_call = launches
    r = results[name]
    assert r["validate"] == L.LH_OK
    assert r["fwd"] == L.LH_OK and r["bwd"] == L.LH_OK, r
    bad = [ln for ln in per_call[name] if ln.endswith("BAD")]
    assert not bad, bad
    names = " ".join(per_call[name])
    for k in ("select_kernel", "attn", "scatter_bwd" if "span" not in name else "scatter_span_bwd"):
        assert k in names, (k, per_call[name])
