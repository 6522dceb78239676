"""Build libabla.so (the HIP kernels and the C-ABI) in-tree for gfx950.

Usage: python block_sparse_attention_21_amd/build.py [-v]   (or __graft_entry__.build())
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libabla.so")
PROBE_LIB = os.path.join(PKG, "libabla_probe.so")  # matrix-core rate probes for the benchmark
OBJ = os.path.join(PKG, "_build")

SOURCES = ["abla_api.hip", "k_reorder.hip", "k_mask.hip", "k_attn.hip", "k_attn_bwd.hip"]
PROBE_SOURCES = ["probe_mfma.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I" + INCLUDE, "-I" + CSRC,
    # No packed-FP32 VALU instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libabla.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every source and link libabla.so (and the benchmark's libabla_probe.so); always
    rebuilds. Returns the path of libabla.so."""
    os.makedirs(OBJ, exist_ok=True)
    cc = hipcc()
    srcs = SOURCES + PROBE_SOURCES
    objs = {s: os.path.join(OBJ, s.replace(".hip", ".o")) for s in srcs}
    jobs = [[cc, *FLAGS, "-c", os.path.join(CSRC, s), "-o", objs[s]] for s in srcs]
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    for lib, group in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        tmp = lib + ".tmp"
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", *[objs[s] for s in group],
              "-o", tmp], verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
