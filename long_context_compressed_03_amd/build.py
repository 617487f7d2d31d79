"""Build libcsa.so (all HIP kernels + the C ABI) for gfx950 with hipcc, in-tree.

Each source compiles to its own object in parallel (they share no device
symbols, so no relocatable device code is needed); the objects are then linked
into one shared library.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsa.so")
OBJ = os.path.join(HERE, "_build")
SOURCES = ["abi.hip", "compress.hip", "indexer.hip", "indexer_topk.hip", "topk.hip", "attn.hip",
           "quant.hip", "cache.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    return r.returncode, err


def build(verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ, exist_ok=True)
    srcs = list(SOURCES)
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in srcs]
    cmds = [[hipcc, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, err), s in zip(results, srcs):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {s} ({rc}):\n{err}")
        if err.strip() and verbose:
            print(err)
    tmp = LIB + ".tmp"
    rc, err = _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
