"""Build libpa.so (and the measurement library libpa_probe.so) for gfx950
with hipcc, in-tree.

    python -m paged_kv_cache_240_amd.build      # or build() from Python

Each source is compiled to an object under _build/ (in parallel) and the
objects are linked into paged_kv_cache_240_amd/libpa.so (the paged-attention
ABI, include/pa.h) and libpa_probe.so (the device-ceiling probes,
include/pa_probe.h, used by the benchmark).  Every call recompiles.  All device code is built with packed fp32 arithmetic disabled;
the store kernel additionally with FMA contraction off (its fp32 operation
order is part of its contract).
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
PROBE_LIB = os.path.join(PKG, "libpa_probe.so")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
PER_FILE = {"k_cache_store.hip": ["-ffp-contract=off"]}
SOURCES = ["pa_api.cpp", "k_cache_store.hip", "k_decode.hip", "k_decode_multi.hip", "k_prefill_chunk.hip", "k_blocks.hip",
           "k_norm_act.hip", "block_manager.cpp", "pa_noalloc.hip"]
PROBE_SOURCES = ["probe_api.cpp", "k_probe.hip"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa)")


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *COMMON, *PER_FILE.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r, cmd


def _link(lib, objs):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False):
    """Compile every source and link libpa.so and libpa_probe.so; raises on any
    compiler error.  Returns the path of libpa.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    objs = {}
    for src, obj, r, cmd in results:
        noise = "\n".join(l for l in r.stderr.splitlines()
                          if "packed-fp32-ops' is not a recognized feature" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{noise}")
        if verbose and noise.strip():
            print(noise, file=sys.stderr)
        objs[src] = obj
    _link(LIB, [objs[s] for s in SOURCES])
    _link(PROBE_LIB, [objs[s] for s in PROBE_SOURCES])
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
