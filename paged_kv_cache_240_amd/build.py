"""Build libpa.so for gfx950 with hipcc, in-tree.

    python -m paged_kv_cache_240_amd.build      # or build() from Python

Each source is compiled to an object under _build/ (in parallel) and the
objects are linked into paged_kv_cache_240_amd/libpa.so.  Every call
recompiles.  All device code is built with packed fp32 arithmetic disabled;
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
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
PER_FILE = {"k_cache_store.hip": ["-ffp-contract=off"]}
SOURCES = ["pa_api.cpp", "k_cache_store.hip", "k_decode.hip", "k_decode_multi.hip", "k_prefill.hip", "k_blocks.hip",
           "k_norm_act.hip", "k_probe.hip", "block_manager.cpp"]


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


def build(verbose=False):
    """Compile every source and link libpa.so; raises on any compiler error."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for src, obj, r, cmd in results:
        noise = "\n".join(l for l in r.stderr.splitlines()
                          if "packed-fp32-ops' is not a recognized feature" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{noise}")
        if verbose and noise.strip():
            print(noise, file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libpa.so failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
