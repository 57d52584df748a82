"""The host C++ of libpa under AddressSanitizer and UndefinedBehaviorSanitizer.

block_manager.cpp (free list, ref counts, prefix hash map, LRU list iterators,
fork / copy-on-write / swap bookkeeping) and pa_api.cpp (argument validation,
partition choice, workspace sizing) are compiled for the host with g++ and
-fsanitize=address,undefined into a stand-alone library whose kernel launchers
are stand-ins that launch nothing (tests/host/launch_stubs.cpp).  The block
manager and ABI test suites then run in a child process against that library,
with the sanitizer runtime preloaded and every finding fatal.  CPU only: no GPU
code is built or run.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_240_amd", "csrc")
ROCM = "/opt/rocm"


def _libasan():
    gcc = shutil.which("gcc")
    if not gcc:
        return None
    p = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def build_sanitized(out_dir):
    """The host sources built with ASan + UBSan; returns the library path."""
    lib = os.path.join(out_dir, "libpa_host_asan.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           os.path.join(CSRC, "block_manager.cpp"), os.path.join(CSRC, "pa_api.cpp"),
           os.path.join(ROOT, "tests", "host", "launch_stubs.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stderr
    return lib


CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import paged_kv_cache_240_amd as pa
pa.library_path = {lib!r}
import pytest
rc = pytest.main(["-q", "-p", "no:cacheprovider", {bm!r}, {abi!r},
                  "-k", "not exports_every and not probe_library"])
maps = open("/proc/self/maps").read()
print("SANITIZED_LIBRARY_MAPPED", {lib!r} in maps)
sys.exit(rc)
"""


@pytest.mark.skipif(shutil.which("g++") is None or _libasan() is None
                    or not os.path.exists(f"{ROCM}/lib/libamdhip64.so"),
                    reason="needs g++, its libasan and the ROCm host runtime")
def test_block_manager_and_abi_under_asan_ubsan(tmp_path):
    lib = build_sanitized(str(tmp_path))
    env = dict(os.environ)
    env["LD_PRELOAD"] = _libasan()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:detect_stack_use_after_return=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(root=ROOT, lib=lib, bm=os.path.join(ROOT, "tests", "test_block_manager.py"),
                        abi=os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=str(tmp_path), timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "SANITIZED_LIBRARY_MAPPED True" in out, out[-4000:]
    assert " passed" in out
