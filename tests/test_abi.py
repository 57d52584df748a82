"""The C ABI: libpa.so loads, exports every symbol include/pa.h declares, and
rejects bad arguments on the host before enqueueing anything.  CPU only: every
call here fails validation, so no kernel is ever launched."""

import ctypes
import os
import re

import pytest

import paged_kv_cache_240_amd as pa
from paged_kv_cache_240_amd import probes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")
PROBE_HEADER = os.path.join(ROOT, "include", "pa_probe.h")

OK, NULL, SHAPE, UNSUP, WS, HIP, MEM = range(7)
P = ctypes.c_void_p(0x1000)  # a non-null dummy pointer: never dereferenced on these paths


def declared_symbols(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ("pa_cache_store", "pa_decode", "pa_decode_partitions", "pa_decode_combine",
              "pa_decode_step", "pa_decode_step_partitions",
              "pa_decode_workspace_bytes", "pa_decode_partition_size", "pa_prefill",
              "pa_decode_multi", "pa_decode_multi_workspace_bytes",
              "pa_status_str"):
        assert s in syms


def test_library_exports_every_declared_symbol():
    lib = pa.load()
    for s in declared_symbols():
        assert hasattr(lib, s), s
    assert os.path.samefile(pa.library_path, os.path.join(ROOT, "paged_kv_cache_240_amd", "libpa.so"))


def test_status_strings():
    lib = pa.load()
    for code, name in pa.STATUS.items():
        assert lib.pa_status_str(code).decode().startswith(name)
    assert lib.pa_status_str(99)


def _store(**kw):
    a = dict(q=P, k=P, v=P, kc=P, vc=P, slots=P, pos=P, cs=P, T=4, Hq=12, Hkv=2, D=128, bs=16,
             nb=64, max_pos=100)
    a.update(kw)
    return pa.load().pa_cache_store(a["q"], a["k"], a["v"], a["kc"], a["vc"], a["slots"], a["pos"],
                                    a["cs"], a["T"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["nb"],
                                    a["max_pos"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), NULL), (dict(v=None), NULL), (dict(kc=None), NULL), (dict(vc=None), NULL),
    (dict(slots=None), NULL), (dict(pos=None), NULL), (dict(cs=None), NULL),
    (dict(T=-1), SHAPE), (dict(Hq=13), SHAPE), (dict(Hkv=0), SHAPE), (dict(D=96), UNSUP),
    (dict(D=256), UNSUP), (dict(bs=32), UNSUP), (dict(bs=0), SHAPE), (dict(Hq=18, Hkv=2), UNSUP),
    (dict(nb=0), SHAPE), (dict(max_pos=0), SHAPE), (dict(T=0), OK),
])
def test_cache_store_validation(kw, code):
    assert _store(**kw) == code


def _decode(**kw):
    a = dict(out=P, q=P, kc=P, vc=P, bt=P, cl=P, B=2, Hq=12, Hkv=2, D=128, bs=16, mb=8, mcl=128,
             scale=0.088, ps=-1, ws=None, wsb=0)
    a.update(kw)
    return pa.load().pa_decode(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["B"], a["Hq"],
                               a["Hkv"], a["D"], a["bs"], a["mb"], a["mcl"], a["scale"], a["ps"],
                               a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), NULL), (dict(q=None), NULL), (dict(kc=None), NULL), (dict(vc=None), NULL),
    (dict(bt=None), NULL), (dict(cl=None), NULL),
    (dict(B=-1), SHAPE), (dict(Hq=7), SHAPE), (dict(D=80), UNSUP), (dict(bs=8), UNSUP),
    (dict(mb=0), SHAPE), (dict(mcl=-1), SHAPE), (dict(mcl=129), SHAPE),
    (dict(ps=24), SHAPE), (dict(ps=-2), SHAPE),
    (dict(ps=16, ws=None, wsb=0), WS), (dict(ps=16, ws=P, wsb=100), WS),
    (dict(Hq=20, Hkv=2), UNSUP), (dict(B=0), OK),
])
def test_decode_validation(kw, code):
    assert _decode(**kw) == code


def test_workspace_size_formula():
    lib = pa.load()
    # fp32 [B][Hq][NP][D] partials + fp32 [B][Hq][NP] log-sum-exps
    assert lib.pa_decode_workspace_bytes(16, 12, 2, 128, 8192, 512) == 16 * 12 * 16 * 129 * 4
    assert lib.pa_decode_workspace_bytes(3, 2, 1, 64, 33, 16) == 3 * 2 * 3 * 65 * 4
    assert lib.pa_decode_workspace_bytes(3, 2, 1, 64, 33, 0) == 0
    assert lib.pa_decode_workspace_bytes(3, 2, 1, 64, 33, 24) == 0
    assert lib.pa_decode_workspace_bytes(-1, 2, 1, 64, 33, 16) == 0


def test_partition_choice():
    # the rule (256 compute units assumed without a GPU): one pass when the (sequence, KV
    # head) pairs give every CU a workgroup or the context fits 128 tokens; else the smallest
    # of 128 / 256 / 512 keeping the grid within 2 workgroups per CU and 64 partitions per
    # sequence; else 512, doubled while a sequence would need more than 64 partitions
    lib = pa.load()
    for (B, Hkv, L), want in [((1, 2, 2048), 128), ((4, 2, 2048), 128), ((64, 2, 2512), 512), ((64, 2, 1024), 256),
                              ((8, 2, 4096), 128), ((4, 2, 8192), 128), ((16, 2, 8192), 512),
                              ((32, 2, 4096), 512), ((1, 2, 8192), 128), ((1, 2, 16384), 256),
                              ((1, 2, 32768), 512), ((1, 2, 65536), 1024), ((4, 1, 33), 0), ((1, 2, 128), 0),
                              ((1, 2, 129), 128), ((1, 2, 512), 128), ((128, 2, 2048), 0), ((127, 2, 2048), 512),
                              ((1000, 8, 4096), 0), ((0, 2, 100), 0)]:
        assert lib.pa_decode_partition_size(B, Hkv, L) == want, (B, Hkv, L)


@pytest.mark.parametrize("kw,code", [
    (dict(o=None), NULL), (dict(ps=0), SHAPE), (dict(ps=20), SHAPE), (dict(D=48), UNSUP),
    (dict(B=-2), SHAPE), (dict(B=0), OK),
])
def test_decode_stage_validation(kw, code):
    lib = pa.load()
    a = dict(o=P, B=2, D=128, ps=64)
    a.update(kw)
    assert lib.pa_decode_partitions(a["o"], P, P, P, P, P, P, a["B"], 12, 2, a["D"], 16, 8, 128,
                                    0.1, a["ps"], None) == code
    if "o" not in kw:
        assert lib.pa_decode_combine(P, P, P, P, a["B"], 12, a["D"], 128, a["ps"], None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), NULL), (dict(qsl=None), NULL), (dict(D=32), UNSUP), (dict(Hq=5), SHAPE),
    (dict(T=-1), SHAPE), (dict(mql=10, T=4), SHAPE), (dict(bs=64), UNSUP), (dict(T=0), OK),
])
def test_prefill_validation(kw, code):
    a = dict(out=P, qsl=P, B=2, T=16, Hq=12, Hkv=2, D=128, bs=16, mb=8, mql=8)
    a.update(kw)
    assert pa.load().pa_prefill(a["out"], P, P, P, P, P, a["qsl"], a["B"], a["T"], a["Hq"],
                                a["Hkv"], a["D"], a["bs"], a["mb"], a["mql"], 0.1, None) == code


def _multi(**kw):
    a = dict(out=P, q=P, kc=P, vc=P, bt=P, cl=P, B=2, NQ=5, Hq=12, Hkv=2, D=128, bs=16, mb=8,
             mcl=128, scale=0.088, ps=64, ws=None, wsb=0)
    a.update(kw)
    return pa.load().pa_decode_multi(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["B"],
                                     a["NQ"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["mb"], a["mcl"],
                                     a["scale"], a["ps"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), NULL), (dict(q=None), NULL), (dict(bt=None), NULL), (dict(cl=None), NULL),
    (dict(NQ=0), SHAPE), (dict(NQ=-2), SHAPE), (dict(NQ=6), UNSUP), (dict(Hq=16, Hkv=2, NQ=5), UNSUP),
    (dict(Hq=8, Hkv=1, NQ=4, B=0), OK), (dict(D=80), UNSUP), (dict(bs=32), UNSUP),
    (dict(mcl=129), SHAPE), (dict(ps=24), SHAPE), (dict(ps=-2), SHAPE),
    (dict(ps=64, ws=None), WS), (dict(ps=64, ws=P, wsb=100), WS), (dict(B=0), OK),
])
def test_decode_multi_validation(kw, code):
    assert _multi(**kw) == code


def test_decode_multi_workspace_is_per_query_decode_workspace():
    lib = pa.load()
    for B, NQ, L, P in [(16, 5, 8192, 512), (3, 2, 100, 16), (1, 1, 2048, 64)]:
        one = lib.pa_decode_workspace_bytes(B, 12, 2, 128, L, P)
        assert lib.pa_decode_multi_workspace_bytes(B, NQ, 12, 2, 128, L, P) == NQ * one
        assert one == B * 12 * (-(-L // P)) * 129 * 4
    assert lib.pa_decode_multi_workspace_bytes(4, 0, 12, 2, 128, 100, 16) == 0


def test_decode_multi_library_partition_choice():
    # -1: decode's choice, except 512 -> 1024 when two row tiles (NQ * G > 16) still give every CU
    # a workgroup at 1024 tokens (no GPU here: the library assumes 256 CUs)
    lib = pa.load()
    assert lib.pa_decode_partition_size(16, 2, 8192) == 512
    assert lib.pa_decode_multi_workspace_bytes(16, 5, 12, 2, 128, 8192, -1) == \
        lib.pa_decode_multi_workspace_bytes(16, 5, 12, 2, 128, 8192, 1024)
    # one 16-row tile (NQ * G <= 16): decode's choice
    assert lib.pa_decode_multi_workspace_bytes(16, 2, 12, 2, 128, 8192, -1) == \
        lib.pa_decode_multi_workspace_bytes(16, 2, 12, 2, 128, 8192, 512)
    # a 1024-token grid below the CU count: decode's choice
    assert lib.pa_decode_multi_workspace_bytes(8, 5, 12, 2, 128, 8192, -1) == \
        lib.pa_decode_multi_workspace_bytes(8, 5, 12, 2, 128, 8192, lib.pa_decode_partition_size(8, 2, 8192))


def _copy(**kw):
    a = dict(kc=P, vc=P, src=P, dst=P, n=4, Hkv=2, D=128, bs=16, nb=64)
    a.update(kw)
    return pa.load().pa_copy_blocks(a["kc"], a["vc"], a["src"], a["dst"], a["n"], a["Hkv"], a["D"],
                                    a["bs"], a["nb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kc=None), NULL), (dict(vc=None), NULL), (dict(src=None), NULL), (dict(dst=None), NULL),
    (dict(n=-1), SHAPE), (dict(Hkv=0), SHAPE), (dict(D=96), UNSUP), (dict(bs=32), UNSUP),
    (dict(bs=0), SHAPE), (dict(nb=-1), SHAPE), (dict(nb=0), SHAPE),
    (dict(n=0), OK), (dict(n=0, src=None, dst=None), OK),
])
def test_copy_blocks_validation(kw, code):
    assert _copy(**kw) == code


def _swap(**kw):
    a = dict(dk=P, dv=P, sk=P, sv=P, src=P, dst=P, n=4, Hkv=2, D=128, bs=16)
    a.update(kw)
    return pa.load().pa_swap_blocks(a["dk"], a["dv"], a["sk"], a["sv"], a["src"], a["dst"], a["n"],
                                    a["Hkv"], a["D"], a["bs"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dk=None), NULL), (dict(dv=None), NULL), (dict(sk=None), NULL), (dict(sv=None), NULL),
    (dict(src=None), NULL), (dict(dst=None), NULL), (dict(n=-3), SHAPE), (dict(D=32), UNSUP),
    (dict(bs=8), UNSUP), (dict(n=0), OK), (dict(n=0, src=None), OK),
])
def test_swap_blocks_validation(kw, code):
    assert _swap(**kw) == code


@pytest.mark.parametrize("args,code", [
    ((None, None, P, P, 4, 64, 1e-6), NULL), ((P, None, None, P, 4, 64, 1e-6), NULL),
    ((P, None, P, None, 4, 64, 1e-6), NULL), ((P, None, P, P, -1, 64, 1e-6), SHAPE),
    ((P, None, P, P, 4, 0, 1e-6), SHAPE), ((P, None, P, P, 4, 60, 1e-6), UNSUP),
    ((P, None, P, P, 4, 16392, 1e-6), UNSUP), ((P, None, P, P, 4, 64, -1.0), SHAPE),
    ((P, None, P, P, 4, 64, float("nan")), SHAPE), ((P, P, P, P, 0, 64, 1e-6), OK),
])
def test_rmsnorm_validation(args, code):
    assert pa.load().pa_rmsnorm_residual(*args, None) == code


@pytest.mark.parametrize("args,code", [
    ((None, P, 4, 64), NULL), ((P, None, 4, 64), NULL), ((P, P, -1, 64), SHAPE),
    ((P, P, 4, 0), SHAPE), ((P, P, 4, 12), UNSUP), ((P, P, 0, 64), OK),
])
def test_swiglu_validation(args, code):
    assert pa.load().pa_swiglu(*args, None) == code


def _step(**kw):
    a = dict(out=P, q=P, k=P, v=P, kc=P, vc=P, bt=P, cl=P, cs=P, B=2, Hq=12, Hkv=2, D=128, bs=16,
             mb=8, mcl=128, max_pos=128, scale=0.088, ps=-1, ws=None, wsb=0)
    a.update(kw)
    return pa.load().pa_decode_step(a["out"], a["q"], a["k"], a["v"], a["kc"], a["vc"], a["bt"],
                                    a["cl"], a["cs"], a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"],
                                    a["mb"], a["mcl"], a["max_pos"], a["scale"], a["ps"], a["ws"],
                                    a["wsb"], None)


WS16 = 2 * 12 * 8 * 129 * 4   # the pa_decode workspace at B=2, Hq=12, D=128, 128 tokens, P=16


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), NULL), (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL),
    (dict(kc=None), NULL), (dict(vc=None), NULL), (dict(bt=None), NULL), (dict(cl=None), NULL),
    (dict(cs=None), NULL),
    (dict(B=-1), SHAPE), (dict(Hq=7), SHAPE), (dict(D=80), UNSUP), (dict(bs=8), UNSUP),
    (dict(mb=0), SHAPE), (dict(mcl=129), SHAPE), (dict(max_pos=127), SHAPE),
    (dict(ps=24), SHAPE), (dict(ps=-2), SHAPE),
    (dict(ps=16, ws=None, wsb=0), WS), (dict(ps=16, ws=P, wsb=WS16 - 1), WS),
    (dict(Hq=20, Hkv=2), UNSUP), (dict(B=0), OK),
])
def test_decode_step_validation(kw, code):
    assert _step(**kw) == code


def test_probe_library_is_separate():
    """The measurement kernels live in libpa_probe.so (include/pa_probe.h), not in the
    paged-attention library: pa.h declares none of them and libpa.so exports none."""
    assert not [s for s in declared_symbols() if s.startswith("pa_probe")]
    lib = pa.load()
    for s in declared_symbols(PROBE_HEADER):
        assert not hasattr(lib, s), s
    plib = probes.load()
    for s in declared_symbols(PROBE_HEADER):
        assert hasattr(plib, s), s
    assert os.path.samefile(probes.library_path, os.path.join(ROOT, "paged_kv_cache_240_amd", "libpa_probe.so"))


def test_probe_validation():
    lib = probes.load()
    assert lib.pa_probe_stream_read(None, 16, P, 1, None) == NULL
    assert lib.pa_probe_stream_read(P, 16, None, 1, None) == NULL
    assert lib.pa_probe_stream_read(P, 0, P, 1, None) == SHAPE
    assert lib.pa_probe_stream_read(P, 24, P, 1, None) == SHAPE
    assert lib.pa_probe_stream_read(P, 16, P, 0, None) == SHAPE
    assert lib.pa_probe_gather_read(None, 4096, P, None) == NULL
    assert lib.pa_probe_gather_read(P, 4096, None, None) == NULL
    assert lib.pa_probe_gather_read(P, 0, P, None) == SHAPE
    assert lib.pa_probe_gather_read(P, 4095, P, None) == SHAPE
    assert lib.pa_probe_gather_read(P, 3 * 4096, P, None) == SHAPE  # tile count not a power of two
    assert lib.pa_probe_gather_read_groups(0) == 0
    assert lib.pa_probe_gather_read_groups(4096) == 1
    assert lib.pa_probe_gather_read_groups(1 << 31) == (1 << 31) // 4096 // 16  # 4 waves x 4 tiles
    assert lib.pa_probe_mfma_bf16(1, None, 1, None) == NULL
    assert lib.pa_probe_mfma_bf16(0, P, 1, None) == SHAPE
    assert lib.pa_probe_mfma_bf16(1, P, 0, None) == SHAPE
    assert lib.pa_probe_issue_mix(1, 1, None, 1, None) == NULL
    assert lib.pa_probe_issue_mix(0, 1, P, 1, None) == SHAPE
    assert lib.pa_probe_issue_mix(4, 1, P, 1, None) == SHAPE
    assert lib.pa_probe_issue_mix(3, 0, P, 1, None) == SHAPE
    assert lib.pa_probe_issue_mix(3, 1, P, 0, None) == SHAPE


def _sp(**kw):
    a = dict(out=P, q=P, kc=P, vc=P, bt=P, cl=P, gs=P, pl=P, B=4, ng=1, mg=4, mp=32, Hq=12, Hkv=2,
             D=128, bs=16, mb=8, mcl=128, ms=128, scale=0.088, ps=64, ws=P, wsb=1 << 30)
    a.update(kw)
    return pa.load().pa_decode_shared_prefix(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"],
                                             a["gs"], a["pl"], a["B"], a["ng"], a["mg"], a["mp"],
                                             a["Hq"], a["Hkv"], a["D"], a["bs"], a["mb"], a["mcl"],
                                             a["ms"], a["scale"], a["ps"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), NULL), (dict(pl=None), NULL), (dict(gs=None), NULL), (dict(q=None), NULL),
    (dict(ng=-1), SHAPE), (dict(mp=-16), SHAPE), (dict(mp=24), SHAPE), (dict(mp=144), SHAPE),
    (dict(mg=0), SHAPE), (dict(mg=5), SHAPE), (dict(ps=0), SHAPE), (dict(ps=24), SHAPE),
    (dict(ms=-1), SHAPE), (dict(ms=129), SHAPE),
    (dict(ws=None), WS), (dict(wsb=100), WS), (dict(ps=16, mcl=1024, ms=1024, mp=128, mb=64), UNSUP),
    (dict(D=80), UNSUP), (dict(B=0, ng=0), OK),
])
def test_shared_prefix_validation(kw, code):
    assert _sp(**kw) == code


def test_shared_prefix_workspace_size():
    lib = pa.load()
    # slots = ceil(max_suffix_len / P) + ceil(max_prefix / 128)
    assert lib.pa_decode_shared_prefix_workspace_bytes(64, 12, 2, 128, 1024, 2000, 512) == \
        64 * 12 * (2 + 16) * 129 * 4
    assert lib.pa_decode_shared_prefix_workspace_bytes(4, 12, 2, 128, 128, 0, 64) == 4 * 12 * 2 * 129 * 4
    assert lib.pa_decode_shared_prefix_workspace_bytes(4, 12, 2, 128, 128, 0, 24) == 0


def test_noalloc_refuses_more_than_its_array():
    """pa_decode_noalloc checks the workspace it would need against its 16 MiB
    array before touching the device (no GPU is used here)."""
    lib = pa.load()
    assert lib.pa_decode_workspace_bytes(256, 12, 2, 128, 32768, 512) > 16 << 20
    assert lib.pa_decode_noalloc(P, P, P, P, P, P, 256, 12, 2, 128, 16, 2048, 32768, 0.088, 512,
                                 None) == WS
    assert lib.pa_decode_noalloc(P, P, P, P, P, P, 2, 12, 2, 128, 16, 8, 128, 0.088, 24, None) == SHAPE
