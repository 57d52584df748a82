"""ctypes binding of libpa_probe.so, the device-ceiling measurement kernels
(include/pa_probe.h): a streaming read, a scrambled 4 KiB-tile gather and bf16
matrix-core chains, and an issue-mix probe (matrix products beside exp2/FMA
chains).  Used by the benchmark to report what the device reaches
beside its published figures; not part of the paged-attention ABI."""

import ctypes
import os

import torch

from . import Call, _ptr, _stream

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa_probe.so")

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_SIGS = {
    "pa_probe_stream_read": (ctypes.c_int, [_p, _i64, _p, _i32, _p]),
    "pa_probe_mfma_bf16": (ctypes.c_int, [_i32, _p, _i32, _p]),
    "pa_probe_gather_read_groups": (ctypes.c_int64, [_i64]),
    "pa_probe_gather_read": (ctypes.c_int, [_p, _i64, _p, _p]),
    "pa_probe_issue_mix": (ctypes.c_int, [_i32, _i32, _p, _i32, _p]),
}
_lib = None


def load():
    """Load libpa_probe.so (once).  Raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"libpa_probe.so is not built ({library_path}); run "
                              "`python -m paged_kv_cache_240_amd.build`")
        lib = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class ProbeCall(Call):
    """A Call on libpa_probe.so."""

    __slots__ = ()

    def __init__(self, name, args, result=None, keep=()):
        super().__init__(name, args, result, keep, lib=load())


def prepare_probe_stream_read(buf, grid=2048, sums=None):
    """pa_probe_stream_read over a contiguous device tensor; returns a callable whose
    result is the per-workgroup uint32 sums (as int32) of the buffer's 32-bit words."""
    dev = buf.device
    if not buf.is_contiguous() or buf.numel() * buf.element_size() % 16:
        raise ValueError("buf must be contiguous and a multiple of 16 bytes")
    if sums is None:
        sums = torch.empty(grid, dtype=torch.int32, device=dev)
    return ProbeCall("pa_probe_stream_read", (_ptr(buf), buf.numel() * buf.element_size(), _ptr(sums),
                                              grid, _stream(dev)), result=sums, keep=(buf,))


def prepare_probe_gather_read(buf, sums=None):
    """pa_probe_gather_read over a contiguous device tensor (a power-of-two count of
    4 KiB tiles); returns a callable whose result is the per-workgroup uint32 sums
    (as int32) of the buffer's 32-bit words."""
    dev = buf.device
    nbytes = buf.numel() * buf.element_size()
    tiles = nbytes // 4096
    if not buf.is_contiguous() or nbytes % 4096 or tiles & (tiles - 1):
        raise ValueError("buf must be contiguous and a power-of-two count of 4 KiB tiles")
    groups = load().pa_probe_gather_read_groups(nbytes)
    if sums is None:
        sums = torch.empty(groups, dtype=torch.int32, device=dev)
    return ProbeCall("pa_probe_gather_read", (_ptr(buf), nbytes, _ptr(sums), _stream(dev)),
                     result=sums, keep=(buf,))


def prepare_probe_mfma_bf16(iters, grid, device, out=None):
    """pa_probe_mfma_bf16; returns a callable whose result is out fp32 [4 * grid]."""
    if out is None:
        out = torch.empty(4 * grid, dtype=torch.float32, device=device)
    return ProbeCall("pa_probe_mfma_bf16", (int(iters), _ptr(out), int(grid), _stream(out.device)),
                     result=out)


def prepare_probe_issue_mix(mode, iters, grid, device, out=None):
    """pa_probe_issue_mix: mode 1 (products), 2 (exp2 + FMA chains) or 3 (both);
    returns a callable whose result is the fp32 [256 * grid] per-thread values."""
    if out is None:
        out = torch.empty(256 * grid, dtype=torch.float32, device=device)
    return ProbeCall("pa_probe_issue_mix", (int(mode), int(iters), _ptr(out), int(grid), _stream(out.device)),
                     result=out)
