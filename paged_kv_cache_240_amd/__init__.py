"""Python binding of libpa: paged KV-cache attention on MI355X (gfx950).

Thin ctypes wrappers with the names of the C ABI (include/pa.h).  They check
dtypes, shapes, devices and contiguity, allocate outputs and workspaces with
torch (torch provides device memory and streams only) and pass raw pointers
and torch's current stream to the library.  Every step of the computation
runs in the HIP kernels of libpa.so; there is no fallback: if the library is
missing, load() raises.

    import paged_kv_cache_240_amd as pa
    pa.cache_store(q, k, v, k_cache, v_cache, slot_mapping, positions, cos_sin)
    out = pa.decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len)
    out = pa.prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                     scale, max_query_len)
"""

import ctypes
import os

import torch

__all__ = ["load", "PAError", "Call", "cache_store", "decode", "decode_partitions",
           "decode_combine", "prefill", "prepare_cache_store", "prepare_decode",
           "prepare_decode_partitions", "prepare_decode_combine", "prepare_prefill",
           "decode_workspace_bytes", "decode_partition_size", "decode_multi", "prepare_decode_multi",
           "decode_multi_workspace_bytes", "copy_blocks", "swap_blocks", "prepare_copy_blocks",
           "prepare_swap_blocks", "BlockManager", "rmsnorm_residual", "prepare_rmsnorm_residual",
           "swiglu", "prepare_swiglu", "BLOCK_SIZE", "library_path",
           "STATUS"]

BLOCK_SIZE = 16
_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libpa.so")
STATUS = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED",
          4: "PA_ERR_WORKSPACE", 5: "PA_ERR_HIP", 6: "PA_ERR_MEMORY", 7: "PA_ERR_CAPACITY"}

_lib = None

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

_SIGS = {
    "pa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_cache_store": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                      _i64, _i32, _p]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_partition_size": (_i32, [_i32, _i32, _i32]),
    "pa_decode_shared_prefix_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_shared_prefix": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                               _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _p,
                                               _sz, _p]),
    "pa_decode_step": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _i32, _i32, _f32, _i32, _p, _sz, _p]),
    "pa_decode_step_partitions": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32,
                                                 _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _p]),
    "pa_decode": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                 _f32, _i32, _p, _sz, _p]),
    "pa_decode_noalloc": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _f32, _i32, _p]),
    "pa_decode_partitions": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _i32, _f32, _i32, _p]),
    "pa_decode_combine": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p]),
    "pa_prefill": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                  _i32, _i32, _f32, _p]),
    "pa_decode_multi_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_copy_blocks": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _i64, _p]),
    "pa_rmsnorm_residual": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _f32, _p]),
    "pa_swiglu": (ctypes.c_int, [_p, _p, _i64, _i32, _p]),
    "pa_bm_create": (_p, [_i32, _i32, _i32]),
    "pa_bm_destroy": (None, [_p]),
    "pa_bm_num_free_blocks": (_i32, [_p]),
    "pa_bm_num_cached_blocks": (_i32, [_p]),
    "pa_bm_num_free_host_blocks": (_i32, [_p]),
    "pa_bm_block_ref": (_i32, [_p, _i32]),
    "pa_bm_add_sequence": (ctypes.c_int, [_p, _i64, _p, _i32, _p]),
    "pa_bm_commit": (ctypes.c_int, [_p, _i64, _i32]),
    "pa_bm_append_token": (ctypes.c_int, [_p, _i64, _i32, _p, _p, _p]),
    "pa_bm_fork": (ctypes.c_int, [_p, _i64, _i64]),
    "pa_bm_free_sequence": (ctypes.c_int, [_p, _i64]),
    "pa_bm_seq_len": (_i32, [_p, _i64]),
    "pa_bm_block_table": (ctypes.c_int, [_p, _i64, _p, _i32, _p]),
    "pa_bm_slots": (ctypes.c_int, [_p, _i64, _i32, _i32, _p]),
    "pa_bm_swap_out": (ctypes.c_int, [_p, _i64, _p, _p, _i32, _p]),
    "pa_bm_swap_in": (ctypes.c_int, [_p, _i64, _p, _p, _i32, _p]),
    "pa_swap_blocks": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _p]),
    "pa_decode_multi": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _i32, _f32, _i32, _p, _sz, _p]),
}


class PAError(RuntimeError):
    """A libpa entry point returned a status other than PA_OK."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {load().pa_status_str(status).decode()}")


def load():
    """Load libpa.so (once).  Raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"libpa.so is not built ({library_path}); run "
                              "`python -m paged_kv_cache_240_amd.build`")
        lib = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class Call:
    """One library call, validated and marshalled once.

    Calling the object enqueues the operation again with the same pointers,
    sizes and stream (no per-call Python checks), e.g. once per decode step
    while the tensors stay in place.  `result` is what the call writes.
    call(stream) enqueues on another torch stream instead (every entry point
    takes its stream last), e.g. the capture stream of a HIP graph.
    """

    __slots__ = ("name", "fn", "args", "result", "keep")

    def __init__(self, name, args, result=None, keep=(), lib=None):
        self.name = name
        self.fn = getattr(lib if lib is not None else load(), name)
        self.args = args
        self.result = result
        self.keep = keep  # the tensors whose pointers are in args stay alive with the call

    def __call__(self, stream=None):
        args = self.args
        if stream is not None:
            args = args[:-1] + (ctypes.c_void_p(stream.cuda_stream),)
        st = self.fn(*args)
        if st != 0:
            raise PAError(self.name, st)
        return self.result


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, dtype, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() and t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")


def _cache_dims(k_cache, v_cache):
    _check(k_cache, "k_cache", torch.bfloat16, 4)
    _check(v_cache, "v_cache", torch.bfloat16, 4, k_cache.device)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    nb, hkv, bs, d = k_cache.shape
    return nb, hkv, bs, d


def cache_store(q, k, v, k_cache, v_cache, slot_mapping, positions, cos_sin):
    """Fused rotate-half RoPE + KV-cache store (pa_cache_store); q rotated in place.

    q bf16 [T, Hq, D] or None; k, v bf16 [T, Hkv, D]; caches bf16 [NB, Hkv, 16, D];
    slot_mapping, positions int32 [T]; cos_sin float32 [max_pos, D].
    """
    prepare_cache_store(q, k, v, k_cache, v_cache, slot_mapping, positions, cos_sin)()


def prepare_cache_store(q, k, v, k_cache, v_cache, slot_mapping, positions, cos_sin):
    """Validated pa_cache_store call (see cache_store) on the current stream."""
    nb, hkv, bs, d = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _check(k, "k", torch.bfloat16, 3, dev)
    _check(v, "v", torch.bfloat16, 3, dev)
    T = k.shape[0]
    if k.shape != (T, hkv, d) or v.shape != (T, hkv, d):
        raise ValueError("k and v must be [T, Hkv, D] matching the cache")
    hq = 0
    if q is not None:
        _check(q, "q", torch.bfloat16, 3, dev)
        if q.shape[0] != T or q.shape[2] != d:
            raise ValueError("q must be [T, Hq, D]")
        hq = q.shape[1]
    for name, t in (("slot_mapping", slot_mapping), ("positions", positions)):
        _check(t, name, torch.int32, 1, dev)
        if t.shape[0] != T:
            raise ValueError(f"{name} must have T={T} entries")
    _check(cos_sin, "cos_sin", torch.float32, 2, dev)
    if cos_sin.shape[1] != d:
        raise ValueError("cos_sin must be [max_pos, D]")
    return Call("pa_cache_store", (_ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(slot_mapping), _ptr(positions), _ptr(cos_sin), T, hq, hkv,
                                   d, bs, nb, cos_sin.shape[0], _stream(dev)),
                keep=(q, k, v, k_cache, v_cache, slot_mapping, positions, cos_sin))


def decode_workspace_bytes(B, Hq, Hkv, D, max_context_len, partition_size=-1):
    return int(load().pa_decode_workspace_bytes(B, Hq, Hkv, D, max_context_len, partition_size))


def decode_partition_size(B, Hkv, max_context_len):
    return int(load().pa_decode_partition_size(B, Hkv, max_context_len))


def _decode_common(q, k_cache, v_cache, block_tables, context_lens):
    nb, hkv, bs, d = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _check(q, "q", torch.bfloat16, 3, dev)
    B, hq, dq = q.shape
    if dq != d:
        raise ValueError("q head_dim differs from the cache's")
    _check(block_tables, "block_tables", torch.int32, 2, dev)
    _check(context_lens, "context_lens", torch.int32, 1, dev)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables and context_lens must have one row per sequence")
    return dev, B, hq, hkv, d, bs, block_tables.shape[1]


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
           partition_size=-1, out=None, workspace=None):
    """Paged GQA decode (pa_decode).  Returns out bf16 [B, Hq, D].

    max_context_len must bound context_lens (it sizes the grid).  partition_size:
    0 single pass, >0 split-K with that many tokens per partition, -1 library's choice.
    """
    return prepare_decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                          partition_size, out, workspace)()


def prepare_decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                   partition_size=-1, out=None, workspace=None):
    """Validated pa_decode call (see decode); allocates out/workspace once."""
    dev, B, hq, hkv, d, bs, mb = _decode_common(q, k_cache, v_cache, block_tables, context_lens)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", torch.bfloat16, 3, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    P = decode_partition_size(B, hkv, max_context_len) if partition_size == -1 else partition_size
    need = decode_workspace_bytes(B, hq, hkv, d, max_context_len, P) if P > 0 else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check(workspace, "workspace", workspace.dtype, None, dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return Call("pa_decode", (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                              _ptr(context_lens), B, hq, hkv, d, bs, mb, int(max_context_len),
                              float(scale), P, _ptr(workspace), wbytes, _stream(dev)),
                result=out, keep=(q, k_cache, v_cache, block_tables, context_lens, workspace))


def decode_step(q, k, v, k_cache, v_cache, block_tables, context_lens, cos_sin, scale,
                max_context_len, partition_size=-1, out=None, workspace=None):
    """The decode step with the store folded into the decode kernel (pa_decode_step):
    the new token (q, k, v not rotated, one per sequence, at position L-1) is rotated,
    its K/V row stored in the cache, and out = attention over the L tokens; the same
    results as cache_store + decode.  q is not modified.  Returns out bf16 [B, Hq, D]."""
    return prepare_decode_step(q, k, v, k_cache, v_cache, block_tables, context_lens, cos_sin,
                               scale, max_context_len, partition_size, out, workspace)()


def prepare_decode_step(q, k, v, k_cache, v_cache, block_tables, context_lens, cos_sin, scale,
                        max_context_len, partition_size=-1, out=None, workspace=None):
    """Validated pa_decode_step call (see decode_step); allocates out/workspace once."""
    dev, B, hq, hkv, d, bs, mb = _decode_common(q, k_cache, v_cache, block_tables, context_lens)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, torch.bfloat16, 3, dev)
        if t.shape != (B, hkv, d):
            raise ValueError(f"{name} must be [B, Hkv, D] matching the cache")
    _check(cos_sin, "cos_sin", torch.float32, 2, dev)
    if cos_sin.shape[1] != d:
        raise ValueError("cos_sin must be [max_pos, D]")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", torch.bfloat16, 3, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    P = decode_partition_size(B, hkv, max_context_len) if partition_size == -1 else partition_size
    need = decode_workspace_bytes(B, hq, hkv, d, max_context_len, P) if P > 0 else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check(workspace, "workspace", workspace.dtype, None, dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return Call("pa_decode_step", (_ptr(out), _ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(block_tables), _ptr(context_lens), _ptr(cos_sin), B, hq, hkv,
                                   d, bs, mb, int(max_context_len), cos_sin.shape[0], float(scale), P,
                                   _ptr(workspace), wbytes, _stream(dev)),
                result=out, keep=(q, k, v, k_cache, v_cache, block_tables, context_lens, cos_sin,
                                  workspace))


def decode_step_partitions(q, k, v, k_cache, v_cache, block_tables, context_lens, cos_sin, scale,
                           max_context_len, partition_size, o_part=None, lse=None):
    """First stage of decode_step (pa_decode_step_partitions): the store folded into the
    split-K partition kernel.  Returns (o_part fp32 [B, Hq, NP, D], lse fp32 [B, Hq, NP])."""
    return prepare_decode_step_partitions(q, k, v, k_cache, v_cache, block_tables, context_lens,
                                          cos_sin, scale, max_context_len, partition_size, o_part,
                                          lse)()


def prepare_decode_step_partitions(q, k, v, k_cache, v_cache, block_tables, context_lens, cos_sin,
                                   scale, max_context_len, partition_size, o_part=None, lse=None):
    """Validated pa_decode_step_partitions call (see decode_step_partitions)."""
    dev, B, hq, hkv, d, bs, mb = _decode_common(q, k_cache, v_cache, block_tables, context_lens)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, torch.bfloat16, 3, dev)
        if t.shape != (B, hkv, d):
            raise ValueError(f"{name} must be [B, Hkv, D] matching the cache")
    _check(cos_sin, "cos_sin", torch.float32, 2, dev)
    if cos_sin.shape[1] != d:
        raise ValueError("cos_sin must be [max_pos, D]")
    P = int(partition_size)
    if P <= 0:
        raise ValueError("partition_size must be a positive multiple of 16")
    np_ = max(1, -(-int(max_context_len) // P))
    if o_part is None:
        o_part = torch.empty((B, hq, np_, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, hq, np_), dtype=torch.float32, device=dev)
    _check(o_part, "o_part", torch.float32, 4, dev)
    _check(lse, "lse", torch.float32, 3, dev)
    if tuple(o_part.shape) != (B, hq, np_, d) or tuple(lse.shape) != (B, hq, np_):
        raise ValueError("o_part / lse have the wrong shape")
    return Call("pa_decode_step_partitions",
                (_ptr(o_part), _ptr(lse), _ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                 _ptr(block_tables), _ptr(context_lens), _ptr(cos_sin), B, hq, hkv, d, bs, mb,
                 int(max_context_len), cos_sin.shape[0], float(scale), P, _stream(dev)),
                result=(o_part, lse),
                keep=(q, k, v, k_cache, v_cache, block_tables, context_lens, cos_sin))


def decode_shared_prefix(q, k_cache, v_cache, block_tables, context_lens, group_start, prefix_lens,
                         scale, max_context_len, max_group_size, max_prefix, max_suffix_len=None,
                         partition_size=-1, out=None, workspace=None):
    """Decode with the prefixes shared by groups of sequences read once
    (pa_decode_shared_prefix).  group_start int32 [NG+1]: group i is sequences
    group_start[i] .. group_start[i+1]-1; prefix_lens int32 [B]: shared tokens of
    each sequence (whole blocks, 0 outside groups); max_suffix_len bounds L_b - prefix
    (default max_context_len).  Returns out bf16 [B, Hq, D]."""
    return prepare_decode_shared_prefix(q, k_cache, v_cache, block_tables, context_lens, group_start,
                                        prefix_lens, scale, max_context_len, max_group_size,
                                        max_prefix, max_suffix_len, partition_size, out, workspace)()


def prepare_decode_shared_prefix(q, k_cache, v_cache, block_tables, context_lens, group_start,
                                 prefix_lens, scale, max_context_len, max_group_size, max_prefix,
                                 max_suffix_len=None, partition_size=-1, out=None, workspace=None):
    """Validated pa_decode_shared_prefix call (see decode_shared_prefix)."""
    dev, B, hq, hkv, d, bs, mb = _decode_common(q, k_cache, v_cache, block_tables, context_lens)
    _check(prefix_lens, "prefix_lens", torch.int32, 1, dev)
    if prefix_lens.shape[0] != B:
        raise ValueError("prefix_lens must have B entries")
    ng = 0
    if group_start is not None:
        _check(group_start, "group_start", torch.int32, 1, dev)
        ng = group_start.shape[0] - 1
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", torch.bfloat16, 3, dev)
    if max_suffix_len is None:
        max_suffix_len = max_context_len
    need = int(load().pa_decode_shared_prefix_workspace_bytes(B, hq, hkv, d, int(max_suffix_len),
                                                               int(max_prefix), int(partition_size)))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check(workspace, "workspace", workspace.dtype, None, dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return Call("pa_decode_shared_prefix",
                (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
                 _ptr(group_start), _ptr(prefix_lens), B, ng, int(max_group_size), int(max_prefix), hq,
                 hkv, d, bs, mb, int(max_context_len), int(max_suffix_len), float(scale),
                 int(partition_size),
                 _ptr(workspace), wbytes, _stream(dev)),
                result=out, keep=(q, k_cache, v_cache, block_tables, context_lens, group_start,
                                  prefix_lens, workspace))


def decode_multi_workspace_bytes(B, NQ, Hq, Hkv, D, max_context_len, partition_size=-1):
    return int(load().pa_decode_multi_workspace_bytes(B, NQ, Hq, Hkv, D, max_context_len,
                                                      partition_size))


def decode_multi(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                 partition_size=-1, out=None, workspace=None):
    """Multi-query paged decode for speculative verification (pa_decode_multi).

    q bf16 [B, NQ, Hq, D]: query i of sequence b sits at position L_b - NQ + i and
    attends keys up to it.  Returns out bf16 [B, NQ, Hq, D].
    """
    return prepare_decode_multi(q, k_cache, v_cache, block_tables, context_lens, scale,
                                max_context_len, partition_size, out, workspace)()


def prepare_decode_multi(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                         partition_size=-1, out=None, workspace=None):
    """Validated pa_decode_multi call (see decode_multi); allocates out/workspace once."""
    nb, hkv, bs, d = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _check(q, "q", torch.bfloat16, 4, dev)
    B, nq, hq, dq = q.shape
    if dq != d:
        raise ValueError("q head_dim differs from the cache's")
    _check(block_tables, "block_tables", torch.int32, 2, dev)
    _check(context_lens, "context_lens", torch.int32, 1, dev)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables and context_lens must have one row per sequence")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", torch.bfloat16, 4, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    P = int(partition_size)  # -1 is resolved by the library (pa_decode_multi's own rule)
    need = decode_multi_workspace_bytes(B, nq, hq, hkv, d, max_context_len, P) if P != 0 else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check(workspace, "workspace", workspace.dtype, None, dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return Call("pa_decode_multi", (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(block_tables), _ptr(context_lens), B, nq, hq, hkv, d, bs,
                                    block_tables.shape[1], int(max_context_len), float(scale), P,
                                    _ptr(workspace), wbytes, _stream(dev)),
                result=out, keep=(q, k_cache, v_cache, block_tables, context_lens, workspace))


def _pool_dims(t, name):
    """A [num_blocks, Hkv, 16, D] bf16 pool on the device or in pinned host memory."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 4:
        raise ValueError(f"{name} must be a bf16 [num_blocks, Hkv, 16, D] tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda" and not t.is_pinned():
        raise ValueError(f"{name} must be on the GPU or in pinned host memory")
    if t.shape[2] != BLOCK_SIZE:
        raise ValueError(f"{name}: block size must be {BLOCK_SIZE}")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")
    return t.shape[1], t.shape[3]


def copy_blocks(k_cache, v_cache, src_blocks, dst_blocks):
    """Copy-on-write block copies inside one pool pair (pa_copy_blocks)."""
    prepare_copy_blocks(k_cache, v_cache, src_blocks, dst_blocks)()


def prepare_copy_blocks(k_cache, v_cache, src_blocks, dst_blocks):
    nb, hkv, bs, d = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _check(src_blocks, "src_blocks", torch.int32, 1, dev)
    _check(dst_blocks, "dst_blocks", torch.int32, 1, dev)
    n = src_blocks.shape[0]
    if dst_blocks.shape[0] != n:
        raise ValueError("src_blocks and dst_blocks must have the same length")
    return Call("pa_copy_blocks", (_ptr(k_cache), _ptr(v_cache), _ptr(src_blocks), _ptr(dst_blocks),
                                   n, hkv, d, bs, nb, _stream(dev)),
                keep=(k_cache, v_cache, src_blocks, dst_blocks))


def swap_blocks(dst_k, dst_v, src_k, src_v, src_blocks, dst_blocks):
    """Block moves between two pool pairs (pa_swap_blocks); either side may be
    pinned host memory (swap-out / swap-in over PCIe).  The id lists live on the GPU."""
    prepare_swap_blocks(dst_k, dst_v, src_k, src_v, src_blocks, dst_blocks)()


def prepare_swap_blocks(dst_k, dst_v, src_k, src_v, src_blocks, dst_blocks):
    dims = {_pool_dims(t, n) for t, n in ((dst_k, "dst_k"), (dst_v, "dst_v"), (src_k, "src_k"),
                                          (src_v, "src_v"))}
    if len(dims) != 1:
        raise ValueError("all four pools must share Hkv and head_dim")
    (hkv, d), = dims
    if src_blocks.device.type != "cuda":
        raise ValueError("src_blocks/dst_blocks must be on the GPU")
    dev = src_blocks.device
    _check(src_blocks, "src_blocks", torch.int32, 1, dev)
    _check(dst_blocks, "dst_blocks", torch.int32, 1, dev)
    n = src_blocks.shape[0]
    if dst_blocks.shape[0] != n:
        raise ValueError("src_blocks and dst_blocks must have the same length")
    return Call("pa_swap_blocks", (_ptr(dst_k), _ptr(dst_v), _ptr(src_k), _ptr(src_v),
                                   _ptr(src_blocks), _ptr(dst_blocks), n, hkv, d, BLOCK_SIZE,
                                   _stream(dev)),
                keep=(dst_k, dst_v, src_k, src_v, src_blocks, dst_blocks))


def decode_partitions(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                      partition_size, o_part=None, lse=None):
    """First split-K stage (pa_decode_partitions).

    Returns (o_part fp32 [B, Hq, NP, D], lse fp32 [B, Hq, NP]), NP = ceil(max_context_len / P);
    entries of empty partitions are left as they were.
    """
    return prepare_decode_partitions(q, k_cache, v_cache, block_tables, context_lens, scale,
                                     max_context_len, partition_size, o_part, lse)()


def prepare_decode_partitions(q, k_cache, v_cache, block_tables, context_lens, scale,
                              max_context_len, partition_size, o_part=None, lse=None):
    """Validated pa_decode_partitions call (see decode_partitions)."""
    dev, B, hq, hkv, d, bs, mb = _decode_common(q, k_cache, v_cache, block_tables, context_lens)
    P = int(partition_size)
    if P <= 0:
        raise ValueError("partition_size must be a positive multiple of 16")
    np_ = max(1, -(-int(max_context_len) // P))
    if o_part is None:
        o_part = torch.empty((B, hq, np_, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, hq, np_), dtype=torch.float32, device=dev)
    _check(o_part, "o_part", torch.float32, 4, dev)
    _check(lse, "lse", torch.float32, 3, dev)
    if tuple(o_part.shape) != (B, hq, np_, d) or tuple(lse.shape) != (B, hq, np_):
        raise ValueError("o_part / lse have the wrong shape")
    return Call("pa_decode_partitions",
                (_ptr(o_part), _ptr(lse), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                 _ptr(context_lens), B, hq, hkv, d, bs, mb, int(max_context_len), float(scale), P,
                 _stream(dev)),
                result=(o_part, lse), keep=(q, k_cache, v_cache, block_tables, context_lens))


def decode_combine(o_part, lse, context_lens, max_context_len, partition_size, out=None):
    """Second split-K stage (pa_decode_combine).  Returns out bf16 [B, Hq, D]."""
    return prepare_decode_combine(o_part, lse, context_lens, max_context_len, partition_size, out)()


def prepare_decode_combine(o_part, lse, context_lens, max_context_len, partition_size, out=None):
    """Validated pa_decode_combine call (see decode_combine)."""
    dev = o_part.device
    _check(o_part, "o_part", torch.float32, 4, dev)
    _check(lse, "lse", torch.float32, 3, dev)
    _check(context_lens, "context_lens", torch.int32, 1, dev)
    B, hq, np_, d = o_part.shape
    if tuple(lse.shape) != (B, hq, np_) or context_lens.shape[0] != B:
        raise ValueError("shapes of o_part, lse and context_lens disagree")
    if np_ != max(1, -(-int(max_context_len) // int(partition_size))):
        raise ValueError("o_part's partition count does not match max_context_len / partition_size")
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, 3, dev)
    return Call("pa_decode_combine", (_ptr(out), _ptr(o_part), _ptr(lse), _ptr(context_lens), B, hq,
                                      d, int(max_context_len), int(partition_size), _stream(dev)),
                result=out, keep=(o_part, lse, context_lens))


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale,
            max_query_len, out=None):
    """Causal paged chunked prefill (pa_prefill).  Returns out bf16 [T, Hq, D]."""
    return prepare_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale,
                           max_query_len, out)()


def prepare_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale,
                    max_query_len, out=None):
    """Validated pa_prefill call (see prefill)."""
    nb, hkv, bs, d = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _check(q, "q", torch.bfloat16, 3, dev)
    T, hq, dq = q.shape
    if dq != d:
        raise ValueError("q head_dim differs from the cache's")
    _check(block_tables, "block_tables", torch.int32, 2, dev)
    _check(context_lens, "context_lens", torch.int32, 1, dev)
    _check(query_start_loc, "query_start_loc", torch.int32, 1, dev)
    B = context_lens.shape[0]
    if block_tables.shape[0] != B or query_start_loc.shape[0] != B + 1:
        raise ValueError("block_tables / query_start_loc do not match context_lens")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", torch.bfloat16, 3, dev)
    return Call("pa_prefill", (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                               _ptr(context_lens), _ptr(query_start_loc), B, T, hq, hkv, d, bs,
                               block_tables.shape[1], int(max_query_len), float(scale),
                               _stream(dev)),
                result=out, keep=(q, k_cache, v_cache, block_tables, context_lens, query_start_loc))


def rmsnorm_residual(x, weight, residual=None, eps=1e-6, out=None):
    """Fused residual add + RMSNorm (pa_rmsnorm_residual).  x, residual bf16 [T, H]
    (residual updated in place to x + residual); weight bf16 [H].  Returns out."""
    return prepare_rmsnorm_residual(x, weight, residual, eps, out)()


def prepare_rmsnorm_residual(x, weight, residual=None, eps=1e-6, out=None):
    dev = x.device
    _check(x, "x", torch.bfloat16, 2, dev)
    T, H = x.shape
    _check(weight, "weight", torch.bfloat16, 1, dev)
    if weight.shape[0] != H:
        raise ValueError("weight must have H entries")
    if residual is not None:
        _check(residual, "residual", torch.bfloat16, 2, dev)
        if residual.shape != x.shape:
            raise ValueError("residual must have x's shape")
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", torch.bfloat16, 2, dev)
    return Call("pa_rmsnorm_residual", (_ptr(out), _ptr(residual), _ptr(x), _ptr(weight), T, H,
                                        float(eps), _stream(dev)),
                result=out, keep=(x, weight, residual, out))


def swiglu(gate_up, out=None):
    """Fused SwiGLU (pa_swiglu): gate_up bf16 [T, 2I] -> silu(gate) * up, bf16 [T, I]."""
    return prepare_swiglu(gate_up, out)()


def prepare_swiglu(gate_up, out=None):
    dev = gate_up.device
    _check(gate_up, "gate_up", torch.bfloat16, 2, dev)
    T, I2 = gate_up.shape
    if I2 % 2:
        raise ValueError("gate_up must hold gate and up halves")
    if out is None:
        out = torch.empty((T, I2 // 2), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, 2, dev)
    return Call("pa_swiglu", (_ptr(out), _ptr(gate_up), T, I2 // 2, _stream(dev)), result=out,
                keep=(gate_up, out))


class BlockManager:
    """The C++ host block manager of libpa (pa_bm_*): block tables, slot mappings,
    prefix reuse by content, copy-on-write after fork, swap bookkeeping."""

    def __init__(self, num_blocks, num_host_blocks=0, block_size=BLOCK_SIZE):
        self._lib = load()
        self._h = self._lib.pa_bm_create(int(num_blocks), int(num_host_blocks), int(block_size))
        if not self._h:
            raise ValueError("pa_bm_create: bad sizes (block_size must be 16)")

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _ok(self, name, st):
        if st != 0:
            raise PAError(name, st)

    @property
    def num_free_blocks(self):
        return int(self._lib.pa_bm_num_free_blocks(self._h))

    @property
    def num_cached_blocks(self):
        return int(self._lib.pa_bm_num_cached_blocks(self._h))

    @property
    def num_free_host_blocks(self):
        return int(self._lib.pa_bm_num_free_host_blocks(self._h))

    def block_ref(self, block):
        return int(self._lib.pa_bm_block_ref(self._h, int(block)))

    def add_sequence(self, seq_id, tokens):
        """Returns the number of prompt tokens already cached (reused blocks)."""
        arr = (ctypes.c_int32 * len(tokens))(*[int(t) for t in tokens])
        n = ctypes.c_int32()
        self._ok("pa_bm_add_sequence", self._lib.pa_bm_add_sequence(
            self._h, int(seq_id), arr, len(tokens), ctypes.byref(n)))
        return n.value

    def commit(self, seq_id, n_computed_tokens):
        self._ok("pa_bm_commit", self._lib.pa_bm_commit(self._h, int(seq_id), int(n_computed_tokens)))

    def append_token(self, seq_id, token):
        """Returns (slot, cow) with cow = (src_block, dst_block) or None."""
        slot, src, dst = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        self._ok("pa_bm_append_token", self._lib.pa_bm_append_token(
            self._h, int(seq_id), int(token), ctypes.byref(slot), ctypes.byref(src), ctypes.byref(dst)))
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def fork(self, parent_id, child_id):
        self._ok("pa_bm_fork", self._lib.pa_bm_fork(self._h, int(parent_id), int(child_id)))

    def free_sequence(self, seq_id):
        self._ok("pa_bm_free_sequence", self._lib.pa_bm_free_sequence(self._h, int(seq_id)))

    def seq_len(self, seq_id):
        return int(self._lib.pa_bm_seq_len(self._h, int(seq_id)))

    def block_table(self, seq_id):
        n = ctypes.c_int32()
        st = self._lib.pa_bm_block_table(self._h, int(seq_id), None, 0, ctypes.byref(n))
        if st not in (0, 7):
            raise PAError("pa_bm_block_table", st)
        out = (ctypes.c_int32 * max(1, n.value))()
        self._ok("pa_bm_block_table", self._lib.pa_bm_block_table(
            self._h, int(seq_id), out, n.value, ctypes.byref(n)))
        return list(out[:n.value])

    def slots(self, seq_id, start, n):
        out = (ctypes.c_int32 * max(1, n))()
        self._ok("pa_bm_slots", self._lib.pa_bm_slots(self._h, int(seq_id), int(start), int(n), out))
        return list(out[:n])

    def _swap(self, fn, seq_id):
        cap = max(1, len(self.block_table(seq_id)) if fn == "pa_bm_swap_out" else 4096)
        while True:
            a, b = (ctypes.c_int32 * cap)(), (ctypes.c_int32 * cap)()
            n = ctypes.c_int32()
            st = getattr(self._lib, fn)(self._h, int(seq_id), a, b, cap, ctypes.byref(n))
            if st == 7 and n.value > cap:
                cap = n.value
                continue
            self._ok(fn, st)
            return list(a[:n.value]), list(b[:n.value])

    def swap_out(self, seq_id):
        """Returns (device_blocks, host_blocks): copy device -> host with pa_swap_blocks."""
        return self._swap("pa_bm_swap_out", seq_id)

    def swap_in(self, seq_id):
        """Returns (host_blocks, device_blocks): copy host -> device with pa_swap_blocks."""
        return self._swap("pa_bm_swap_in", seq_id)
