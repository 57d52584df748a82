"""pa_decode_noalloc -- pa_decode with its split-K workspace in the library's own
device array -- against pa_decode on the same inputs, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input (so it reuses the
array the first one filled), each bit-identical to pa_decode with a caller
workspace; a request whose workspace would exceed the array is refused on the
host with PA_ERR_WORKSPACE."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_attention_close
from workloads import as_bits

pytestmark = pytest.mark.gpu

WS = 4  # PA_ERR_WORKSPACE
SCRATCH = 16 << 20


def _noalloc(pa, b, partition_size):
    lib = pa.load()
    out = torch.empty_like(b.q)
    P = ctypes.c_void_p
    print(f"pa_decode_noalloc B={b.B} L<={b.max_context_len} P={partition_size}", flush=True)
    st = lib.pa_decode_noalloc(P(out.data_ptr()), P(b.q.data_ptr()), P(b.k_cache.data_ptr()),
                               P(b.v_cache.data_ptr()), P(b.block_tables.data_ptr()),
                               P(b.context_lens.data_ptr()), b.B, b.Hq, b.Hkv, b.D, 16,
                               b.block_tables.shape[1], b.max_context_len, b.scale, partition_size,
                               P(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.pa_status_str(st)
    torch.cuda.synchronize()
    return out


def _with_workspace(pa, b, partition_size):
    out = pa.decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.scale,
                    b.max_context_len, partition_size=partition_size)
    torch.cuda.synchronize()
    return out


def test_two_calls_then_a_smaller_one(gpu):
    pa = gpu
    # 1: the long-context layer (16 x 8192 tokens, 512-token partitions: 1.6 MB of partials)
    big = W.long_decode_layer(0, device="cuda")
    pa.cache_store(big.q, big.k, big.v, big.k_cache, big.v_cache, big.slot_mapping, big.positions, big.cos_sin)
    assert pa.decode_workspace_bytes(big.B, big.Hq, big.Hkv, big.D, big.max_context_len, 512) <= SCRATCH
    y1 = _noalloc(pa, big, 512)
    assert torch.equal(y1, _with_workspace(pa, big, 512))
    # 2: a smaller, ragged batch with the library's partition choice, into the same array
    small = W.decode_batch([1, 15, 16, 33, 700, 1000], 12, 2, 128, 512, 4242, theta=1e6, poison=True,
                           table_fill=W.INT32_MIN, device="cuda")
    pa.cache_store(small.q, small.k, small.v, small.k_cache, small.v_cache, small.slot_mapping,
                   small.positions, small.cos_sin)
    y2 = _noalloc(pa, small, -1)
    assert torch.equal(y2, _with_workspace(pa, small, -1))
    ref = oracle.decode(as_bits(small.q), as_bits(small.k_cache), as_bits(small.v_cache),
                        small.block_tables.cpu().numpy(), small.context_lens.cpu().numpy(), small.scale)
    assert_attention_close(y2, ref, "pa_decode_noalloc, ragged batch")
    # 3: the first input again, after the smaller call changed the array's contents
    y3 = _noalloc(pa, big, 512)
    assert torch.equal(y3, y1)


def test_refuses_more_than_the_array(gpu):
    pa = gpu
    lib = pa.load()
    B, Hq, Hkv, D, L = 256, 12, 2, 128, 32768
    assert pa.decode_workspace_bytes(B, Hq, Hkv, D, L, 512) > SCRATCH
    t = torch.zeros(64, dtype=torch.int32, device="cuda")
    P = ctypes.c_void_p(t.data_ptr())
    # max_blocks = 1 would fail pa_decode's own shape check too: nothing can launch
    st = lib.pa_decode_noalloc(P, P, P, P, P, P, B, Hq, Hkv, D, 16, 1, L, 0.088, 512, None)
    assert st == WS, lib.pa_status_str(st)
