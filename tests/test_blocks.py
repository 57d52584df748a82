"""pa_copy_blocks / pa_swap_blocks (copy-on-write and swap of whole KV blocks)
against the oracle, bit for bit."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import gpu_decode, gpu_store
from workloads import as_bits

pytestmark = pytest.mark.gpu


def _pool(nb, hkv, d, seed, device="cuda", pin=False):
    g = torch.Generator().manual_seed(seed)
    bits = torch.randint(-2 ** 15, 2 ** 15, (nb, hkv, 16, d), generator=g, dtype=torch.int16)
    t = bits.view(torch.bfloat16)
    if pin:
        return t.pin_memory()
    return t.to(device)


def _ids(values, device="cuda"):
    return torch.tensor(values, dtype=torch.int32, device=device)


@pytest.mark.parametrize("hkv,d", [(2, 128), (1, 64), (8, 128)])
def test_copy_on_write_in_device_pools(gpu, hkv, d):
    kc, vc = _pool(64, hkv, d, 1), _pool(64, hkv, d, 2)
    src = [3, 17, 17, 40, 0, 63]
    dst = [50, 51, 9, 10, 11, 12]
    k_ref = oracle.copy_blocks(as_bits(kc), as_bits(kc), src, dst)
    v_ref = oracle.copy_blocks(as_bits(vc), as_bits(vc), src, dst)
    gpu.copy_blocks(kc, vc, _ids(src), _ids(dst))
    torch.cuda.synchronize()
    assert np.array_equal(as_bits(kc), k_ref) and np.array_equal(as_bits(vc), v_ref)


def test_swap_out_and_back_in(gpu):
    hkv, d = 2, 128
    kc, vc = _pool(256, hkv, d, 3), _pool(256, hkv, d, 4)
    hk, hv = _pool(32, hkv, d, 5, pin=True), _pool(32, hkv, d, 6, pin=True)
    seq = list(range(100, 120, 2)) + [7, 255]         # a preempted sequence's blocks
    slots = list(range(3, 3 + len(seq)))              # host slots
    hk_ref = oracle.copy_blocks(as_bits(hk), as_bits(kc), seq, slots)
    hv_ref = oracle.copy_blocks(as_bits(hv), as_bits(vc), seq, slots)
    gpu.swap_blocks(hk, hv, kc, vc, _ids(seq), _ids(slots))        # swap out (device -> host)
    torch.cuda.synchronize()
    assert np.array_equal(hk.view(torch.int16).numpy().view(np.uint16), hk_ref)
    assert np.array_equal(hv.view(torch.int16).numpy().view(np.uint16), hv_ref)
    # swap in to newly allocated device blocks of a second pool pair
    kc2, vc2 = _pool(128, hkv, d, 7), _pool(128, hkv, d, 8)
    new = [127 - i for i in range(len(seq))]
    k2_ref = oracle.copy_blocks(as_bits(kc2), hk_ref, slots, new)
    v2_ref = oracle.copy_blocks(as_bits(vc2), hv_ref, slots, new)
    gpu.swap_blocks(kc2, vc2, hk, hv, _ids(slots), _ids(new))      # swap in (host -> device)
    torch.cuda.synchronize()
    assert np.array_equal(as_bits(kc2), k2_ref) and np.array_equal(as_bits(vc2), v2_ref)
    assert np.array_equal(as_bits(kc2)[new], as_bits(kc)[seq])


def test_empty_copy_is_a_no_op(gpu):
    kc, vc = _pool(8, 2, 128, 9), _pool(8, 2, 128, 10)
    before = as_bits(kc).copy()
    gpu.copy_blocks(kc, vc, _ids([]), _ids([]))
    torch.cuda.synchronize()
    assert np.array_equal(as_bits(kc), before)


class _PtrAttr(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int), ("device", ctypes.c_int), ("devicePointer", ctypes.c_void_p),
                ("hostPointer", ctypes.c_void_p), ("isManaged", ctypes.c_int),
                ("allocationFlags", ctypes.c_uint)]


def _runtime_sees_as_accessible(ptr):
    """What the HIP runtime reports for a host pointer (query only, nothing launched)."""
    hip = ctypes.CDLL("libamdhip64.so")
    a = _PtrAttr()
    rc = hip.hipPointerGetAttributes(ctypes.byref(a), ctypes.c_void_p(ptr))
    hip.hipGetLastError()
    return rc == 0 and (a.type == 2 or (a.type == 1 and a.devicePointer))


def test_pageable_host_memory_is_refused(gpu):
    # the C library checks every pointer before launching: plain (pageable) host
    # memory is neither device memory nor mapped for the device
    lib = gpu.load()
    kc, vc = _pool(8, 2, 128, 11), _pool(8, 2, 128, 12)
    host = np.zeros((8, 2, 16, 128), dtype=np.uint16)
    if _runtime_sees_as_accessible(host.ctypes.data):
        pytest.skip("this runtime maps pageable memory for the device; nothing to refuse")
    hp = ctypes.c_void_p(host.ctypes.data)
    ids = _ids([0, 1])
    st = lib.pa_swap_blocks(hp, hp, ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(vc.data_ptr()),
                            ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(ids.data_ptr()), 2, 2,
                            128, 16, None)
    assert st == 6  # PA_ERR_MEMORY
    assert not host.any()
    # and the refusal leaves no error behind for the next call
    gpu.copy_blocks(kc, vc, _ids([0]), _ids([5]))
    torch.cuda.synchronize()
    assert torch.equal(kc[5].view(torch.int16), kc[0].view(torch.int16))  # bits: the pool holds NaN patterns


def test_copy_on_write_keeps_decode_bit_identical(gpu):
    # two sequences share a 2-block prefix; one gets private copies of those blocks
    # (copy-on-write) and its table points at them: decode is unchanged, bit for bit
    b = W.decode_batch([40, 40], 12, 2, 128, 16, 90, shared_prefix=([0, 1], 2))
    g = b.to("cuda")
    gpu_store(gpu, g)
    ref = gpu_decode(gpu, g, 0)
    bt = g.block_tables.cpu().numpy()
    free = np.setdiff1d(np.arange(16), bt[bt >= 0])[:2]
    gpu.copy_blocks(g.k_cache, g.v_cache, _ids(bt[1, :2].tolist()), _ids(free.tolist()))
    g.block_tables[1, :2] = torch.from_numpy(free.astype(np.int32)).cuda()
    out = gpu_decode(gpu, g, 0)
    assert torch.equal(out, ref)
