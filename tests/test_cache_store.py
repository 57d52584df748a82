"""pa_cache_store on the GPU against the oracle: bit-exact pools and queries."""

import numpy as np
import pytest
import torch

import workloads as W
from parity import gpu_store, oracle_store
from workloads import as_bits

pytestmark = pytest.mark.gpu


def _check_exact(gpu, b_host, g):
    q_ref, kc_ref, vc_ref = oracle_store(b_host)
    assert np.array_equal(as_bits(g.k_cache), kc_ref), "k_cache differs"
    assert np.array_equal(as_bits(g.v_cache), vc_ref), "v_cache differs"
    assert np.array_equal(as_bits(g.q), q_ref), "rotated q differs"


@pytest.mark.parametrize("make", [W.tiny_decode, lambda: W.tiny_decode(poison=True), W.qwen_decode,
                                  W.cb_step, W.chunked_prefill],
                         ids=["tiny", "tiny-poison", "qwen", "cb-step", "chunked-prefill"])
def test_store_bit_exact(gpu, make):
    b = make()
    g = b.to("cuda")
    gpu_store(gpu, g)
    _check_exact(gpu, b, g)


def test_store_padding_and_no_query(gpu):
    b = W.decode_batch([5, 40, 17, 64, 3], 12, 2, 128, 64, 77, theta=1e6)
    b.slot_mapping[[1, 3]] = -1  # padding tokens
    g = b.to("cuda")
    q_before = g.q.clone()
    gpu_store(gpu, g)
    _check_exact(gpu, b, g)
    assert torch.equal(g.q[1], q_before[1]) and torch.equal(g.q[3], q_before[3])
    # without q only the pool changes, with the same bits
    g2 = b.to("cuda")
    gpu.cache_store(None, g2.k, g2.v, g2.k_cache, g2.v_cache, g2.slot_mapping, g2.positions,
                    g2.cos_sin)
    torch.cuda.synchronize()
    assert torch.equal(g2.k_cache, g.k_cache) and torch.equal(g2.v_cache, g.v_cache)
    assert torch.equal(g2.q, q_before)


def test_store_untouched_slots_are_canaries(gpu):
    b = W.decode_batch([33, 1, 16], 4, 4, 64, 16, 78, theta=1e4)
    g = b.to("cuda")
    canary = 0x5A5A
    g.k_cache.view(torch.int16).fill_(canary)
    g.v_cache.view(torch.int16).fill_(canary)
    gpu_store(gpu, g)
    kc = as_bits(g.k_cache)
    written = np.zeros(kc.shape[:1] + kc.shape[2:3], bool)
    for s in b.slot_mapping.tolist():
        written[s // 16, s % 16] = True
    untouched = ~written[:, None, :, None].repeat(kc.shape[1], 1).repeat(kc.shape[3], 3)
    assert (kc[untouched] == canary).all() and (as_bits(g.v_cache)[untouched] == canary).all()
    assert (kc[~untouched] != canary).any()


def test_store_position_zero_is_identity(gpu):
    b = W.decode_batch([1, 1, 1], 2, 2, 128, 8, 79, theta=1e6)  # every token at position 0
    g = b.to("cuda")
    q0 = g.q.clone()
    gpu_store(gpu, g)
    assert torch.equal(g.q, q0)
    for i, s in enumerate(b.slot_mapping.tolist()):
        assert torch.equal(g.k_cache[s // 16, :, s % 16], g.k[i])


def test_store_large_positions(gpu):
    # positions near the end of a long table (angles up to ~8191 rad on pair 0)
    b = W.decode_batch([8190, 8191, 8192], 12, 2, 128, 1536, 80, theta=1e6)
    g = b.to("cuda")
    gpu_store(gpu, g)
    _check_exact(gpu, b, g)
