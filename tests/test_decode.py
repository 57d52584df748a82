"""pa_decode (single pass and split-K + combine) on the GPU against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import (assert_attention_close, gpu_decode, gpu_store, oracle_decode, oracle_store)
from workloads import as_bits

pytestmark = pytest.mark.gpu


def _store_then_decode(pa, b, partitions):
    """Store the new tokens, decode, and compare with the oracle doing the same."""
    q_ref, kc_ref, vc_ref = oracle_store(b)
    ref = oracle_decode(q_ref, kc_ref, vc_ref, b)
    g = b.to("cuda")
    gpu_store(pa, g)
    outs = {}
    for P in partitions:
        out = gpu_decode(pa, g, P)
        outs[P] = out
        assert_attention_close(out, ref, f"{b.name} P={P}")
    return g, ref, outs


@pytest.mark.parametrize("poison", [False, True])
def test_tiny_decode(gpu, poison):
    b = W.tiny_decode(poison=poison)
    g, ref, outs = _store_then_decode(gpu, b, [0, 16, 32, -1])
    # L = 1: the output is the new token's value row, exactly, in every head
    v0 = g.v[0, 0]
    for out in outs.values():
        assert torch.equal(out[0, 0], v0) and torch.equal(out[0, 1], v0)


def test_qwen_decode_shape(gpu):
    b = W.qwen_decode()
    g = b.to("cuda")
    ref = oracle_decode(as_bits(b.q), as_bits(b.k_cache), as_bits(b.v_cache), b)
    for P in (0, 16, 64, 512, -1):
        assert_attention_close(gpu_decode(gpu, g, P), ref, f"qwen P={P}")


@pytest.mark.parametrize("poison", [False, True])
def test_cb_step(gpu, poison):
    b = W.cb_step(poison=poison)
    _store_then_decode(gpu, b, [0, 512, -1])


def test_long_decode_one_layer_full_size(gpu):
    # the long-context layer exactly as the benchmark runs it: split-K of 512 tokens
    b = W.long_decode_layer(0)
    _store_then_decode(gpu, b, [512])


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8])
def test_head_shapes_and_ragged_lengths(gpu, D, G):
    lens = [0, 1, 2, 15, 16, 17, 100, 511, 512, 513, 1000]
    Hkv = 2 if G <= 4 else 1
    b = W.decode_batch([max(L, 1) for L in lens], G * Hkv, Hkv, D, 512, 1000 + 10 * G + D,
                       theta=1e4)
    b.context_lens = torch.tensor(lens, dtype=torch.int32)  # one empty sequence
    ref = oracle_decode(as_bits(b.q), as_bits(b.k_cache), as_bits(b.v_cache), b)
    g = b.to("cuda")
    # partitions of 2, 4 and 8 blocks per wave (up to 128, 256 and 512 tokens), and a single pass
    for P in (0, 16, 48, 128, 208, 256, 512, -1):
        out = gpu_decode(gpu, g, P)
        assert_attention_close(out, ref, f"G={G} D={D} P={P}")
        assert (out[0] == 0).all()


def test_wide_score_range(gpu):
    # q scaled by 64 (exact in bf16): scores spread over hundreds
    b = W.decode_batch([1, 17, 300, 1025, 4096], 12, 2, 128, 512, 1090, theta=1e4)
    b.q = (b.q.float() * 64).to(torch.bfloat16)
    ref = oracle_decode(as_bits(b.q), as_bits(b.k_cache), as_bits(b.v_cache), b)
    g = b.to("cuda")
    for P in (0, 16, 64, 512, -1):
        assert_attention_close(gpu_decode(gpu, g, P), ref, f"q x 64 P={P}")


def test_block_permutation_and_rerun_bit_identical(gpu):
    b = W.cb_step()
    g = b.to("cuda")
    out1 = gpu_decode(gpu, g, -1)
    out1b = gpu_decode(gpu, g, -1)
    assert torch.equal(out1, out1b)
    sigma = torch.randperm(b.num_blocks, generator=torch.Generator().manual_seed(5))
    kc2 = torch.empty_like(b.k_cache)
    vc2 = torch.empty_like(b.v_cache)
    kc2[sigma] = b.k_cache
    vc2[sigma] = b.v_cache
    bt = b.block_tables.long()
    bt2 = torch.where(bt >= 0, sigma[bt.clamp(min=0)], bt).to(torch.int32)
    out2 = gpu.decode(g.q, kc2.cuda(), vc2.cuda(), bt2.cuda(), g.context_lens, b.scale,
                      b.max_context_len, partition_size=-1)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


def test_aliased_prefix_equals_private_copies(gpu):
    # sequences 0-31 of the continuous-batching step read one shared 125-block prefix;
    # giving each its own copy of those blocks changes no output bit
    b = W.cb_step()
    g = b.to("cuda")
    out_alias = gpu_decode(gpu, g, 512)
    bt = b.block_tables.clone()
    extra = 31 * 125  # a private copy of the prefix for sequences 1..31, appended to the pool
    kc = torch.cat([b.k_cache, torch.zeros((extra,) + tuple(b.k_cache.shape[1:]), dtype=torch.bfloat16)])
    vc = torch.cat([b.v_cache, torch.zeros((extra,) + tuple(b.v_cache.shape[1:]), dtype=torch.bfloat16)])
    nxt = b.num_blocks
    for s in range(1, 32):
        for j in range(125):
            src = int(bt[s, j])
            kc[nxt] = kc[src]
            vc[nxt] = vc[src]
            bt[s, j] = nxt
            nxt += 1
    out_priv = gpu.decode(g.q, kc.cuda(), vc.cuda(), bt.cuda(), g.context_lens, b.scale,
                          b.max_context_len, partition_size=512)
    torch.cuda.synchronize()
    assert torch.equal(out_alias, out_priv)


def test_stages_equal_fused_call_and_oracle_partials(gpu):
    b = W.decode_batch([1, 47, 300, 700], 12, 2, 128, 256, 81, theta=1e6)
    g = b.to("cuda")
    P = 128
    o_part, lse = gpu.decode_partitions(g.q, g.k_cache, g.v_cache, g.block_tables,
                                        g.context_lens, b.scale, b.max_context_len, P)
    out = gpu.decode_combine(o_part, lse, g.context_lens, b.max_context_len, P)
    torch.cuda.synchronize()
    assert torch.equal(out, gpu_decode(gpu, g, P))
    # partials against the oracle's Flash-Decode partials
    qb, kc, vc = as_bits(b.q), as_bits(b.k_cache), as_bits(b.v_cache)
    o_part, lse = o_part.cpu().numpy(), lse.cpu().numpy()
    for s, L in enumerate(b.context_lens.tolist()):
        K, V = oracle.gather_sequence_kv(kc, vc, b.block_tables[s].numpy(), L)
        m, l, o = oracle.decode_partials(oracle.bf16_to_f64(qb[s]), K, V, L, b.scale, P)
        n = -(-L // P)
        ref_o = o / l[:, :, None]                            # [n, Hq, D]
        ref_lse = (m + np.log(l)) / np.log(2.0)              # base 2
        assert np.abs(o_part[s, :, :n].transpose(1, 0, 2) - ref_o).max() < 2e-3
        assert np.abs(lse[s, :, :n].T - ref_lse).max() < 1e-4 * (1 + np.abs(ref_lse).max())


def test_empty_batch_and_empty_sequences(gpu):
    b = W.decode_batch([3, 3], 4, 2, 64, 4, 82)
    g = b.to("cuda")
    g.context_lens.zero_()
    for P in (0, 16):
        out = gpu.decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, b.scale, 16,
                         partition_size=P)
        torch.cuda.synchronize()
        assert (out == 0).all()
