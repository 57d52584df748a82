"""pa_decode_step (RoPE + store of the new token folded into the split-K decode
kernel, then the reduce) against the same step as separate calls
(pa_cache_store, then pa_decode with the same partition size), bit for bit --
output and both pools, NaN poison included -- and against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_attention_close, gpu_decode, gpu_store, oracle_decode, oracle_store
from workloads import as_bits

pytestmark = pytest.mark.gpu


def _separate(pa, b, P):
    g = b.to("cuda")
    gpu_store(pa, g)
    return gpu_decode(pa, g, P), g


def _fused(pa, b, P, workspace=None):
    g = b.to("cuda")
    q0 = g.q.clone()
    out = pa.decode_step(g.q, g.k, g.v, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                         g.cos_sin, g.scale, g.max_context_len, partition_size=P, workspace=workspace)
    torch.cuda.synchronize()
    assert torch.equal(g.q, q0), "q is only read"
    return out, g


def _same_bits(a, b):
    return np.array_equal(as_bits(a), as_bits(b))


def _check(pa, b, partitions, label):
    q_ref, kc_ref, vc_ref = oracle_store(b)
    ref = oracle_decode(q_ref, kc_ref, vc_ref, b)
    for P in partitions:
        print(f"{label} P={P}", flush=True)
        o_sep, g_sep = _separate(pa, b, P)
        o_fus, g_fus = _fused(pa, b, P)
        assert _same_bits(o_fus, o_sep), f"{label} P={P}: output differs from store + decode"
        assert _same_bits(g_fus.k_cache, g_sep.k_cache), f"{label} P={P}: K pool"
        assert _same_bits(g_fus.v_cache, g_sep.v_cache), f"{label} P={P}: V pool"
        assert_attention_close(o_fus, ref, f"{label} P={P}")


@pytest.mark.parametrize("poison", [False, True])
def test_tiny(gpu, poison):
    _check(gpu, W.tiny_decode(poison=poison), [0, 16, 32, -1], f"tiny poison={poison}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 6, 8])
def test_ragged_lengths_and_partition_edges(gpu, D, G):
    # new token in row 0 of its block (L = 16k + 1), alone in its partition (L = nP + 1),
    # last row of a block, one token, and ranges longer than one 512-token chunk
    lens = [1, 2, 15, 16, 17, 33, 65, 100, 129, 511, 512, 513, 1000, 1025, 1600]
    Hkv = 2 if G <= 4 else 1
    b = W.decode_batch(lens, G * Hkv, Hkv, D, 512, 5100 + 10 * G + D, theta=1e4, poison=True,
                       table_fill=W.INT32_MIN)
    _check(gpu, b, [0, 16, 48, 64, 128, 144, 256, 512, 1024, -1], f"G={G} D={D}")


def test_qwen_batch1(gpu):
    _check(gpu, W.qwen_decode(), [0, 64, -1], "qwen B=1 L=2048")


def test_cb_step_shared_prefix(gpu):
    _check(gpu, W.cb_step(poison=True), [512, -1], "cb step B=64")


def test_long_context_layer_full_size(gpu):
    # the long-context layer exactly as the benchmark runs it: partitions of 512 tokens
    _check(gpu, W.long_decode_layer(0), [512], "long B=16 L=8192")


def test_repeated_calls_and_workspace_reuse(gpu):
    # one workspace (stale bytes from earlier calls are never read) across repeated calls
    # and other batch shapes
    b = W.decode_batch([700, 33, 1200, 5], 12, 2, 128, 256, 5201, theta=1e4)
    P = 64
    ws = torch.full((1 << 20,), 255, dtype=torch.uint8, device="cuda")

    def step(g):
        o = gpu.decode_step(g.q, g.k, g.v, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                            g.cos_sin, g.scale, g.max_context_len, partition_size=P, workspace=ws)
        torch.cuda.synchronize()
        return o

    g = b.to("cuda")
    o1 = step(g)
    for _ in range(3):   # the new row is rewritten with the same bits: the same output each time
        assert _same_bits(step(g), o1)
    for lens, seed in (([300, 64], 5202), ([90] * 12, 5203)):
        b2 = W.decode_batch(lens, 12, 2, 128, 128, seed, theta=1e4)
        o_sep, _ = _separate(gpu, b2, P)
        assert _same_bits(step(b2.to("cuda")), o_sep)


def test_empty_sequences(gpu):
    # L = 0: zero output, nothing written; the others as the separate calls with that slot skipped
    lens = [40, 0, 17, 0]
    b = W.decode_batch([max(L, 1) for L in lens], 12, 2, 128, 64, 5203, theta=1e4, poison=True)
    b.context_lens = torch.tensor(lens, dtype=torch.int32)
    b.slot_mapping = torch.where(b.context_lens > 0, b.slot_mapping, torch.full_like(b.slot_mapping, -1))
    for P in (0, 16):
        o_sep, g_sep = _separate(gpu, b, P)
        o_fus, g_fus = _fused(gpu, b, P)
        assert _same_bits(o_fus, o_sep) and (o_fus[1] == 0).all() and (o_fus[3] == 0).all()
        assert _same_bits(g_fus.k_cache, g_sep.k_cache) and _same_bits(g_fus.v_cache, g_sep.v_cache)


def test_stages_equal_the_separate_stages(gpu):
    # pa_decode_step_partitions writes the partials pa_decode_partitions writes after the
    # store (bit for bit), and the new rows; pa_decode_combine then gives pa_decode_step's out
    b = W.decode_batch([1, 17, 700, 1025], 12, 2, 128, 256, 5204, theta=1e4, poison=True)
    P = 64
    g1 = b.to("cuda")
    gpu_store(gpu, g1)
    o1, l1 = gpu.decode_partitions(g1.q, g1.k_cache, g1.v_cache, g1.block_tables, g1.context_lens,
                                   g1.scale, g1.max_context_len, P)
    g2 = b.to("cuda")
    o2, l2 = gpu.decode_step_partitions(g2.q, g2.k, g2.v, g2.k_cache, g2.v_cache, g2.block_tables,
                                        g2.context_lens, g2.cos_sin, g2.scale, g2.max_context_len, P)
    torch.cuda.synchronize()
    lens = b.context_lens.numpy()
    for s, L in enumerate(lens):   # partitions past ceil(L/P) are not written
        n = -(-int(L) // P)
        assert torch.equal(o1[s, :, :n], o2[s, :, :n]) and torch.equal(l1[s, :, :n], l2[s, :, :n])
    assert _same_bits(g1.k_cache, g2.k_cache) and _same_bits(g1.v_cache, g2.v_cache)
    out = gpu.decode_combine(o2, l2, g2.context_lens, g2.max_context_len, P)
    o_step, _ = _fused(gpu, b, P)
    assert _same_bits(out, o_step)
