"""pa_decode_multi (speculative verification: NQ causal queries per sequence)
against the oracle's chunked prefill with chunks of NQ rows."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_attention_close, gpu_store, oracle_store
from workloads import as_bits

pytestmark = pytest.mark.gpu


def _oracle(qbits, kc, vc, b, nq):
    out = oracle.prefill(qbits, kc, vc, b.block_tables.cpu().numpy(), b.context_lens.cpu().numpy(),
                         b.query_start_loc.cpu().numpy(), b.scale)
    return out.reshape(b.B, nq, b.Hq, b.D)


def _run(pa, b, nq, partitions, label):
    q_ref, kc_ref, vc_ref = oracle_store(b)
    ref = _oracle(q_ref, kc_ref, vc_ref, b, nq)
    g = b.to("cuda")
    gpu_store(pa, g)
    q = g.q.view(b.B, nq, b.Hq, b.D)
    outs = {}
    for P in partitions:
        out = pa.decode_multi(q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, g.scale,
                              g.max_context_len, partition_size=P)
        torch.cuda.synchronize()
        assert_attention_close(out, ref, f"{label} P={P}")
        outs[P] = out
    return g, q, ref, outs


def test_spec_verify_workload(gpu):
    # 16 sequences x 8192 tokens, 5 queries each (4 drafts), Qwen head shape; 512-token partitions
    # and the library choice (1024: one 8-wave chunk per workgroup)
    _run(gpu, W.spec_verify(), 5, [512, -1], "spec verify 16x8192")


@pytest.mark.parametrize("nq", [1, 2, 5])
def test_ragged_lengths_qwen_shape(gpu, nq):
    lens = [nq, nq + 1, 16, 17, 33, 100, 511, 512, 513, 1500, 2048]
    b = W.verify_batch(lens, nq, 12, 2, 128, 512, 3300 + nq, poison=True, table_fill=W.INT32_MIN)
    _run(gpu, b, nq, [0, 16, 64, 512, 1024, -1], f"ragged nq={nq}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,Hkv,nq", [(1, 2, 16), (2, 1, 5), (3, 2, 10), (6, 2, 5), (8, 1, 4),
                                      (8, 1, 2), (4, 2, 3)])
def test_head_shapes(gpu, D, G, Hkv, nq):
    # rows nq*G from 6 to 32: one or two 16-row tiles
    lens = [nq, 40, 77, 300, 1025]
    b = W.verify_batch(lens, nq, G * Hkv, Hkv, D, 256, 3400 + 7 * G + nq + D, theta=1e4,
                       poison=True, table_fill=W.INT32_MIN)
    _run(gpu, b, nq, [0, 64, 512, 768, 1024], f"G={G} Hkv={Hkv} nq={nq} D={D}")


def test_wide_score_range(gpu):
    # q scaled by 64 (exact in bf16): a row maximum taken too low would overflow
    lens = [5, 40, 300, 1025, 2048]
    b = W.verify_batch(lens, 5, 12, 2, 128, 512, 3450, theta=1e4)
    b.q = (b.q.float() * 64).to(torch.bfloat16)
    _run(gpu, b, 5, [0, 64, 512, -1], "q x 64")


def test_one_query_is_decode(gpu):
    # NQ = 1 is a decode step: both entry points agree with the oracle and closely with each other
    b = W.verify_batch([1, 15, 16, 33, 700, 2048], 1, 12, 2, 128, 256, 3501)
    g, q, ref, outs = _run(gpu, b, 1, [0, 64], "nq=1")
    dec = gpu.decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, g.scale,
                     g.max_context_len, partition_size=64)
    torch.cuda.synchronize()
    assert_attention_close(dec, ref.reshape(b.B, b.Hq, b.D), "pa_decode")
    diff = (dec.float() - outs[64].view(b.B, b.Hq, b.D).float()).abs().max().item()
    assert diff <= 2 ** -4, diff


def test_matches_prefill_entry_point(gpu):
    # the same step through pa_prefill (chunks of NQ rows): both within tolerance of the oracle
    b = W.verify_batch([5, 64, 1000, 3000], 5, 12, 2, 128, 512, 3502)
    g, q, ref, outs = _run(gpu, b, 5, [-1], "vs prefill")
    pre = gpu.prefill(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, g.query_start_loc,
                      g.scale, g.max_query_len)
    torch.cuda.synchronize()
    assert_attention_close(pre.view(b.B, 5, b.Hq, b.D), ref, "pa_prefill")


def test_single_key_rows_are_v(gpu):
    # L = NQ: query 0 sees exactly one key, so its output is that key's V row (bit-exact)
    nq = 5
    b = W.verify_batch([nq, nq, nq], nq, 12, 2, 128, 64, 3503)
    g, q, ref, outs = _run(gpu, b, nq, [0, 16], "L=NQ")
    v_first = g.v[::nq]  # value rows of each sequence's first new token [B, Hkv, D]
    for P, out in outs.items():
        for h in range(b.Hq):
            assert torch.equal(out[:, 0, h], v_first[:, h // (b.Hq // b.Hkv)]), (P, h)


def test_empty_sequences(gpu):
    # sequences with L = 0 give zeros; their neighbours are unchanged, bit for bit
    nq = 3
    b = W.verify_batch([nq, 50], nq, 12, 2, 128, 64, 3504)
    g = b.to("cuda")
    gpu_store(gpu, g)
    q2 = g.q.view(2, nq, 12, 128)
    fill = torch.full_like(g.block_tables[:1], W.INT32_MIN)
    bt4 = torch.cat([fill, g.block_tables[:1], fill, g.block_tables[1:]]).contiguous()
    lens4 = torch.tensor([0, nq, 0, 50], dtype=torch.int32, device="cuda")
    q4 = torch.stack([torch.full_like(q2[0], float("nan")), q2[0], q2[1], q2[1]]).contiguous()
    for P in (0, 16):
        ref = gpu.decode_multi(q2, g.k_cache, g.v_cache, g.block_tables, g.context_lens, g.scale, 50,
                               partition_size=P)
        out = gpu.decode_multi(q4, g.k_cache, g.v_cache, bt4, lens4, g.scale, 50, partition_size=P)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[2]) == 0
        assert torch.equal(out[1], ref[0]) and torch.equal(out[3], ref[1])


def test_rerun_and_permutation_bit_identical(gpu):
    nq = 5
    b = W.verify_batch([300, 1000], nq, 12, 2, 128, 256, 3505)
    g = b.to("cuda")
    gpu_store(gpu, g)
    q = g.q.view(2, nq, 12, 128)
    o1 = gpu.decode_multi(q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, g.scale, 1000, 64)
    o2 = gpu.decode_multi(q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, g.scale, 1000, 64)
    # move every block to a new physical id: same output, bit for bit
    perm = torch.randperm(g.k_cache.shape[0], generator=torch.Generator().manual_seed(7))
    kc2 = torch.empty_like(g.k_cache)
    vc2 = torch.empty_like(g.v_cache)
    kc2[perm.cuda()] = g.k_cache
    vc2[perm.cuda()] = g.v_cache
    bt2 = torch.where(g.block_tables >= 0, perm.cuda().to(torch.int32)[g.block_tables.clamp(min=0).long()],
                      g.block_tables)
    o3 = gpu.decode_multi(q, kc2, vc2, bt2, g.context_lens, g.scale, 1000, 64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
