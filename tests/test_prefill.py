"""pa_prefill (causal paged chunked prefill on matrix cores) against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_attention_close, gpu_store, oracle_store
from workloads import as_bits

pytestmark = pytest.mark.gpu


def _oracle_prefill(qbits, kc, vc, b):
    return oracle.prefill(qbits, kc, vc, b.block_tables.cpu().numpy(), b.context_lens.cpu().numpy(),
                          b.query_start_loc.cpu().numpy(), b.scale)


def _gpu_prefill(pa, g):
    out = pa.prefill(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, g.query_start_loc,
                     g.scale, g.max_query_len)
    torch.cuda.synchronize()
    return out


def _store_then_prefill(pa, b, label):
    q_ref, kc_ref, vc_ref = oracle_store(b)
    ref = _oracle_prefill(q_ref, kc_ref, vc_ref, b)
    g = b.to("cuda")
    gpu_store(pa, g)
    out = _gpu_prefill(pa, g)
    e = assert_attention_close(out, ref, label)
    return g, out, ref, e


def test_chunked_prefill_workload(gpu):
    # 4 sequences: 2048 cached tokens + a 512-token chunk, Qwen head shape, theta 1e6
    _store_then_prefill(gpu, W.chunked_prefill(), "chunked prefill 4x(2048+512)")


def test_chunked_prefill_poisoned(gpu):
    _store_then_prefill(gpu, W.chunked_prefill(poison=True), "chunked prefill, NaN-poisoned pool")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,Hkv", [(1, 2), (2, 1), (3, 2), (6, 2), (8, 1)])
def test_ragged_chunks(gpu, D, G, Hkv):
    prefix = [0, 7, 16, 100, 33, 0, 250]
    chunk = [1, 5, 16, 17, 129, 64, 300]
    b = W.prefill_batch(prefix, chunk, G * Hkv, Hkv, D, 256, 3000 + 17 * G + D, theta=1e4,
                        poison=True, table_fill=W.INT32_MIN)
    _store_then_prefill(gpu, b, f"ragged G={G} Hkv={Hkv} D={D}")


def test_chunks_of_one_token(gpu):
    # a chunk of one row is a decode step
    b = W.prefill_batch([0, 15, 16, 500, 2047], [1] * 5, 12, 2, 128, 256, 3101, theta=1e6)
    _store_then_prefill(gpu, b, "chunks of one")


def test_empty_chunks_and_long_prompt(gpu):
    # sequences with no new rows are skipped; a whole 1000-token prompt in one chunk
    b = W.prefill_batch([40, 0, 16, 0], [0, 1000, 0, 3], 12, 2, 128, 256, 3102, theta=1e6)
    g, out, ref, _ = _store_then_prefill(gpu, b, "empty chunks")
    assert b.T == 1003


def test_wide_score_range(gpu):
    # q scaled by 64 (exact in bf16): scores spread over hundreds, so a row
    # maximum taken too low by more than about 2^7 in the exponent would
    # overflow the bf16 probabilities and show as a non-finite output
    b = W.prefill_batch([0, 40, 300, 1000], [130, 64, 200, 24], 12, 2, 128, 256, 3104, theta=1e4)
    b.q = (b.q.float() * 64).to(torch.bfloat16)
    _store_then_prefill(gpu, b, "q x 64")


def test_rerun_bit_identical(gpu):
    b = W.prefill_batch([100, 3], [200, 77], 12, 2, 128, 64, 3103, theta=1e6)
    g = b.to("cuda")
    gpu_store(gpu, g)
    o1 = _gpu_prefill(gpu, g)
    o2 = _gpu_prefill(gpu, g)
    assert torch.equal(o1, o2)
