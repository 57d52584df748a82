"""Seeded random sweeps over the shapes the kernels support: head grouping
G = 1..8 with one or two KV heads, head_dim 64 / 128, ragged lengths drawn
around block and partition edges, partition sizes, NaN poison.  Each case is
checked against the oracle; the decode step is also checked bit for bit
against the separate store + decode.  Every case prints what it runs."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_attention_close, gpu_decode, gpu_store, oracle_decode, oracle_store
from workloads import as_bits

pytestmark = pytest.mark.gpu


def _shape(rng):
    D = int(rng.choice([64, 128]))
    G = int(rng.integers(1, 9))
    Hkv = int(rng.choice([1, 2])) if G <= 4 else 1
    return D, G, Hkv


def _length(rng, hi):
    kind = rng.integers(4)
    if kind == 0:
        return int(rng.integers(1, hi + 1))
    if kind == 1:   # first row of a block
        return int(16 * rng.integers(0, hi // 16) + 1)
    if kind == 2:   # last row of a block
        return int(16 * rng.integers(1, hi // 16 + 1))
    return int(min(hi, 64 * rng.integers(1, hi // 64 + 1) + int(rng.choice([0, 1]))))  # partition edges


def _same_bits(a, b):
    return np.array_equal(as_bits(a), as_bits(b))


@pytest.mark.parametrize("case", range(16))
def test_decode_and_decode_step(gpu, case):
    rng = np.random.default_rng(8000 + case)
    D, G, Hkv = _shape(rng)
    B = int(rng.integers(1, 7))
    lens = [_length(rng, 2000) for _ in range(B)]
    P = int(rng.choice([0, -1, 16 * int(rng.integers(1, 48))]))
    poison = bool(rng.integers(2))
    nb = sum(-(-L // 16) for L in lens) + 8
    print(f"decode case {case}: D={D} G={G} Hkv={Hkv} lens={lens} P={P} poison={poison}", flush=True)
    b = W.decode_batch(lens, G * Hkv, Hkv, D, nb, 8100 + case, theta=float(rng.choice([1e4, 1e6])),
                       poison=poison, table_fill=W.INT32_MIN if poison else -1)
    q_ref, kc_ref, vc_ref = oracle_store(b)
    ref = oracle_decode(q_ref, kc_ref, vc_ref, b)
    g = b.to("cuda")
    gpu_store(gpu, g)
    out = gpu_decode(gpu, g, P)
    assert_attention_close(out, ref, f"decode case {case}")
    g2 = b.to("cuda")
    o2 = gpu.decode_step(g2.q, g2.k, g2.v, g2.k_cache, g2.v_cache, g2.block_tables, g2.context_lens,
                         g2.cos_sin, g2.scale, g2.max_context_len, partition_size=P)
    torch.cuda.synchronize()
    assert _same_bits(o2, out) and _same_bits(g2.k_cache, g.k_cache) and _same_bits(g2.v_cache, g.v_cache)


@pytest.mark.parametrize("case", range(12))
def test_multi_query_decode(gpu, case):
    rng = np.random.default_rng(8200 + case)
    D, G, Hkv = _shape(rng)
    nq = int(rng.integers(1, 32 // G + 1))
    nq = min(nq, 6)
    B = int(rng.integers(1, 5))
    lens = [max(nq, _length(rng, 1500)) for _ in range(B)]
    P = int(rng.choice([0, -1, 64 * int(rng.integers(1, 17))]))  # up to 1024: the 8-wave chunks
    print(f"multi case {case}: D={D} G={G} Hkv={Hkv} nq={nq} lens={lens} P={P}", flush=True)
    b = W.verify_batch(lens, nq, G * Hkv, Hkv, D, sum(-(-L // 16) for L in lens) + 8, 8300 + case,
                       poison=True, table_fill=W.INT32_MIN)
    q_ref, kc_ref, vc_ref = oracle_store(b)
    ref = oracle.prefill(q_ref, kc_ref, vc_ref, b.block_tables.numpy(), b.context_lens.numpy(),
                         b.query_start_loc.numpy(), b.scale).reshape(B, nq, G * Hkv, D)
    g = b.to("cuda")
    gpu_store(gpu, g)
    out = gpu.decode_multi(g.q.view(B, nq, G * Hkv, D), g.k_cache, g.v_cache, g.block_tables,
                           g.context_lens, g.scale, g.max_context_len, partition_size=P)
    torch.cuda.synchronize()
    assert_attention_close(out, ref, f"multi case {case}")


@pytest.mark.parametrize("case", range(8))
def test_shared_prefix_decode(gpu, case):
    # random groups of sequences sharing whole-block prefixes, sequences in no group,
    # random suffix partitions: the one-launch form or the matrix-core group pass
    rng = np.random.default_rng(8600 + case)
    D, G, Hkv = _shape(rng)
    B = int(rng.integers(2, 13))
    ngroups = int(rng.integers(1, 4))
    cuts = sorted(int(x) for x in rng.choice(np.arange(1, B), size=min(ngroups, B - 1), replace=False))
    bounds = [0] + cuts
    groups, prefix = [], [0] * B
    for gi in range(len(bounds) - 1 + (1 if rng.integers(2) else 0)):
        first = bounds[gi]
        end = bounds[gi + 1] if gi + 1 < len(bounds) else B
        if end - first < 1 or rng.integers(4) == 0:
            continue                                  # sometimes leave a run ungrouped
        pre = 16 * int(rng.integers(1, 80))
        groups.append((first, end, pre))
        for sidx in range(first, end):
            prefix[sidx] = pre
    lens = [prefix[i] + _length(rng, 700) for i in range(B)]
    P = int(rng.choice([-1, 16 * int(rng.integers(1, 33))]))
    print(f"shared-prefix case {case}: D={D} G={G} Hkv={Hkv} groups={groups} lens={lens} P={P}",
          flush=True)
    nb = sum(-(-L // 16) for L in lens) + 8
    b = W.decode_batch(lens, G * Hkv, Hkv, D, nb, 8700 + case, theta=1e4, poison=True,
                       table_fill=W.INT32_MIN)
    bt = b.block_tables.clone()
    for first, end, pre in groups:
        for sidx in range(first + 1, end):
            bt[sidx, :pre // 16] = bt[first, :pre // 16]
    b.block_tables = bt
    q_ref, kc_ref, vc_ref = oracle_store(b)
    ref = oracle_decode(q_ref, kc_ref, vc_ref, b)
    g = b.to("cuda")
    gpu_store(gpu, g)
    start = torch.tensor([f for f, _, _ in groups] + [groups[-1][1]] if groups else [0],
                         dtype=torch.int32, device="cuda")
    pre_t = torch.tensor(prefix, dtype=torch.int32, device="cuda")
    max_group = max([e - f for f, e, _ in groups], default=1)
    out = gpu.decode_shared_prefix(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                                   start if groups else None, pre_t, g.scale, g.max_context_len,
                                   max_group, max(prefix), max(L - p for L, p in zip(lens, prefix)),
                                   partition_size=P)
    torch.cuda.synchronize()
    assert_attention_close(out, ref, f"shared-prefix case {case}")


@pytest.mark.parametrize("case", range(8))
def test_chunked_prefill(gpu, case):
    rng = np.random.default_rng(8400 + case)
    D, G, Hkv = _shape(rng)
    B = int(rng.integers(1, 5))
    prefix = [int(rng.choice([0, _length(rng, 1200)])) for _ in range(B)]
    chunk = [int(rng.choice([0, 1, _length(rng, 300)])) for _ in range(B)]
    if sum(chunk) == 0:
        chunk[0] = 1
    print(f"prefill case {case}: D={D} G={G} Hkv={Hkv} prefix={prefix} chunk={chunk}", flush=True)
    nb = sum(-(-(p + c) // 16) for p, c in zip(prefix, chunk)) + 8
    b = W.prefill_batch(prefix, chunk, G * Hkv, Hkv, D, nb, 8500 + case, theta=1e4, poison=True,
                        table_fill=W.INT32_MIN)
    q_ref, kc_ref, vc_ref = oracle_store(b)
    ref = oracle.prefill(q_ref, kc_ref, vc_ref, b.block_tables.numpy(), b.context_lens.numpy(),
                         b.query_start_loc.numpy(), b.scale)
    g = b.to("cuda")
    gpu_store(gpu, g)
    out = gpu.prefill(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, g.query_start_loc,
                      g.scale, g.max_query_len)
    torch.cuda.synchronize()
    assert_attention_close(out, ref, f"prefill case {case}")
