"""pa_decode_shared_prefix (the prefix a group of sequences shares is attended
once for the whole group, each sequence's suffix by split-K, one reduce)
against the oracle's plain paged attention, and against pa_decode."""

import numpy as np
import pytest
import torch

import workloads as W
from parity import assert_attention_close, gpu_decode, gpu_store, oracle_decode, oracle_store
from workloads import as_bits

pytestmark = pytest.mark.gpu


def _groups(b, groups):
    """Make each group (first, end, prefix_tokens) share its first member's prefix blocks."""
    bt = b.block_tables.clone()
    prefix = torch.zeros(b.B, dtype=torch.int32)
    for first, end, pre in groups:
        nb = pre // 16
        for s in range(first + 1, end):
            bt[s, :nb] = bt[first, :nb]
        prefix[first:end] = pre
    b.block_tables = bt
    start = torch.tensor([g[0] for g in groups] + [groups[-1][1]] if groups else [0], dtype=torch.int32)
    return start, prefix


def _run(pa, b, groups, partitions, label):
    start, prefix = _groups(b, groups)
    q_ref, kc_ref, vc_ref = oracle_store(b)
    ref = oracle_decode(q_ref, kc_ref, vc_ref, b)
    g = b.to("cuda")
    gpu_store(pa, g)
    max_group = max([e - f for f, e, _ in groups], default=1)
    max_prefix = int(prefix.max())
    outs = {}
    for P in partitions:
        print(f"{label} P={P}", flush=True)
        max_suffix = int((g.context_lens.cpu() - prefix).max())
        out = pa.decode_shared_prefix(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                                      start.cuda() if groups else None, prefix.cuda(), g.scale,
                                      g.max_context_len, max_group, max_prefix, max_suffix,
                                      partition_size=P)
        torch.cuda.synchronize()
        assert_attention_close(out, ref, f"{label} P={P}")
        outs[P] = out
    return g, outs


@pytest.mark.parametrize("poison", [False, True])
def test_cb_step_shared_system_prompt(gpu, poison):
    # 32 sequences share a 2000-token prefix (125 blocks), 32 have none
    b = W.cb_step(poison=poison)
    _run(gpu, b, [(0, 32, 2000)], [512, -1], f"cb step poison={poison}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 6, 8])
def test_several_groups(gpu, D, G):
    # prefixes of one block, two whole 128-token partitions, a partial partition, a
    # prefix that is the whole sequence (empty suffix), and sequences in no group
    lens = [48, 60, 300, 260, 257, 700, 417, 33, 1100, 405, 400, 90]
    groups = [(0, 3, 48), (3, 6, 256), (8, 11, 400)]
    Hkv = 2 if G <= 4 else 1
    b = W.decode_batch(lens, G * Hkv, Hkv, D, 512, 6100 + 10 * G + D, theta=1e4, poison=True,
                       table_fill=W.INT32_MIN)
    _run(gpu, b, groups, [16, 64, 512, 1024, -1], f"G={G} D={D}")  # 1024: the three-launch path


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 3, 5, 7])
def test_group_split_over_items(gpu, D, G):
    # a group of 13 sequences: the one-launch form splits it into items of 16 // G
    # sequences (a partial last item unless 16 // G divides 13; rows past 16 // G * G
    # padding), over a 576-token prefix (a partial 512-token prefix partition)
    lens = [576 + 16 + 37 * i for i in range(13)] + [300, 45]
    Hkv = 2 if G <= 4 else 1
    b = W.decode_batch(lens, G * Hkv, Hkv, D, 1024, 6300 + 10 * G + D, theta=1e4, poison=True,
                       table_fill=W.INT32_MIN)
    _run(gpu, b, [(0, 13, 576)], [64, 512, -1], f"13-sequence group G={G} D={D}")


def test_without_groups_equals_decode(gpu):
    # every prefix 0: the same partitions and reduce as pa_decode, bit for bit
    b = W.decode_batch([1, 17, 500, 1000, 33], 12, 2, 128, 256, 6201, theta=1e4)
    g, outs = _run(gpu, b, [], [64, 512], "no groups")
    for P, out in outs.items():
        ref = gpu_decode(gpu, g, P)
        assert torch.equal(out, ref), f"P={P}"


def test_group_is_one_sequence(gpu):
    # a group of one: the prefix path and the suffix path on the same sequence
    b = W.decode_batch([900, 130], 12, 2, 128, 128, 6202, theta=1e4)
    _run(gpu, b, [(0, 1, 512), (1, 2, 128)], [64, 256], "singleton groups")


def test_large_group_longer_prefix_partitions(gpu):
    # 128 sequences on a 4096-token prefix: the library takes prefix partitions longer
    # than 128 tokens here (several key steps per workgroup)
    lens = [4096 + 16 + 7 * (i % 9) for i in range(128)]
    b = W.decode_batch(lens, 12, 2, 128, 128 * 6 + 256 + 64, 6203, theta=1e6,
                       shared_prefix=(list(range(128)), 256))
    _run(gpu, b, [(0, 128, 4096)], [64], "128 x 4096")


def test_large_group_eight_heads_head_dim_64(gpu):
    # 96 sequences (G = 8, D = 64) on a 6144-token prefix: 576 prefix items of two
    # sequences at 512 tokens would not fit one per CU, so the group pass runs on the
    # matrix cores (the chunked-prefill kernel's 96-row workgroups), then the suffixes,
    # then the reduce
    lens = [6144 + 16 + 5 * (i % 7) for i in range(96)]
    b = W.decode_batch(lens, 8, 1, 64, 96 * 3 + 384 + 64, 6204, theta=1e6,
                       shared_prefix=(list(range(96)), 384))
    _run(gpu, b, [(0, 96, 6144)], [64, -1], "96 x 6144, G=8, D=64")
