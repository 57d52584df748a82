"""Structure of the seeded synthetic workloads (CPU only)."""

import json
import os

import numpy as np
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_tables(b, allow_shared=None):
    bt = b.block_tables.numpy()
    lens = b.context_lens.numpy()
    owners = {}
    for s, L in enumerate(lens):
        n = -(-int(L) // 16)
        row = bt[s, :n]
        assert ((row >= 0) & (row < b.num_blocks)).all()
        for j, blk in enumerate(row):
            owners.setdefault(int(blk), []).append((s, j))
    for blk, refs in owners.items():
        if len(refs) > 1:
            assert allow_shared is not None
            # shared blocks sit at the same logical index in every owner
            assert len({j for _, j in refs}) == 1 and refs[0][1] < allow_shared
    return owners


def _check_slots(b):
    bt = b.block_tables.numpy()
    qsl = b.query_start_loc.numpy()
    slots, pos = b.slot_mapping.numpy(), b.positions.numpy()
    for s in range(b.B):
        for i in range(qsl[s], qsl[s + 1]):
            p = int(pos[i])
            assert slots[i] == bt[s, p // 16] * 16 + p % 16
            assert p < int(b.context_lens[s])
    assert len(np.unique(slots[slots >= 0])) == (slots >= 0).sum()


def test_tiny_decode():
    b = W.tiny_decode()
    assert b.context_lens.tolist() == [1, 15, 16, 33]
    assert (b.Hq, b.Hkv, b.D, b.num_blocks) == (2, 1, 64, 32)
    assert b.positions.tolist() == [0, 14, 15, 32]
    assert abs(b.scale - 0.125) < 1e-15 and b.theta == 1e4
    owners = _check_tables(b)
    assert len(owners) == 6
    _check_slots(b)
    p = W.tiny_decode(poison=True)
    assert (p.block_tables.numpy()[0, 1:] == W.INT32_MIN).all()
    # poison: unread slots are NaN, read slots finite
    kc = p.k_cache.float()
    assert torch.isnan(kc).any()
    bt = p.block_tables.numpy()
    for s, L in enumerate(p.context_lens.tolist()):
        for t in range(L):
            assert torch.isfinite(kc[bt[s, t // 16], :, t % 16]).all()


def test_qwen_decode():
    b = W.qwen_decode()
    assert (b.Hq, b.Hkv, b.D, b.B, b.num_blocks) == (12, 2, 128, 1, 4096)
    assert b.context_lens.tolist() == [2048] and b.max_blocks == 128
    _check_tables(b)
    _check_slots(b)


def test_cb_step_shared_prefix():
    fx = json.load(open(os.path.join(GOLDEN, "paging_examples.json")))["shared_prefix_2000"]
    assert fx["prefix_tokens"] == 16 * fx["full_blocks"]
    b = W.cb_step()
    lens = b.context_lens.numpy()
    assert b.B == 64
    assert ((lens[:32] >= 2016) & (lens[:32] <= 2512)).all()
    assert ((lens[32:] >= 64) & (lens[32:] <= 1024)).all()
    owners = _check_tables(b, allow_shared=fx["full_blocks"])
    shared = [blk for blk, refs in owners.items() if len(refs) > 1]
    assert len(shared) == 125 and all(len(owners[blk]) == 32 for blk in shared)
    _check_slots(b)
    # the new token always lands in a private block (no copy-on-write needed)
    bt = b.block_tables.numpy()
    for s in range(32):
        assert len(owners[int(bt[s, (lens[s] - 1) // 16])]) == 1
    logical = W.kv_bytes_logical(lens, 2, 128)
    unique = W.kv_bytes_unique(bt, lens, 2, 128)
    assert unique == logical - 31 * 2000 * 1024


def test_long_decode_layer_structure():
    b = W.long_decode_layer(0, batch=2, context=1024)
    assert b.num_blocks == 128 and b.context_lens.tolist() == [1024, 1024]
    owners = _check_tables(b)
    assert len(owners) == 128  # the pool is used exactly
    _check_slots(b)
    # about 1% of key rows scaled by 8 (exact powers of two in bf16)
    b2 = W.long_decode_layer(0, batch=2, context=1024)
    assert torch.equal(b.k_cache, b2.k_cache)  # seeded
    assert b.meta["partition_size"] == 512


def test_chunked_prefill():
    b = W.chunked_prefill()
    assert b.context_lens.tolist() == [2560] * 4
    assert b.query_start_loc.tolist() == [0, 512, 1024, 1536, 2048]
    assert b.positions[:3].tolist() == [2048, 2049, 2050] and int(b.positions[-1]) == 2559
    assert b.theta == 1e6 and b.T == 2048
    _check_tables(b)
    _check_slots(b)


def test_request_20_tokens_example():
    fx = json.load(open(os.path.join(GOLDEN, "paging_examples.json")))["request_20_tokens"]
    tables, used = W.deal_block_tables([fx["tokens"]], 8, np.random.default_rng(0))
    assert used == fx["blocks_needed"]
    # a static reservation of 128 tokens would hold 20 of them; pages of 16 hold 20 of 32
    assert fx["tokens"] / fx["static_reservation"] < fx["tokens"] / (16 * used)


def test_seeded_reproducible():
    a, b = W.cb_step(), W.cb_step()
    assert torch.equal(a.block_tables, b.block_tables) and torch.equal(a.q, b.q)
    assert not torch.equal(W.cb_step(seed=1).q, a.q)
