"""End to end: a synthetic continuous-batching loop whose block tables, slot
mappings, prefix reuse, copy-on-write and swaps all come from the C++ block
manager, with every attention output of every step checked against plain
unpaged attention computed by the oracle from the tokens alone."""

import numpy as np
import pytest
import torch

import oracle
from parity import assert_attention_close
from workloads import as_bits
from workloads.cb_loop import Loop, make_requests

pytestmark = pytest.mark.gpu


class _Reference:
    """Unpaged attention from token ids: K/V of (token, position), RoPE by the oracle."""

    def __init__(self, loop):
        self.k_tab = loop.k_tab.view(torch.int16).numpy().view(np.uint16)
        self.v_tab = loop.v_tab.view(torch.int16).numpy().view(np.uint16)
        cs = loop.cos_sin.cpu().numpy()
        half = loop.D // 2
        self.cos, self.sin = cs[:, :half], cs[:, half:]
        self.scale = loop.scale

    def kv(self, tokens):
        pos = np.arange(len(tokens))
        k = self.k_tab[tokens, pos]                                  # [L, Hkv, D]
        k = oracle.rope_rotate_half(k, self.cos[pos][:, None, :], self.sin[pos][:, None, :])
        return oracle.bf16_to_f64(k), oracle.bf16_to_f64(self.v_tab[tokens, pos])

    def rows(self, q_bits, positions, tokens):
        """Outputs of consecutive query rows at `positions` over the sequence `tokens`."""
        q = oracle.rope_rotate_half(q_bits, self.cos[positions][:, None, :], self.sin[positions][:, None, :])
        K, V = self.kv(np.asarray(tokens))
        L = int(positions[-1]) + 1
        return oracle.attend_sequence(oracle.bf16_to_f64(q), K[:L], V[:L], L, self.scale)


def _check_run(loop, requests):
    ref = _Reference(loop)
    stats = dict(steps=0, prefill_rows=0, decode_rows=0, cached=0, cows=0, swaps=0)
    for st in loop.run(requests):
        torch.cuda.synchronize()
        qb = as_bits(st.q)
        stats["steps"] += 1
        stats["cows"] += len(st.cows)
        stats["swaps"] += len(st.swaps)
        for i, (rid, first, n, L) in enumerate(st.prefill):
            pos = np.array([st.rows[first + j][1] for j in range(n)])
            stats["prefill_rows"] += n
            stats["cached"] += L - n
            want = ref.rows(qb[first:first + n], pos, st.history[rid])
            start = sum(p[2] for p in st.prefill[:i])
            assert_attention_close(st.out_prefill[start:start + n], want, f"prefill rid={rid}")
        for i, (rid, row, L) in enumerate(st.decode):
            pos = np.array([st.rows[row][1]])
            stats["decode_rows"] += 1
            want = ref.rows(qb[row:row + 1], pos, st.history[rid])
            assert_attention_close(st.out_decode[i:i + 1], want, f"decode rid={rid} L={L}")
    return stats


def test_loop_with_prefix_reuse_forks_and_swaps(gpu):
    reqs = make_requests(12, seed=2409)
    reqs[1].fork_at = 2        # parallel sample: the sibling shares every block
    reqs[4].fork_at = 5
    reqs[2].swap_at = 3        # preempted for one step: blocks go to host memory and come back
    reqs[7].swap_at = 1
    loop = Loop(12, 2, 128, num_blocks=120, num_host_blocks=32, max_pos=256, seed=2410, max_batch=6)
    stats = _check_run(loop, reqs)
    # every mechanism was exercised: cached prefixes, copy-on-write, swap out and in
    assert stats["cached"] > 0 and stats["cows"] > 0 and stats["swaps"] > 0
    assert stats["prefill_rows"] > 0 and stats["decode_rows"] > 50
    # everything returned: only cached (released, hashed) blocks remain out of the free list
    assert loop.bm.num_free_blocks == 120 and loop.bm.num_free_host_blocks == 32


def test_loop_under_block_pressure(gpu):
    # a pool too small for all requests at once: admission waits, cached blocks get evicted
    reqs = make_requests(10, seed=2411, max_new=(8, 20))
    loop = Loop(12, 2, 128, num_blocks=40, num_host_blocks=8, max_pos=256, seed=2412, max_batch=8)
    stats = _check_run(loop, reqs)
    assert stats["decode_rows"] > 50
    assert loop.bm.num_free_blocks == 40
