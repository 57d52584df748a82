"""A synthetic continuous-batching loop driving the library through the host
block manager (the mini-llm-engine post, §3.2: after every step finished
sequences leave and waiting requests join; §3.1, §3.4, §3.5: block tables,
prefix reuse, copy-on-write and swap come from the block manager).

No model and no weights: a token's K and V rows are a fixed pseudo-random
function of (token id, position), so equal prefixes have equal K/V and cached
blocks are valid to reuse; queries are fresh random rows each step.  Each step
runs, in order: the copy-on-write block copies the manager asked for, the
fused RoPE + store of the prefill rows, pa_prefill for the sequences being
prefilled (only their uncached prompt tokens) and pa_decode_step (store
folded into the decode kernel) for the others.
Sampling is a seeded draw of the next token id.

`run` yields one record per step (the rows stored and the outputs), so a test
can check every output against plain unpaged attention.

Decode rows go through pa_decode_step, which stores the new token at the
position its block table gives (no slot mapping), so the loop also checks
that the slot the manager hands out and its table agree.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

import paged_kv_cache_240_amd as pa
from workloads import rope_cos_sin_table


@dataclass
class Request:
    rid: int
    prompt: list
    max_new: int
    tokens: list = field(default_factory=list)   # prompt + generated
    fork_at: int = -1                            # generated count at which to fork a sibling
    swap_at: int = -1                            # generated count at which to swap out for a step


@dataclass
class Step:
    rows: list          # (rid, position, token) per stored row, in store order
    q: torch.Tensor     # the rows' queries before the store rotated them in place
    prefill: list       # (rid, first_row, n_rows, context_len)
    decode: list        # (rid, row, context_len)
    history: dict       # rid -> token ids 0 .. context_len-1 of every sequence in the step
    out_prefill: torch.Tensor
    out_decode: torch.Tensor
    cows: list
    swaps: list


def make_requests(n, seed, vocab=64, systems=((48,), (100,)), max_new=(4, 16)):
    """Requests built from a few shared system prompts plus unique suffixes."""
    rng = np.random.default_rng(seed)
    sys_prompts = [rng.integers(0, vocab, size=s[0]).tolist() for s in systems]
    reqs = []
    for i in range(n):
        base = sys_prompts[i % len(sys_prompts)]
        suffix = rng.integers(0, vocab, size=int(rng.integers(1, 40))).tolist()
        r = Request(i, base + suffix, int(rng.integers(*max_new)))
        r.tokens = list(r.prompt)
        reqs.append(r)
    return reqs


class Loop:
    def __init__(self, Hq, Hkv, D, num_blocks, num_host_blocks, max_pos, seed, vocab=64,
                 device="cuda", max_batch=8):
        self.Hq, self.Hkv, self.D = Hq, Hkv, D
        self.dev = torch.device(device)
        self.bm = pa.BlockManager(num_blocks, num_host_blocks)
        g = torch.Generator().manual_seed(seed)
        self.k_tab = torch.randn((vocab, max_pos, Hkv, D), generator=g).to(torch.bfloat16)
        self.v_tab = torch.randn((vocab, max_pos, Hkv, D), generator=g).to(torch.bfloat16)
        self.kc = torch.randn((num_blocks, Hkv, 16, D), generator=g).to(torch.bfloat16).to(self.dev)
        self.vc = torch.randn((num_blocks, Hkv, 16, D), generator=g).to(torch.bfloat16).to(self.dev)
        self.hk = torch.zeros((max(1, num_host_blocks), Hkv, 16, D), dtype=torch.bfloat16).pin_memory()
        self.hv = torch.zeros_like(self.hk).pin_memory()
        self.cos_sin = rope_cos_sin_table(1e6, D, max_pos).to(self.dev)
        self.scale = 1.0 / float(np.sqrt(D))
        self.rng = np.random.default_rng(seed + 1)
        self.qgen = torch.Generator().manual_seed(seed + 2)
        self.vocab, self.max_batch = vocab, max_batch

    def _ids(self, values):
        return torch.tensor(values, dtype=torch.int32, device=self.dev)

    def run(self, requests):
        waiting = list(requests)
        running = {}          # rid -> Request (prefilled, decoding)
        swapped = {}          # rid -> Request swapped out for one whole step
        next_rid = max(r.rid for r in requests) + 1
        while waiting or running or swapped:
            rows, prefill, decode, cows, swaps = [], [], [], [], []
            back = [rid for rid, (r, wait) in swapped.items() if wait <= 0]
            for rid in swapped:
                swapped[rid] = (swapped[rid][0], swapped[rid][1] - 1)
            # decode: one new token per running sequence
            for rid, r in list(running.items()):
                tok = r.tokens[-1]
                pos = len(r.tokens) - 1
                # (the last sampled token is stored now; it was appended to r.tokens at sampling)
                slot, cow = self.bm.append_token(rid, tok)
                if cow is not None:
                    cows.append(cow)
                decode.append((rid, len(rows), pos + 1))
                rows.append((rid, pos, tok, slot))
            # admit new requests while the batch allows and the pool keeps room for every
            # admitted sequence to finish (so decode never runs out of blocks)
            def blocks_to_finish(req):
                total = -(-(len(req.prompt) + req.max_new) // 16) + 1  # +1: a copy-on-write block
                held = 0 if req.rid in swapped else len(self.bm.block_table(req.rid))
                return max(0, total - held)
            reserve = sum(blocks_to_finish(x) for x in running.values()) + \
                sum(blocks_to_finish(x) for x, _ in swapped.values())
            while waiting and len(running) < self.max_batch:
                r = waiting[0]
                if self.bm.num_free_blocks - reserve < -(-(len(r.prompt) + r.max_new) // 16) + 1:
                    break
                try:
                    cached = self.bm.add_sequence(r.rid, r.prompt)
                except pa.PAError:
                    break
                reserve += blocks_to_finish(r)
                waiting.pop(0)
                n = len(r.prompt) - cached
                slots = self.bm.slots(r.rid, cached, n)
                prefill.append((r.rid, len(rows), n, len(r.prompt)))
                for i in range(n):
                    rows.append((r.rid, cached + i, r.prompt[cached + i], slots[i]))
                running[r.rid] = r
            # then bring back what sat out the previous step (into whatever blocks are free now)
            for rid in back:
                r, _ = swapped.pop(rid)
                try:
                    host, devb = self.bm.swap_in(rid)
                except pa.PAError:
                    swapped[rid] = (r, 0)  # no room yet: stays out
                    continue
                pa.swap_blocks(self.kc, self.vc, self.hk, self.hv, self._ids(host), self._ids(devb))
                swaps.append(("in", rid, host, devb))
                slot, cow = self.bm.append_token(rid, r.tokens[-1])
                if cow is not None:
                    cows.append(cow)
                decode.append((rid, len(rows), len(r.tokens)))
                rows.append((rid, len(r.tokens) - 1, r.tokens[-1], slot))
                running[rid] = r
            if not rows:
                if swapped:
                    continue
                break
            if cows:
                pa.copy_blocks(self.kc, self.vc, self._ids([c[0] for c in cows]),
                               self._ids([c[1] for c in cows]))
            T = len(rows)
            q = torch.randn((T, self.Hq, self.D), generator=self.qgen).to(torch.bfloat16).to(self.dev)
            q_raw = q.clone()
            history = {rid: list(running[rid].tokens[:self.bm.seq_len(rid)]) for rid in {r[0] for r in rows}}
            tok_idx = torch.tensor([r[2] for r in rows])
            pos_idx = torch.tensor([r[1] for r in rows])
            k = self.k_tab[tok_idx, pos_idx].to(self.dev)
            v = self.v_tab[tok_idx, pos_idx].to(self.dev)
            out_p = out_d = None
            if prefill:
                pre_rows = [i for _, s0, n, _ in prefill for i in range(s0, s0 + n)]
                idx = torch.tensor(pre_rows, device=self.dev)
                qp = q[idx].contiguous()
                pa.cache_store(qp, k[idx].contiguous(), v[idx].contiguous(), self.kc, self.vc,
                               self._ids([rows[i][3] for i in pre_rows]),
                               self._ids([rows[i][1] for i in pre_rows]), self.cos_sin)
                bt = self._tables([p[0] for p in prefill])
                lens = self._ids([p[3] for p in prefill])
                qsl = self._ids(np.concatenate([[0], np.cumsum([p[2] for p in prefill])]).tolist())
                out_p = pa.prefill(qp, self.kc, self.vc, bt, lens, qsl, self.scale,
                                   max(p[2] for p in prefill))
            if decode:
                idx = torch.tensor([s0 for _, s0, _ in decode], device=self.dev)
                bt = self._tables([d[0] for d in decode])
                lens = self._ids([d[2] for d in decode])
                for (rid, row, L), t in zip(decode, bt.cpu().numpy()):
                    assert rows[row][3] == t[(L - 1) // 16] * 16 + (L - 1) % 16, "slot and table disagree"
                out_d = pa.decode_step(q[idx].contiguous(), k[idx].contiguous(), v[idx].contiguous(),
                                       self.kc, self.vc, bt, lens, self.cos_sin, self.scale,
                                       max(d[2] for d in decode))
            # the stored tokens are computed: register their full blocks
            for rid in {r[0] for r in rows}:
                self.bm.commit(rid, self.bm.seq_len(rid))
            yield Step([(r[0], r[1], r[2]) for r in rows], q_raw, prefill, decode, history, out_p, out_d,
                       cows, swaps)
            # sample, finish, fork and swap
            for rid, r in list(running.items()):
                r.tokens.append(int(self.rng.integers(0, self.vocab)))
                gen = len(r.tokens) - len(r.prompt)
                if gen >= r.max_new:
                    self.bm.free_sequence(rid)
                    del running[rid]
                elif gen == r.fork_at and self.bm.num_free_blocks > 2 * (-(-(len(r.prompt) + r.max_new) // 16) + 1):
                    child = Request(next_rid, r.prompt, r.max_new, list(r.tokens[:-1]))
                    child.tokens.append(int(self.rng.integers(0, self.vocab)))  # a different sample
                    self.bm.fork(rid, next_rid)
                    running[next_rid] = child
                    next_rid += 1
                elif gen == r.swap_at:
                    devb, host = self.bm.swap_out(rid)
                    pa.swap_blocks(self.hk, self.hv, self.kc, self.vc, self._ids(devb), self._ids(host))
                    swapped[rid] = (running.pop(rid), 1)

    def _tables(self, rids):
        tabs = [self.bm.block_table(r) for r in rids]
        width = max(len(t) for t in tabs)
        out = np.full((len(tabs), width), -1, dtype=np.int32)
        for i, t in enumerate(tabs):
            out[i, :len(t)] = t
        return torch.from_numpy(out).to(self.dev)
