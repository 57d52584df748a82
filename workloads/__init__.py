"""Seeded synthetic inputs for paged KV-cache attention.

This module only makes inputs: random bf16 tensors, block tables dealt from
seeded permutations of a physical-block pool, context lengths, slot mappings
and the RoPE angle table.  It is shared by the tests, the benchmark and the
oracle's callers, and contains none of the attention, RoPE-rotation or
reduction arithmetic that the library and the oracle compute.

Recipe (all seeded; numpy PCG64 for integers, torch's generator for normal
bf16 values, fp32 N(0,1) rounded to bf16 by torch's cast):
  * a pool of NB physical blocks, each [Hkv, 16, D] for K and for V
    (mini-llm-engine post, §3.1: 16-token blocks);
  * physical ids dealt in order from a seeded permutation of range(NB), so
    every sequence's blocks are scattered over the pool (its block table maps
    logical block j to a random physical id; nano-vllm commentary, FAQ Q2);
  * a shared prefix is the same physical ids at the head of several tables
    (mini-llm-engine post, §3.4: shared blocks with ref_count > 1);
  * slot_mapping[i] = table[pos_i // 16] * 16 + pos_i % 16 is what a scheduler
    hands the store for a new token at position pos_i (it is an input of the
    store; the store itself never looks at block tables);
  * cos_sin[p] = [cos(p * f_j) | sin(p * f_j)], f_j = theta^(-2j/D), j < D/2,
    computed in float64 and rounded once to float32 (the RoPE frequency
    table a model builds once; both the library and the oracle receive it).
"""

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

BLOCK_SIZE = 16
INT32_MIN = -(2 ** 31)


def as_bits(t):
    """bf16 torch tensor -> numpy uint16 bit patterns (a copy on the host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a):
    """numpy uint16 bf16 bit patterns -> bf16 torch tensor (host)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def rope_cos_sin_table(theta, head_dim, max_pos):
    """float32 [max_pos, head_dim]: cos in the first half, sin in the second."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * j / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    tab = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    return torch.from_numpy(tab)


def normal_bf16(shape, gen, device="cpu"):
    """N(0,1) float32 draws rounded to bf16 by torch's cast."""
    return torch.randn(shape, generator=gen, dtype=torch.float32, device=device).to(torch.bfloat16)


def _torch_gen(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


@dataclass
class PagedBatch:
    """One step's worth of paged-attention inputs (host or device tensors).

    New-token rows (q, k, v, slot_mapping, positions) are packed by sequence;
    sequence b owns rows query_start_loc[b] .. query_start_loc[b+1]-1.  For a
    decode step every sequence has exactly one new row.  context_lens counts
    every cached token of a sequence, the new rows included.
    """
    Hq: int
    Hkv: int
    D: int
    num_blocks: int
    k_cache: torch.Tensor          # bf16 [NB, Hkv, 16, D]
    v_cache: torch.Tensor          # bf16 [NB, Hkv, 16, D]
    block_tables: torch.Tensor     # int32 [B, max_blocks]
    context_lens: torch.Tensor     # int32 [B]
    q: torch.Tensor                # bf16 [T, Hq, D]
    k: torch.Tensor                # bf16 [T, Hkv, D]
    v: torch.Tensor                # bf16 [T, Hkv, D]
    slot_mapping: torch.Tensor     # int32 [T]
    positions: torch.Tensor        # int32 [T]
    query_start_loc: torch.Tensor  # int32 [B+1]
    cos_sin: torch.Tensor          # float32 [max_pos, D]
    theta: float
    scale: float
    block_size: int = BLOCK_SIZE
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return int(self.context_lens.shape[0])

    @property
    def T(self):
        return int(self.q.shape[0])

    @property
    def max_blocks(self):
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self):
        return int(self.context_lens.max().item()) if self.B else 0

    @property
    def max_query_len(self):
        d = self.query_start_loc[1:] - self.query_start_loc[:-1]
        return int(d.max().item()) if self.B else 0

    def to(self, device):
        kw = {}
        for f in ("k_cache", "v_cache", "block_tables", "context_lens", "q", "k", "v",
                  "slot_mapping", "positions", "query_start_loc", "cos_sin"):
            kw[f] = getattr(self, f).to(device)
        return replace(self, **kw)

    def clone(self):
        kw = {}
        for f in ("k_cache", "v_cache", "block_tables", "context_lens", "q", "k", "v",
                  "slot_mapping", "positions", "query_start_loc", "cos_sin"):
            kw[f] = getattr(self, f).clone()
        return replace(self, **kw, meta=dict(self.meta))


def deal_block_tables(lens, num_blocks, rng, shared_prefix=None, table_fill=-1,
                      max_blocks=None, block_size=BLOCK_SIZE):
    """Block tables dealt from one seeded permutation of the pool.

    shared_prefix: optional (seq_ids, n_blocks): those sequences start with the
    same n_blocks physical ids (dealt first).  Every other block is private,
    dealt in order, sequence by sequence.  Entries past a sequence's last
    block hold table_fill.
    """
    lens = [int(x) for x in lens]
    need = [-(-L // block_size) for L in lens]
    if max_blocks is None:
        max_blocks = max(1, max(need) if need else 1)
    perm = rng.permutation(num_blocks)
    cursor = 0
    tables = np.full((len(lens), max_blocks), table_fill, dtype=np.int64)
    shared_ids = set()
    if shared_prefix is not None:
        seq_ids, n_pre = shared_prefix
        pre = perm[cursor:cursor + n_pre]
        cursor += n_pre
        for b in seq_ids:
            tables[b, :n_pre] = pre
        shared_ids = set(int(b) for b in seq_ids)
    for b, n in enumerate(need):
        start = shared_prefix[1] if b in shared_ids else 0
        cnt = n - start
        if cnt < 0:
            raise ValueError("shared prefix longer than the sequence")
        if cursor + cnt > num_blocks:
            raise ValueError("pool too small for the requested lengths")
        tables[b, start:n] = perm[cursor:cursor + cnt]
        cursor += cnt
    return tables.astype(np.int32), cursor


def _slot_of(table_row, pos, block_size=BLOCK_SIZE):
    return int(table_row[pos // block_size]) * block_size + pos % block_size


def _fill_pools(NB, Hkv, D, gen, device, poison, tables, lens, block_size=BLOCK_SIZE):
    """K/V pools; with poison, every slot no sequence reads holds bf16 NaN."""
    shape = (NB, Hkv, block_size, D)
    k_cache = normal_bf16(shape, gen, device)
    v_cache = normal_bf16(shape, gen, device)
    if poison:
        used = torch.zeros((NB, block_size), dtype=torch.bool)
        for b, L in enumerate(lens):
            t = np.arange(int(L))
            blk = torch.from_numpy(np.asarray(tables[b])[t // block_size].astype(np.int64))
            used[blk, torch.from_numpy(t % block_size)] = True
        used = used.to(device)[:, None, :, None].expand(shape)
        nan = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=device)
        k_cache = torch.where(used, k_cache, nan)
        v_cache = torch.where(used, v_cache, nan)
    return k_cache, v_cache


def decode_batch(lens, Hq, Hkv, D, num_blocks, seed, theta=1e4, shared_prefix=None,
                 poison=False, table_fill=-1, max_blocks=None, device="cpu",
                 max_pos=None, name=""):
    """A decode step: one new token per sequence at position L - 1.

    The pool holds every sequence's history (tokens 0 .. L-2) plus random
    values elsewhere (NaN elsewhere with poison); the new token's q/k/v are
    separate rows, to be rotated and stored by the store step.
    """
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    if (lens < 1).any():
        raise ValueError("a decode step needs at least the new token (L >= 1)")
    tables, _ = deal_block_tables(lens, num_blocks, rng, shared_prefix, table_fill, max_blocks)
    gen = _torch_gen(rng.integers(2 ** 62), device)
    k_cache, v_cache = _fill_pools(num_blocks, Hkv, D, gen, device, poison, tables, lens)
    B = len(lens)
    q = normal_bf16((B, Hq, D), gen, device)
    k = normal_bf16((B, Hkv, D), gen, device)
    v = normal_bf16((B, Hkv, D), gen, device)
    pos = lens - 1
    slots = np.array([_slot_of(tables[b], int(pos[b])) for b in range(B)], dtype=np.int32)
    if max_pos is None:
        max_pos = int(lens.max())
    return PagedBatch(
        Hq=Hq, Hkv=Hkv, D=D, num_blocks=num_blocks,
        k_cache=k_cache, v_cache=v_cache,
        block_tables=torch.from_numpy(tables).to(device),
        context_lens=torch.from_numpy(lens.astype(np.int32)).to(device),
        q=q, k=k, v=v,
        slot_mapping=torch.from_numpy(slots).to(device),
        positions=torch.from_numpy(pos.astype(np.int32)).to(device),
        query_start_loc=torch.arange(B + 1, dtype=torch.int32, device=device),
        cos_sin=rope_cos_sin_table(theta, D, max_pos).to(device),
        theta=float(theta), scale=1.0 / float(np.sqrt(D)), name=name,
    )


def prefill_batch(prefix_lens, chunk_lens, Hq, Hkv, D, num_blocks, seed, theta=1e6,
                  poison=False, table_fill=-1, device="cpu", name=""):
    """A chunked-prefill step: sequence b has prefix_lens[b] cached tokens and
    a new chunk of chunk_lens[b] tokens at positions prefix .. prefix+chunk-1.

    The prefix K/V are written straight into the pool (already rotated); the
    chunk's blocks are dealt after the prefix blocks from the same permutation
    (freshly allocated), and the chunk's q/k/v rows go through the store step.
    """
    rng = np.random.default_rng(seed)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    chunk_lens = np.asarray(chunk_lens, dtype=np.int64)
    lens = prefix_lens + chunk_lens
    tables, _ = deal_block_tables(lens, num_blocks, rng, None, table_fill)
    gen = _torch_gen(rng.integers(2 ** 62), device)
    # Only the prefix counts as written history; chunk slots are written by the store.
    k_cache, v_cache = _fill_pools(num_blocks, Hkv, D, gen, device, poison, tables, prefix_lens)
    T = int(chunk_lens.sum())
    q = normal_bf16((T, Hq, D), gen, device)
    k = normal_bf16((T, Hkv, D), gen, device)
    v = normal_bf16((T, Hkv, D), gen, device)
    pos = np.concatenate([np.arange(p, p + c) for p, c in zip(prefix_lens, chunk_lens)]).astype(np.int64) \
        if T else np.zeros(0, dtype=np.int64)
    seq_of_row = np.repeat(np.arange(len(lens)), chunk_lens)
    slots = np.array([_slot_of(tables[seq_of_row[i]], int(pos[i])) for i in range(T)], dtype=np.int32)
    qsl = np.concatenate([[0], np.cumsum(chunk_lens)]).astype(np.int32)
    return PagedBatch(
        Hq=Hq, Hkv=Hkv, D=D, num_blocks=num_blocks,
        k_cache=k_cache, v_cache=v_cache,
        block_tables=torch.from_numpy(tables).to(device),
        context_lens=torch.from_numpy(lens.astype(np.int32)).to(device),
        q=q, k=k, v=v,
        slot_mapping=torch.from_numpy(slots).to(device),
        positions=torch.from_numpy(pos.astype(np.int32)).to(device),
        query_start_loc=torch.from_numpy(qsl).to(device),
        cos_sin=rope_cos_sin_table(theta, D, max(1, int(lens.max()))).to(device),
        theta=float(theta), scale=1.0 / float(np.sqrt(D)), name=name,
    )


def verify_batch(lens, nq, Hq, Hkv, D, num_blocks, seed, theta=1e6, poison=False, table_fill=-1,
                 device="cpu", name=""):
    """A speculative-verification step: sequence b has lens[b] tokens of which
    the last nq (the last accepted token and nq - 1 drafts) are new and go
    through the store; q viewed as [B, nq, Hq, D] holds their queries."""
    lens = np.asarray(lens, dtype=np.int64)
    return prefill_batch(lens - nq, [nq] * len(lens), Hq, Hkv, D, num_blocks, seed, theta=theta,
                         poison=poison, table_fill=table_fill, device=device, name=name)


def spec_verify(seed=2406, device="cpu", batch=16, context=8192, nq=5, poison=False):
    """Verification of 4 draft tokens (5 queries per sequence) at the Qwen2.5-1.5B head
    shape: 16 sequences of 8192 tokens, 16-token blocks dealt from a pool of exactly the
    blocks needed."""
    nb = batch * (-(-context // 16))
    return verify_batch([context] * batch, nq, QWEN_HQ, QWEN_HKV, QWEN_D, nb, seed, theta=1e6,
                        poison=poison, device=device,
                        name=f"spec verify {batch}x{context}, {nq} queries")


# --------------------------------------------------------------------------
# The five workloads at their stated sizes.
# --------------------------------------------------------------------------

QWEN_HQ, QWEN_HKV, QWEN_D = 12, 2, 128   # Qwen2.5-1.5B attention head shape


def tiny_decode(seed=2401, poison=False, device="cpu"):
    """4 sequences, L = {1, 15, 16, 33}, 2 query / 1 KV head, D = 64, 32 blocks."""
    return decode_batch([1, 15, 16, 33], 2, 1, 64, 32, seed, theta=1e4, poison=poison,
                        table_fill=INT32_MIN if poison else -1, device=device,
                        name="tiny paged decode (B=4, L={1,15,16,33}, 2q/1kv, D=64)")


def qwen_decode(seed=2402, device="cpu"):
    """Batch 1, context 2048, Qwen head shape, 4096-block pool."""
    return decode_batch([2048], QWEN_HQ, QWEN_HKV, QWEN_D, 4096, seed, theta=1e6, device=device,
                        name="Qwen2.5-1.5B decode shape (B=1, L=2048)")


def cb_step_lens(seed=2403):
    """Context lengths of the continuous-batching step.

    Sequences 0-31 carry a shared 2000-token prefix (125 whole blocks) plus a
    private suffix of U{16..512} tokens; sequences 32-63 have L ~ U{64..1024}.
    """
    rng = np.random.default_rng([seed, 1])
    suffix = rng.integers(16, 512, size=32, endpoint=True)
    rest = rng.integers(64, 1024, size=32, endpoint=True)
    return np.concatenate([2000 + suffix, rest])


def cb_step(seed=2403, poison=False, device="cpu"):
    lens = cb_step_lens(seed)
    return decode_batch(lens, QWEN_HQ, QWEN_HKV, QWEN_D, 4096, seed, theta=1e6,
                        shared_prefix=(list(range(32)), 125), poison=poison,
                        table_fill=INT32_MIN if poison else -1, device=device,
                        name="continuous-batching decode step (B=64, 32 share a 2000-token prefix)")


LONG_B, LONG_L, LONG_LAYERS, LONG_PARTITION = 16, 8192, 28, 512


def long_decode_layer(layer, seed=2404, device="cpu", batch=LONG_B, context=LONG_L):
    """One layer of the long-context flash-decode workload.

    16 sequences x 8192 tokens fill an 8192-block pool exactly.  1% of key rows
    (drawn per pool row, i.e. per layer, sequence, token and KV head) are
    multiplied by 8, which is exact in bf16.
    """
    nb = batch * context // BLOCK_SIZE
    b = decode_batch([context] * batch, QWEN_HQ, QWEN_HKV, QWEN_D, nb, [seed, layer],
                     theta=1e6, device=device,
                     name=f"long-context flash-decode layer {layer} (B={batch}, L={context})")
    gen = _torch_gen(np.random.default_rng([seed, layer, 7]).integers(2 ** 62), device)
    mask = torch.rand((nb, QWEN_HKV, BLOCK_SIZE, 1), generator=gen, device=device) < 0.01
    b.k_cache = torch.where(mask, b.k_cache * 8, b.k_cache)
    kmask = torch.rand((batch, QWEN_HKV, 1), generator=gen, device=device) < 0.01
    b.k = torch.where(kmask, b.k * 8, b.k)
    b.meta["partition_size"] = LONG_PARTITION
    return b


def chunked_prefill(seed=2405, poison=False, device="cpu"):
    """4 sequences: 2048 cached tokens each plus a new 512-token chunk (theta 1e6)."""
    return prefill_batch([2048] * 4, [512] * 4, QWEN_HQ, QWEN_HKV, QWEN_D, 1024, seed,
                         theta=1e6, poison=poison, table_fill=INT32_MIN if poison else -1,
                         device=device,
                         name="paged chunked prefill (4 x (2048 cached + 512 new))")


def kv_bytes_logical(context_lens, Hkv, D, elem_bytes=2):
    """Bytes of K and V a decode step must read: sum_b L_b * Hkv * D * 2 * 2."""
    return int(np.asarray(context_lens, dtype=np.int64).sum()) * Hkv * D * 2 * elem_bytes


def kv_bytes_unique(block_tables, context_lens, Hkv, D, elem_bytes=2, block_size=BLOCK_SIZE):
    """Bytes of distinct (block, row) slots referenced by the step."""
    bt = np.asarray(block_tables).astype(np.int64)
    ids = []
    for b, L in enumerate(np.asarray(context_lens)):
        t = np.arange(int(L))
        ids.append(bt[b, t // block_size] * block_size + t % block_size)
    n = len(np.unique(np.concatenate(ids))) if ids else 0
    return n * Hkv * D * 2 * elem_bytes
