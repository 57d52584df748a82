"""Paged attention in fp64 (oracle): decode, split-K partials + combine, prefill.

What is computed.  The pages never write the attention formula out; they name
paged prefill and decode kernels built on Flash-Attention ideas (Pico-vLLM
write-up, §2 "kernel layer") and Flash Decode (H200 comparison section).  Both
are exact reformulations of softmax attention, so this oracle computes the
plain definition:

  out[i, h, :] = sum_t softmax_t(scale * q[i, h] . K[t, g]) * V[t, g]
  with g = h // (Hq / Hkv)  (grouped-query attention: consecutive query heads
  share one KV head; Pico-vLLM write-up, §1 "model layer", GQA)

K and V of a sequence are gathered token by token through its block table:
logical token t lives in physical block block_table[t // block_size] at row
t % block_size (mini-llm-engine post, §3.1 Paged KV Cache; nano-vllm
commentary, FAQ Q2).  Only t < L is read; table entries past ceil(L/16) are
never touched.

A chunk of C new query rows of a sequence with L cached tokens (L includes the
chunk) puts row i at absolute position L - C + i; it sees keys t <= L - C + i:
the whole cached prefix plus a causal triangle inside the chunk
(mini-llm-engine post, §3.3 Chunked Prefill).  Decode is the case C = 1.

All arithmetic is float64.  A sequence with L = 0 has no keys: its output is
zero (a reading; the pages do not cover empty sequences).
"""

import numpy as np

from .bf16 import bf16_to_f64


def gather_sequence_kv(k_cache, v_cache, block_table_row, L, block_size=16):
    """K, V of one sequence as float64 [L, Hkv, D], gathered via its table."""
    t = np.arange(int(L))
    blk = np.asarray(block_table_row)[t // block_size].astype(np.int64)
    row = t % block_size
    K = bf16_to_f64(k_cache[blk, :, row, :])
    V = bf16_to_f64(v_cache[blk, :, row, :])
    return K, V


def attend_sequence(q_rows, K, V, L, scale):
    """Causal attention of C query rows (float64 [C, Hq, D]) over L keys.

    Row i sees keys 0 .. L - C + i.  Returns float64 [C, Hq, D].
    """
    C, Hq, D = q_rows.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((C, Hq, D), dtype=np.float64)
    for i in range(C):
        n_vis = L - C + i + 1
        if n_vis <= 0:
            continue
        for h in range(Hq):
            g = h // G
            s = scale * (K[:n_vis, g, :] @ q_rows[i, h, :])
            w = np.exp(s - s.max())
            out[i, h, :] = (w @ V[:n_vis, g, :]) / w.sum()
    return out


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, block_size=16):
    """Single-token decode for every sequence: float64 [B, Hq, D].

    q: uint16 [B, Hq, D] (already rotated); block_tables: int [B, max_blocks];
    context_lens: int [B], each counting every cached token including the new
    one, whose query sits at position L - 1.
    """
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        K, V = gather_sequence_kv(k_cache, v_cache, block_tables[b], L, block_size)
        out[b] = attend_sequence(bf16_to_f64(q[b])[None], K, V, L, scale)[0]
    return out


def decode_partials(q_b, K, V, L, scale, partition_size):
    """Flash-Decode partials of one sequence (float64).

    Partition p covers tokens [p*P, min((p+1)*P, L)).  For each query head it
    holds m_p = the largest scaled score, l_p = sum exp(s - m_p) and
    o_p = sum exp(s - m_p) * v (unnormalised).  Returns (m [n, Hq],
    l [n, Hq], o [n, Hq, D]) with n = ceil(L / P); empty partitions do not
    exist.
    """
    Hq, D = q_b.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    n = -(-int(L) // partition_size)
    m = np.zeros((n, Hq))
    l = np.zeros((n, Hq))
    o = np.zeros((n, Hq, D))
    for p in range(n):
        t0, t1 = p * partition_size, min((p + 1) * partition_size, L)
        for h in range(Hq):
            g = h // G
            s = scale * (K[t0:t1, g, :] @ q_b[h])
            m[p, h] = s.max()
            w = np.exp(s - m[p, h])
            l[p, h] = w.sum()
            o[p, h] = w @ V[t0:t1, g, :]
    return m, l, o


def combine_partials(m, l, o):
    """Log-sum-exp combine of partials: float64 [Hq, D].

    M = max_p m_p, w_p = exp(m_p - M), out = sum_p w_p o_p / sum_p w_p l_p.
    """
    M = m.max(axis=0)
    w = np.exp(m - M[None, :])
    num = (w[:, :, None] * o).sum(axis=0)
    den = (w * l).sum(axis=0)
    return num / den[:, None]


def decode_split(q, k_cache, v_cache, block_tables, context_lens, scale,
                 partition_size, block_size=16):
    """Decode evaluated partition by partition, then combined: [B, Hq, D]."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        K, V = gather_sequence_kv(k_cache, v_cache, block_tables[b], L, block_size)
        m, l, o = decode_partials(bf16_to_f64(q[b]), K, V, L, scale, partition_size)
        out[b] = combine_partials(m, l, o)
    return out


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
            scale, block_size=16):
    """Causal chunked prefill over the paged cache: float64 [T, Hq, D].

    q: uint16 [T, Hq, D] packed by sequence; sequence b owns rows
    query_start_loc[b] .. query_start_loc[b+1]-1 (C_b rows) and has
    context_lens[b] = L_b cached tokens, the chunk's own keys included.
    """
    T, Hq, D = q.shape
    out = np.zeros((T, Hq, D), dtype=np.float64)
    B = len(context_lens)
    for b in range(B):
        r0, r1 = int(query_start_loc[b]), int(query_start_loc[b + 1])
        C, L = r1 - r0, int(context_lens[b])
        if C == 0:
            continue
        if C > L:
            raise ValueError("a chunk cannot be longer than its context")
        K, V = gather_sequence_kv(k_cache, v_cache, block_tables[b], L, block_size)
        out[r0:r1] = attend_sequence(bf16_to_f64(q[r0:r1]), K, V, L, scale)
    return out
