"""Fused rotate-half RoPE + KV-cache store (oracle).

What is computed (Pico-vLLM write-up, §1 "model layer": RoPE written by hand,
rotate_half done in place; §2 "kernel layer": the position encoding is fused
with the write into the KV cache; mini-llm-engine post, §3.1: the cache is a
pool of 16-token physical blocks addressed through a per-sequence table):

  for each new token i with slot s_i >= 0 and position p_i:
    blk = s_i // block_size, row = s_i % block_size
    k_cache[blk, g, row, :] = bf16(rope(k[i, g, :], p_i))   for every KV head g
    v_cache[blk, g, row, :] = v[i, g, :]  (bit copy)         for every KV head g
    q[i, h, :]              = bf16(rope(q[i, h, :], p_i))   for every query head h
  a token with s_i < 0 is padding: nothing is read or written for it.

Readings where the pages are silent (each listed in the design notes):
  * rotate-half pairs element j with element j + D/2 (half split, not
    interleaved), because the page names rotate_half;
  * the angles come in as an fp32 table cos_sin[p] = [cos(p*f_j) | sin(p*f_j)]
    for j < D/2, an input of the operation shared by both sides;
  * each output element is two fp32 products and one fp32 add or subtract,
    each rounded to nearest even, with no fused multiply-add, then rounded to
    bf16 (nearest even).  numpy float32 arithmetic does exactly this.
"""

import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16_rne


def rope_rotate_half(x_bits, cos, sin):
    """Rotate-half RoPE on bf16 rows, in the pinned fp32 operation order.

    x_bits: uint16 [..., D] bf16 bit patterns.
    cos, sin: float32 [..., D/2], broadcastable against x's leading dims.
    Returns uint16 [..., D]: bf16(y) with
      y[j]       = fl32(fl32(a_j * c_j) - fl32(b_j * s_j))
      y[j + D/2] = fl32(fl32(b_j * c_j) + fl32(a_j * s_j))
    where a_j = x[j], b_j = x[j + D/2], j < D/2.
    """
    x = bf16_to_f32(x_bits)
    half = x.shape[-1] // 2
    a = x[..., :half]
    b = x[..., half:]
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    ac = np.multiply(a, c, dtype=np.float32)
    bs = np.multiply(b, s, dtype=np.float32)
    bc = np.multiply(b, c, dtype=np.float32)
    as_ = np.multiply(a, s, dtype=np.float32)
    y_lo = np.subtract(ac, bs, dtype=np.float32)
    y_hi = np.add(bc, as_, dtype=np.float32)
    return f32_to_bf16_rne(np.concatenate([y_lo, y_hi], axis=-1))


def cache_store(q, k, v, k_cache, v_cache, slot_mapping, positions, cos_sin,
                block_size=16):
    """Oracle of the fused RoPE + slot-mapped KV store.

    q: uint16 [T, Hq, D] or None; k, v: uint16 [T, Hkv, D];
    k_cache, v_cache: uint16 [NB, Hkv, block_size, D];
    slot_mapping, positions: int [T]; cos_sin: float32 [max_pos, D].
    Returns new arrays (q_out or None, k_cache_out, v_cache_out); the inputs
    are not modified.  Tokens are visited one at a time, in order.
    """
    k_out = np.array(k_cache, dtype=np.uint16, copy=True)
    v_out = np.array(v_cache, dtype=np.uint16, copy=True)
    q_out = None if q is None else np.array(q, dtype=np.uint16, copy=True)
    T = len(slot_mapping)
    D = k.shape[-1]
    half = D // 2
    for i in range(T):
        slot = int(slot_mapping[i])
        if slot < 0:
            continue
        pos = int(positions[i])
        c = cos_sin[pos, :half]
        s = cos_sin[pos, half:]
        blk, row = divmod(slot, block_size)
        for g in range(k.shape[1]):
            k_out[blk, g, row, :] = rope_rotate_half(k[i, g, :], c, s)
            v_out[blk, g, row, :] = v[i, g, :]
        if q_out is not None:
            for h in range(q_out.shape[1]):
                q_out[i, h, :] = rope_rotate_half(q[i, h, :], c, s)
    return q_out, k_out, v_out
