"""Block copies between KV pools (test infrastructure, CPU only).

Follows the mini-llm-engine post: §3.4 (a block shared by several sequences,
ref_count > 1, is copied to a newly allocated block before one of them writes
it: copy-on-write) and §3.5 (a preempted sequence's blocks move to host memory
and come back into new device blocks: swap-out / swap-in).  Both are the same
operation on whole blocks: the [Hkv][16][D] tile of a source block id becomes
the tile of a destination block id, bit for bit.
"""

import numpy as np


def copy_blocks(dst_pool, src_pool, src_ids, dst_ids):
    """dst[dst_ids[i]] = src[src_ids[i]] for every i; returns a new dst pool.

    Pools are arrays [num_blocks, Hkv, 16, D] of any dtype (bf16 bit patterns
    here); src and dst may be the same pool (copy-on-write), in which case
    every tile is read from the pool as it was before the call."""
    src = np.array(src_pool, copy=True)
    out = np.array(dst_pool, copy=True)
    for s, d in zip(np.asarray(src_ids).tolist(), np.asarray(dst_ids).tolist()):
        out[d] = src[s]
    return out
