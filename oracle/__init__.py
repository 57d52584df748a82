"""CPU oracle for paged KV-cache attention (test infrastructure, not product).

This package is the slow, plainly written reference that the HIP path is checked
against.  It is test infrastructure: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it.  The product
library never routes through it, and it imports nothing from the product
package or its C library.

Sources (the four pages this work follows, cited by title and section):
  * "Pico-vLLM" write-up (zingnex forum): §1 model layer (RoPE, GQA, in-place
    rotate_half), §2 kernel layer (paged prefill kernel, paged decode kernel,
    fused RoPE + KV-cache store, Flash-Attention-style tiling), H200 comparison
    section (Flash Decode).
  * "mini-llm-engine" post (liangqianxing): §3.1 Paged KV Cache (16-token
    blocks, per-sequence logical->physical block table), §3.3 Chunked Prefill
    (prefill ranges), §3.4 Prefix Caching (shared blocks, ref_count > 1,
    copy-on-write), §3.5 CPU Swap, §3.6 Speculative Decoding (verification
    is a prefill of the draft rows).
  * "nano-vllm" commentary (ai-stack), FAQ Q2 (logical-to-physical block map).
  * "LLM-Inference-Engine" write-up (zingnex forum), "dynamic request injection"
    (prefill is compute-bound, decode is bandwidth-bound).

Modules:
  bf16       bf16 <-> fp32/fp64 conversions written from the IEEE-754 definition.
  store      fused rotate-half RoPE + slot-mapped scatter into the block pool,
             in a pinned fp32 operation order (bit-exact target).
  attention  fp64 paged attention: decode, split-K partials + log-sum-exp
             combine, and causal chunked prefill (multi-query verification is
             the chunked prefill with chunks of NQ rows).
  blocks     whole-block copies between pools (copy-on-write, swap).
  block_manager  plain-Python model of the host block manager's policy.
  layer_ops  fused residual add + RMSNorm and fused SwiGLU.

Every function here is pinned by ``tests/test_oracle.py`` against something
other than itself (closed forms, library routines, invariants, brute force).
No function of this package is "parity unpinned".
"""

from . import bf16, store, attention, blocks, layer_ops  # noqa: F401
from .bf16 import (  # noqa: F401
    bf16_to_f32,
    bf16_to_f64,
    f32_to_bf16_rne,
    f64_to_bf16_rne,
    bf16_ulp,
)
from .store import rope_rotate_half, cache_store  # noqa: F401
from .attention import (  # noqa: F401
    gather_sequence_kv,
    attend_sequence,
    decode,
    decode_partials,
    combine_partials,
    decode_split,
    prefill,
)
from .blocks import copy_blocks  # noqa: F401
from .layer_ops import rmsnorm_residual, swiglu  # noqa: F401
