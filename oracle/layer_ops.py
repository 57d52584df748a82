"""The elementwise neighbours of attention in a decoder layer (test
infrastructure, CPU only): fused residual add + RMSNorm and fused SwiGLU
(Pico-vLLM write-up, §2 kernel layer), written from their definitions.

rmsnorm_residual: r' = bf16(x + r) (the sum of two bf16 values is exact in
fp64, then rounded to nearest even); out = w * r' / sqrt(mean(r'^2) + eps) in
fp64.  swiglu: out = silu(gate) * up with silu(g) = g / (1 + e^-g), in fp64.
"""

import numpy as np

from .bf16 import bf16_to_f64, f64_to_bf16_rne


def rmsnorm_residual(x_bits, weight_bits, residual_bits=None, eps=1e-6):
    """x, residual: uint16 [T, H] bf16 bits; weight: uint16 [H].
    Returns (out float64 [T, H], new residual uint16 [T, H] or None)."""
    x = bf16_to_f64(x_bits)
    if residual_bits is not None:
        new_r = f64_to_bf16_rne(x + bf16_to_f64(residual_bits))
        h = bf16_to_f64(new_r)
    else:
        new_r = None
        h = x
    w = bf16_to_f64(weight_bits)
    rms = np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return w * h / rms, new_r


def swiglu(gate_up_bits):
    """gate_up: uint16 [T, 2I] bf16 bits ([gate | up]).  Returns float64 [T, I]."""
    gu = bf16_to_f64(gate_up_bits)
    i = gu.shape[-1] // 2
    g, u = gu[..., :i], gu[..., i:]
    with np.errstate(over="ignore"):   # e^-g = inf for very negative g: the quotient is then -0
        return g / (1.0 + np.exp(-g)) * u
