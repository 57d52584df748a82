"""Shared helpers of the GPU parity tests: run the library and the oracle on the
same seeded inputs and compare.

Attention tolerance (bf16 outputs y against the fp64 oracle x):
  max criterion   max(|y - x| - ulp_bf16(x)/2) <= 1e-2
  mean criterion  mean|y - bf16_rne(x)|          <= 1e-3
Rounding x to bf16 alone can move it by half a bf16 ulp (0.0156 for |x| in
[4, 8)), so the allowance of the max-abs bar is measured beyond that rounding,
and the mean-abs bar against the correctly rounded oracle.  Raw max/mean abs
errors are returned too.
"""

import numpy as np
import torch

import oracle
from workloads import as_bits, from_bits

MAX_TOL = 1e-2
MEAN_TOL = 1e-3


def attention_errors(y, x):
    """y: bf16 tensor (any device); x: float64 numpy array of the same shape."""
    yb = as_bits(y)
    yf = oracle.bf16_to_f64(yb)
    x = np.asarray(x, dtype=np.float64)
    excess = np.abs(yf - x) - oracle.bf16_ulp(x) / 2
    rne = oracle.bf16_to_f64(oracle.f64_to_bf16_rne(x))
    return {
        "max_excess": float(excess.max()) if x.size else 0.0,
        "mean_vs_rne": float(np.abs(yf - rne).mean()) if x.size else 0.0,
        "raw_max": float(np.abs(yf - x).max()) if x.size else 0.0,
        "raw_mean": float(np.abs(yf - x).mean()) if x.size else 0.0,
        "finite": bool(np.isfinite(yf).all()),
    }


def assert_attention_close(y, x, label=""):
    e = attention_errors(y, x)
    assert e["finite"], f"{label}: non-finite output"
    assert e["max_excess"] <= MAX_TOL, f"{label}: {e}"
    assert e["mean_vs_rne"] <= MEAN_TOL, f"{label}: {e}"
    return e


def oracle_store(b):
    """Oracle store of a workload's new rows: (q bits, k_cache bits, v_cache bits)."""
    return oracle.cache_store(as_bits(b.q), as_bits(b.k), as_bits(b.v), as_bits(b.k_cache),
                              as_bits(b.v_cache), b.slot_mapping.cpu().numpy(),
                              b.positions.cpu().numpy(), b.cos_sin.cpu().numpy())


def gpu_store(pa, g):
    """Library store on a device copy g (modified in place)."""
    pa.cache_store(g.q, g.k, g.v, g.k_cache, g.v_cache, g.slot_mapping, g.positions, g.cos_sin)
    torch.cuda.synchronize()


def oracle_decode(qbits, kc, vc, b):
    return oracle.decode(qbits, kc, vc, b.block_tables.cpu().numpy(),
                         b.context_lens.cpu().numpy(), b.scale)


def gpu_decode(pa, g, partition_size=-1, q=None):
    out = pa.decode(g.q if q is None else q, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                    g.scale, g.max_context_len, partition_size=partition_size)
    torch.cuda.synchronize()
    return out


def to_device_bits(a, device="cuda"):
    return from_bits(a).to(device)
