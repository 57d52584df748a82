"""Shared helpers of the GPU parity tests: run the library and the oracle on the
same seeded inputs and compare.

Attention tolerance (bf16 outputs y against the fp64 oracle x), the bar of
1e-2 max-abs and 1e-3 mean-abs on bf16 outputs:
  literal   max|y - x| <= 1e-2 and mean|y - x| <= 1e-3, asserted on every case
            whose oracle output stays below 4 in magnitude (there half a bf16
            ulp is at most 0.0078, so the max bar leaves room beyond rounding).
            The mean bar is asserted where the correctly rounded oracle itself,
            mean|bf16_rne(x) - x|, is at most 0.75e-3: for outputs spread like
            N(0,1) that floor is about 1.1e-3, which no bf16 output can beat.
  rounding  max(|y - x| - ulp_bf16(x)/2) <= 1e-2 and mean|y - bf16_rne(x)| <= 1e-3,
            asserted on every case: the allowance measured beyond the rounding
            of x to bf16 (half an ulp is 0.0156 for |x| in [4, 8)).
Every error figure is returned, with the rounding floor and which bars applied.
"""

import numpy as np
import torch

import oracle
from workloads import as_bits, from_bits

MAX_TOL = 1e-2
MEAN_TOL = 1e-3
LITERAL_BELOW = 4.0        # literal max/mean bars apply when max|x| < this
LITERAL_MEAN_FLOOR = 0.75e-3  # ... and the mean bar when the rounding floor is at most this


def attention_errors(y, x):
    """y: bf16 tensor (any device); x: float64 numpy array of the same shape."""
    yb = as_bits(y)
    yf = oracle.bf16_to_f64(yb)
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return {"max_excess": 0.0, "mean_vs_rne": 0.0, "raw_max": 0.0, "raw_mean": 0.0,
                "rne_floor_mean": 0.0, "max_abs_x": 0.0, "literal_max": True,
                "literal_mean": True, "finite": True}
    excess = np.abs(yf - x) - oracle.bf16_ulp(x) / 2
    rne = oracle.bf16_to_f64(oracle.f64_to_bf16_rne(x))
    max_abs_x = float(np.abs(x).max())
    floor = float(np.abs(rne - x).mean())
    return {
        "max_excess": float(excess.max()),
        "mean_vs_rne": float(np.abs(yf - rne).mean()),
        "raw_max": float(np.abs(yf - x).max()),
        "raw_mean": float(np.abs(yf - x).mean()),
        "rne_floor_mean": floor,
        "max_abs_x": max_abs_x,
        "literal_max": max_abs_x < LITERAL_BELOW,
        "literal_mean": max_abs_x < LITERAL_BELOW and floor <= LITERAL_MEAN_FLOOR,
        "finite": bool(np.isfinite(yf).all()),
    }


def assert_attention_close(y, x, label=""):
    e = attention_errors(y, x)
    assert e["finite"], f"{label}: non-finite output"
    assert e["max_excess"] <= MAX_TOL, f"{label}: {e}"
    assert e["mean_vs_rne"] <= MEAN_TOL, f"{label}: {e}"
    if e["literal_max"]:
        assert e["raw_max"] <= MAX_TOL, f"{label}: literal max-abs bar: {e}"
    if e["literal_mean"]:
        assert e["raw_mean"] <= MEAN_TOL, f"{label}: literal mean-abs bar: {e}"
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
