"""pa_rmsnorm_residual and pa_swiglu against the oracle.

Bar: the residual written back is bit-exact (the fp32 sum of two bf16 values
is exact, then rounded to nearest even); the outputs are one fp32 computation
rounded once to bf16, so each may differ from the fp64 value x by half a bf16
ulp plus fp32 arithmetic error: |y - x| - ulp_bf16(x)/2 <= 2^-14 |x|.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import as_bits

pytestmark = pytest.mark.gpu

QWEN_H, QWEN_I = 1536, 8960


def _close(y, x, label):
    yf = oracle.bf16_to_f64(as_bits(y))
    excess = np.abs(yf - x) - oracle.bf16_ulp(x) / 2 - 2.0 ** -14 * np.abs(x)
    assert np.isfinite(yf).all(), label
    assert excess.max() <= 0, f"{label}: {excess.max()}"


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("T,H", [(1, QWEN_H), (64, QWEN_H), (4096, QWEN_H), (7, 64), (33, 384),
                                 (5, 4096), (3, 16384)])
def test_rmsnorm_residual(gpu, T, H):
    x, r, w = _rand((T, H), T + H), _rand((T, H), T + H + 1, 0.5), _rand((H,), H)
    want, new_r = oracle.rmsnorm_residual(as_bits(x), as_bits(w), as_bits(r), eps=1e-6)
    xg, rg, wg = x.cuda(), r.cuda(), w.cuda()
    out = gpu.rmsnorm_residual(xg, wg, rg, eps=1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(as_bits(rg), new_r), "residual written back bit-exact"
    _close(out, want, f"rmsnorm T={T} H={H}")


def test_rmsnorm_without_residual(gpu):
    x, w = _rand((100, QWEN_H), 1, 3.0), _rand((QWEN_H,), 2)
    want, _ = oracle.rmsnorm_residual(as_bits(x), as_bits(w), None, eps=1e-5)
    xg = x.cuda()
    out = gpu.rmsnorm_residual(xg, w.cuda(), None, eps=1e-5)
    torch.cuda.synchronize()
    _close(out, want, "rmsnorm, no residual")
    assert torch.equal(xg.cpu(), x)  # x is only read


def test_rmsnorm_tiny_and_zero_rows(gpu):
    # an all-zero row normalises to zeros (eps keeps it finite); tiny rows to their direction
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    x[1] = 1e-20
    x[2, ::3] = -3.0
    w = torch.ones(256, dtype=torch.bfloat16)
    want, _ = oracle.rmsnorm_residual(as_bits(x), as_bits(w), None, eps=1e-6)
    out = gpu.rmsnorm_residual(x.cuda(), w.cuda(), None, eps=1e-6)
    torch.cuda.synchronize()
    _close(out, want, "zero/tiny rows")
    assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[3]) == 0


@pytest.mark.parametrize("T,I", [(1, QWEN_I), (64, QWEN_I), (2048, QWEN_I), (3, 8), (17, 136)])
def test_swiglu(gpu, T, I):
    gu = _rand((T, 2 * I), T * 7 + I, 3.0)
    want = oracle.swiglu(as_bits(gu))
    out = gpu.swiglu(gu.cuda())
    torch.cuda.synchronize()
    _close(out, want, f"swiglu T={T} I={I}")


def test_swiglu_extremes(gpu):
    # zero, tiny and huge gates; large negative gates across the switch to the
    # scaled form (near -44.4) and beyond the overflow of e^-g (below -88.7), whose
    # results are tiny normals, then subnormals, then zero
    gate = torch.tensor([0.0, 1.0, -1.0, 80.0, -80.0, 1e-30, -1e-30, 3.0e38,
                         -44.0, -45.0, -60.0, -89.0, -95.0, -100.0, -120.0, -3.0e38], dtype=torch.float32)
    up = torch.tensor([1.0, 2.0, -2.0, 0.5, 7.0, 1.0, 1.0, 1e-37,
                       3.0, -3.0, 1.0, 1.0, 2.0, -1.0, 1.0, 1.0], dtype=torch.float32)
    gu = torch.cat([gate, up]).view(1, 32).to(torch.bfloat16)
    want = oracle.swiglu(as_bits(gu))
    assert want[0, 11] != 0 and abs(want[0, 11]) > 2.0 ** -126   # -89: a normal result
    out = gpu.swiglu(gu.cuda())
    torch.cuda.synchronize()
    _close(out, want, "extremes")
