"""The device-ceiling probes: the streaming read sees every 32-bit word of the
buffer exactly once (its per-workgroup sums add up to the buffer's word sum mod
2^32, computed here on the host), the MFMA probe's accumulators end at the
exact value its operands of ones give, and the issue-mix probe's products do the
same beside its exp2/FMA chains."""

import numpy as np
import pytest
import torch

from paged_kv_cache_240_amd import probes

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,grid", [(16, 1), (4096, 3), (1 << 20, 64), ((1 << 24) + 48, 2048)])
def test_stream_read_sees_every_word_once(gpu, nbytes, grid):
    g = torch.Generator().manual_seed(nbytes)
    words = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    want = int(words.numpy().view(np.uint32).astype(np.uint64).sum() % (1 << 32))
    sums = probes.prepare_probe_stream_read(words.cuda(), grid=grid)()
    torch.cuda.synchronize()
    got = int(sums.cpu().numpy().view(np.uint32).astype(np.uint64).sum() % (1 << 32))
    assert got == want


@pytest.mark.parametrize("nbytes", [4096, 8192, 16384, 1 << 20, 1 << 24])
def test_gather_read_sees_every_word_once(gpu, nbytes):
    """Every 4 KiB tile is visited once under the scrambled order (sizes below and
    above one wave's 4 tiles and one workgroup's 16)."""
    g = torch.Generator().manual_seed(nbytes + 1)
    words = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    want = int(words.numpy().view(np.uint32).astype(np.uint64).sum() % (1 << 32))
    call = probes.prepare_probe_gather_read(words.cuda())
    sums = call()
    torch.cuda.synchronize()
    assert sums.numel() == max(1, nbytes // 4096 // 16)
    got = int(sums.cpu().numpy().view(np.uint32).astype(np.uint64).sum() % (1 << 32))
    assert got == want


@pytest.mark.parametrize("iters,grid", [(1, 1), (7, 3), (1000, 512)])
def test_mfma_probe_exact(gpu, iters, grid):
    out = probes.prepare_probe_mfma_bf16(iters, grid, "cuda")()
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.full((4 * grid,), 128.0 * iters))


def _issue_mix_products_only(iters):
    """Host value of a mode-1 lane: eight accumulators of 64 * iters each, then the
    16 untouched chain values 1e-3 * (lane + k), added in the kernel's fp32 order."""
    lane = np.arange(256) % 64
    acc = np.zeros(256, dtype=np.float32)
    for _ in range(8):
        acc = (acc + np.float32(64.0 * iters)).astype(np.float32)
    for k in range(16):
        acc = (acc + (np.float32(1e-3) * (lane + k).astype(np.float32)).astype(np.float32)).astype(np.float32)
    return acc


@pytest.mark.parametrize("iters,grid", [(1, 1), (5, 3), (256, 256)])
def test_issue_mix_probe(gpu, iters, grid):
    outs = {}
    for mode in (1, 2, 3):
        outs[mode] = probes.prepare_probe_issue_mix(mode, iters, grid, "cuda")().cpu()
        again = probes.prepare_probe_issue_mix(mode, iters, grid, "cuda")().cpu()
        torch.cuda.synchronize()
        assert torch.isfinite(outs[mode]).all() and torch.equal(outs[mode], again)
    want = np.tile(_issue_mix_products_only(iters), grid)
    assert np.array_equal(outs[1].numpy(), want)
    # both kinds of work in one wave: the products' exact part plus the chains' part
    assert torch.allclose(outs[3], outs[2] + 512.0 * iters, rtol=4e-6, atol=1e-3)  # 16 roundings at 512 * iters
