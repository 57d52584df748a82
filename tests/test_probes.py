"""The device-ceiling probes: the streaming read sees every 32-bit word of the
buffer exactly once (its per-workgroup sums add up to the buffer's word sum mod
2^32, computed here on the host), and the MFMA probe's accumulators end at the
exact value its operands of ones give."""

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
