"""Prepared library calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay, with eager work and synchronisations between replays,
gives the eager result bit for bit.  The library records no memset and
allocates nothing while enqueueing, so its launches capture as they are."""

import numpy as np
import pytest
import torch

import workloads as W
from workloads import as_bits

pytestmark = pytest.mark.gpu


def _step_calls(pa, layers, P):
    calls, outs = [], []
    for g in layers:
        o_part = torch.empty((g.B, g.Hq, -(-g.max_context_len // P), g.D), dtype=torch.float32, device="cuda")
        lse = torch.empty(o_part.shape[:3], dtype=torch.float32, device="cuda")
        out = torch.empty_like(g.q)
        calls.append(pa.prepare_decode_step_partitions(g.q, g.k, g.v, g.k_cache, g.v_cache, g.block_tables,
                                                       g.context_lens, g.cos_sin, g.scale,
                                                       g.max_context_len, P, o_part, lse))
        calls.append(pa.prepare_decode_combine(o_part, lse, g.context_lens, g.max_context_len, P, out))
        outs.append(out)
    return calls, outs


def test_decode_step_graph_replays(gpu):
    layers = [W.decode_batch([300 + 97 * i, 1024, 17, 600], 12, 2, 128, 256, 9000 + i, theta=1e6).to("cuda")
              for i in range(4)]
    P = 128
    calls, outs = _step_calls(gpu, layers, P)
    for c in calls:
        c()
    torch.cuda.synchronize()
    eager = [as_bits(o).copy() for o in outs]
    for o in outs:
        o.zero_()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        for c in calls:
            c(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.zero_()                       # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(as_bits(o), eager[i]), f"replay {rep} layer {i}"
        calls[1]()                          # an eager library call between replays too
        torch.cuda.synchronize()


def test_prefill_graph_replays(gpu):
    b = W.prefill_batch([100, 0, 33], [64, 17, 200], 12, 2, 128, 64, 9100, theta=1e6).to("cuda")
    gpu.cache_store(b.q, b.k, b.v, b.k_cache, b.v_cache, b.slot_mapping, b.positions, b.cos_sin)
    pre = gpu.prepare_prefill(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                              b.query_start_loc, b.scale, b.max_query_len)
    ref = as_bits(pre()).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        pre(s)
    torch.cuda.synchronize()
    for rep in range(3):
        pre.result.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(as_bits(pre.result), ref), f"replay {rep}"
