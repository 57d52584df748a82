"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

Headline workload (the long-context flash-decode): 16 sequences x 8192 cached
tokens, 12 query / 2 KV heads (the Qwen2.5-1.5B attention shape), head_dim
128, 16-token blocks, split-K partitions of 512 tokens, 28 independent layer
caches run back to back (3.76 GB of K/V, far beyond the 256 MB last-level
cache, so every step reads HBM).  One step = for each of the 28 layers: RoPE
and KV-cache store of the step's 16 new tokens, the split-K partitions and
the log-sum-exp reduce -- pa_decode_step, two launches per layer (the store
folded into the partition kernel, then the reduce), bit-identical to
pa_cache_store + pa_decode (also timed, as `separate_calls`).  All inputs are synthetic, seeded, resident in HBM.

Printed: one JSON line.  value = effective KV GB/s of the whole step (K/V
bytes the 28 layers read / step time).  roofline = the step's partition
kernel (the store folded in; dominant) timed per launch with HIP events on its
stream, against 8 TB/s.  cpu_baseline = the CPU oracle on a bounded sample of the same
workload.  Extra keys: the separate calls, the batch-1 2048-token decode call,
the continuous-batching step, speculative verification, block copies, the
layer ops and the chunked prefill.

Other modes (for profiling with rocprofv3, committed so profile commands run
committed files only):
    python bench.py --mode decode-kernel   # 3 x 28 launches of the step's partition kernel
    python bench.py --mode partition-kernel  # 3 x 28 launches of the unfused partition kernel
    python bench.py --mode prefill-kernel  # 20 launches of the prefill kernel only
    python bench.py --mode verify-kernel  # 3 x 28 calls of pa_decode_multi (5 queries per sequence)
    python bench.py --mode cb-cold  # continuous-batching step, 10 cold calls of each path
    python bench.py --mode copy-calibration  # torch copy of 1 GiB (FETCH/WRITE_SIZE scale)
    python bench.py --mode issue-probe  # matrix products beside exp2/FMA chains, 1-3 waves per SIMD
    python bench.py --mode write-traffic --pmc F_STEP W_STEP F_COPY W_COPY
        # profiles/decode_partitions_traffic.json from the four counter folders
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import paged_kv_cache_240_amd as pa  # noqa: E402
from paged_kv_cache_240_amd import probes  # noqa: E402
import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
LONG_P = W.LONG_PARTITION
STEP_KERNEL = "decode_kernel<128, 6, true, true, true, 8, false>"


def _sync():
    torch.cuda.synchronize()


def _event():
    return torch.cuda.Event(enable_timing=True)


def kernel_source_hash(name):
    with open(os.path.join(ROOT, "paged_kv_cache_240_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


# ---------------------------------------------------------------------------
# Workload set-up
# ---------------------------------------------------------------------------

def make_long_layers(layers, device):
    """The layer caches with their library calls prepared once (validated and
    marshalled; each call then costs one C call, as in a serving loop)."""
    out = []
    for layer in range(layers):
        b = W.long_decode_layer(layer, device=device)
        P = LONG_P
        np_ = -(-b.max_context_len // P)
        o_part = torch.empty((b.B, b.Hq, np_, b.D), dtype=torch.float32, device=device)
        lse = torch.empty((b.B, b.Hq, np_), dtype=torch.float32, device=device)
        dout = torch.empty((b.B, b.Hq, b.D), dtype=torch.bfloat16, device=device)
        b.meta["store"] = pa.prepare_cache_store(b.q, b.k, b.v, b.k_cache, b.v_cache,
                                                 b.slot_mapping, b.positions, b.cos_sin)
        b.meta["partitions"] = pa.prepare_decode_partitions(b.q, b.k_cache, b.v_cache, b.block_tables,
                                                            b.context_lens, b.scale, b.max_context_len,
                                                            P, o_part, lse)
        b.meta["combine"] = pa.prepare_decode_combine(o_part, lse, b.context_lens, b.max_context_len,
                                                      P, dout)
        # the step with the store folded in reads q unrotated; its own copy, so the separate
        # store's in-place rotation of b.q cannot change what it is given.  pa_decode_step is
        # exactly these two calls on the same workspace
        q_raw = b.q.clone()
        b.meta["q_raw"] = q_raw
        o2 = torch.empty_like(o_part)
        l2 = torch.empty_like(lse)
        b.meta["step_partitions"] = pa.prepare_decode_step_partitions(
            q_raw, b.k, b.v, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.cos_sin,
            b.scale, b.max_context_len, P, o2, l2)
        b.meta["step_combine"] = pa.prepare_decode_combine(o2, l2, b.context_lens, b.max_context_len,
                                                           P, torch.empty_like(dout))
        out.append(b)
    return out


def store(b):
    b.meta["store"]()


def partitions(b):
    b.meta["partitions"]()


def combine(b):
    b.meta["combine"]()


def fused_step(b):
    b.meta["step_partitions"]()
    b.meta["step_combine"]()


def fused_partitions(b):
    b.meta["step_partitions"]()


def step_kernel_bytes(b):
    """Algorithmic bytes of one launch of the step's partition kernel (the store
    folded in): K and V of every context token (the new token's row read from its
    input instead), the queries, the cos/sin row of each sequence's position, the
    block table and the lengths read; the new K/V rows written.  The split-K
    partials are workspace, not counted."""
    kv = W.kv_bytes_logical(b.context_lens.cpu().numpy(), b.Hkv, b.D)
    new_rows = b.B * b.Hkv * b.D * 2 * 2
    return (kv + b.q.numel() * 2 + b.B * b.D * 4 + b.B * (-(-b.max_context_len // 16)) * 4 + b.B * 4
            + new_rows)


def partition_kernel_bytes(b):
    """Algorithmic bytes one partition-kernel launch must read: K and V of every
    context token, the queries, the block table and the context lengths."""
    kv = W.kv_bytes_logical(b.context_lens.cpu().numpy(), b.Hkv, b.D)
    return kv + b.q.numel() * 2 + b.B * (-(-b.max_context_len // 16)) * 4 + b.B * 4


# ---------------------------------------------------------------------------
# Headline: long-context decode steps
# ---------------------------------------------------------------------------

def run_long(layers, steps, warmup):
    """Windows over the same prepared calls, each bracketed by one pair of HIP
    events on the library's stream (torch's current stream):
      step      pa_decode_step for every layer (partitions with the store folded
                in, then the reduce)                             -> value
      stepk     the step's partition launches alone             -> roofline
      separate  store + partitions + combine for every layer
      decode    partitions + combine for every layer
      kernel    the unfused partition launches alone
    No event sits inside a window, so none adds its own cost to what is timed."""
    L = layers

    def step():
        for b in L:
            fused_step(b)

    def step_kernel():
        for b in L:
            fused_partitions(b)

    def separate():
        for b in L:
            store(b)
            partitions(b)
            combine(b)

    def decode_only():
        for b in L:
            partitions(b)
            combine(b)

    def kernel_only():
        for b in L:
            partitions(b)

    def window(fn):
        for _ in range(warmup):
            fn()
        _sync()
        t0, t1 = _event(), _event()
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        _sync()
        return t0.elapsed_time(t1) / steps

    return {"step_ms": window(step), "step_kernel_us": window(step_kernel) * 1000 / len(L),
            "separate_ms": window(separate),
            "decode_only_ms": window(decode_only),
            "partition_us": window(kernel_only) * 1000 / len(L)}


def run_graph(layers, steps, warmup):
    """The same 28-layer decode step captured once in a HIP graph and replayed
    (what a serving loop does to spare the per-launch host cost)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for b in layers:
            b.meta["step_partitions"](s)
            b.meta["step_combine"](s)
    _sync()
    for _ in range(warmup):
        g.replay()
    _sync()
    t0, t1 = _event(), _event()
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    _sync()
    ms = t0.elapsed_time(t1) / steps
    kv = sum(W.kv_bytes_logical(b.context_lens.cpu().numpy(), b.Hkv, b.D) for b in layers)
    return {"us_per_layer": round(ms * 1000 / len(layers), 2), "kv_GBps": round(kv / (ms * 1e-3) / 1e9, 1),
            "note": "pa_decode_step's two launches per layer, 28 layers, captured once and replayed"}


def run_verify(layers, steps, warmup, nq=5):
    """Speculative verification over the same 28 layer caches: nq queries per
    sequence (the last accepted token and nq-1 drafts) through pa_decode_multi
    with the library's partition choice (1024 tokens at this shape), one call per
    layer, back to back (cold caches)."""
    gen = torch.Generator(device=layers[0].q.device)
    gen.manual_seed(2407)
    calls = []
    for b in layers:
        q = torch.randn((b.B, nq, b.Hq, b.D), generator=gen, device=b.q.device).to(torch.bfloat16)
        calls.append(pa.prepare_decode_multi(q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                                             b.scale, b.max_context_len, -1))

    def run():
        for c in calls:
            c()
    for _ in range(warmup):
        run()
    _sync()
    t0, t1 = _event(), _event()
    t0.record()
    for _ in range(steps):
        run()
    t1.record()
    _sync()
    us = t0.elapsed_time(t1) * 1000 / steps / len(layers)
    kv = W.kv_bytes_logical(layers[0].context_lens.cpu().numpy(), layers[0].Hkv, layers[0].D)
    return {"queries_per_sequence": nq, "us_per_layer_call": round(us, 2),
            "kv_GBps": round(kv / us / 1e3, 1), "pct_of_hbm_peak": round(kv / us / 1e3 / HBM_PEAK_GBPS * 100, 2),
            "partition_size": 1024,
            "note": "pa_decode_multi with the library's partition choice (1024 tokens: one chunk of 8 waves "
                    "per workgroup) + combine, 28 layer caches of 16 x 8192 tokens"}


# ---------------------------------------------------------------------------
# Context measurements (the other decode shapes and the prefill)
# ---------------------------------------------------------------------------

def time_calls(fn, reps, warm=10):
    for _ in range(warm):
        fn()
    _sync()
    e0, e1 = _event(), _event()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    _sync()
    return e0.elapsed_time(e1) * 1000 / reps


def time_each(fn, reps, scrub=None, warm=10):
    """Per-call times in us (one pair of HIP events around each call), as
    median / p10 / p90.  With scrub (a device tensor of 1 GiB), the tensor is
    rewritten before every call, outside the timed window, so the call starts
    with cold caches (the 256 MB last-level cache included)."""
    for _ in range(warm):
        fn()
    _sync()
    t = []
    e0, e1 = _event(), _event()
    for _ in range(reps):
        if scrub is not None:
            scrub.add_(1)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        t.append(e0.elapsed_time(e1) * 1000)
    t = np.sort(np.array(t))
    return {"median_us": round(float(np.median(t)), 2), "p10_us": round(float(np.percentile(t, 10)), 2),
            "p90_us": round(float(np.percentile(t, 90)), 2), "reps": reps}


def issue_mix_table(device, iters=4096, verbose=False):
    """pa_probe_issue_mix: per launch, each wave runs `iters` iterations of 16 products
    (mode 1), 32 exp2 + FMA steps per lane (mode 2) or both (mode 3); one to three waves
    per SIMD (grid = CUs x waves); SIMD cycles per iteration at the nominal 2.4 GHz clock.
    overlap_saved_frac: the share of the two separate times that running both saves."""
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    table = []
    for wps in (1, 2, 3):
        row = {"waves_per_simd": wps}
        for mode, name in ((1, "products"), (2, "exp2_fma"), (3, "both")):
            call = probes.prepare_probe_issue_mix(mode, iters, cus * wps, device)
            us = time_calls(call, 5, warm=2)
            row[name + "_us"] = round(us, 2)
            row[name + "_cycles_per_iter"] = round(us * 1e-6 * 2.4e9 / iters)
        row["overlap_saved_frac"] = round(1 - row["both_us"] / (row["products_us"] + row["exp2_fma_us"]), 3)
        table.append(row)
        if verbose:
            print(json.dumps(row), flush=True)
    return table


def run_ceilings(device, layer_bytes):
    """Measured device limits beside the published ones:
      * a grid-stride streaming read of a 2 GiB buffer (eight times the
        last-level cache; best of four grid sizes);
      * a one-pass gather of the same buffer in scrambled 4 KiB tiles (a paged
        K/V read without its arithmetic) -- the read ceiling;
      * that gather over one layer's bytes per launch, each launch on another
        slice of the buffer (cold): the floor for one decode launch's reads;
      * bf16 matrix-core throughput (4 independent chains per wave)."""
    res = {"nominal_hbm_GBps": HBM_PEAK_GBPS, "nominal_mfma_bf16_TFLOPs": MFMA_BF16_PEAK_TFLOPS}
    nbytes = 1 << 31
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=device)
    best = 0.0
    for grid in (1024, 2048, 4096, 8192):
        us = time_calls(probes.prepare_probe_stream_read(buf, grid), 10, warm=2)
        best = max(best, nbytes / us / 1e3)
    res["stream_read_GBps"] = round(best, 1)
    us = time_calls(probes.prepare_probe_gather_read(buf), 10, warm=2)
    res["gather_read_GBps"] = round(nbytes / us / 1e3, 1)
    res["read_ceiling_GBps"] = max(res["stream_read_GBps"], res["gather_read_GBps"])
    slices = [probes.prepare_probe_gather_read(buf[i * (layer_bytes // 4):(i + 1) * (layer_bytes // 4)])
              for i in range(nbytes // layer_bytes)]
    state = {"i": 0}

    def one_layer():
        slices[state["i"] % len(slices)]()
        state["i"] += 1

    us = time_calls(one_layer, 4 * len(slices), warm=len(slices))
    res["gather_read_one_layer"] = {"bytes": layer_bytes, "us_per_launch": round(us, 2),
                                    "GBps": round(layer_bytes / us / 1e3, 1)}
    del slices, buf
    iters, best = 20000, 0.0
    for grid in (512, 1024):
        us = time_calls(probes.prepare_probe_mfma_bf16(iters, grid, device), 3, warm=1)
        best = max(best, grid * 4 * iters * 4 * 16384 / us / 1e6)
    res["mfma_bf16_TFLOPs"] = round(best, 1)
    res["issue_mix"] = issue_mix_table(device)
    res["note"] = ("pa_probe_stream_read, pa_probe_gather_read, pa_probe_mfma_bf16, pa_probe_issue_mix on this device; "
                   "read_ceiling = the faster of the two reads")
    return res


def run_context(device):
    res = {}
    scrub = torch.zeros(1 << 28, dtype=torch.int32, device=device)  # 1 GiB
    # batch 1, 2048 tokens: store + decode, library-chosen partitions, warm
    b = W.qwen_decode(device=device)
    q_raw = b.q.clone()  # the decode step takes q unrotated; the separate store rotates b.q in place
    P = pa.decode_partition_size(b.B, b.Hkv, b.max_context_len)
    dec = pa.prepare_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.scale,
                            b.max_context_len, partition_size=P)
    st = pa.prepare_cache_store(b.q, b.k, b.v, b.k_cache, b.v_cache, b.slot_mapping, b.positions,
                                b.cos_sin)

    def step2():
        st()
        dec()

    us = time_calls(dec, 1000)
    dstep = pa.prepare_decode_step(q_raw, b.k, b.v, b.k_cache, b.v_cache, b.block_tables,
                                   b.context_lens, b.cos_sin, b.scale, b.max_context_len)
    res["qwen_b1_l2048"] = {"decode_us_per_call": round(us, 2), "partition_size": P,
                            "store_plus_decode_us": round(time_calls(step2, 1000), 2),
                            "decode_step_us_per_call": round(time_calls(dstep, 1000), 2),
                            "kv_GBps": round(W.kv_bytes_logical([2048], 2, 128) / us / 1e3, 1),
                            "per_call_warm": time_each(dec, 1000),
                            "per_call_cold": time_each(dec, 50, scrub),
                            "note": "decode_us_per_call: pa_decode, 1000 back-to-back calls in one event "
                                    "window; store_plus_decode_us: pa_cache_store + pa_decode; "
                                    "decode_step_us_per_call: pa_decode_step (RoPE + store folded in); "
                                    "per_call_*: pa_decode with one event pair around each call "
                                    "(adds the event cost)"}
    # continuous-batching step: 64 sequences, 32 share a 2000-token prefix
    b = W.cb_step(device=device)
    P = pa.decode_partition_size(b.B, b.Hkv, b.max_context_len)
    dec3 = pa.prepare_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.scale,
                             b.max_context_len, partition_size=P)

    us = time_calls(dec3, 200)
    lens = b.context_lens.cpu().numpy()
    logical = W.kv_bytes_logical(lens, 2, 128)
    unique = W.kv_bytes_unique(b.block_tables.cpu().numpy(), lens, 2, 128)
    cold = time_each(dec3, 50, scrub)
    # the same step with the 2000-token prefix of sequences 0-31 read once for the group
    prefix = torch.zeros(b.B, dtype=torch.int32, device=device)
    prefix[:32] = 2000
    sp = pa.prepare_decode_shared_prefix(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                                         torch.tensor([0, 32], dtype=torch.int32, device=device), prefix,
                                         b.scale, b.max_context_len, 32, 2000,
                                         int((b.context_lens - prefix).max()), -1)
    us_sp = time_calls(sp, 200)
    cold_sp = time_each(sp, 50, scrub)
    res["cb_step_b64_shared_prefix"] = {
        "decode_us_per_call": round(us_sp, 2), "suffix_partition_size": "library's choice",
        "kv_unique_GBps_warm": round(unique / us_sp / 1e3, 1),
        "per_call_cold": cold_sp,
        "kv_unique_GBps_cold": round(unique / cold_sp["median_us"] / 1e3, 1),
        "unique_frac_of_hbm_peak_cold": round(unique / cold_sp["median_us"] / 1e3 / HBM_PEAK_GBPS, 4),
        "note": "pa_decode_shared_prefix: one partition launch of prefix items (2 sequences x 6 heads "
                "over 512 prefix tokens) and suffix items, then one reduce; at this size (32 sequences, "
                "2 MB of prefix) pa_decode is faster"}
    # the floor of the cold protocol: a one-element add, and pa_decode on a 4-sequence batch of
    # the same shape (two sequences on a 2000-token prefix + 16 tokens, two of 64 tokens)
    tiny = torch.zeros(1, device=device)
    fb = W.decode_batch([2016, 2016, 64, 64], W.QWEN_HQ, W.QWEN_HKV, W.QWEN_D, 512, 9, theta=1e6,
                        shared_prefix=([0, 1], 125), device=device)
    dec_f = pa.prepare_decode(fb.q, fb.k_cache, fb.v_cache, fb.block_tables, fb.context_lens, fb.scale,
                              fb.max_context_len, partition_size=P)
    res["cold_protocol_floor"] = {"one_element_add_us": time_each(lambda: tiny.add_(1), 50, scrub)["median_us"],
                                  "pa_decode_4_sequences_us": time_each(dec_f, 50, scrub)["median_us"],
                                  "note": "the same event window after the same 1 GiB rewrite, on "
                                          "launches with next to no bytes"}
    # many sequences on one long prefix: 128 x (4096 shared + 128 own) tokens
    lens = [4096 + 128] * 128
    bb = W.decode_batch(lens, W.QWEN_HQ, W.QWEN_HKV, W.QWEN_D, 128 * 8 + 256 + 64, 2414, theta=1e6,
                        shared_prefix=(list(range(128)), 256), device=device)
    Pb = pa.decode_partition_size(bb.B, bb.Hkv, bb.max_context_len)
    dec_b = pa.prepare_decode(bb.q, bb.k_cache, bb.v_cache, bb.block_tables, bb.context_lens, bb.scale,
                              bb.max_context_len, Pb)
    pre_b = torch.full((128,), 4096, dtype=torch.int32, device=device)
    sp_b = pa.prepare_decode_shared_prefix(bb.q, bb.k_cache, bb.v_cache, bb.block_tables, bb.context_lens,
                                           torch.tensor([0, 128], dtype=torch.int32, device=device), pre_b,
                                           bb.scale, bb.max_context_len, 128, 4096, 128, -1)
    uniq = W.kv_bytes_unique(bb.block_tables.cpu().numpy(), bb.context_lens.cpu().numpy(), 2, 128)
    us_d, us_s = time_calls(dec_b, 50), time_calls(sp_b, 50)
    res["shared_prefix_128x4096"] = {"decode_us": round(us_d, 2), "shared_prefix_us": round(us_s, 2),
                                     "speedup": round(us_d / us_s, 2), "kv_unique_bytes": int(uniq),
                                     "kv_logical_bytes": int(W.kv_bytes_logical(lens, 2, 128)),
                                     "note": "pa_decode vs pa_decode_shared_prefix, warm"}
    res["cb_step_b64"] = {"decode_us_per_call": round(us, 2), "partition_size": P,
                          "kv_logical_GBps": round(logical / us / 1e3, 1),
                          "kv_unique_GBps_warm": round(unique / us / 1e3, 1),
                          "per_call_cold": cold,
                          "kv_unique_GBps_cold": round(unique / cold["median_us"] / 1e3, 1),
                          "unique_frac_of_hbm_peak_cold": round(unique / cold["median_us"] / 1e3 / HBM_PEAK_GBPS, 4),
                          "kv_unique_bytes": int(unique), "kv_logical_bytes": int(logical),
                          "note": "warm: 28.5 MB of unique K/V stays in the last-level cache; cold: a 1 GiB "
                                  "rewrite before each call, outside the timed window"}
    # chunked prefill: 4 x (2048 cached + 512 new), store then prefill
    b = W.chunked_prefill(device=device)
    pst = pa.prepare_cache_store(b.q, b.k, b.v, b.k_cache, b.v_cache, b.slot_mapping, b.positions,
                                 b.cos_sin)
    pre = pa.prepare_prefill(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                             b.query_start_loc, b.scale, b.max_query_len)
    pst()
    wins = sorted(time_calls(pre, 100) for _ in range(5))
    us_pre = wins[len(wins) // 2]
    us_store = time_calls(pst, 50)
    pre_cold = time_each(pre, 50, scrub)
    store_cold = time_each(pst, 50, scrub)
    flops = prefill_flops(b)
    store_bytes = chunk_store_bytes(b)
    res["chunked_prefill"] = {"prefill_us": round(us_pre, 2),
                              "prefill_us_windows": [round(w, 2) for w in wins],
                              "prefill_cold": pre_cold,
                              "store_us": round(us_store, 2),
                              "store_cold": store_cold,
                              "store_bytes": store_bytes,
                              "store_GBps_warm": round(store_bytes / us_store / 1e3, 1),
                              "store_GBps_cold": round(store_bytes / store_cold["median_us"] / 1e3, 1),
                              "prefill_TFLOPs": round(flops / us_pre / 1e6, 1),
                              "mfma_bf16_frac": round(flops / us_pre / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                              "prefill_TFLOPs_cold": round(flops / pre_cold["median_us"] / 1e6, 1),
                              "mfma_bf16_frac_cold": round(flops / pre_cold["median_us"] / 1e6 /
                                                           MFMA_BF16_PEAK_TFLOPS, 4),
                              "flop": flops,
                              "note": "warm: back-to-back calls in one event window; cold: one event pair "
                                      "around each call after a 1 GiB rewrite (median, p10, p90)"}
    return res


def run_blocks(device):
    """Copy-on-write and swap of whole blocks at the Qwen2.5-1.5B head shape (8 KiB per
    block and pool): 2048 device-to-device copies, and 1024 blocks out to pinned host
    memory and back (over PCIe).  Rates count bytes read plus bytes written."""
    nb, hkv, d = 8192, W.QWEN_HKV, W.QWEN_D
    kc = torch.randn((nb, hkv, 16, d), device=device).to(torch.bfloat16)
    vc = torch.randn((nb, hkv, 16, d), device=device).to(torch.bfloat16)
    g = torch.Generator().manual_seed(2408)
    perm = torch.randperm(nb, generator=g).to(torch.int32)
    src, dst = perm[:2048].to(device), perm[4096:6144].to(device)
    cow = pa.prepare_copy_blocks(kc, vc, src, dst)
    blk = hkv * 16 * d * 2
    us = time_calls(cow, 50)
    res = {"cow_2048_blocks_us": round(us, 2), "cow_GBps": round(2 * 2 * 2048 * blk / us / 1e3, 1)}
    hk = torch.empty((1024, hkv, 16, d), dtype=torch.bfloat16).pin_memory()
    hv = torch.empty((1024, hkv, 16, d), dtype=torch.bfloat16).pin_memory()
    slots = torch.arange(1024, dtype=torch.int32, device=device)
    seq = perm[:1024].to(device)
    out_ = pa.prepare_swap_blocks(hk, hv, kc, vc, seq, slots)
    in_ = pa.prepare_swap_blocks(kc, vc, hk, hv, slots, perm[6144:7168].to(device))
    us_out, us_in = time_calls(out_, 20, warm=3), time_calls(in_, 20, warm=3)
    moved = 2 * 1024 * blk
    res.update({"swap_out_1024_blocks_us": round(us_out, 1), "swap_out_GBps": round(moved / us_out / 1e3, 2),
                "swap_in_1024_blocks_us": round(us_in, 1), "swap_in_GBps": round(moved / us_in / 1e3, 2)})
    return res


def run_layer_ops(device):
    """Fused RMSNorm + residual add and SwiGLU at the Qwen2.5-1.5B widths (hidden 1536,
    intermediate 8960), for a prefill-sized batch of tokens and a decode-sized one.
    Rates count bytes read plus bytes written once each."""
    res = {}
    g = torch.Generator().manual_seed(2413)
    H, I = 1536, 8960
    for T in (4096, 16):
        x = torch.randn((T, H), generator=g).to(torch.bfloat16).to(device)
        r = torch.randn((T, H), generator=g).to(torch.bfloat16).to(device)
        w = torch.randn((H,), generator=g).to(torch.bfloat16).to(device)
        norm = pa.prepare_rmsnorm_residual(x, w, r, eps=1e-6)
        us = time_calls(norm, 200)
        moved = 4 * T * H * 2 + H * 2          # x, r in; r', out out; the weight
        res[f"rmsnorm_residual_T{T}_H{H}"] = {"us": round(us, 2), "GBps": round(moved / us / 1e3, 1)}
        gu = torch.randn((T, 2 * I), generator=g).to(torch.bfloat16).to(device)
        act = pa.prepare_swiglu(gu)
        us = time_calls(act, 200)
        moved = 3 * T * I * 2                  # gate and up in, the product out
        res[f"swiglu_T{T}_I{I}"] = {"us": round(us, 2), "GBps": round(moved / us / 1e3, 1)}
    return res


def chunk_store_bytes(b):
    """Algorithmic bytes of the chunk's RoPE + store: q read and written, k and v
    read, their rows written to the pools, one cos/sin row per token read."""
    T = b.q.shape[0]
    return T * ((2 * b.Hq + 4 * b.Hkv) * b.D * 2 + b.D * 4)


def prefill_flops(b):
    """4 * D multiply-adds... per visible (row, key) pair: QK^T and PV, 2 flop each."""
    qsl = b.query_start_loc.cpu().numpy()
    lens = b.context_lens.cpu().numpy()
    pairs = 0
    for s in range(b.B):
        C, L = int(qsl[s + 1] - qsl[s]), int(lens[s])
        pairs += sum(L - C + i + 1 for i in range(C))
    return pairs * b.Hq * 4 * b.D


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the headline workload
# ---------------------------------------------------------------------------

def _blas_threads():
    """Threads numpy's BLAS may use (the oracle's matrix-vector products)."""
    try:
        from threadpoolctl import threadpool_info
        n = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return max(n)
    except ImportError:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(layers, budget_s):
    """The oracle's fp64 decode over (sequence, layer) pairs of the headline
    workload, cycling through the layers until about budget_s seconds of oracle
    time are spent."""
    import oracle  # test infrastructure; used here only for the CPU baseline leg
    from workloads import as_bits
    host = []
    for b in layers:
        host.append((as_bits(b.k_cache), as_bits(b.v_cache), b.block_tables.cpu().numpy(),
                     b.context_lens.cpu().numpy(), as_bits(b.q), b))
    done_bytes = 0
    pairs = 0
    t_total = 0.0
    threads = _blas_threads()
    while t_total < budget_s:
        for kc, vc, bt, cl, qb, b in host:
            for s in range(b.B):
                t0 = time.perf_counter()
                oracle.decode(qb[s:s + 1], kc, vc, bt[s:s + 1], cl[s:s + 1], b.scale)
                t_total += time.perf_counter() - t0
                done_bytes += W.kv_bytes_logical(cl[s:s + 1], b.Hkv, b.D)
                pairs += 1
                if t_total >= budget_s:
                    break
            if t_total >= budget_s:
                break
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(done_bytes / t_total / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model,
            "sample": f"fp64 numpy oracle decode of {pairs} (sequence, layer) pairs of the "
                      f"long-context workload (8192 tokens x 2 KV heads each), {t_total:.1f} s"}


def _errors(y, x):
    """Errors of the bf16 output y (device tensor) against the fp64 oracle x: raw
    max/mean |y - x|; the max beyond half a bf16 ulp of x and the mean against x
    rounded to bf16 (the reading used where |x| >= 4); the count of |x| >= 2."""
    import oracle
    from workloads import as_bits
    yf = oracle.bf16_to_f64(as_bits(y))
    x = np.asarray(x, dtype=np.float64)
    d = np.abs(yf - x)
    rne = oracle.bf16_to_f64(oracle.f64_to_bf16_rne(x))
    return {"raw_max_abs": float(d.max()), "raw_mean_abs": float(d.mean()),
            "max_beyond_half_ulp": float((d - oracle.bf16_ulp(x) / 2).max()),
            "mean_vs_bf16_rne": float(np.abs(yf - rne).mean()),
            "rne_floor_mean": float(np.abs(rne - x).mean()),
            "max_abs_x": float(np.abs(x).max()), "n_abs_x_ge_2": int((np.abs(x) >= 2).sum()),
            "n": int(x.size)}


def oracle_errors(layers, device):
    """The oracle on the inputs of configs 1-5 beside the library's outputs on the
    same inputs, with the launch configurations the timings use.  Sampled where the
    oracle would take long: two of the 28 long-context layers; eight rows of each
    chunked-prefill sequence (row i of a chunk equals decode at length L - C + i + 1)."""
    import oracle  # test infrastructure; run here only in the oracle leg of the bench
    from workloads import as_bits
    t0 = time.perf_counter()
    res = {}
    # 1: tiny decode, store then single pass and 16-token partitions
    b = W.tiny_decode(device=device)
    qr, kc, vc = oracle.cache_store(as_bits(b.q), as_bits(b.k), as_bits(b.v), as_bits(b.k_cache),
                                   as_bits(b.v_cache), b.slot_mapping.cpu().numpy(),
                                   b.positions.cpu().numpy(), b.cos_sin.cpu().numpy())
    pa.cache_store(b.q, b.k, b.v, b.k_cache, b.v_cache, b.slot_mapping, b.positions, b.cos_sin)
    _sync()
    store_exact = bool(np.array_equal(as_bits(b.k_cache), kc) and np.array_equal(as_bits(b.v_cache), vc)
                       and np.array_equal(as_bits(b.q), qr))
    ref = oracle.decode(qr, kc, vc, b.block_tables.cpu().numpy(), b.context_lens.cpu().numpy(), b.scale)
    res["1_tiny"] = {"store_bit_exact": store_exact,
                     "single_pass": _errors(pa.decode(b.q, b.k_cache, b.v_cache, b.block_tables,
                                                      b.context_lens, b.scale, b.max_context_len, 0), ref),
                     "split_16": _errors(pa.decode(b.q, b.k_cache, b.v_cache, b.block_tables,
                                                   b.context_lens, b.scale, b.max_context_len, 16), ref)}
    # 2 and 3: library-chosen partitions, as timed
    for name, b in (("2_qwen_b1_l2048", W.qwen_decode(device=device)), ("3_cb_step_b64", W.cb_step(device=device))):
        y = pa.decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.scale, b.max_context_len)
        ref = oracle.decode(as_bits(b.q), as_bits(b.k_cache), as_bits(b.v_cache), b.block_tables.cpu().numpy(),
                            b.context_lens.cpu().numpy(), b.scale)
        res[name] = _errors(y, ref)
    # 4: the headline decode step (store folded in, 512-token partitions, reduce) on two layers
    e4 = {}
    for li in sorted({0, len(layers) - 1}):
        b = layers[li]
        fused_step(b)
        _sync()
        y = b.meta["step_combine"].result
        qr, kc, vc = oracle.cache_store(as_bits(b.meta["q_raw"]), as_bits(b.k), as_bits(b.v),
                                       as_bits(b.k_cache), as_bits(b.v_cache), b.slot_mapping.cpu().numpy(),
                                       b.positions.cpu().numpy(), b.cos_sin.cpu().numpy())
        ref = oracle.decode(qr, kc, vc, b.block_tables.cpu().numpy(), b.context_lens.cpu().numpy(), b.scale)
        e4[f"layer_{li}"] = _errors(y, ref)
    res["4_long_step"] = e4
    # 5: store then prefill; rows 0, 1, 63, 64, 255, 256, 510, 511 of each chunk, all heads
    b = W.chunked_prefill(device=device)
    qr, kc, vc = oracle.cache_store(as_bits(b.q), as_bits(b.k), as_bits(b.v), as_bits(b.k_cache),
                                   as_bits(b.v_cache), b.slot_mapping.cpu().numpy(),
                                   b.positions.cpu().numpy(), b.cos_sin.cpu().numpy())
    pa.cache_store(b.q, b.k, b.v, b.k_cache, b.v_cache, b.slot_mapping, b.positions, b.cos_sin)
    y = pa.prefill(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.query_start_loc,
                   b.scale, b.max_query_len)
    _sync()
    store_exact = bool(np.array_equal(as_bits(b.k_cache), kc) and np.array_equal(as_bits(b.v_cache), vc)
                       and np.array_equal(as_bits(b.q), qr))
    qsl = b.query_start_loc.cpu().numpy()
    lens = b.context_lens.cpu().numpy()
    bt = b.block_tables.cpu().numpy()
    rows, dec_lens, dec_tab = [], [], []
    for s in range(b.B):
        C, L = int(qsl[s + 1] - qsl[s]), int(lens[s])
        for i in (0, 1, 63, 64, 255, 256, C - 2, C - 1):
            rows.append(int(qsl[s]) + i)
            dec_lens.append(L - C + i + 1)
            dec_tab.append(bt[s])
    ref = oracle.decode(qr[rows], kc, vc, np.array(dec_tab), np.array(dec_lens), b.scale)
    res["5_chunked_prefill"] = {"store_bit_exact": store_exact,
                                "prefill_sampled_rows": _errors(y[torch.tensor(rows, device=device)], ref)}
    res["note"] = ("raw_*: |y - x| against the fp64 oracle; max_beyond_half_ulp / mean_vs_bf16_rne: "
                   "the reading used where |x| >= 4; rne_floor_mean: mean |bf16(x) - x|, what a "
                   "correctly rounded output already has")
    res["oracle_s"] = round(time.perf_counter() - t0, 1)
    return res


def load_traffic(kernel_file, kernel_name):
    """HBM bytes per launch measured with rocprofv3 counters, if taken on the current kernel."""
    path = os.path.join(ROOT, "profiles", "decode_partitions_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != kernel_source_hash(kernel_file) or rec.get("kernel") != kernel_name:
        return None
    return rec.get("hbm_bytes_per_launch")


def _pmc_per_dispatch(folder, counter, kernel):
    """Mean and count of one counter per dispatch of the kernels whose name contains
    `kernel`, from a rocprofv3 --pmc csv folder (rows summed per dispatch)."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    per = {}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter or kernel not in row.get("Kernel_Name", ""):
                    continue
                key = (fn, row.get("Dispatch_Id"))
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"{counter}: no dispatch of {kernel!r} in {folder}")
    vals = list(per.values())
    return sum(vals) / len(vals), len(vals)


def write_traffic(dirs, path=None):
    """profiles/decode_partitions_traffic.json from four counter passes: FETCH_SIZE and
    WRITE_SIZE of `--mode decode-kernel`, then of `--mode copy-calibration` (a 1 GiB
    device copy whose true bytes scale the counters)."""
    fetch_step, write_step, fetch_copy, write_copy = dirs
    fk, n = _pmc_per_dispatch(fetch_step, "FETCH_SIZE", STEP_KERNEL)
    wk, _ = _pmc_per_dispatch(write_step, "WRITE_SIZE", STEP_KERNEL)
    fc, _ = _pmc_per_dispatch(fetch_copy, "FETCH_SIZE", "__amd_rocclr_copyBuffer")
    wc, _ = _pmc_per_dispatch(write_copy, "WRITE_SIZE", "__amd_rocclr_copyBuffer")
    copy_bytes = 1 << 30
    fscale = copy_bytes / (fc * 1024)
    wscale = copy_bytes / (wc * 1024)
    rd = int(round(fk * 1024 * fscale))
    wr = int(round(wk * 1024 * wscale))
    b = W.long_decode_layer(0, device=torch.device("cpu"))
    rec = {
        "kernel": STEP_KERNEL,
        "source": "paged_kv_cache_240_amd/csrc/k_decode.hip",
        "source_sha256_16": kernel_source_hash("k_decode.hip"),
        "workload": "long-context decode step, one layer: B=16, L=8192, Hq=12, Hkv=2, D=128, partition 512 "
                    "(grid 16x2x16); the new token's RoPE + store folded in",
        "fetch_size_kib_per_launch": round(fk, 1),
        "write_size_kib_per_launch": round(wk, 1),
        "fetch_scale": round(fscale, 5),
        "write_scale": round(wscale, 5),
        "hbm_read_bytes_per_launch": rd,
        "hbm_write_bytes_per_launch": wr,
        "hbm_bytes_per_launch": rd + wr,
        "algorithmic_bytes_per_launch": step_kernel_bytes(b),
        "launches": n,
    }
    path = path or os.path.join(ROOT, "profiles", "decode_partitions_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=2)
        f.write("\n")
    print(json.dumps(rec))


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=W.LONG_LAYERS)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true")
    ap.add_argument("--mode", default="bench",
                    choices=["bench", "decode-kernel", "partition-kernel", "prefill-kernel",
                             "verify-kernel", "cb-cold", "copy-calibration", "write-traffic",
                             "issue-probe"])
    ap.add_argument("--pmc", nargs=4, metavar=("FETCH_STEP", "WRITE_STEP", "FETCH_COPY", "WRITE_COPY"),
                    help="write-traffic: the four rocprofv3 --pmc output folders")
    args = ap.parse_args()

    if args.mode == "write-traffic":
        write_traffic(args.pmc)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence or KV head with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    pa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.mode == "issue-probe":
        table = issue_mix_table(dev, verbose=True)
        print(json.dumps({"mode": "issue-probe", "iters": 4096,
                          "cus": torch.cuda.get_device_properties(dev).multi_processor_count, "rows": table}))
        return
    if args.mode == "copy-calibration":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        _sync()
        for _ in range(3):
            dst.copy_(src)
        _sync()
        print(json.dumps({"mode": "copy-calibration", "bytes_read": n, "bytes_written": n}))
        return
    if args.mode in ("decode-kernel", "partition-kernel"):
        Ls = make_long_layers(args.layers, dev)
        fn = fused_partitions if args.mode == "decode-kernel" else partitions
        _sync()
        for _ in range(3):
            for b in Ls:
                fn(b)
        _sync()
        nbytes = step_kernel_bytes(Ls[0]) if args.mode == "decode-kernel" else partition_kernel_bytes(Ls[0])
        print(json.dumps({"mode": args.mode, "launches": 3 * len(Ls), "bytes_per_launch": nbytes}))
        return
    if args.mode == "verify-kernel":
        # speculative verification as the bench times it: pa_decode_multi (5 queries per
        # sequence, the library's partition choice) over the 28 layer caches, 3 times
        layers = make_long_layers(args.layers, dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(2407)
        calls = []
        for b in layers:
            q = torch.randn((b.B, 5, b.Hq, b.D), generator=gen, device=dev).to(torch.bfloat16)
            calls.append(pa.prepare_decode_multi(q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                                                 b.scale, b.max_context_len, -1))
        _sync()
        for _ in range(3):
            for c in calls:
                c()
        _sync()
        print(json.dumps({"mode": "verify-kernel", "calls": 3 * len(calls)}))
        return
    if args.mode == "cb-cold":
        # the continuous-batching step, cold: 10 calls of pa_decode (library partition), then 10
        # of pa_decode_shared_prefix, each after a 1 GiB rewrite (for counter and trace runs)
        b = W.cb_step(device=dev)
        scrub = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        P = pa.decode_partition_size(b.B, b.Hkv, b.max_context_len)
        dec = pa.prepare_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.scale,
                                b.max_context_len, P)
        prefix = torch.zeros(b.B, dtype=torch.int32, device=dev)
        prefix[:32] = 2000
        sp = pa.prepare_decode_shared_prefix(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                                             torch.tensor([0, 32], dtype=torch.int32, device=dev), prefix,
                                             b.scale, b.max_context_len, 32, 2000,
                                             int((b.context_lens - prefix).max()), -1)
        for fn in (dec, sp):
            for _ in range(10):
                scrub.add_(1)
                _sync()
                fn()
                _sync()
        print(json.dumps({"mode": "cb-cold", "calls": [10, 10], "partition_size": P}))
        return
    if args.mode == "prefill-kernel":
        b = W.chunked_prefill(device=dev)
        pa.cache_store(b.q, b.k, b.v, b.k_cache, b.v_cache, b.slot_mapping, b.positions, b.cos_sin)
        pre = pa.prepare_prefill(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                                 b.query_start_loc, b.scale, b.max_query_len)
        for _ in range(20):
            pre()
        _sync()
        print(json.dumps({"mode": "prefill-kernel", "launches": 20, "flop_per_launch": prefill_flops(b)}))
        return

    layers = make_long_layers(args.layers, dev)
    _sync()
    t = run_long(layers, args.steps, args.warmup)
    step_ms = t["step_ms"]
    nl = len(layers)
    kv_step = sum(W.kv_bytes_logical(b.context_lens.cpu().numpy(), b.Hkv, b.D) for b in layers)
    value = kv_step / (step_ms * 1e-3) / 1e9
    launch_us = t["step_kernel_us"]         # the step's partition kernel, back to back
    launch_bytes = step_kernel_bytes(layers[0])
    achieved = launch_bytes / (launch_us * 1e-6) / 1e9
    part_bytes = partition_kernel_bytes(layers[0])
    traffic = load_traffic("k_decode.hip", STEP_KERNEL)
    line = {
        "metric": "paged-attn decode effective KV GB/s (% of HBM peak); us/call at Qwen2.5-1.5B shape",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "long-context flash-decode step: 28 layer caches x (RoPE+store of 16 new "
                        "tokens, split-K decode, LSE reduce) = pa_decode_step each (two launches)",
            "batch": layers[0].B, "context_len": layers[0].max_context_len,
            "q_heads": layers[0].Hq, "kv_heads": layers[0].Hkv, "head_dim": layers[0].D,
            "block_size": 16, "partition_size": LONG_P, "layers": nl,
            "kv_bytes_per_step": kv_step,
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "us_per_layer_call": round(step_ms * 1000 / nl, 2),
        "separate_calls": {
            "note": "pa_cache_store + pa_decode (partitions, reduce): three launches per layer, same results",
            "us_per_layer": round(t["separate_ms"] * 1000 / nl, 2),
            "kv_GBps": round(kv_step / (t["separate_ms"] * 1e-3) / 1e9, 1),
            "decode_only_us_per_layer": round(t["decode_only_ms"] * 1000 / nl, 2),
            "partition_kernel_avg_us": round(t["partition_us"], 3),
            "partition_kernel_GBps": round(part_bytes / (t["partition_us"] * 1e-6) / 1e9, 1),
            "partition_kernel_frac": round(part_bytes / (t["partition_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        },
        "roofline": {
            "kernel": STEP_KERNEL + " (split-K partitions with the RoPE + store of the new token)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": launch_bytes,
            "avg_launch_us": round(launch_us, 3),
            "launches_timed": args.steps * nl,
        },
    }
    if not args.no_context:
        line["context"] = run_context(dev)
        line["context"]["decode_step_graph"] = run_graph(layers, args.steps, args.warmup)
        line["context"]["spec_verify_16x8192"] = run_verify(layers, args.steps, args.warmup)
        line["context"]["block_copies"] = run_blocks(dev)
        line["context"]["layer_ops"] = run_layer_ops(dev)
        # the second configuration the bandwidth bar is judged on: the continuous-batching
        # step with cold caches, on unique K/V bytes, through the faster of its two paths
        cb, sp = line["context"]["cb_step_b64"], line["context"]["cb_step_b64_shared_prefix"]
        best = min((cb, "pa_decode"), (sp, "pa_decode_shared_prefix"),
                   key=lambda r: r[0]["per_call_cold"]["median_us"])
        line["cb_step_cold"] = {"entry_point": best[1], "us": best[0]["per_call_cold"]["median_us"],
                                "kv_unique_bytes": cb["kv_unique_bytes"],
                                "unique_frac_of_hbm_peak": best[0]["unique_frac_of_hbm_peak_cold"],
                                "protocol_floor": line["context"]["cold_protocol_floor"]}
        kv_layer = W.kv_bytes_logical(layers[0].context_lens.cpu().numpy(), layers[0].Hkv, layers[0].D)
        dc = line["device_ceilings"] = run_ceilings(dev, kv_layer)
        line["roofline"]["frac_of_measured_read"] = round(line["roofline"]["achieved"] / dc["read_ceiling_GBps"], 4)
        # the launch against a pure read of the same K/V bytes in one launch
        line["roofline"]["frac_of_one_layer_read"] = round(
            dc["gather_read_one_layer"]["us_per_launch"] / line["roofline"]["avg_launch_us"], 4)
    if not args.no_cpu_baseline:
        # the oracle leg: the CPU baseline, then the errors of every config against the oracle
        line["cpu_baseline"] = cpu_baseline(layers, args.cpu_budget)
        line["errors"] = oracle_errors(layers, dev)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line))


if __name__ == "__main__":
    main()
