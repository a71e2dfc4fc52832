#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on MI355X.

A step is one pass of the whole path over one batch of the Qwen3-0.6B-shaped
decode layer (256 sequences, 16 Q / 8 KV heads, head_dim 128, bf16, block
size 256, context lengths uniform in [128, 4096]): slot addressing of the new
tokens, the K/V scatter, the split-K decode pass and the log-sum-exp merge.
Inputs are resident in HBM before the timed region.  The JSON line reports
the whole step's algorithmic bytes per second as `value`, the decode pass's
own HBM roofline, and the CPU oracle timed on a bounded sample of the same
batch (whose outputs are also compared with the GPU's).  Extras: the
chunked-prefill workload (8 x (1024 cached + 256 new) tokens), and a mixed
serving step (256 decode rows + those 8 chunks) in one pa_attention_mixed
launch against separate decode and prefill launches, and decode steps of
several batch sizes replayed from HIP graphs against eager launches.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_bytes(w):
    """Algorithmic bytes of one decode call: live K/V rows once, q, out, live table entries."""
    elt = 2 if w.dtype == "bf16" else 4
    kv = int(w.seq_lens_k.sum()) * w.kv_bytes_per_token
    q = w.num_seqs * w.num_q_heads * w.head_dim * elt
    bt = int(np.ceil(w.seq_lens_k / w.block_size).sum()) * 4 + w.num_seqs * 4
    return kv, q, bt


def store_bytes(w):
    """New K/V rows read and written, plus slot-addressing metadata."""
    rows = w.num_new_tokens * w.kv_bytes_per_token
    meta = w.num_seqs * (4 + 4 + 4) + w.num_new_tokens * 4 * 2
    return 2 * rows + meta


def time_decode(args):
    import torch

    import paged_kv_cache_67_amd as pk
    from paged_kv_cache_67_amd import harness
    from workloads import make_config

    log("generating the Qwen3-0.6B decode batch (seed 67002)")
    w = make_config(2)
    dw = harness.DeviceWorkload(w, "cuda", partition_size=args.partition)
    dw.load_history()
    torch.cuda.synchronize()
    P = args.partition
    max_ctx = w.max_seqlen_k
    split = dw.workspace is not None
    log(f"sum(ctx)={int(w.seq_lens_k.sum())} partition={P} split={split}")

    def step(ev=None):
        dw.store_paged()  # a1 slot addressing + a2 scatter, one launch
        if ev is not None:
            ev[0].record()
        if split:
            pk.pa_decode_partitions(dw.out, dw.q, dw.k_cache, dw.v_cache, dw.block_table,
                                    dw.seq_lens_k, w.scale, max_ctx, P, dw.workspace)
            if ev is not None:
                ev[1].record()
            pk.pa_decode_merge(dw.out, dw.workspace, dw.seq_lens_k, w.num_kv_heads, max_ctx, P)
        else:
            dw.attention()
            if ev is not None:
                ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    k_ms = np.array([a.elapsed_time(b) for a, b in evs])
    log(f"step {ms_step * 1e3:.1f} us; decode pass mean {k_ms.mean() * 1e3:.1f} us "
        f"(median {np.median(k_ms) * 1e3:.1f})")

    # component times, each in a loop of its own (not part of the reported step time)
    comp = {}
    for name, fn in (("store_paged", dw.store_paged), ("slot_mapping", dw.slot_mapping),
                     ("store", dw.store)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(50):
            fn()
        b.record()
        torch.cuda.synchronize()
        comp[name + "_us"] = round(a.elapsed_time(b) / 50 * 1e3, 2)
    if split:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(50):
            pk.pa_decode_merge(dw.out, dw.workspace, dw.seq_lens_k, w.num_kv_heads, max_ctx, P)
        b.record()
        torch.cuda.synchronize()
        comp["merge_us"] = round(a.elapsed_time(b) / 50 * 1e3, 2)
    step()
    torch.cuda.synchronize()
    return w, dw, ms_step, float(k_ms.mean()), comp, P


def time_prefill(args):
    """pa_prefill_paged on the chunked-prefill workload.

    One launch per buffer set (6 sets, ~90 MB each, more than the 256 MB Infinity Cache) is
    captured in a HIP graph, and the graph is replayed between two events, so the time is
    the GPU's and not Python's launch rate.
    """
    import torch

    from paged_kv_cache_67_amd import harness
    from workloads import make_config

    log("prefill: generating 8 x (1024 cached + 256 new) tokens")
    w = make_config(4)
    sets = []
    for _ in range(6):
        dw = harness.DeviceWorkload(w, "cuda")
        dw.load_history()
        dw.slot_mapping()
        dw.store()
        sets.append(dw)
    torch.cuda.synchronize()
    L, lq = int(w.seq_lens_k[0]), int(w.new_lens[0])
    pairs = sum(L - lq + i + 1 for i in range(lq))  # causal-masked (query, key) pairs per head
    flops = 4.0 * w.head_dim * pairs * w.num_q_heads * w.num_seqs
    reps = max(10, args.steps // 5)

    def all_sets():
        for dw in sets:
            dw.attention()

    us = _graph_us(all_sets, reps) / len(sets)
    tf = flops / (us * 1e-6) / 1e12
    log(f"prefill {us:.1f} us per launch (graph replay), {tf:.1f} TFLOP/s")
    res = {"workload": w.name, "kernel": "pa_prefill_paged", "us_per_launch": round(us, 2),
           "launches_timed": 5 * reps * len(sets), "gflop": round(flops / 1e9, 3),
           "tflops": round(tf, 1), "peak_tflops": BF16_PEAK_TFLOPS,
           "frac_of_peak": round(tf / BF16_PEAK_TFLOPS, 4), "buffer_sets": len(sets),
           "timing": "HIP graph of one launch per buffer set, replayed between two events"}
    for dw in sets:  # the same inputs stored as fp16
        dw.k_cache, dw.v_cache = dw.k_cache.to(torch.float16), dw.v_cache.to(torch.float16)
        dw.q, dw.out = dw.q.to(torch.float16), dw.out.to(torch.float16)
    torch.cuda.synchronize()
    us16 = _graph_us(all_sets, reps) / len(sets)
    tf16 = flops / (us16 * 1e-6) / 1e12
    log(f"prefill fp16 {us16:.1f} us per launch, {tf16:.1f} TFLOP/s")
    res["f16"] = {"us_per_launch": round(us16, 2), "tflops": round(tf16, 1),
                  "frac_of_peak": round(tf16 / BF16_PEAK_TFLOPS, 4)}
    return res


def time_other_decode(args):
    """pa_decode (both passes), and the whole step (store + decode as two calls and as one
    pa_decode_append), on the two other decode workloads: Qwen2.5-0.5B shape
    (batch 64, 14 Q / 2 KV heads, d64, block 16) and the skewed long-context batch (one
    32768-token sequence and seven of 512).  Each fits in the 256 MB Infinity Cache, so
    the launches rotate over enough buffer sets (own pools) to touch about 1 GB, one
    launch per set captured in a HIP graph and replayed between two events."""
    import torch

    from paged_kv_cache_67_amd import harness
    from workloads import make_config

    res = {}
    for idx in (1, 3):
        w = make_config(idx)
        kv, q, bt = decode_bytes(w)
        nbytes = kv + 2 * q + bt
        pool = 2 * int(np.prod(w.pool_shape)) * (2 if w.dtype == "bf16" else 4)
        nsets = int(min(16, max(2, -(-(1 << 30) // pool))))
        sets = []
        for _ in range(nsets):
            dw = harness.DeviceWorkload(w, "cuda")
            dw.load_history()
            dw.slot_mapping()
            dw.store()
            sets.append(dw)
        torch.cuda.synchronize()

        def all_sets():
            for dw in sets:
                dw.attention()

        def two_calls():
            for dw in sets:
                dw.store_paged(write_slots=False)
                dw.attention()

        def one_call():
            for dw in sets:
                dw.attention_append()

        reps = max(10, args.steps // 10)
        us = _graph_us(all_sets, reps) / nsets
        us_two = _graph_us(two_calls, reps) / nsets
        us_one = _graph_us(one_call, reps) / nsets
        gbs = nbytes / (us * 1e-6) / 1e9
        log(f"{w.name}: pa_decode {us:.1f} us, {gbs:.1f} GB/s over {nsets} buffer sets; "
            f"step (store + decode) {us_two:.1f} us as two calls, {us_one:.1f} us as "
            f"pa_decode_append")
        res[w.name] = {"us_per_call": round(us, 2), "algorithmic_bytes": int(nbytes),
                       "GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                       "buffer_sets": nsets, "us_step_store_then_decode": round(us_two, 2),
                       "us_step_decode_append": round(us_one, 2)}
        del sets
        torch.cuda.empty_cache()
    res["timing"] = ("HIP graph of one pa_decode per buffer set, replayed between two events; "
                     "the steps: pa_store_kv_paged + pa_decode, and pa_decode_append")
    return res


def _graph_us(fn, reps, rounds=5):
    """Per-call GPU time of fn() (a few launches on the current stream), by HIP graph replay."""
    import torch
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / reps)
    return float(np.median(per))


def time_graphs(w, dw, args):
    """Decode steps (slot addressing + store + decode + merge: one pa_decode_append call) for
    the first n sequences of the decode batch: launched eagerly from Python against replayed
    from the HIP graph
    of their batch bucket, with the inputs staged into the graph's fixed buffers each step
    (one pa_copy_many launch) and with them already in place (bare replay)."""
    import torch

    import paged_kv_cache_67_amd as pk
    from paged_kv_cache_67_amd.graphs import GraphedDecode

    runner = GraphedDecode(dw.k_cache, dw.v_cache, w.num_q_heads, w.block_table.shape[1],
                           w.max_seqlen_k, w.scale, max_batch=w.num_seqs)
    steps = max(50, args.steps)
    res = {}
    for n in (1, 8, 64, w.num_seqs):
        q, kn, vn = dw.q[:n], dw.k_new[:n], dw.v_new[:n]
        bt, ctx = dw.block_table[:n], dw.seq_lens_k[:n]
        out = torch.empty_like(q)
        nbytes = pk.pa_decode_workspace_size(n, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                             w.max_seqlen_k, 0)
        ws = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device="cuda")

        def eager():  # the captured step, called directly on the caller's tensors
            pk.pa_decode_append(out, q, kn, vn, dw.k_cache, dw.v_cache, bt, ctx, w.scale,
                                max_context_len=w.max_seqlen_k, partition_size=0, workspace=ws)

        def graphed():
            runner.step(q, kn, vn, bt, ctx)

        graphed()  # captures the bucket and leaves these inputs in its buffers
        replay = runner.graphs[runner.bucket(n)].replay

        timing = {}
        for name, fn in (("eager", eager), ("graph", graphed), ("replay", replay)):
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            timing[name] = e0.elapsed_time(e1) * 1e3 / steps
        same = bool(torch.equal(out, runner.out[:n]))
        res[str(n)] = {"bucket": runner.bucket(n), "us_eager": round(timing["eager"], 2),
                       "us_graph_with_input_copies": round(timing["graph"], 2),
                       "us_graph_replay": round(timing["replay"], 2), "outputs_identical": same}
        log(f"graphs: batch {n}: eager {timing['eager']:.1f} us/step; graph (bucket "
            f"{runner.bucket(n)}) {timing['replay']:.1f} us/step with the inputs in its buffers, "
            f"{timing['graph']:.1f} with the inputs staged in by one pa_copy_many; identical {same}")
    return {"workload": w.name, "steps": steps, "by_batch": res,
            "timing": "events around back-to-back steps launched from Python"}


def time_f16_decode(w, dw, args):
    """pa_decode (both passes) on the decode batch with bf16 storage and with the same
    inputs converted to fp16 on the device (same shapes and bytes), by HIP graph replay."""
    import torch

    import paged_kv_cache_67_amd as pk

    nbytes = pk.pa_decode_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                         w.max_seqlen_k, 0)
    ws = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device="cuda")
    kv, q, bt = decode_bytes(w)
    res = {}
    reps = max(20, args.steps // 5)
    for name, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        kc, vc, qq = dw.k_cache.to(tdt), dw.v_cache.to(tdt), dw.q.to(tdt)
        out = torch.empty_like(qq)
        us = _graph_us(lambda: pk.pa_decode(out, qq, kc, vc, dw.block_table, dw.seq_lens_k, w.scale,
                                            max_context_len=w.max_seqlen_k, partition_size=0,
                                            workspace=ws), reps)
        gbs = (kv + 2 * q + bt) / (us * 1e-6) / 1e9
        res[name] = {"us_pa_decode": round(us, 2), "GBps": round(gbs, 1)}
        log(f"pa_decode {name}: {us:.1f} us, {gbs:.1f} GB/s (both passes, graph replay)")
        del kc, vc, qq, out
        torch.cuda.empty_cache()
    return {"workload": w.name, **res}


def time_copy_blocks(w, dw, args):
    """pa_copy_blocks over the decode pool: copy-on-write copies of n whole blocks (K and
    V), sources and destinations drawn without overlap, launched back to back between two
    events (a graph replay costs more than a small copy here).  Bytes moved: n x block
    bytes x 2 pools, read once and written once."""
    import torch

    import paged_kv_cache_67_amd as pk

    rng = np.random.default_rng(67007)
    block_bytes = w.block_size * w.num_kv_heads * w.head_dim * 2
    res = {}
    for n in sorted({16, min(256, w.num_blocks // 2), w.num_blocks // 2}):
        ids = rng.permutation(w.num_blocks)[:2 * n].astype(np.int32)
        pairs = torch.from_numpy(ids.reshape(2, n).T.copy()).cuda()
        reps = max(20, args.steps // 5)
        for _ in range(3):
            pk.pa_copy_blocks(dw.k_cache, dw.v_cache, pairs)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            pk.pa_copy_blocks(dw.k_cache, dw.v_cache, pairs)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        moved = 4 * n * block_bytes
        gbs = moved / (us * 1e-6) / 1e9
        res[str(n)] = {"us": round(us, 2), "bytes": moved, "GBps": round(gbs, 1)}
        log(f"pa_copy_blocks: {n} blocks of {block_bytes} B (K and V): {us:.1f} us, "
            f"{gbs:.1f} GB/s")
    return {"workload": w.name, "block_bytes": block_bytes, "by_pairs": res}


def time_mixed(args):
    """A mixed serving step: 256 decode rows + 8 chunks of 256 new tokens over 1024 cached,
    one pa_attention_mixed call against separate pa_decode + pa_prefill_paged calls on the
    same pool (both captured in HIP graphs and replayed)."""
    import torch

    import paged_kv_cache_67_amd as pk
    from paged_kv_cache_67_amd import harness
    from workloads import make_mixed

    log("mixed: generating 256 decode rows + 8 x (1024 cached + 256 new)")
    w = make_mixed()
    dw = harness.DeviceWorkload(w, "cuda")
    dw.load_history()
    dw.slot_mapping()
    dw.store()
    torch.cuda.synchronize()
    dec = np.flatnonzero(w.new_lens == 1)
    nd = len(dec)
    assert np.array_equal(dec, np.arange(nd)), "decode rows lead the batch"
    q_d, q_p = dw.q[:nd], dw.q[nd:]
    out_d, out_p = torch.empty_like(q_d), torch.empty_like(q_p)
    bt_d, bt_p = dw.block_table[:nd], dw.block_table[nd:]
    ctx_d = dw.seq_lens_k[:nd]
    cu_q_p = (dw.cu_q[nd:] - dw.cu_q[nd]).contiguous()
    cu_k_p = (dw.cu_k[nd:] - dw.cu_k[nd]).contiguous()
    max_ctx_d = int(w.seq_lens_k[:nd].max())
    nbytes = pk.pa_decode_workspace_size(nd, w.num_q_heads, w.num_kv_heads, w.head_dim, max_ctx_d, 0)
    ws_d = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device="cuda")
    max_q_p, max_k_p = int(w.new_lens[nd:].max()), int(w.seq_lens_k[nd:].max())

    def separate():
        pk.pa_decode(out_d, q_d, dw.k_cache, dw.v_cache, bt_d, ctx_d, w.scale,
                     max_context_len=max_ctx_d, partition_size=0, workspace=ws_d)
        pk.pa_prefill_paged(out_p, q_p, dw.k_cache, dw.v_cache, bt_p, cu_q_p, cu_k_p, max_q_p,
                            max_k_p, w.scale, causal=True)

    reps = max(20, args.steps // 5)
    us_mixed = _graph_us(dw.attention_mixed, reps)
    us_sep = _graph_us(separate, reps)
    us_dec = _graph_us(lambda: pk.pa_decode(out_d, q_d, dw.k_cache, dw.v_cache, bt_d, ctx_d,
                                            w.scale, max_context_len=max_ctx_d, partition_size=0,
                                            workspace=ws_d), reps)
    us_pf = _graph_us(lambda: pk.pa_prefill_paged(out_p, q_p, dw.k_cache, dw.v_cache, bt_p,
                                                   cu_q_p, cu_k_p, max_q_p, max_k_p, w.scale,
                                                   causal=True), reps)
    same = bool(torch.equal(dw.out[:nd], out_d) and torch.equal(dw.out[nd:], out_p))
    log(f"mixed step {us_mixed:.1f} us in one launch (+ merge); separate decode + prefill "
        f"{us_sep:.1f} us (decode {us_dec:.1f}, prefill {us_pf:.1f}); outputs identical: {same}")
    return {"workload": w.name, "decode_rows": nd, "prefill_chunks": int(w.num_seqs - nd),
            "us_mixed_launch": round(us_mixed, 2), "us_separate_launches": round(us_sep, 2),
            "us_decode_alone": round(us_dec, 2), "us_prefill_alone": round(us_pf, 2),
            "outputs_identical": same,
            "timing": "HIP graph of the call(s), replayed between two events"}


def _oracle_sample(w, kp, vp, gpu, seconds):
    """The oracle's slot mapping, store and fp64 decode, sequence by sequence in a fixed
    random order, until `seconds` have passed; returns what it did and its errors."""
    import oracle
    order = np.random.default_rng(0).permutation(w.num_seqs)
    done, errs, nbytes = [], [], 0
    wall0, cpu0 = time.perf_counter(), time.process_time()
    for b in order:
        sl = slice(int(b), int(b) + 1)
        slots = oracle.slot_mapping(w.block_table[sl], np.array([0, 1]), w.seq_lens_k[sl], w.block_size)
        oracle.store_kv(kp, vp, w.k_new[sl], w.v_new[sl], slots)
        out = oracle.decode(w.q[sl], kp, vp, w.block_table[sl], w.seq_lens_k[sl], w.scale, w.dtype)
        done.append(int(b))
        errs.append(np.abs(out[0] - gpu[b]))
        kv, q, bt = decode_bytes_sample(w, int(b))
        nbytes += kv + 2 * q + bt
        if time.perf_counter() - wall0 >= seconds:
            break
    wall = time.perf_counter() - wall0
    return done, np.stack(errs), nbytes, wall, time.process_time() - cpu0


def host_cpu():
    """The host's CPU facts: os.cpu_count(), the CPUs this process may run on, the model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"cpu_count": os.cpu_count(), "affinity": affinity, "cpu_model": model}


# Oracle worker processes share the parent's pools (fork, copy-on-write) and take whole
# sequences; they are started from a child process that has not touched the GPU.
_OW = {}


def _oracle_seq(b):
    import oracle
    w, kp, vp = _OW["w"], _OW["kp"], _OW["vp"]
    sl = slice(int(b), int(b) + 1)
    slots = oracle.slot_mapping(w.block_table[sl], np.array([0, 1]), w.seq_lens_k[sl], w.block_size)
    oracle.store_kv(kp, vp, w.k_new[sl], w.v_new[sl], slots)
    oracle.decode(w.q[sl], kp, vp, w.block_table[sl], w.seq_lens_k[sl], w.scale, w.dtype)
    kv, q, bt = decode_bytes_sample(w, int(b))
    return kv + 2 * q + bt


def _oracle_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        _OW["limit"] = threadpool_limits(limits=1)
    except ImportError:
        pass


def oracle_all_cores(seconds, workers):
    """Child-process leg: the oracle over the same batch's sequences (same random order) in
    `workers` processes of one thread each for about `seconds`; prints one JSON line."""
    import multiprocessing as mp

    import oracle
    from workloads import make_config
    w = make_config(2)
    kp, vp = w.empty_pool(), w.empty_pool()
    oracle.store_kv(kp, vp, w.k_hist, w.v_hist,
                    oracle.slot_mapping(w.block_table, w.cu_seqlens_hist, w.hist_lens, w.block_size))
    _OW.update(w=w, kp=kp, vp=vp)
    # the batch's sequences in the parent's random order, repeated so that the pool stays
    # busy for the whole interval (a repeat rewrites the same rows and recomputes the rows)
    order = [int(b) for b in np.random.default_rng(0).permutation(w.num_seqs)] * 200
    done = nbytes = 0
    with mp.get_context("fork").Pool(workers, initializer=_oracle_worker_init) as pool:
        t0 = time.perf_counter()
        for nb in pool.imap_unordered(_oracle_seq, order):
            done += 1
            nbytes += nb
            if time.perf_counter() - t0 >= seconds:
                break
        wall = time.perf_counter() - t0
        pool.terminate()
    print(json.dumps({"done": done, "bytes": int(nbytes), "wall": wall}), flush=True)


def cpu_baseline(w, dw, seconds):
    """Time the CPU oracle on bounded samples of the same batch: in this process on one
    thread (its outputs are compared with the GPU rows), then in a child process over one
    single-thread worker per available CPU (at most 16)."""
    import subprocess

    import oracle
    from paged_kv_cache_67_amd import harness

    log("cpu baseline: building oracle pools (not timed)")
    kp, vp = w.empty_pool(), w.empty_pool()
    oracle.store_kv(kp, vp, w.k_hist, w.v_hist,
                    oracle.slot_mapping(w.block_table, w.cu_seqlens_hist, w.hist_lens, w.block_size))
    gpu = oracle.to_f64(harness.from_device(dw.out), w.dtype)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            done, err, nbytes, wall, cpu = _oracle_sample(w, kp, vp, gpu, seconds)
    except ImportError:
        done, err, nbytes, wall, cpu = _oracle_sample(w, kp, vp, gpu, seconds)
    log(f"cpu baseline, one thread: {len(done)} sequences in {wall:.1f} s; parity max "
        f"{err.max():.2e} mean {err.mean():.2e}")
    facts = host_cpu()
    one = {"value": round(nbytes / wall / 1e9, 4), "unit": "GB/s", "cores": 1,
           "sample": f"{len(done)} of {w.num_seqs} sequences (random order, seed 0): slot "
                     f"mapping, store and fp64 decode, {wall:.1f} s wall",
           "busy_ratio": round(cpu / wall, 2)}
    workers = max(1, min(16, facts["affinity"] or 1))
    base = None
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-leg",
                        str(seconds), str(workers)], capture_output=True, text=True,
                       timeout=seconds + 240)
    if r.returncode == 0 and r.stdout.strip():
        leg = json.loads(r.stdout.strip().splitlines()[-1])
        log(f"cpu baseline, {workers} processes: {leg['done']} sequences in {leg['wall']:.1f} s")
        base = {"value": round(leg["bytes"] / leg["wall"] / 1e9, 4), "unit": "GB/s",
                "cores": workers, "kind": "oracle",
                "sample": f"{leg['done']} sequence decodes (the batch's {w.num_seqs} in the same "
                          f"order, repeated), {workers} single-thread processes, "
                          f"{leg['wall']:.1f} s wall",
                **facts, "threads_per_process": 1, "one_thread": one}
    else:
        log(f"cpu baseline: all-cores leg failed ({r.returncode}): {r.stderr[-500:]}")
        base = {**one, "kind": "oracle", **facts, "note": "all-cores leg failed; one thread only"}
    return (base,
            {"sample_seqs": len(done), "max_err": float(err.max()), "mean_err": float(err.mean()),
             "ok": bool(err.max() <= 2e-2 and err.mean() <= 2e-3 and np.all(np.isfinite(gpu)))})


def time_ceiling(args):
    """Read ceiling of the decode pass: pa_read_ceiling over two pools of 4096 blocks in the
    decode's layout (block 256 x 8 KV heads x 128, bf16: 512 KiB per block and pool, 4 GiB in
    all, 16 times the last-level cache), blocks in random order (the decode's pattern) and in
    address order, at several grid sizes; median of 5 rounds of 10 launches between events."""
    import torch

    import paged_kv_cache_67_amd as pk

    nb, bs, hkv, d = 4096, 256, 8, 128
    kc = torch.empty((nb, bs, hkv, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    kc.view(torch.int16).random_()
    vc.view(torch.int16).random_()
    nbytes = 2 * kc.numel() * kc.element_size()
    orders = {"random_blocks": torch.from_numpy(
        np.random.default_rng(67009).permutation(nb).astype(np.int32)).cuda(),
        "address_order": torch.arange(nb, dtype=torch.int32, device="cuda")}
    res = {"bytes_per_launch": nbytes}
    for name, ids in orders.items():
        by = {}
        for grid in (128, 192, 256, 512, 1024):
            sink = torch.empty(8 * grid, dtype=torch.int32, device="cuda")
            for _ in range(2):
                pk.pa_read_ceiling(kc, vc, ids, grid, sink)
            torch.cuda.synchronize()
            per = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(10):
                    pk.pa_read_ceiling(kc, vc, ids, grid, sink)
                e1.record()
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) * 1e3 / 10)
            us = float(np.median(per))
            by[str(grid)] = round(nbytes / (us * 1e-6) / 1e9, 1)
        best = max(by, key=lambda k: by[k])
        res[name] = {"GBps": by[best], "grid": int(best), "by_grid_GBps": by}
        log(f"read ceiling ({name}): {by[best]:.0f} GB/s at {best} workgroups; {by}")
    del kc, vc
    torch.cuda.empty_cache()
    return res


def time_tp_shard(args):
    """One TP=2 rank's share of the decode batch (8 Q / 4 KV heads, the same contexts):
    pa_decode (both passes) by HIP graph replay."""
    import torch

    from paged_kv_cache_67_amd import harness
    from workloads import make_tp_shard

    w = make_tp_shard(2)
    dw = harness.DeviceWorkload(w, "cuda")
    dw.load_history()
    dw.slot_mapping()
    dw.store()
    torch.cuda.synchronize()
    kv, q, bt = decode_bytes(w)
    nbytes = kv + 2 * q + bt
    us = _graph_us(dw.attention, max(20, args.steps // 5))
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"{w.name}: pa_decode {us:.1f} us, {gbs:.1f} GB/s")
    del dw
    torch.cuda.empty_cache()
    return {"workload": w.name, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
            "us_per_call": round(us, 2), "algorithmic_bytes": int(nbytes), "GBps": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "timing": "HIP graph of one pa_decode, replayed between two events"}


PROFILE = os.path.join(ROOT, "profiles", "decode_qwen3-0.6b-b256.md")
# The sources the decode first pass is compiled from, hashed in this order.
DECODE_SRCS = [os.path.join(ROOT, "paged_kv_cache_67_amd", "csrc", f)
               for f in ("pa_decode.hip", "pa_decode_dev.h", "pa_decode_plan.h", "pa_internal.h")]


def measured_traffic():
    """HBM bytes per first-pass launch from the committed counter summary.

    The summary records the sha256 of the decode sources it was measured on
    (DECODE_SRCS concatenated); if the kernel has changed since, the figure no
    longer applies (None).
    """
    import hashlib
    import re
    try:
        text = open(PROFILE).read()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch=(\d+) source_sha256=([0-9a-f]{64})", text)
    if not m:
        return None
    h = hashlib.sha256()
    for path in DECODE_SRCS:
        h.update(open(path, "rb").read())
    src = h.hexdigest()
    return int(m.group(1)) if m.group(2) == src else None


def copy_calibration():
    """A 1 GiB device-to-device copy: known bytes for scaling the FETCH/WRITE counters."""
    import torch
    x = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log("copy calibration: 3 x 1 GiB copies done")


def decode_bytes_sample(w, b):
    elt = 2 if w.dtype == "bf16" else 4
    L = int(w.seq_lens_k[b])
    return (L * w.kv_bytes_per_token, w.num_q_heads * w.head_dim * elt,
            int(math.ceil(L / w.block_size)) * 4 + 4)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-mixed", action="store_true")
    ap.add_argument("--no-graphs", action="store_true")
    ap.add_argument("--no-f16", action="store_true")
    ap.add_argument("--no-other-decode", action="store_true",
                    help="skip the Qwen2.5-0.5B and skewed long-context decode timings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="finish with 3 x 1 GiB device copies (counter calibration runs)")
    ap.add_argument("--partition", type=int, default=0,
                    help="decode split: 0 balanced (default), -1 single pass, P fixed partitions")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-tp-shard", action="store_true")
    ap.add_argument("--oracle-leg", nargs=2, metavar=("SECONDS", "WORKERS"),
                    help=argparse.SUPPRESS)  # internal: the all-cores oracle leg (no GPU)
    args = ap.parse_args()
    if args.oracle_leg:
        oracle_all_cores(float(args.oracle_leg[0]), int(args.oracle_leg[1]))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the paged-attention path needs no collective (a "
              "multi-GPU run shards sequences or KV heads, each GPU running this same step on "
              "its share); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import paged_kv_cache_67_amd as pk
    pk.lib()  # fails loudly if libpa.so is not built

    w, dw, ms_step, pass_ms, comp, P = time_decode(args)
    kv, q, bt = decode_bytes(w)
    pass_bytes = kv + q + bt                       # what the split-K pass must read
    step_bytes = kv + 2 * q + bt + store_bytes(w)  # + out, + the scatter and its metadata
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = pass_bytes / (pass_ms * 1e-3) / 1e9

    result = {
        "metric": "paged decode µs/step + achieved HBM GB/s (% of peak), Qwen3-0.6B shape",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.num_seqs, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size,
            "context_lens": "uniform [128, 4096], seed 67002",
            "sum_context_tokens": int(w.seq_lens_k.sum()),
            "split": {0: "balanced split-K", -1: "single pass"}.get(P, f"fixed {P}-token partitions"),
            "step": "pa_store_kv_paged (slot addressing + store) + pa_decode_partitions + pa_decode_merge",
            "step_bytes": int(step_bytes),
        },
        "roofline": {
            "kernel": "decode first pass (pa_decode_partitions)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "algorithmic_bytes": int(pass_bytes),
            "avg_launch_us": round(pass_ms * 1e3, 2),
        },
        "components_us": comp,
    }
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline(w, dw, args.cpu_seconds)
        result["cpu_baseline"] = base
        result["parity"] = parity
        if not parity["ok"]:
            result["value"] = None
            result["note"] = "parity failed on the oracle sample: no time reported"
    else:
        result["cpu_baseline"] = None
    extra = {}
    if not args.no_ceiling:
        ceil = time_ceiling(args)
        extra["read_ceiling"] = ceil
        c = ceil["random_blocks"]["GBps"]
        result["roofline"]["ceiling"] = {
            "GBps": c, "kind": "pa_read_ceiling: the decode's loads over random 512 KiB blocks",
            "frac": round(achieved / c, 4)}
    if not args.no_f16:
        extra["f16_decode"] = time_f16_decode(w, dw, args)
    if not args.no_graphs:
        extra["graphs"] = time_graphs(w, dw, args)
    extra["copy_blocks"] = time_copy_blocks(w, dw, args)  # overwrites pool blocks: runs last
    del dw
    torch.cuda.empty_cache()
    if not args.no_prefill:
        extra["prefill"] = time_prefill(args)
        torch.cuda.empty_cache()
    if not args.no_other_decode:
        extra["other_decode"] = time_other_decode(args)
        torch.cuda.empty_cache()
    if not args.no_mixed:
        extra["mixed"] = time_mixed(args)
        torch.cuda.empty_cache()
    if not args.no_tp_shard:
        extra["tp2_rank"] = time_tp_shard(args)
    if extra:
        result["extra"] = extra
    if args.copy_calibration:
        copy_calibration()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
