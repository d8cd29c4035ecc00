#!/usr/bin/env python3
"""Paged single-token decode attention on one MI355X: µs/step and achieved HBM GB/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads main|all]

A step is one decode call (split-KV partition kernel + log-sum-exp combine)
over one batch, launched through the C ABI. Steps are captured in one HIP
graph and replayed; every step reads the next cold copy of the paged pool
(copies totalling >= 1 GiB of touched pages, so the 256 MB last-level cache
cannot serve them). Inputs are resident in HBM before the timed region.

The JSON line reports the wide serving batch: 64 sequences with KV lengths
drawn uniformly from [2048, 65536], page 832, split-KV partitions of 4096
tokens and the log-sum-exp combine -- the largest decode workload, about
9.4 GB of K/V per step. The other decode workloads are reported in
"workloads", each with its own roofline block. "roofline" is the split kernel
alone, timed with HIP events around a graph of back-to-back launches on the
stream it runs on. "cpu_baseline" is the fp64 oracle timed on this host's
cores on the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MAIN = "wide_64seq_b832_p4096"
EXTRA = ["tiny_l1024_b64", "long_l8192_b832", "long_l16384_b832", "long_l32768_b832",
         "ab_l32768_b784", "ab_l32768_b832", "batched_8seq_t131072_b832",
         "wide_64seq_b832_auto", "serving_1024seq_b832"]
PEAK_GBPS = 8000.0            # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
COLD_BYTES = 1 << 30          # touched bytes the replicas must span
# KV appends timed next to decode: (new tokens, page size). One new token for
# each sequence of the 64-sequence batch, and one 32768-token prefill chunk.
APPEND_WORKLOADS = {"append_decode_64tok_b832": (64, 832),
                    "append_chunk_32768tok_b832": (32768, 832)}
# Decode times the page832 article reports for its page-contiguous Triton kernel
# on a Hygon DCU (gfx936), same head layout, q = 1, page 832 (context only).
PAGES_US = {"long_l8192_b832": 80.010, "long_l16384_b832": 122.411,
            "long_l32768_b832": 278.832}
# the decode kernels and the host plan that picks their variants: the recorded
# traffic holds only while both are unchanged
KERNEL_SRC = [os.path.join(ROOT, "paged_kv_cache_36_amd", "csrc", f)
              for f in ("pkv_kernels.hip", "pkv_plan.cpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sha():
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measure(name, steps, warmup, torch, pkv, synth, **case_overrides):
    case = synth.make_case(name, device="cuda", **case_overrides)
    nbytes = case.algorithmic_bytes()
    copies = max(1, math.ceil(COLD_BYTES / nbytes))
    if copies > 1:
        k_big, v_big, tables = synth.replicate(case, copies)
    else:
        k_big, v_big, tables = case.k_cache, case.v_cache, case.block_table[None]
    max_len = case.max_seq_len
    prm = pkv.make_params(case.q, k_big, v_big, tables[0], case.block_size, case.scale,
                          max_len, case.partition_tokens)
    plan = pkv.plan(prm)
    out = torch.empty_like(case.q)
    ws_bytes = max(pkv.workspace_bytes(prm), 256)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    n_parts = plan["num_partitions"]
    rows = case.num_seqs * 24 * n_parts
    o_part = torch.empty((rows * 256,), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((rows,), dtype=torch.float32, device="cuda")

    def step(i):
        pkv.decode(case.q, k_big, v_big, tables[i % copies], case.seq_lens, case.block_size,
                   case.scale, max_seq_len=max_len, partition_tokens=case.partition_tokens,
                   out=out, workspace=ws)

    balanced = bool(plan["balanced"])

    def split_only(i):
        # the split launch pkv_decode makes for this plan, alone
        if balanced:
            pkv.split_balanced(prm, case.q, k_big, v_big, tables[i % copies], case.seq_lens, ws)
        else:
            pkv.split(prm, case.q, k_big, v_big, tables[i % copies], case.seq_lens, o_part,
                      lse_part)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
    torch.cuda.synchronize()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i)
        return g

    g_step = capture(step, steps)
    g_split = capture(split_only, steps)
    g_warm = capture(lambda i: step(0), steps)

    def timed(graph):
        """Replay on `stream`, events on the same stream; returns (wall s, gpu ms)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            e0.record(stream)
            graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1)

    for g in (g_step, g_split, g_warm):   # first replays off the clock
        timed(g)

    # timed region: exactly `steps` steps, synchronized on both sides
    wall_s, gpu_ms = timed(g_step)
    # the split kernel alone, back to back, HIP events on its stream
    _, split_ms = timed(g_split)
    split_us = split_ms * 1e3 / steps
    # warm: the same step repeated on one copy (cache-resident where it fits)
    _, warm_ms = timed(g_warm)
    warm_us = warm_ms * 1e3 / steps
    if gpu_ms > wall_s * 1e3 * 1.01 or nbytes / (split_us * 1e-6) > 2 * PEAK_GBPS * 1e9:
        raise RuntimeError(f"implausible timing for {name}: wall {wall_s * 1e3:.3f} ms, "
                           f"events {gpu_ms:.3f} ms, split {split_us:.3f} us")

    us_step = wall_s * 1e6 / steps
    # after the timed region: five more replays of the same graph, their median
    # (the repeat protocol of the decode microbenchmark; outside the K timed steps)
    repeats = sorted(timed(g_step)[0] * 1e6 / steps for _ in range(5))
    kernel = "balanced_split_kernel" if balanced else "split_decode_kernel"
    res = {
        "workload": name, "num_seqs": case.num_seqs, "total_tokens": sum(case.lens),
        "max_seq_len": max_len, "block_size": case.block_size,
        "split": "balanced" if balanced else "fixed",
        "partition_tokens": 0 if balanced else plan["partition_tokens"],
        "num_partitions": 0 if balanced else n_parts,
        "split_workgroups": plan["split_workgroups"], "cold_copies": copies, "steps": steps,
        "algorithmic_bytes": nbytes,
        "us_per_step": round(us_step, 3),
        "us_per_step_median5": round(repeats[2], 3),
        "gpu_us_per_step": round(gpu_ms * 1e3 / steps, 3),
        "split_us": round(split_us, 3),
        "warm_us_per_step": round(warm_us, 3),
        "gbps_step": round(nbytes / (us_step * 1e-6) / 1e9, 1),
        "gbps_split": round(nbytes / (split_us * 1e-6) / 1e9, 1),
    }
    res["frac_peak_step"] = round(res["gbps_step"] / PEAK_GBPS, 4)
    res["frac_peak_split"] = round(res["gbps_split"] / PEAK_GBPS, 4)
    res["roofline"] = {
        "bound": "hbm", "kernel": kernel,
        "achieved": res["gbps_split"], "peak": PEAK_GBPS, "unit": "GB/s",
        "frac": res["frac_peak_split"], "traffic": traffic_for(res),
        "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": res["split_us"],
    }
    if name in PAGES_US:
        res["pages_dcu_us"] = PAGES_US[name]
    log(json.dumps(res))
    del g_step, g_split, g_warm, k_big, v_big, tables, case
    torch.cuda.empty_cache()
    return res


def measure_append(name, num_tokens, block_size, steps, warmup, torch, pkv, synth):
    """KV append of `num_tokens` new tokens (K and V, 4 KV heads x 256) into a
    page-832 cache: each step writes the next cold copy of the rows into its own
    pages. Algorithmic bytes: 2 KiB read + 2 KiB written per token for each of
    K and V."""
    nbytes = num_tokens * 4 * 256 * 2 * 2 * 2
    copies = max(1, min(64, math.ceil(COLD_BYTES / nbytes)))
    rows_k, rows_v, slots, pages = synth.append_bench_inputs(num_tokens, block_size, copies,
                                                             seed=77)
    kc = torch.empty((pages, block_size, 4, 256), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    stream = torch.cuda.Stream()

    def step(i):
        c = i % copies
        pkv.append(rows_k[c], rows_v[c], slots[c], kc, vc)

    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            step(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        g.replay()
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    # the library moves two tokens per wave from 2048 tokens of 4 x 256 rows
    kernel = "append_pairs_kernel" if num_tokens >= 2048 else "append_kernel"
    res = {"workload": name, "kernel": kernel, "tokens": num_tokens,
           "block_size": block_size, "cold_copies": copies, "steps": steps,
           "algorithmic_bytes": nbytes, "us_per_append": round(us, 3),
           "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
           "frac_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_GBPS, 4)}
    log(json.dumps(res))
    del g, rows_k, rows_v, slots, kc, vc
    torch.cuda.empty_cache()
    return res


def prefill_flops(num_q, seq_len, hq=24, d=256):
    """Algorithmic flops of causal tail-Q prefill: every (query, visible key,
    head) pair costs 2 d for q.k and 2 d for p.v."""
    pairs = num_q * (seq_len - num_q) + num_q * (num_q + 1) // 2
    return pairs * hq * 4 * d


def measure_prefill(name, steps, warmup, torch, pkv, synth):
    """Tail-Q prefill of one workload, graph-replayed; bf16 MFMA-bound."""
    case, q_new = synth.make_prefill_case(name, device="cuda")
    nq, length = q_new.shape[0], case.lens[0]
    flops = prefill_flops(nq, length)
    out = torch.empty_like(q_new)
    bt = case.block_table[0]
    stream = torch.cuda.Stream()
    prm = pkv.prefill_params(q_new, case.k_cache, case.v_cache, bt, length, case.block_size,
                             case.scale)
    splits = pkv.prefill_key_splits(prm)
    ws_bytes = pkv.prefill_workspace_bytes(prm)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None

    def step(i):
        pkv.prefill(q_new, case.k_cache, case.v_cache, bt, length, case.block_size, case.scale,
                    out=out, workspace=ws)

    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            step(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        g.replay()
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    tflops = flops / (us * 1e-6) / 1e12
    kernel = "prefill_kernel" if splits == 1 else "prefill_kernel+prefill_combine_kernel"
    res = {"workload": name, "kernel": kernel, "num_q": nq, "seq_len": length,
           "block_size": case.block_size, "key_splits": splits, "steps": steps,
           "algorithmic_flops": flops,
           "us_per_call": round(us, 2), "tflops": round(tflops, 1),
           "frac_peak_bf16_mfma": round(tflops / PEAK_BF16_TFLOPS, 4)}
    log(json.dumps(res))
    del g, case, q_new, out, ws
    torch.cuda.empty_cache()
    return res


def measure_compress(name, steps, warmup, torch, pkv, synth):
    """Paged window compression of one of the 12 shapes, graph-replayed over
    cold replicas of the state cache. Algorithmic bytes: every window row read
    once (4 KiB: 512 fp32 values + 512 fp32 scores) plus the fp32 output.
    Also times the finalizer alone (RMSNorm, INT8/RoPE packing, KV-page
    scatter of every output), the whole operator as two calls and as one
    call (pkv_compress_pack, the finalizer fused into the last kernel)."""
    case = synth.make_compress_case(name, device="cuda")
    n, c = case.num_outputs, case.compress_ratio
    rows = sum(min(int(p) + 1, c) for p in case.positions[case.boundaries].tolist())
    nbytes = rows * 2 * case.head_dim * 4 + n * case.head_dim * 4
    copies = max(1, math.ceil(COLD_BYTES / nbytes))
    caches = [case.state_cache] + [case.state_cache.clone() for _ in range(copies - 1)]
    prm = pkv.compress_params(case.state_cache, case.token_to_req, case.boundaries,
                              case.block_table, c)
    splits = pkv.compress_splits(prm)
    out = torch.empty((n, case.head_dim), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(pkv.compress_workspace_bytes(prm), 256), dtype=torch.uint8,
                     device="cuda")
    # the finalizer's inputs: fp32 weight and cos/sin table, every output
    # packed into its own slot of a shuffled KV page pool
    gen = torch.Generator().manual_seed(7)
    t = case.positions.shape[0]
    weight = (torch.rand(case.head_dim, generator=gen) + 0.5).cuda()
    rows = int(case.positions.max()) + 1
    th = torch.rand((rows, 32), generator=gen) * 6.283
    cos_sin = torch.cat([torch.cos(th), torch.sin(th)], 1).cuda()
    kv_pages = (n + 63) // 64 + 1
    slots = torch.full((t,), -1, dtype=torch.int64)
    slots[case.boundaries.cpu()] = torch.randperm(kv_pages * 64, generator=gen)[:n]
    slots = slots.cuda()
    kv = torch.zeros((kv_pages, pkv.KV_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()

    def step(i):
        pkv.compress(caches[i % copies], case.token_to_req, case.positions, case.boundaries,
                     case.block_table, c, out=out, workspace=ws)

    def finalize(i):
        pkv.compress_finalize(out, case.positions, case.boundaries, weight, cos_sin, slots, kv, c)

    def operator(i):
        step(i)
        finalize(i)

    def pack(i):
        # the same operator in one call: the finalizer inside the last kernel
        pkv.compress_pack(caches[i % copies], case.token_to_req, case.positions, case.boundaries,
                          case.block_table, c, weight, cos_sin, slots, kv, workspace=ws)

    def timed(fn):
        with torch.cuda.stream(stream):
            for i in range(warmup):
                fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                fn(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            g.replay()
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    us = timed(step)
    us_fin = timed(finalize)
    us_op = timed(operator)
    us_pack = timed(pack)
    gbps = nbytes / (us * 1e-6) / 1e9
    res = {"workload": name, "kernel": "compress_split_kernel" + ("+compress_combine_kernel"
                                                                 if splits > 1 else ""),
           "num_outputs": n, "compress_ratio": c, "tokens": int(t),
           "num_splits": splits, "workgroups": n * splits, "cold_copies": copies,
           "steps": steps, "algorithmic_bytes": nbytes, "us_per_call": round(us, 3),
           "gbps": round(gbps, 1), "frac_peak": round(gbps / PEAK_GBPS, 4),
           "finalize_us": round(us_fin, 3), "operator_us": round(us_op, 3),
           "pack_us": round(us_pack, 3)}
    log(json.dumps(res))
    del caches, case, out, ws, kv
    torch.cuda.empty_cache()
    return res


def read_probe(torch, pkv, reps=20):
    """Streaming read of 2 GiB of random bytes. The rate depends on how long the
    memory has been streaming: on an idle GPU it reads about 5 % faster than
    after a few seconds of sustained reads (the state the timed decode steps run
    in, after their off-the-clock replays); the contents of the bytes make no
    measurable difference."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    buf = torch.randint(0, 256, (2 << 30,), dtype=torch.uint8, device="cuda", generator=gen)
    sink = torch.empty(pkv.api.probe_sink_floats(), dtype=torch.float32, device="cuda")
    for _ in range(3):
        pkv.probe_read(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        pkv.probe_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbps = buf.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return round(gbps, 1)


def copy_probe(torch, pkv, nbytes=1 << 30, reps=5):
    """A plain copy kernel of known size (the counter calibration reference)."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        pkv.probe_copy(dst, src)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} launches of {nbytes} bytes")


def host_cpu():
    """Usable CPUs of this process and the CPU model string."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def _host_bits(t):
    import numpy as np
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def cpu_baseline(name=MAIN, budget_s=30.0):
    """The fp64 oracle (as it stands) on the host, one thread, on one step of
    `name`: sequence by sequence, the bf16 -> fp64 conversion of its q, K and
    V and the oracle's decode are timed; drawing the data and copying it to
    the host are not. Sequences are taken in order until the step is done or
    the budget is spent; a partial step is scaled by tokens."""
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import decode as od
    from paged_kv_cache_36_amd import synth

    case = synth.make_case(name, device="cuda")
    q_bits = _host_bits(case.q)
    total = sum(case.lens)
    el = 0.0
    done_tok = done_seq = 0
    with threadpool_limits(limits=1):
        for s in range(case.num_seqs):
            k_bits, v_bits = _host_bits(case.keys(s)), _host_bits(case.values(s))
            t0 = time.perf_counter()
            od.decode_batch(od.bf16_bits_to_f64(q_bits[s:s + 1]), [od.bf16_bits_to_f64(k_bits)],
                            [od.bf16_bits_to_f64(v_bits)], case.scale)
            el += time.perf_counter() - t0
            done_tok += case.lens[s]
            done_seq += 1
            if el >= budget_s:
                break
    del case
    torch.cuda.empty_cache()
    us = el * 1e6 * total / done_tok
    ncpu, model = host_cpu()
    what = ("one whole step" if done_seq == len(q_bits) else
            f"{done_seq} of {len(q_bits)} sequences ({done_tok} of {total} tokens), scaled by tokens")
    return {"value": round(us, 1), "unit": "us/step", "cores": 1, "kind": "oracle",
            "host_cpus": ncpu, "cpu_model": model,
            "sample": f"{what} of {name} ({len(q_bits)} sequences, {total} tokens, 24 heads; "
                      f"fp64 two-pass numpy, one thread, bf16->fp64 conversion timed), "
                      f"{el:.1f} s timed"}


def cpu_baseline_parallel(name=MAIN, budget_s=10.0):
    """The same oracle (unchanged) run in parallel over (sequence, KV head) on the
    host's cores: each task converts its slice from bf16 and calls the oracle's
    decode for the 6 query heads of one KV head. numpy releases the GIL inside
    its loops, so threads run concurrently; BLAS is held to one thread each.
    Whole steps; the host copy of the data is made once, outside the timing."""
    from concurrent.futures import ThreadPoolExecutor

    import torch
    from threadpoolctl import threadpool_limits

    from oracle import decode as od
    from paged_kv_cache_36_amd import synth

    case = synth.make_case(name, device="cuda")
    q_bits = _host_bits(case.q)
    kv = [(_host_bits(case.keys(s)), _host_bits(case.values(s))) for s in range(case.num_seqs)]
    scale = case.scale
    nseq, total = case.num_seqs, sum(case.lens)
    del case
    torch.cuda.empty_cache()
    tasks = [(s, g) for s in range(nseq) for g in range(4)]
    ncpu, model = host_cpu()
    workers = min(ncpu, len(tasks))

    def task(sg):
        s, g = sg
        q = od.bf16_bits_to_f64(q_bits[s, 6 * g:6 * g + 6])
        k = od.bf16_bits_to_f64(kv[s][0][:, g:g + 1])
        v = od.bf16_bits_to_f64(kv[s][1][:, g:g + 1])
        return od.attention_decode(q, k, v, scale)

    n = 0
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(task, tasks))
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    us = el * 1e6 / n
    return {"value": round(us, 1), "unit": "us/step", "cores": workers, "kind": "oracle",
            "host_cpus": ncpu, "cpu_model": model,
            "sample": f"{n} whole steps of {name} ({nseq} sequences, {total} tokens), "
                      f"{workers} threads over its {len(tasks)} (sequence, KV head) pairs, "
                      f"{el:.1f} s"}


def cpu_baseline_rows(budget_s=3.0):
    """The oracles of the rows built beside decode, as they stand, timed on the
    host with one BLAS thread on bounded samples of their bench workloads and
    scaled to one call: prefill on sampled query rows of q = 4096, L = 32768;
    the append scatter on a slice of the 32768-token chunk; the compression
    and its finalizer on sampled outputs of 8 x 16384 tokens at C = 128.
    Input conversion to fp64 is inside each timed region."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import append as oa
    from oracle import compress as oc
    from oracle import decode as od
    from oracle import prefill as opf
    from paged_kv_cache_36_amd import synth

    def timed(fn):
        n = 0
        t0 = time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                return el / n, n, el

    out = {}
    ncpu, model = host_cpu()
    with threadpool_limits(limits=1):
        # prefill: 4 query rows (all 24 heads) per call of the oracle
        case, q_new = synth.make_prefill_case("prefill_q4096_l32768_b832", device="cpu")
        qb = q_new.view(torch.int16).numpy().view(np.uint16)
        kb = case.k_logical.view(torch.int16).numpy().view(np.uint16)
        vb = case.v_logical.view(torch.int16).numpy().view(np.uint16)
        rows = [0, 1365, 2730, 4095]
        conv = {}

        def convert():
            conv["q"] = od.bf16_bits_to_f64(qb)
            conv["k"] = od.bf16_bits_to_f64(kb)
            conv["v"] = od.bf16_bits_to_f64(vb)

        tc, _, _ = timed(convert)
        t, n, el = timed(lambda: opf.attention_prefill(conv["q"], conv["k"], conv["v"],
                                                       case.scale, rows=rows))
        out["prefill_q4096_l32768_b832"] = {
            "value": round((tc + t / len(rows) * 4096) * 1e6, 1), "unit": "us/call", "cores": 1,
            "kind": "oracle",
            "sample": f"bf16->fp64 conversion of q, K, V timed once ({tc * 1e3:.0f} ms) plus {n} "
                      f"oracle calls on {len(rows)} of 4096 query rows scaled to 4096, {el:.1f} s"}
        del conv
        del case, q_new, qb, kb, vb
        # append: 2048 of the 32768 new tokens into page-832 pages
        rng = np.random.default_rng(0)
        ntok, bsz = 2048, 832
        pool = np.zeros((40, bsz, 4, 256), dtype=np.uint16)
        new = rng.integers(0, 1 << 16, size=(ntok, 4, 256), dtype=np.uint16)
        slots = oa.slots_for_positions(rng.permutation(40), np.arange(ntok), bsz)
        t, n, el = timed(lambda: oa.append_rows(pool, new, slots, bsz))
        out["append_chunk_32768tok_b832"] = {
            "value": round(t / ntok * 32768 * 1e6, 1), "unit": "us/call", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} oracle calls on {ntok} of 32768 tokens (pool copy included), scaled, {el:.1f} s"}
        # compression + finalizer: 16 of the 1024 outputs
        case = synth.make_compress_case("compress_r8_t131072_c128", device="cpu")
        states = case.states.numpy()
        per_req = [states[lo:hi] for lo, hi in (case.req_range(r) for r in range(len(case.lens)))]
        bnd = case.boundaries.numpy()[::64]
        tok = case.token_to_req.numpy()
        pos = case.positions.numpy()
        t, n, el = timed(lambda: oc.compress_outputs(per_req, tok, pos, bnd, 128))
        out["compress_r8_t131072_c128"] = {
            "value": round(t / len(bnd) * case.num_outputs * 1e6, 1), "unit": "us/call",
            "cores": 1, "kind": "oracle",
            "sample": f"{n} oracle calls on {len(bnd)} of {case.num_outputs} outputs, scaled, {el:.1f} s"}
        comp = np.random.default_rng(1).standard_normal((len(bnd), 512))
        cs = np.random.default_rng(2).standard_normal((int(pos.max()) + 1, 64))
        kv = np.zeros((len(bnd) // 64 + 2, oc.KV_PAGE_BYTES), dtype=np.uint8)
        t, n, el = timed(lambda: oc.finalize_outputs(comp, np.ones(512), 1e-6, cs, pos[bnd], 128,
                                                     np.arange(len(bnd)), kv))
        out["compress_finalize_1024"] = {
            "value": round(t / len(bnd) * 1024 * 1e6, 1), "unit": "us/call", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} oracle calls on {len(bnd)} of 1024 outputs, scaled, {el:.1f} s"}
    for v in out.values():
        v["host_cpus"], v["cpu_model"] = ncpu, model
    return out


def traffic_for(res):
    """HBM bytes per split launch from the committed counter runs, or None when
    the kernel source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha():
        return None
    w = t.get("workloads", {}).get(res["workload"])
    if not w:
        return None
    return int(w["fetch_bytes"] + w["write_bytes"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workloads", default="all",
                    help="main, decode (all decode workloads), all, prefill, compress, or one "
                         "workload name (timed alone)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also launch the plain copy kernel (counter calibration runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(decode shards by sequence with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_36_amd as pkv
    from paged_kv_cache_36_amd import synth

    pkv.load()
    torch.cuda.set_device(0)
    log(f"device {torch.cuda.get_device_name(0)}; library {pkv.LIB_PATH}")

    if args.copy_probe:
        copy_probe(torch, pkv)

    if args.workloads not in ("main", "all", "decode", "prefill", "compress"):
        name = args.workloads
        if name in synth.WORKLOADS:
            res = measure(name, args.steps, args.warmup, torch, pkv, synth)
        elif name in synth.PREFILL_WORKLOADS:
            res = measure_prefill(name, args.steps, args.warmup, torch, pkv, synth)
        elif name in synth.COMPRESS_WORKLOADS:
            res = measure_compress(name, args.steps, args.warmup, torch, pkv, synth)
        elif name in APPEND_WORKLOADS:
            res = measure_append(name, *APPEND_WORKLOADS[name], args.steps, args.warmup,
                                 torch, pkv, synth)
        else:
            known = (sorted(synth.WORKLOADS) + sorted(synth.PREFILL_WORKLOADS) +
                     sorted(APPEND_WORKLOADS) + sorted(synth.COMPRESS_WORKLOADS))
            sys.exit(f"unknown workload {name}; choose from {known}")
        print(json.dumps({"workload_only": res}), flush=True)
        return
    # the streaming-read ceiling before any sustained load (for reference; the
    # ceiling the decode is compared with is taken after the workloads)
    probe_idle = read_probe(torch, pkv)
    log(f"read probe on the idle GPU: {probe_idle} GB/s")
    main_res = measure(MAIN, args.steps, args.warmup, torch, pkv, synth)
    extra = []
    if args.workloads in ("all", "decode"):
        # the other decode workloads run 10 us to 1.5 ms per step: 200 replays at least,
        # so the host-side synchronisation around the replay stays small against the work
        for name in EXTRA:
            extra.append(measure(name, max(min(args.steps, 400), 200), args.warmup, torch, pkv,
                                 synth))
    appends = []
    if args.workloads == "all":
        # one new token per sequence of the wide batch, and a 32768-token
        # prefill chunk written into page-832 pages
        for name, cap in (("append_decode_64tok_b832", 400), ("append_chunk_32768tok_b832", 100)):
            appends.append(measure_append(name, *APPEND_WORKLOADS[name], min(args.steps, cap),
                                          args.warmup, torch, pkv, synth))
    prefills = []
    if args.workloads in ("all", "prefill"):
        for name in sorted(synth.PREFILL_WORKLOADS):
            prefills.append(measure_prefill(name, min(args.steps, 20), min(args.warmup, 3),
                                            torch, pkv, synth))
    compresses = []
    if args.workloads in ("all", "compress"):
        for name in sorted(synth.COMPRESS_WORKLOADS, key=lambda w: synth.COMPRESS_WORKLOADS[w]):
            compresses.append(measure_compress(name, min(args.steps, 100), args.warmup, torch,
                                               pkv, synth))
    probe = read_probe(torch, pkv)
    log(f"read probe (2 GiB streaming read of random bytes) after the workloads: {probe} GB/s")

    cpu = None if args.no_cpu_baseline else cpu_baseline()
    cpu_par = None if args.no_cpu_baseline else cpu_baseline_parallel()
    cpu_rows = None if args.no_cpu_baseline or args.workloads != "all" else cpu_baseline_rows()
    if not args.no_cpu_baseline:
        for r in extra:
            if r["workload"] == "batched_8seq_t131072_b832":
                r["cpu_baseline"] = cpu_baseline(r["workload"], budget_s=5.0)

    us = main_res["us_per_step"]
    line = {
        "metric": "paged decode attention µs/step and achieved HBM GB/s vs peak (bf16, GQA6)",
        "value": us,
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        # the pages quote no decode time for this workload (only single
        # sequences of 8K-32K tokens on other hardware: see "workloads")
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V in a NaN-poisoned shuffled page pool)",
        "config": {"workload": MAIN, "num_seqs": main_res["num_seqs"],
                   "kv_tokens_total": main_res["total_tokens"],
                   "max_seq_len": main_res["max_seq_len"], "block_size": 832,
                   "partition_tokens": main_res["partition_tokens"],
                   "q_heads": 24, "kv_heads": 4, "head_size": 256,
                   "split": main_res["split"],
                   "split_workgroups": main_res["split_workgroups"],
                   "cold_copies": main_res["cold_copies"]},
        "gbps": main_res["gbps_step"],
        "frac_peak_step": main_res["frac_peak_step"],
        "roofline": dict(main_res["roofline"],
                         # the same rate against the measured streaming-read ceiling
                         frac_of_read_probe=(round(main_res["gbps_split"] / probe, 4)
                                             if probe else None)),
        "cpu_baseline": cpu,
        "cpu_baseline_parallel": cpu_par,
        "cpu_baseline_rows": cpu_rows,
        "read_probe_gbps": probe,
        "read_probe_idle_gbps": probe_idle,
        "workloads": [main_res] + extra,
        "append": appends,
        "prefill": prefills,
        "compress": compresses,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
