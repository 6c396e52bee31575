#!/usr/bin/env python3
"""Paged decode attention benchmark on one MI355X.

One step = the whole decode hot path over one batch: the KV write of each
sequence's new token (reshape_and_cache) followed by decode attention over the
paged cache (decode kernel + split-K reduce).  Inputs are the seeded synthetic
workload, resident in HBM before timing starts.

Prints ONE JSON line.  ``value`` is whole-step throughput in GB/s of
algorithmic bytes (K/V of every context token once -- shared prefix pages once,
each new token's row read once -- plus q in, out, the block-table entries used,
the lengths, and the new rows written with their slots); ``seqs_per_s`` is
sequences decoded per second.  ``roofline`` rates the
decode kernel alone (its launches timed with HIP events on the library's
stream) against the MI355X HBM peak; ``cpu_baseline`` is the float64 oracle
on the host cores over a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama7b",
                    help="workload: tiny, llama7b, gqa, shared_prefix, long_context")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="override the workload's partition size (0 = single pass)")
    ap.add_argument("--block-size", type=int, default=None,
                    help="lay the pool out in blocks of this many tokens (8, 16, 32; default: "
                         "the workload's 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--two-call", action="store_true",
                    help="step = pa_reshape_and_cache then pa_paged_attention_decode (default: "
                         "pa_reshape_and_decode, the KV write inside the decode launch)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="also time plain streaming HBM traffic for context: a sum over 4 GiB "
                         "(reads) and a 2 GiB device copy (reads + writes), torch kernels")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode call per step (profiling aid)")
    ap.add_argument("--pool-copies", type=int, default=2,
                    help="copies of the KV pool used in turn by consecutive steps, so that no "
                         "step finds its K/V in the 256 MB Infinity Cache from the step "
                         "before (1 = re-read the same pool every step)")
    ap.add_argument("--loop-steps", type=int, default=0,
                    help="also time this many steps of a multi-step decode loop driven by the "
                         "host block manager (one new token per sequence per step)")
    ap.add_argument("--block-ops", action="store_true",
                    help="also time pa_copy_blocks (device) and pa_swap_blocks (device <-> "
                         "pinned host) on blocks of this workload's pool")
    ap.add_argument("--query-len", type=int, default=0,
                    help="also time pa_paged_attention_multi_query with this many new query "
                         "tokens per sequence (causal over each context's last tokens)")
    ap.add_argument("--no-config-rows", action="store_true",
                    help="skip the per-workload rows (by default every workload of the five "
                         "is also timed for a few steps and checked against the oracle)")
    ap.add_argument("--row-steps", type=int, default=20,
                    help="timed steps of each per-workload row")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before warmup, as the "
                         "known-size reference for HBM byte counters")
    return ap.parse_args(argv)


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed (string
    literals in these sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the decode kernel sources' code (comments and layout
    ignored) and of the compiler flags they are built with, to tell whether
    stored counters still describe the code being run."""
    from paged_kv_cache_269_amd import build as hipbuild
    h = hashlib.sha256()
    for f in ("common.h", "items.h", "launch.h", "mfma_tile.h", "decode_valu.hip",
              "decode_mfma.hip", "prefix.hip", "reduce.hip", "reshape_and_cache.hip", "api.cpp"):
        with open(os.path.join(ROOT, "paged_kv_cache_269_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    # flags with the checkout's own path taken out (it differs between machines)
    flags = [f.replace(ROOT, "<root>") for f in hipbuild.COMMON_FLAGS]
    h.update(" ".join([hipbuild.HIPCC.rsplit("/", 1)[-1], hipbuild.ARCH] + flags).encode())
    return h.hexdigest()[:16]


def stored_traffic(config: str):
    """HBM bytes per step (all of a step's kernels) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel sources
    and this workload."""
    path = os.path.join(ROOT, "profiles", f"decode_{config}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source-hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm-bytes-per-step:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_bytes) or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def cpu_baseline(w, target_s: float):
    """The oracle, untuned, on a prefix of the workload's sequences sized to
    about target_s seconds on all host threads."""
    import numpy as np
    import oracle
    from paged_kv_cache_269_amd import workloads as W

    threads = oracle.max_threads()
    Hq = w.num_q_heads

    def run(nseq, nthreads=threads):
        seqs = np.repeat(np.arange(nseq), Hq)
        heads = np.tile(np.arange(Hq), nseq)
        t0 = time.perf_counter()
        oracle.decode_rows(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale,
                           w.dtype, seqs, heads, num_threads=nthreads)
        return time.perf_counter() - t0

    t1 = run(1)
    n = int(min(w.num_seqs, max(1, target_s / max(t1, 1e-6))))
    dt = run(n) if n > 1 else t1
    reps = 1
    if n == w.num_seqs and dt < target_s / 2:
        # the whole workload is short: repeat it to about target_s, take the median
        reps = int(min(20, max(2, target_s / max(dt, 1e-6))))
        dt = float(sorted([dt] + [run(n) for _ in range(reps - 1)])[reps // 2])
    sub_lens = w.context_lens[:n].astype(np.int64)
    per_tok = W.kv_bytes_per_token(w.num_kv_heads, w.head_dim, w.elem_bytes)
    if w.shared_prefix_blocks:
        prefix = 16 * w.shared_prefix_blocks
        kv = (prefix + int((sub_lens - prefix).sum())) * per_tok
    else:
        kv = int(sub_lens.sum()) * per_tok
    result = {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
              "kind": "oracle", "seqs_per_s": round(n / dt, 3), "seconds": round(dt, 3),
              "sample": f"first {n} of {w.num_seqs} sequences, all {Hq} query heads, "
                        f"float64 C oracle with OpenMP, median of {reps} run(s)",
              "cpu_model": _cpu_model()}
    if w.name in ("tiny", "llama7b") and threads > 1:
        # the same sample on one thread, for the two smallest workloads
        dt1 = run(n, 1)
        result["single_thread_value"] = round(kv / dt1 / 1e9, 4)
    return result


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_ceiling(dev):
    """Plain streaming HBM rates on this GPU for context next to the 8 TB/s
    nominal peak: torch's sum over a 4 GiB fp16 tensor (reads) and a 2 GiB
    device-to-device copy (reads + writes), each the median of 10 timed
    calls with HIP events."""
    import numpy as np
    import torch
    x = torch.ones(2 << 30, dtype=torch.float16, device=dev)       # 4 GiB
    y = torch.empty(1 << 30, dtype=torch.float16, device=dev)      # 2 GiB
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)) * 1e-3

    t_sum = timed(lambda: x.sum(dtype=torch.float32))
    t_copy = timed(lambda: y.copy_(x[: 1 << 30]))
    out = {"sum_4GiB_read_GBps": round(x.numel() * 2 / t_sum / 1e9, 1),
           "copy_2GiB_read_write_GBps": round(2 * y.numel() * 2 / t_copy / 1e9, 1),
           "note": "torch kernels, median of 10; nominal HBM peak 8000 GB/s"}
    del x, y
    torch.cuda.empty_cache()
    return out


def decode_loop(args, w, dev):
    """Multi-step decode through the library's host block manager: each step
    appends one token to every sequence (the manager hands out the slots and
    takes a new block at each 16-token boundary) and exports the block tables
    and lengths into a pinned host buffer; the device part -- one copy of that
    buffer and one pa_reshape_and_decode call (KV write inside the decode
    launch) -- is a captured HIP graph, replayed
    once per step.  Two buffer/graph sets alternate so that the host fills one
    while the device reads the other.  The workload's context lengths are the
    prompts; their K/V is whatever the freshly allocated pool holds (timing
    only; the multi-step GPU test checks results)."""
    import numpy as np
    import torch
    import paged_kv_cache_269_amd as pa
    from paged_kv_cache_269_amd import workloads as W

    S, Wm = args.loop_steps, 8
    B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    lens = w.context_lens.astype(np.int64)
    final = lens + S + Wm
    N = int(((final + 15) // 16).sum() * 1.05) + 16
    M = int((final.max() + 15) // 16)
    maxlen = int(final.max())
    tdt = W.torch_dtype(w.dtype)
    gen = torch.Generator(device=dev).manual_seed(7)
    kc = torch.randn((N, Hkv, 16, D), generator=gen, device=dev).to(tdt)
    vc = torch.randn((N, Hkv, 16, D), generator=gen, device=dev).to(tdt)
    q = torch.randn((B, Hq, D), generator=gen, device=dev).to(tdt)
    knew = torch.randn((B, Hkv, D), generator=gen, device=dev).to(tdt)
    vnew = torch.randn((B, Hkv, D), generator=gen, device=dev).to(tdt)
    out = torch.empty_like(q)
    ws = pa.decode_workspace(B, Hq, D, maxlen, w.partition_size, device=dev)
    bm = pa.BlockManager(N, 16)
    ids = np.arange(B, dtype=np.int64)
    for s in range(B):
        bm.allocate(s, int(lens[s]))
    # one packed int32 buffer per set: [slots (B int64) | tables (B x M) | lens (B)]
    n32 = 2 * B + B * M + B
    sets = []
    for _ in range(2):
        h = torch.empty(n32, dtype=torch.int32).pin_memory()
        dvb = torch.empty(n32, dtype=torch.int32, device=dev)
        hn = h.numpy()
        sets.append(dict(
            h=h, d=dvb,
            slots=hn[:2 * B].view(np.int64), bt=hn[2 * B:2 * B + B * M].reshape(B, M),
            cl=hn[2 * B + B * M:],
            d_slots=dvb[:2 * B].view(torch.int64), d_bt=dvb[2 * B:2 * B + B * M].view(B, M),
            d_cl=dvb[2 * B + B * M:], done=None))

    def device_part(st, stream):
        st["d"].copy_(st["h"], non_blocking=True)
        pa.reshape_and_decode(out, q, knew, vnew, kc, vc, st["d_slots"], st["d_bt"], st["d_cl"],
                              w.scale, maxlen, partition_size=w.partition_size, workspace=ws,
                              stream=stream)

    # fill both sets once (valid tables) and capture one graph per set
    for st in sets:
        bm.block_tables(ids, M, 0, out=(st["bt"], st["cl"]))
        st["slots"][:] = -1                     # no KV write during capture warm-up
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for st in sets:
            device_part(st, side)               # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for st in sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            device_part(st, torch.cuda.current_stream())
        st["graph"] = g
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step(i):
        st = sets[i % 2]
        if st["done"] is not None:
            st["done"].synchronize()            # the previous copy out of this buffer has run
        bm.append_batch(ids, st["slots"])
        bm.block_tables(ids, M, 0, out=(st["bt"], st["cl"]))
        st["graph"].replay()
        if st["done"] is None:
            st["done"] = torch.cuda.Event()
        st["done"].record(stream)

    for i in range(Wm):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    host_s = 0.0
    for i in range(Wm, Wm + S):
        h0 = time.perf_counter()
        step(i)
        host_s += time.perf_counter() - h0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the device part alone, replayed back to back
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(20):
        sets[i % 2]["graph"].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    dev_us = e0.elapsed_time(e1) * 1e3 / 20
    bm.close()
    return {"steps": S, "sequences": B, "ms_per_step": round(wall * 1e3 / S, 4),
            "tokens_per_s": round(B * S / wall, 1),
            "host_ms_per_step": round(host_s * 1e3 / S, 4),
            "device_graph_us_per_step": round(dev_us, 2),
            "pool_blocks": N,
            "note": "per step: block-manager appends + table export on the host, then one HIP "
                    "graph (packed H2D copy, pa_reshape_and_decode)"}


def block_ops(w, dev):
    """Copy-on-write copies and swaps on this workload's block shape: 2048
    random (src, dst) pairs copied inside the pool (both caches), and 1024
    blocks of the K cache swapped out to pinned host memory and back."""
    import numpy as np
    import torch
    import paged_kv_cache_269_amd as pa
    from paged_kv_cache_269_amd import workloads as W

    Hkv, D = w.num_kv_heads, w.head_dim
    tdt = W.torch_dtype(w.dtype)
    N = 8192
    kc = torch.randn((N, Hkv, 16, D), device=dev).to(tdt)
    vc = torch.randn((N, Hkv, 16, D), device=dev).to(tdt)
    block_bytes = kc[0].numel() * kc.element_size()
    rng = np.random.default_rng(0)
    perm = rng.permutation(N)
    pairs = torch.from_numpy(np.stack([perm[:2048], perm[2048:4096]], 1).astype(np.int32)).to(dev)
    for _ in range(3):
        pa.copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        pa.copy_blocks(kc, vc, pairs)
    e1.record()
    torch.cuda.synchronize()
    copy_us = e0.elapsed_time(e1) * 1e3 / reps
    copy_bytes = 2 * 2 * 2048 * block_bytes          # read + write, K and V
    host = torch.empty((1024, Hkv, 16, D), dtype=tdt).pin_memory()
    out_pairs = np.stack([perm[4096:5120], rng.permutation(1024)], 1)   # scattered, no runs
    in_pairs = out_pairs[:, ::-1].copy()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / 5

    out_us = timed(lambda: pa.swap_blocks(kc, host, out_pairs))
    in_us = timed(lambda: pa.swap_blocks(host, kc, in_pairs))
    sw_bytes = 1024 * block_bytes
    # the same moves in one kernel through the pinned buffer's device mapping
    out_p = torch.from_numpy(np.ascontiguousarray(out_pairs, dtype=np.int64)).to(dev)
    in_p = torch.from_numpy(np.ascontiguousarray(in_pairs, dtype=np.int64)).to(dev)
    mout_us = timed(lambda: pa.swap_blocks_mapped(kc, host, out_p))
    min_us = timed(lambda: pa.swap_blocks_mapped(host, kc, in_p))
    return {"block_bytes_per_cache": block_bytes,
            "copy_pairs": 2048, "copy_us": round(copy_us, 2),
            "copy_GBps": round(copy_bytes / copy_us / 1e3, 1),
            "copy_frac_of_hbm_peak": round(copy_bytes / copy_us / 1e3 / HBM_PEAK_GBPS, 4),
            "swap_blocks": 1024, "swap_out_us": round(out_us, 1), "swap_in_us": round(in_us, 1),
            "swap_out_GBps": round(sw_bytes / out_us / 1e3, 1),
            "swap_in_GBps": round(sw_bytes / in_us / 1e3, 1),
            "swap_mapped_out_us": round(mout_us, 1), "swap_mapped_in_us": round(min_us, 1),
            "swap_mapped_out_GBps": round(sw_bytes / mout_us / 1e3, 1),
            "swap_mapped_in_GBps": round(sw_bytes / min_us / 1e3, 1),
            "note": "copy: read + write of K and V blocks; swap: one cache, scattered blocks, "
                    "one asynchronous copy each; swap_mapped: one kernel through the pinned "
                    "buffer's device mapping"}


def multi_query_bench(args, w, d, pools, part, stream, query_len=None, steps=None,
                      keep=None):
    """The multi-query entry point on this workload's pool: every sequence's
    last ``query_len`` (default ``args.query_len``) context tokens as queries.
    Algorithmic bytes: K/V of every context token once, q in, out, the table
    entries and offsets; re-reads of a tile by the 16-row units of one KV head
    are overhead.  ``keep`` (a dict), if given, receives the spans and the
    last call's output."""
    import numpy as np
    import torch
    import paged_kv_cache_269_amd as pa
    from paged_kv_cache_269_amd import workloads as W

    query_len = args.query_len if query_len is None else query_len
    spans = W.generate_query_spans(w, query_len, seed=7)
    T = spans.num_tokens
    tdt = W.torch_dtype(w.dtype)
    q = torch.from_numpy(spans.q)
    q = (q.view(torch.bfloat16) if w.dtype == "bf16" else q).to(d["q"].device)
    qs = torch.from_numpy(spans.query_start).to(q.device)
    out = torch.empty_like(q)
    assert out.dtype == tdt
    ws = pa.multi_query_workspace(T, w.num_q_heads, w.head_dim, w.max_context_len, part,
                                  device=q.device)

    def call(i):
        kc, vc = pools[i % len(pools)]
        pa.paged_attention_multi_query(out, q, kc, vc, d["block_tables"], d["context_lens"], qs,
                                       w.scale, w.max_context_len, spans.max_query_len,
                                       partition_size=part, workspace=ws, stream=stream)

    for i in range(max(3, args.warmup)):
        call(i)
    torch.cuda.synchronize()
    K = max(10, args.steps if steps is None else steps)
    # calls back to back, one HIP event pair around them (as the decode step)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(K):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / K
    ab = W.algorithmic_bytes(w, unique=True)
    qo = 2 * T * w.num_q_heads * w.head_dim * w.elem_bytes
    nbytes = ab["kv"] + qo + ab["meta"] + 4 * (w.num_seqs + 1)
    flops = W.multi_query_flops(w, spans)
    gbps = nbytes / us / 1e3
    tflops = flops / us / 1e6
    if keep is not None:
        keep["spans"], keep["out"] = spans, out
    return {"entry": "pa_paged_attention_multi_query", "query_len": query_len,
            "query_tokens": T, "partition_size": part, "launch_us_avg": round(us, 2),
            "algorithmic_bytes": nbytes, "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "flops": flops,
            "TFLOPs": round(tflops, 2), "frac_mfma_peak": round(tflops / 2500.0, 5),
            "tokens_per_s": round(T / us * 1e6, 1)}


class Timed:
    """One workload's steps timed on the device (see time_workload)."""


def time_workload(args, name, dev, steps, warmup, block_size=None, partition_size=None):
    """Generate the workload, upload it (``args.pool_copies`` copies of the
    pool), and time ``steps`` decode steps back to back with one HIP event
    pair around them, then ``min(steps, 50)`` single calls with an event pair
    each (their spread).  Returns a Timed holding the workload, its device
    tensors, the last step's output and the timings."""
    import numpy as np
    import torch
    import paged_kv_cache_269_amd as pa
    from paged_kv_cache_269_amd import workloads as W

    w = W.generate(name, poison=False, block_size=block_size)
    part = w.partition_size if partition_size is None else partition_size
    d = W.to_device(w, dev)
    pools = [(d["k_cache"], d["v_cache"])]
    for _ in range(max(1, args.pool_copies) - 1):
        pools.append((d["k_cache"].clone(), d["v_cache"].clone()))
    out = torch.empty_like(d["q"])
    cascade = bool(w.params.get("cascade")) and part == 0
    # one call per step (KV write inside the decode launch) unless the step
    # is asked for as two calls or is decode only
    fused = not (args.two_call or args.decode_only)
    if cascade:   # allocated once, outside the timed loop
        ws = pa.cascade_workspace(w.num_seqs, w.num_q_heads, w.head_dim, device=dev)
    else:
        ws = pa.decode_workspace(w.num_seqs, w.num_q_heads, w.head_dim, w.max_context_len, part,
                                 device=dev)
    stream = torch.cuda.current_stream()

    def reshape(i):
        kc, vc = pools[i % len(pools)]
        pa.reshape_and_cache(d["key"], d["value"], kc, vc, d["slot_mapping"], stream=stream)

    def decode(i):
        kc, vc = pools[i % len(pools)]
        if fused and cascade:
            pa.reshape_and_decode_cascade(out, d["q"], d["key"], d["value"], kc, vc,
                                          d["slot_mapping"], d["block_tables"],
                                          d["context_lens"], w.scale, w.max_context_len,
                                          workspace=ws, stream=stream)
        elif fused:
            pa.reshape_and_decode(out, d["q"], d["key"], d["value"], kc, vc, d["slot_mapping"],
                                  d["block_tables"], d["context_lens"], w.scale,
                                  w.max_context_len, partition_size=part, workspace=ws,
                                  stream=stream)
        elif cascade:
            pa.paged_attention_decode_cascade(out, d["q"], kc, vc, d["block_tables"],
                                              d["context_lens"], w.scale, w.max_context_len,
                                              workspace=ws, stream=stream)
        else:
            pa.paged_attention_decode(out, d["q"], kc, vc, d["block_tables"], d["context_lens"],
                                      w.scale, w.max_context_len, partition_size=part,
                                      workspace=ws, stream=stream)

    def step(i):
        if not (args.decode_only or fused):
            reshape(i)
        decode(i)

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 18           # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # every pool copy sees the KV write before timing starts (the last
    # step's output then belongs to the written pool whichever copy it read)
    for i in range(max(warmup, len(pools))):
        if args.decode_only:
            reshape(i)
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps back to back, one HIP event pair on the library's
    # stream around them (an event pair around every step would add its own
    # gaps between the launches: ~7 us per step measured).
    K = steps
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    for i in range(K):
        step(warmup + i)
    region[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = region[0].elapsed_time(region[1])
    # Spread of single calls, from a separate pass with an event pair around
    # each call (not the timed region).
    nspread = min(K, 50)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(nspread)]
    for i in range(nspread):
        j = warmup + K + i
        if not (args.decode_only or fused):
            reshape(j)
        ev[i][0].record(stream)
        decode(j)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t = Timed()
    t.w, t.d, t.pools, t.ws, t.out, t.part = w, d, pools, ws, out, part
    t.cascade, t.fused, t.stream = cascade, fused, stream
    t.steps, t.wall, t.region_ms = K, wall, region_ms
    t.dec_ms = np.array([a.elapsed_time(b) for a, b in ev])
    ab = W.algorithmic_bytes(w, unique=True)
    t.ab = ab
    t.step_bytes = ab["total"] if args.decode_only else W.step_bytes(w)
    return t


def oracle_check(t):
    """The last step's output against the float64 oracle over every output
    row (the host pools with the oracle's own KV write): max-abs, rel-L2
    over the whole tensor, and the oracle's time on all host threads."""
    import numpy as np
    import torch
    import oracle

    w = t.w
    got = t.out.detach().cpu()
    if w.dtype == "bf16":   # bf16 bits -> the float32 they stand for
        got = (got.view(torch.uint16).numpy().astype(np.uint32) << 16).view(np.float32)
    got = np.asarray(got.numpy() if isinstance(got, torch.Tensor) else got, np.float64)
    oracle.reshape_and_cache(w.key, w.value, w.k_cache, w.v_cache, w.slot_mapping, w.dtype)
    t0 = time.perf_counter()
    ref = oracle.decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale,
                        w.dtype)
    dt = time.perf_counter() - t0
    err = np.abs(got - ref)
    nref = float(np.linalg.norm(ref))
    return {"max_abs": float(err.max()), "rel_l2": float(np.linalg.norm(got - ref) / nref),
            "rows": int(ref.shape[0] * ref.shape[1]),
            "oracle_s": round(dt, 4), "oracle_GBps": round(t.ab["kv"] / dt / 1e9, 3),
            "oracle_cores": oracle.max_threads(), "kind": "oracle"}


def config_row(args, name, dev):
    """One per-workload row: a few timed steps of the workload in its
    benchmark configuration, the spread of single calls, the stored HBM
    traffic, and the output against the oracle."""
    import numpy as np
    import torch

    t = time_workload(args, name, dev, args.row_steps, 3)
    ms = t.wall * 1e3 / t.steps
    us_region = t.region_ms * 1e3 / t.steps
    gbps = t.step_bytes / (us_region * 1e-6) / 1e9
    row = {"entry": _entry(t, args), "partition_size": t.part, "num_seqs": t.w.num_seqs,
           "steps": t.steps, "ms_per_step_wall": round(ms, 4),
           "step_us_avg": round(us_region, 2),
           "single_call_us_median": round(float(np.median(t.dec_ms)) * 1e3, 2),
           "single_call_us_p10": round(float(np.percentile(t.dec_ms, 10)) * 1e3, 2),
           "single_call_us_p90": round(float(np.percentile(t.dec_ms, 90)) * 1e3, 2),
           "algorithmic_bytes_per_step": t.step_bytes, "GBps": round(gbps, 1),
           "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
           "seqs_per_s": round(t.w.num_seqs / (us_region * 1e-6), 1),
           "hbm_traffic_bytes_per_step": stored_traffic(name)}
    row["oracle"] = oracle_check(t)
    del t
    torch.cuda.empty_cache()
    return row


# Multi-token query rows of the default run: (workload, new tokens per
# sequence), at the library's suggested partition size.
MQ_ROWS = (("gqa", 16), ("gqa", 4), ("long_context", 4))


def multi_query_row(args, name, query_len, dev, sample_rows=96):
    """One multi-query row: the workload's pool with its KV write done, calls
    timed back to back, and ``sample_rows`` (token, head) rows of the last
    output against the float64 oracle (the whole output would take the oracle
    minutes at these sizes)."""
    import numpy as np
    import torch
    import paged_kv_cache_269_amd as pa
    from paged_kv_cache_269_amd import workloads as W
    import oracle

    w = W.generate(name, poison=False)
    d = W.to_device(w, dev)
    pools = [(d["k_cache"], d["v_cache"]), (d["k_cache"].clone(), d["v_cache"].clone())]
    stream = torch.cuda.current_stream()
    for kc, vc in pools:
        pa.reshape_and_cache(d["key"], d["value"], kc, vc, d["slot_mapping"], stream=stream)
    torch.cuda.synchronize()
    part = pa.multi_query_partition_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, query_len,
                                         w.max_context_len)
    keep = {}
    row = multi_query_bench(args, w, d, pools, part, stream, query_len=query_len,
                            steps=args.row_steps, keep=keep)
    spans, out = keep["spans"], keep["out"]
    got = out.detach().cpu()
    if w.dtype == "bf16":
        got = (got.view(torch.uint16).numpy().astype(np.uint32) << 16).view(np.float32)
    got = np.asarray(got.numpy() if isinstance(got, torch.Tensor) else got, np.float64)
    T, Hq = got.shape[0], got.shape[1]
    rng = np.random.default_rng(11)
    # the last token of the longest span and random others
    last = int(spans.query_start[int(np.argmax(w.context_lens)) + 1]) - 1
    toks = np.concatenate([[last] * 4, rng.integers(0, T, sample_rows - 4)])
    heads = np.concatenate([[0, Hq // 3, Hq // 2, Hq - 1], rng.integers(0, Hq, sample_rows - 4)])
    oracle.reshape_and_cache(w.key, w.value, w.k_cache, w.v_cache, w.slot_mapping, w.dtype)
    t0 = time.perf_counter()
    ref = oracle.multi_query(spans.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                             spans.query_start, w.scale, w.dtype, rows_token=toks,
                             rows_head=heads)
    dt = time.perf_counter() - t0
    sub = got[toks, heads]
    err = np.abs(sub - ref)
    row["oracle"] = {"max_abs": float(err.max()),
                     "rel_l2": float(np.linalg.norm(sub - ref) / np.linalg.norm(ref)),
                     "rows": int(sample_rows), "rows_total": int(T * Hq),
                     "oracle_s": round(dt, 4), "oracle_cores": oracle.max_threads(),
                     "kind": "oracle"}
    del d, pools, out, keep
    torch.cuda.empty_cache()
    return row


def _entry(t, args):
    if t.fused and t.cascade:
        return "pa_reshape_and_decode_cascade"
    if t.fused:
        return "pa_reshape_and_decode"
    return "pa_paged_attention_decode_cascade" if t.cascade else "pa_paged_attention_decode"


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                                   f"--gpus {args.gpus} is not supported (the library has no "
                                   "multi-GPU path)"}))
        return 2

    import numpy as np
    import torch
    import paged_kv_cache_269_amd as pa
    from paged_kv_cache_269_amd import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    dev = torch.device("cuda:0")
    pa.load_library()

    t = time_workload(args, args.config, dev, args.steps, args.warmup,
                      block_size=args.block_size, partition_size=args.partition_size)
    w, part, cascade, fused = t.w, t.part, t.cascade, t.fused
    d, pools, ws, stream = t.d, t.pools, t.ws, t.stream
    K, wall, region_ms, dec_ms = t.steps, t.wall, t.region_ms, t.dec_ms
    ab, step_bytes = t.ab, t.step_bytes
    ms_per_step = wall * 1e3 / K
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # Roofline of the step's launches over the timed region: one call of
    # pa_reshape_and_decode (the KV write inside the decode kernel) or of
    # pa_reshape_and_decode_cascade (the KV write inside the shared-prefix
    # kernel), or the KV-write kernel and the decode call.
    dec_avg = region_ms / K
    launch_bytes = step_bytes
    achieved = launch_bytes / (dec_avg * 1e-3) / 1e9
    traffic = stored_traffic(args.config)

    result = {
        "metric": "paged decode attention: KV GB/s (% of HBM peak) and seqs/s, 7B shape",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, randomly permuted 16-token blocks)",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size,
                   "kv_dtype": w.dtype, "accumulate": "f32", "partition_size": part,
                   "context_len_mean": float(w.context_lens.mean()),
                   "context_len_max": int(w.max_context_len), "num_blocks": w.num_blocks,
                   "pool_copies": len(pools),
                   "entry": _entry(t, args),
                   "step": ("decode" if args.decode_only else
                            "KV write + decode in one call" if fused else
                            "reshape_and_cache + decode")
                           + (" + split-K reduce" if part and w.max_context_len > part else "")},
        "seqs_per_s": round(w.num_seqs / (ms_per_step * 1e-3), 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "bytes_per_step": {"algorithmic": step_bytes, "kv_unique": ab["kv"],
                           "kv_logical": ab["logical_kv"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": ("pa_reshape_and_decode_cascade (shared-prefix kernel with "
                                "the KV write, decode kernel)" if cascade and fused else
                                "pa_paged_attention_decode_cascade (KV-write kernel, "
                                "shared-prefix kernel, decode kernel)" if cascade and
                                not args.decode_only else
                                "pa_paged_attention_decode_cascade (shared-prefix kernel + "
                                "decode kernel)" if cascade else
                                ("pa_reshape_and_decode (decode kernel with the KV write"
                                 if fused else "pa_paged_attention_decode (decode kernel"
                                 if args.decode_only else
                                 "pa_reshape_and_cache + pa_paged_attention_decode (KV-write "
                                 "kernel, decode kernel")
                                + (" + split-K reduce" if part and w.max_context_len > part
                                   else "") + ")"),
                     "launch_us_avg": round(dec_avg * 1e3, 2),
                     "timing": "HIP events around the timed region / steps",
                     "single_call_us_median": round(float(np.median(dec_ms)) * 1e3, 2),
                     "single_call_us_p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                     "single_call_us_p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2),
                     "algorithmic_bytes_per_step": launch_bytes},
    }
    if args.query_len > 0:
        # the library's suggested partition for multi-token queries, unless
        # one is given (the decode's partitions are sized for one row per head)
        import paged_kv_cache_269_amd as pa
        mq_part = part if args.partition_size is not None else pa.multi_query_partition_size(
            w.num_seqs, w.num_q_heads, w.num_kv_heads, args.query_len, w.max_context_len)
        result["multi_query"] = multi_query_bench(args, w, d, pools, mq_part, stream)
    if args.block_ops:
        result["block_ops"] = block_ops(w, dev)
    if args.read_ceiling:
        result["read_ceiling"] = read_ceiling(dev)
    if args.loop_steps > 0:
        del pools, d, ws
        t.d = t.pools = t.ws = None
        torch.cuda.empty_cache()
        result["decode_loop"] = decode_loop(args, w, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    rows_wanted = not (args.no_config_rows or args.decode_only or args.two_call
                       or args.block_size or args.partition_size is not None
                       or args.query_len or args.loop_steps or args.block_ops)
    if rows_wanted:
        # every workload: a few steps in its benchmark configuration, each
        # checked against the oracle over its whole output
        d = pools = ws = None
        t.d = t.pools = t.ws = None
        torch.cuda.empty_cache()
        rows = {}
        for name in W.CONFIG_ORDER:
            print(f"[bench] row {name}", file=sys.stderr, flush=True)
            rows[name] = config_row(args, name, dev)
        result["configs"] = rows
        mq = {}
        for name, n in MQ_ROWS:
            print(f"[bench] multi-query row {name} {n}", file=sys.stderr, flush=True)
            mq[f"{name}_q{n}"] = multi_query_row(args, name, n, dev)
        result["multi_query_configs"] = mq
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
