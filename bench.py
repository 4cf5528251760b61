"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input: for a
decode workload one paged_attention_decode call (partition kernel + split
merge) for one attention layer; for the mixed workload the slot write plus
one paged_attention_varlen call; for the shared-prefix workload the slot
write plus one cascade_attention call.  Inputs are resident in HBM before
timing.

Prints ONE JSON line.  `value` is achieved HBM GB/s of the whole step
(algorithmic bytes / step time) of the headline workload (the Llama-7B-shaped
MHA decode unless --workload names another); `roofline` is the dominant
kernel's achieved rate against the MI355X peak, from per-launch HIP events
recorded by the library inside the timed region; `per_workload` repeats the
measurement, in the same run, for the GQA decode, the long-context split
decode, the mixed chunked-prefill step and workloads 6-12 (fp8 caches, a
sliding window, a shared-prefix cascade, binary16 caches; default run
only); `cpu_baseline`
times the fp64 CPU oracle on the headline workload (BLAS threads = the
host cores this process may use) and, single-threaded, on the three small
decode workloads.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..12]
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (% of peak) + µs/step, 1 MI355X"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 (and fp16) MFMA, published
MALL_BYTES = 256 << 20         # MI355X last-level (Infinity) cache

HEADLINE = 2                   # Llama-7B-shaped MHA decode
# GQA decode, long-context split decode, mixed step, then the fp8, sliding-window,
# shared-prefix and binary16 workloads
PER_WORKLOAD = (3, 4, 5, 6, 7, 8, 9, 10, 11, 12)

WORKLOAD_DESC = {
    1: "4 seqs, 8/8 heads, head 64, block 16, fp32, seq_lens U[1,256], seed 0",
    2: "64 seqs, 32/32 heads, head 128, block 16, bf16, seq_lens U[200,4096], seed 1",
    3: "256 seqs, 32/8 heads, head 128, block 16, bf16, seq_lens lognormal(median 1024, sigma 0.8) in [16,8192], seed 2",
    4: "8 seqs, 64/8 heads, head 128, block 16, bf16, seq_lens U[32768,131072], 512-token partitions, N(0,0.5), seed 3",
    5: "slot write + varlen: 4 causal chunks of 512 (context U[0,4096]) + 128 decode rows (U[64,4096]), 32/8 heads, head 128, block 32, bf16, seed 4",
    6: "workload 2 (same lengths and pool) over an fp8 e4m3 cache with per-kv-head scales; q/out bf16",
    7: "workload 3 (same lengths and pool) over an fp8 e4m3 cache with per-kv-head scales; q/out bf16",
    8: "workload 4 (same lengths and pool) with a 4096-key sliding window (window_left 4095)",
    9: "slot write + cascade attention: 256 decode requests sharing a 4096-token prefix, own context U[0,1023] + 1 new token, 32/8 heads, head 128, block 16, bf16, seed 5",
    10: "workload 5 (same lengths and pool) over an fp8 e4m3 cache with per-kv-head scales; q/out bf16",
    11: "workload 3 (same lengths and pool) over a binary16 (fp16) cache; q/out fp16",
    12: "workload 5 (same lengths and pool) over a binary16 (fp16) cache; q/out fp16",
}


# Sources that determine each attention kernel's memory traffic: its own
# translation unit, the shared device headers and the host launch logic.
KERNEL_SOURCES = {
    "attn_valu_kernel": ["attn_valu.hip"],
    "attn_mfma_decode_kernel": ["attn_mfma_decode.hip", "attn_mfma_decode.h"],
    "attn_mfma_prefill_kernel": ["attn_mfma_prefill.hip", "attn_mfma_prefill.h"],
    "attn_mixed_kernel": ["attn_mixed.hip", "attn_mfma_decode.h", "attn_mfma_prefill.h",
                          "seq_order.hip"],
    "attn_mfma_prefix_kernel": ["attn_mfma_prefill.hip", "attn_mfma_prefill.h"],
}
COMMON_SOURCES = ["device_common.h", "attn_common.h", "api.cpp"]


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed, so that
    edits of comments alone keep a kernel's stored measurements valid."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code a kernel's counters depend on."""
    d = os.path.join(ROOT, "paged_kv_cache_50_amd", "csrc")
    h = hashlib.sha256()
    for f in COMMON_SOURCES + KERNEL_SOURCES[kernel]:
        h.update(f.encode())
        h.update(_code_only(open(os.path.join(d, f)).read()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload_name: str):
    """HBM bytes per launch of the workload's dominant kernel, measured by
    rocprofv3 FETCH_SIZE / WRITE_SIZE on the current source of that kernel,
    or None when no such measurement exists."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(workload_name)
        if not rec or rec.get("source_hash") != kernel_source_hash(rec["kernel"]):
            return None
    except Exception:
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------------ CPU baseline

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_rate(w, budget_s: float):
    """The fp64 oracle over the workload's (sequence, kv head) pairs in order,
    repeated until the time budget is used.  Returns (GB/s of algorithmic
    bytes, pairs done, seconds)."""
    import oracle
    kc, vc = w.k_cache, w.v_cache
    if w.slot_mapping is not None:
        kc, vc = kc.copy(), vc.copy()
        if w.dtype == "fp8":
            oracle.kv_cache_write_fp8(kc, vc, w.key_new, w.value_new, w.slot_mapping, w.block_size,
                                      w.k_scale, w.v_scale)
        else:
            oracle.kv_cache_write(kc, vc, w.key_new, w.value_new, w.slot_mapping, w.block_size)
    pairs = [(s, h) for s in range(w.num_seqs) for h in range(w.num_kv_heads)]
    # bytes of one (seq, kv head) pair: its K/V tokens plus q/out rows
    e = w.elem_bytes
    g = w.num_heads // w.num_kv_heads
    ql = w.query_lens
    done_bytes = 0
    done = 0
    t0 = time.perf_counter()
    while True:
        s, h = pairs[done % len(pairs)]
        oracle.paged_attention(w.q, kc, vc, w.block_tables, w.seq_lens, w.scale, w.block_size,
                               w.dtype, cu_seqlens_q=w.cu_seqlens_q, causal=w.causal,
                               pairs=[(s, h)], k_scale=w.k_scale, v_scale=w.v_scale,
                               window_left=w.window_left)
        keys = int(w.seq_lens[s]) if w.window_left < 0 else min(int(w.seq_lens[s]), w.window_left + 1)
        if w.common_prefix_len and keys:
            # the cascade's bytes: the shared prefix is credited once per batch
            keys += w.common_prefix_len // w.num_seqs - w.common_prefix_len
        done_bytes += (keys * 2 * w.head_size * e
                       + 2 * int(ql[s]) * g * w.head_size * w.io_bytes)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return done_bytes / el / 1e9, done, el, len(pairs)


def cpu_baseline(w, hosts: dict, budget_s: float = 10.0, single_budget_s: float = 3.0):
    """The oracle as it stands, on this host: on the headline workload with
    the BLAS pool set to the cores this process may use, and single-threaded
    on the three small decode workloads."""
    from threadpoolctl import threadpool_limits
    from paged_kv_cache_50_amd import workloads as W
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(cores):
        rate, done, el, npairs = oracle_rate(w, budget_s)
    rec = {"value": round(rate, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
           "sample": (f"{done} (sequence, kv head) pairs of {w.name} ({done / npairs:.2f} passes) "
                      f"in {el:.1f} s, numpy fp64 oracle, one pair at a time; BLAS pool of "
                      f"{cores} threads (the matrix products), the other NumPy steps on one"),
           "cpu_model": cpu_model(), "blas_threads": cores, "seconds": round(el, 2)}
    single = {}
    with threadpool_limits(1):
        for cfg in (1, 2, 3):
            wc = hosts.get(cfg) or W.make_config(cfg)
            r, d, e, n = oracle_rate(wc, single_budget_s)
            single[wc.name] = {"value": round(r, 4), "unit": "GB/s", "cores": 1,
                               "sample": f"{d} pairs ({d / n:.2f} passes) in {e:.1f} s"}
    rec["single_thread"] = single
    return rec


# ------------------------------------------------------------------ GPU measurement

def spin_cycles_for(us: float, dev) -> int:
    """GPU clock cycles of torch's spin kernel that last about `us` microseconds."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    n = 1 << 20
    torch.cuda._sleep(n)                           # warm
    a.record()
    torch.cuda._sleep(n)
    b.record()
    torch.cuda.synchronize()
    per_cycle_us = a.elapsed_time(b) * 1e3 / n
    return max(1000, int(us / max(per_cycle_us, 1e-9)))


def measure(w, args, dev, ps, cpu_label=False, graph=False) -> dict:
    """Warm-up, then exactly args.steps timed steps between two events on the
    stream (HIP events around the dominant kernel of one step in ten inside
    that region), then, outside it: the per-step distribution, for kernels
    under 50 us a re-timing of the dominant kernel with the queue kept ahead
    of the GPU, and with graph=True a HIP-graph replay.  Before the timed
    region a probe records the XCD the dispatcher starts launches on.

    Everything runs on the current stream except the graph capture, which
    needs streams of its own; capturing moves where the dispatcher starts
    the current stream's later launches, and the decode kernels' speed
    depends on that start by a few per cent, so callers measure every
    workload before they ask for a graph replay."""
    import numpy as np
    import torch
    from paged_kv_cache_50_amd import pagedkv, workloads as W

    dw = W.DevWorkload(w, device=dev)
    S, T = w.num_seqs, w.num_q_rows
    cascade = w.common_prefix_len > 0
    ws_bytes = pagedkv.workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_size,
                                       w.max_seq_len, ps)
    if cascade:
        ws_bytes = max(ws_bytes, pagedkv.cascade_workspace_bytes(
            S, T, w.num_heads, w.num_kv_heads, w.head_size, w.max_seq_len, w.common_prefix_len, ps))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    # A step whose bytes would stay in the 256 MB last-level cache re-reads
    # cached data: rotate copies of the caches so that consecutive steps
    # stream different memory (the tiny fp32 workload is labelled instead).
    B = W.algorithmic_bytes(w)
    caches = [(dw.k_cache, dw.v_cache)]
    cache_resident = False
    if B < 2 * MALL_BYTES:
        if w.k_cache.nbytes * 2 * 4 < (16 << 30) and B > (32 << 20):
            while len(caches) < 4:
                caches.append((dw.k_cache.clone(), dw.v_cache.clone()))
        else:
            cache_resident = True
    opts = pagedkv.CallOptions(**getattr(args, "call_options", {}))
    it = [0]

    def step(plain=False):
        kc, vc = caches[it[0] % len(caches)]
        it[0] += 1
        if w.slot_mapping is not None:
            pagedkv.kv_cache_write(kc, vc, dw.key_new, dw.value_new, dw.slot_mapping,
                                   k_scale=dw.k_scale, v_scale=dw.v_scale)
        if cascade and not plain:
            pagedkv.cascade_attention(dw.out, dw.q, kc, vc, dw.cu_seqlens_q, dw.seq_lens,
                                      dw.block_tables, dw.prefix_blocks, w.common_prefix_len,
                                      w.scale, w.max_query_len, w.max_seq_len, causal=w.causal,
                                      partition_size=ps, workspace=ws, options=opts)
        elif w.cu_seqlens_q is None:
            pagedkv.paged_attention_decode(dw.out, dw.q, kc, vc, dw.block_tables, dw.seq_lens,
                                           w.scale, w.max_seq_len, partition_size=ps, workspace=ws,
                                           k_scale=dw.k_scale, v_scale=dw.v_scale,
                                           window_left=w.window_left, options=opts)
        else:
            pagedkv.paged_attention_varlen(dw.out, dw.q, kc, vc, dw.cu_seqlens_q, dw.seq_lens,
                                           dw.block_tables, w.scale, w.max_query_len,
                                           w.max_seq_len, causal=w.causal, partition_size=ps,
                                           workspace=ws, k_scale=dw.k_scale, v_scale=dw.v_scale,
                                           window_left=w.window_left, options=opts)

    # Warm-up: at least args.warmup steps, and at least args.warmup_s seconds
    # of them, so the chip's clocks settle before timing.
    t0 = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t0 < args.warmup_s:
        step()
        n_warm += 1
        if n_warm % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    launched = opts.launched
    dispatch_xcds = pagedkv.xcd_probe(8)  # where this stream's launches start
    pagedkv.timing_read()                 # drop anything recorded before
    # HIP events around the dominant kernel of one step in ten (each record
    # adds a few microseconds of stream time, so they are sampled)
    pagedkv.timing_enable(True, every_n=10)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    kern_ms = pagedkv.timing_read()
    pagedkv.timing_enable(False)
    ms_per_step = ms_total / args.steps
    assert opts.launched == launched, "the launch form changed during timing"

    # Outside the timed region: the per-step distribution (each step between
    # its own events) and the step replayed as a HIP graph.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    per_step_us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
    graph_us = None
    if graph:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()                                  # warm the side stream
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            g0.record()
            for _ in range(args.steps):
                g.replay()
            g1.record()
            torch.cuda.synchronize()
            graph_us = g0.elapsed_time(g1) * 1e3 / args.steps
            del g
        except Exception as exc:                        # reported, never fatal
            print(f"[bench] graph replay unavailable: {exc}", file=sys.stderr, flush=True)

    # A HIP event that the GPU reaches before the host has queued the next
    # launch also times the host's launch latency, which is not negligible
    # beside a kernel of a few tens of microseconds.  For such kernels, time
    # them again with a spin kernel of about 150 us queued before each step:
    # the host has queued the step long before the GPU gets to its events.
    kavg_events = float(np.mean(kern_ms)) if kern_ms else None
    kavg = kavg_events
    kernel_ms_method = "HIP events around the kernel, one step in ten of the timed region"
    if kavg is not None and kavg < 0.05:
        cycles = spin_cycles_for(150.0, dev)
        pagedkv.timing_read()
        pagedkv.timing_enable(True, every_n=1)
        for _ in range(min(args.steps, 50)):
            torch.cuda._sleep(cycles)
            step()
        torch.cuda.synchronize()
        spun = pagedkv.timing_read()
        pagedkv.timing_enable(False)
        if spun:
            kavg = float(np.median(spun))
            kernel_ms_method = ("HIP events around the kernel, each step queued behind a "
                                "150 us spin kernel (outside the timed region, median of "
                                f"{len(spun)}); timed-region events gave "
                                f"{kavg_events * 1e3:.2f} us")

    plain_us = None
    if cascade:
        # the same step without the cascade (the plain varlen call), outside
        # the timed region
        for _ in range(3):
            step(plain=True)
        p0 = torch.cuda.Event(enable_timing=True)
        p1 = torch.cuda.Event(enable_timing=True)
        n_plain = max(1, args.steps // 5)
        p0.record()
        for _ in range(n_plain):
            step(plain=True)
        p1.record()
        torch.cuda.synchronize()
        plain_us = p0.elapsed_time(p1) * 1e3 / n_plain
    n_copies = len(caches)
    del caches, dw, ws
    torch.cuda.empty_cache()
    return {"ms_per_step": ms_per_step, "kernel_ms": kavg, "kernel_ms_method": kernel_ms_method,
            "kernel_launches_timed": len(kern_ms), "launched": launched,
            "per_step_us": per_step_us, "graph_us": graph_us, "plain_us": plain_us,
            "warmup_steps_run": n_warm, "cache_copies": n_copies,
            "dispatch_xcds": dispatch_xcds,
            "cache_resident": cache_resident, "bytes": B}


def roofline(w, m) -> dict:
    """The dominant kernel of the step, as the library reported it, against
    its roofline: HBM for decode rows, mixed launches and cascades (their
    ideal time is set by the bytes they move), the matrix cores for a
    chunked-prefill launch of its own."""
    import numpy as np
    from paged_kv_cache_50_amd import pagedkv as P, workloads as W
    ran = m["launched"]
    kavg = m["kernel_ms"]
    S, T = w.num_seqs, w.num_q_rows
    e = w.elem_bytes
    B = m["bytes"]
    out_bytes = T * w.num_heads * w.head_size * w.io_bytes
    write_bytes = W.algorithmic_bytes(w) - W.algorithmic_bytes(w, include_write=False)

    def hbm(main_bytes, kernel, **extra):
        achieved = main_bytes / (kavg * 1e-3) / 1e9 if kavg else None
        r = {"bound": "hbm", "achieved": round(achieved, 1) if achieved else None,
             "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(achieved / PEAK_HBM_GBS, 4) if achieved else None,
             "traffic": load_traffic(w.name), "kernel": kernel,
             "kernel_ms": round(kavg, 5) if kavg else None,
             "kernel_ms_method": m["kernel_ms_method"],
             "launches_timed": m["kernel_launches_timed"], "kernel_bytes": int(main_bytes)}
        r.update(extra)
        return r

    ql = w.query_lens
    pre_flops = 0
    for s in range(S):
        if ql[s] > 1:
            ctx = int(w.seq_lens[s]) - int(ql[s])
            pre_flops += 4 * w.num_heads * w.head_size * (int(ql[s]) * ctx
                                                          + int(ql[s]) * (int(ql[s]) + 1) // 2)
    if ran & (P.RAN_CASCADE_ONE | P.RAN_PREFIX):
        # the suffix pass's decode rows stream each request's own keys: its
        # own KV, q in, the suffix result out, the table entries past the
        # prefix; the one-launch form also reads the prefix's K/V once
        L = w.seq_lens.astype(np.int64)
        own = np.where(L > 0, L - w.common_prefix_len, 0)
        nb_own = np.where(L > 0, (L + w.block_size - 1) // w.block_size
                          - w.common_prefix_len // w.block_size, 0)
        main = (int(own.sum()) * 2 * w.num_kv_heads * w.head_size * e + 2 * out_bytes
                + 4 * int(nb_own.sum()) + 4 * (2 * S + 1))
        fused = bool(ran & P.RAN_CASCADE_ONE)
        if fused:
            main += (w.common_prefix_len * 2 * w.num_kv_heads * w.head_size * e
                     + 4 * (w.common_prefix_len // w.block_size))
        pf = W.prefix_flops(w)
        return hbm(main, "cascade launch (prefix pass + decode rows of the suffix pass)" if fused
                   else "cascade suffix pass (decode rows)", prefix_flops=pf,
                   prefix_tflops_over_kernel_time=round(pf / (kavg * 1e-3) / 1e12, 2)
                   if kavg and fused else None)
    if ran & P.RAN_MIXED:
        # prefill tiles and decode rows in one launch: its ideal time is set
        # by the bytes of all rows (HBM); the merge writes the split rows'
        # output, the slot write moves the new tokens
        main = B - out_bytes - write_bytes
        return hbm(main, "mixed prefill + decode launch", prefill_flops=int(pre_flops),
                   prefill_tflops_over_kernel_time=round(pre_flops / (kavg * 1e-3) / 1e12, 2)
                   if kavg else None)
    if ran & (P.RAN_PREFILL_MFMA | P.RAN_PREFILL_VALU):
        achieved = pre_flops / (kavg * 1e-3) / 1e12 if kavg else None
        pre_kv = sum(int(w.seq_lens[s]) for s in range(S) if ql[s] > 1)
        pre_rows = int(sum(int(x) for x in ql if x > 1))
        pre_bytes = (pre_kv * 2 * w.num_kv_heads * w.head_size * e
                     + 2 * pre_rows * w.num_heads * w.head_size * w.io_bytes)
        return {"bound": "mfma", "achieved": round(achieved, 2) if achieved else None,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4) if achieved else None,
                "traffic": load_traffic(w.name), "kernel": "prefill launch",
                "kernel_ms": round(kavg, 5) if kavg else None,
                "kernel_ms_method": m["kernel_ms_method"],
                "launches_timed": m["kernel_launches_timed"],
                "kernel_flops": int(pre_flops), "kernel_bytes": int(pre_bytes)}
    # decode rows: the partition kernel reads every KV token, q and the
    # metadata; when a merge launch follows, it writes out (charged there)
    main = B - write_bytes - (out_bytes if ran & P.RAN_SPLIT_MERGE else 0)
    kernel = ("matrix-core decode" if ran & P.RAN_DECODE_MFMA else "VALU decode") + \
        (" (fp8, two kv heads per wave)" if ran & P.RAN_DECODE_PAIRS else "")
    return hbm(main, kernel)


def record(w, m, steps, ps) -> dict:
    import numpy as np
    from paged_kv_cache_50_amd import pagedkv as P
    gbs = m["bytes"] / (m["ms_per_step"] * 1e-3) / 1e9
    rec = {"us_per_step": round(m["ms_per_step"] * 1e3, 2),
           "gb_per_s": round(gbs, 1),
           "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
           "tokens_per_s": round(w.num_q_rows / (m["ms_per_step"] * 1e-3), 1),
           "step_us_p10_p50_p90": [round(float(np.percentile(m["per_step_us"], q)), 2)
                                   for q in (10, 50, 90)],
           "graph_replay_us_per_step": round(m["graph_us"], 2) if m["graph_us"] else None,
           "kernels_launched": P.CallOptions(launched=m["launched"]).ran(),
           "warmup_steps_run": m["warmup_steps_run"],
           # XCD of the first workgroup of a launch on the timed stream: the
           # decode kernels lay out their columns for a start at XCD 0
           "dispatch_start_xcd": m["dispatch_xcds"][0],
           "roofline": roofline(w, m)}
    if m["cache_copies"] > 1:
        rec["cache_copies_rotated"] = m["cache_copies"]
    if m["cache_resident"]:
        rec["cache_resident"] = (f"{m['bytes'] / 1e6:.1f} MB per step fits the "
                                 f"{MALL_BYTES >> 20} MB last-level cache: a cache-resident rate, "
                                 "not an HBM one")
    return rec


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    # and at least this long: under sustained load the GPU settles within
    # about 3 s (the headline decode measured 352-355 us per step in the
    # first 2.5 s of a process and 342-345 us after 3 s; the mixed and fp8
    # steps were 4-6 % slower after 10 steps than after a second)
    ap.add_argument("--warmup-s", type=float, default=3.0)
    ap.add_argument("--workload", type=int, default=None, choices=list(range(1, 13)),
                    help="measure only this workload (default: the headline MHA decode, plus "
                         "workloads 3-12 as per_workload)")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--call-option", action="append", default=[], metavar="FIELD=VALUE",
                    help="set a pkv_call_options field for the measured calls (e.g. "
                         "mixed_launch=1: prefill chunks and decode rows in separate launches); "
                         "repeatable; the JSON line records them")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 launches) to calibrate "
                         "HBM byte counters, then exit")
    args = ap.parse_args()
    args.call_options = {}
    fields = {"decode_kernel", "prefill_kernel", "fp8_head_pairs", "mixed_launch", "cascade_launch"}
    for item in args.call_option:
        name, _, value = item.partition("=")
        if name not in fields or not value.lstrip("-").isdigit():
            ap.error(f"--call-option takes FIELD=INT with FIELD one of {sorted(fields)}")
        args.call_options[name] = int(value)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on exactly one GPU; --gpus N > 1 is not supported (the "
              "kernels work on one GPU's share of the batch)", file=sys.stderr)
        return 2

    import torch
    from paged_kv_cache_50_amd import pagedkv, workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        return 1
    pagedkv.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_launch": n,
                          "copy_calibration_bytes_written_per_launch": n, "launches": 5}))
        return 0

    head = HEADLINE if args.workload is None else args.workload
    hosts = {}

    def gen(cfg):
        t = time.time()
        w = W.make_config(cfg)
        print(f"[bench] generated {w.name} in {time.time() - t:.1f}s", file=sys.stderr, flush=True)
        return w

    w = gen(head)
    ps = w.partition_size if args.partition_size is None else args.partition_size
    m = measure(w, args, dev, ps)
    r = record(w, m, args.steps, ps)
    print(f"[bench] {w.name}: {r['us_per_step']} us/step", file=sys.stderr, flush=True)
    if head in (1, 2, 3):
        hosts[head] = w

    rec = {
        "metric": METRIC,
        "value": r["gb_per_s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 5),
        "us_per_step": r["us_per_step"],
        "pct_of_peak": r["pct_of_peak"],
        "tokens_per_s": r["tokens_per_s"],
        "step_us_p10_p50_p90": r["step_us_p10_p50_p90"],
        "graph_replay_us_per_step": r["graph_replay_us_per_step"],
        "dispatch_start_xcd": r["dispatch_start_xcd"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "f16": "f16",
                  "fp8": "fp8 e4m3 cache, bf16 q/out"}[w.dtype],
        "data": "synthetic (seeded; shapes and length distributions of the workload)",
        "config": {"workload": w.name, "description": WORKLOAD_DESC[head],
                   "num_seqs": w.num_seqs, "query_rows": w.num_q_rows, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_size": w.head_size,
                   "block_size": w.block_size, "kv_tokens": int(w.seq_lens.sum()),
                   "algorithmic_bytes": int(m["bytes"]), "partition_size": ps,
                   "parallelism": "single GPU"},
        "kernels_launched": r["kernels_launched"],
        "warmup_steps_run": r["warmup_steps_run"],
        **({"call_options": args.call_options} if args.call_options else {}),
        "roofline": r["roofline"],
    }
    for k in ("cache_resident", "cache_copies_rotated"):
        if k in r:
            rec[k] = r[k]
    if w.common_prefix_len > 0:
        rec["cascade"] = {"common_prefix_len": w.common_prefix_len,
                          "plain_form_bytes": int(W.algorithmic_bytes(w, shared_prefix=False)),
                          "plain_call_us_per_step": round(m["plain_us"], 2) if m["plain_us"] else None,
                          "speedup_over_plain_call": round(m["plain_us"] / (m["ms_per_step"] * 1e3), 2)
                          if m["plain_us"] else None}
    kept = []              # (workload, partition size, record) for the graph replays
    if args.workload is None:
        per = {}
        for cfg in PER_WORKLOAD:
            wc = gen(cfg)
            pc = wc.partition_size if args.partition_size is None else args.partition_size
            mc = measure(wc, args, dev, pc)
            rc = record(wc, mc, args.steps, pc)
            rc["description"] = WORKLOAD_DESC[cfg]
            rc["algorithmic_bytes"] = int(mc["bytes"])
            if wc.common_prefix_len > 0 and mc["plain_us"]:
                rc["plain_call_us_per_step"] = round(mc["plain_us"], 2)
            per[wc.name] = rc
            print(f"[bench] {wc.name}: {rc['us_per_step']} us/step", file=sys.stderr, flush=True)
            kept.append((wc, pc, rc))
            if cfg in (1, 2, 3):
                hosts[cfg] = wc
        rec["per_workload"] = per
    # Each step replayed as a HIP graph, after every timed region: capturing
    # a graph moves where the dispatcher starts later launches on this stream.
    warm = argparse.Namespace(**{**vars(args), "warmup": 10, "warmup_s": 0.2})
    for wg, pg, target in [(w, ps, rec)] + kept:
        g_us = measure(wg, warm, dev, pg, graph=True)["graph_us"]
        target["graph_replay_us_per_step"] = round(g_us, 2) if g_us is not None else None
    del kept
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, hosts)
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
