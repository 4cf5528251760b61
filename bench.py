"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input: for a
decode workload one paged_attention_decode call (partition kernel + split
merge) for one attention layer; for the mixed workload the slot write plus
one paged_attention_varlen call; for the shared-prefix workload the slot
write plus one cascade_attention call.  Inputs are resident in HBM before
timing.

Prints ONE JSON line (rank 0).  `value` is achieved HBM GB/s of the whole step
(algorithmic bytes / step time); `roofline` is the dominant kernel's achieved
rate against the MI355X peak, from per-launch HIP events recorded by the
library inside the timed region; `cpu_baseline` times the fp64 CPU oracle on
the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..10]
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
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published

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


def cpu_baseline(w, budget_s: float = 12.0):
    """fp64 oracle over the workload's sequences, repeated until the time
    budget is used (at least one pass over a bounded sample)."""
    import numpy as np
    import oracle
    from paged_kv_cache_50_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
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
    done_pairs = 0
    t0 = time.perf_counter()
    i = 0
    while True:
        s, h = pairs[i % len(pairs)]
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
        done_pairs += 1
        i += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    el = time.perf_counter() - t0
    sample = (f"{done_pairs} (sequence, kv head) pairs of the same workload "
              f"({done_pairs / len(pairs):.2f} passes), numpy fp64 oracle")
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle", "sample": sample, "seconds": round(el, 2)}


def pool_bench(seconds: float = 3.0) -> dict:
    """Host block pool under a serving-like loop (no GPU): 256 live requests
    of 1..2048-token prompts, a third of them sharing one of 8 cached
    2048-token system prompts; each round grows every request by one decode
    token, frees 8 finished requests and admits 8 new ones, and builds the
    block table and slot mapping of the step."""
    import numpy as np
    from paged_kv_cache_50_amd import pagedkv
    rng = np.random.default_rng(0)
    bs, nb = 16, 1 << 20
    pool = pagedkv.BlockPool(nb, bs, prefix_caching=True)
    systems = [rng.integers(0, 32000, 2048).astype(np.int32) for _ in range(8)]
    live, nxt, ops, tokens = {}, 0, 0, 0

    def admit():
        nonlocal nxt, ops, tokens
        n = int(rng.integers(1, 2048))
        toks = rng.integers(0, 32000, n).astype(np.int32)
        if rng.random() < 1 / 3:
            toks = np.concatenate([systems[int(rng.integers(8))], toks])
        if pool.allocate(nxt, len(toks), toks) >= 0:
            pool.cache_full_blocks(nxt, toks, len(toks))
            live[nxt] = len(toks)
            tokens += len(toks)
        nxt += 1
        ops += 2

    for _ in range(256):
        admit()
    t0 = time.perf_counter()
    rounds = 0
    while time.perf_counter() - t0 < seconds:
        for r in list(live):
            live[r] += 1
            pool.allocate(r, live[r])
        ops += len(live)
        tokens += len(live)
        reqs = sorted(live)
        pool.block_table(reqs, max(pool.num_blocks_of(r) for r in reqs))
        for r in reqs:
            pool.slot_mapping(r, live[r] - 1, 1)
        ops += 1 + len(reqs)
        for r in reqs[:8]:
            pool.free(r)
            del live[r]
        ops += 8
        for _ in range(8):
            admit()
        rounds += 1
    el = time.perf_counter() - t0
    pool.close()
    return {"metric": "host block pool operations/s", "value": round(ops / el, 1),
            "unit": "ops/s", "rounds_per_s": round(rounds / el, 1),
            "tokens_allocated_per_s": round(tokens / el, 1), "live_requests": len(live),
            "config": {"num_blocks": nb, "block_size": bs, "prefix_caching": True},
            "note": "host code through the C ABI from Python; each round is one decode step"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the default warm-up is long enough for the chip's clocks to settle: after
    # 10 steps the mixed and fp8 steps still ran 4-6 % slower than after 200
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5, 6, 7, 8, 9, 10])
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 launches) to calibrate "
                         "HBM byte counters, then exit")
    ap.add_argument("--pool", action="store_true",
                    help="only measure the host block pool (no GPU) and exit")
    args = ap.parse_args()
    if args.pool:
        print(json.dumps(pool_bench()), flush=True)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on exactly one GPU; --gpus N > 1 is not supported (the "
              "kernels work on one GPU's share of the batch)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from paged_kv_cache_50_amd import pagedkv, workloads as W
    from tests import gpu_util as G

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

    t_gen = time.time()
    w = W.make_config(args.workload)
    print(f"[bench] generated {w.name} in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)
    ps = w.partition_size if args.partition_size is None else args.partition_size
    dw = G.DevWorkload(w, device=dev)
    S, T = w.num_seqs, w.num_q_rows
    cascade = w.common_prefix_len > 0
    ws_bytes = pagedkv.workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_size,
                                       w.max_seq_len, ps)
    if cascade:
        ws_bytes = max(ws_bytes, pagedkv.cascade_workspace_bytes(
            S, T, w.num_heads, w.num_kv_heads, w.head_size, w.max_seq_len, w.common_prefix_len, ps))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def step(plain=False):
        if w.slot_mapping is not None:
            pagedkv.kv_cache_write(dw.k_cache, dw.v_cache, dw.key_new, dw.value_new,
                                   dw.slot_mapping, k_scale=dw.k_scale, v_scale=dw.v_scale)
        if cascade and not plain:
            pagedkv.cascade_attention(dw.out, dw.q, dw.k_cache, dw.v_cache, dw.cu_seqlens_q,
                                      dw.seq_lens, dw.block_tables, dw.prefix_blocks,
                                      w.common_prefix_len, w.scale, w.max_query_len,
                                      w.max_seq_len, causal=w.causal, partition_size=ps,
                                      workspace=ws)
        elif w.cu_seqlens_q is None:
            pagedkv.paged_attention_decode(dw.out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables,
                                           dw.seq_lens, w.scale, w.max_seq_len,
                                           partition_size=ps, workspace=ws, k_scale=dw.k_scale,
                                           v_scale=dw.v_scale, window_left=w.window_left)
        else:
            pagedkv.paged_attention_varlen(dw.out, dw.q, dw.k_cache, dw.v_cache, dw.cu_seqlens_q,
                                           dw.seq_lens, dw.block_tables, w.scale, w.max_query_len,
                                           w.max_seq_len, causal=w.causal, partition_size=ps,
                                           workspace=ws, k_scale=dw.k_scale, v_scale=dw.v_scale,
                                           window_left=w.window_left)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
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

    # Outside the timed region: the per-step distribution (each step between
    # its own events) and the step replayed as a HIP graph (no host launch
    # overhead).  Same workload, same buffers.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    per_step_us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
    graph_us = None
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

    plain_us = None
    if cascade:
        # the same step without the cascade (the plain varlen call), for
        # comparison; outside the timed region
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

    B = W.algorithmic_bytes(w)
    e = w.elem_bytes
    out_bytes = T * w.num_heads * w.head_size * w.io_bytes
    gbs = B / (ms_per_step * 1e-3) / 1e9
    kavg = float(np.mean(kern_ms)) if kern_ms else None
    if cascade:
        # the dominant launch is the suffix pass (decode rows streaming each
        # request's own keys): its own KV, q in, the suffix result out, and
        # the table entries past the prefix
        L = w.seq_lens.astype(np.int64)
        own = np.where(L > 0, L - w.common_prefix_len, 0)
        nb_own = np.where(L > 0, (L + w.block_size - 1) // w.block_size
                          - w.common_prefix_len // w.block_size, 0)
        main_bytes = (int(own.sum()) * 2 * w.num_kv_heads * w.head_size * e + 2 * out_bytes
                      + 4 * int(nb_own.sum()) + 4 * (2 * S + 1))
        fused = (os.environ.get("PKV_CASCADE_FUSED", "1") != "0" and w.max_query_len <= 1
                 and w.num_heads // w.num_kv_heads >= 4)
        if fused:
            # one launch also runs the prefix pass: the prefix's keys and
            # values once
            main_bytes += (w.common_prefix_len * 2 * w.num_kv_heads * w.head_size * e
                           + 4 * (w.common_prefix_len // w.block_size))
        achieved = main_bytes / (kavg * 1e-3) / 1e9 if kavg else None
        roof = {"bound": "hbm", "achieved": round(achieved, 1) if achieved else None,
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4) if achieved else None,
                "traffic": load_traffic(w.name),
                "kernel_ms": round(kavg, 5) if kavg else None, "launches": len(kern_ms),
                "kernel_bytes": int(main_bytes),
                "kernel": ("cascade launch (prefix pass + decode rows of the suffix pass)"
                           if fused else "cascade suffix pass (decode rows)"),
                "prefix_flops": W.prefix_flops(w),
                "prefix_tflops_over_kernel_time":
                    round(W.prefix_flops(w) / (kavg * 1e-3) / 1e12, 2) if kavg and fused else None}
    elif w.cu_seqlens_q is None:
        # the partition kernel reads every KV token, q and the metadata; the
        # merge kernel writes out (charged to the merge, not here)
        main_bytes = B - out_bytes
        achieved = main_bytes / (kavg * 1e-3) / 1e9 if kavg else None
        roof = {"bound": "hbm", "achieved": round(achieved, 1) if achieved else None,
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4) if achieved else None,
                "traffic": load_traffic(w.name),
                "kernel_ms": round(kavg, 5) if kavg else None, "launches": len(kern_ms),
                "kernel_bytes": int(main_bytes)}
    else:
        flops = W.attention_flops(w)
        ql = w.query_lens
        pre_flops = 0
        for s in range(S):
            if ql[s] > 1:
                ctx = int(w.seq_lens[s]) - int(ql[s])
                pre_flops += 4 * w.num_heads * w.head_size * (int(ql[s]) * ctx + int(ql[s]) * (int(ql[s]) + 1) // 2)
        # bytes the prefill part must move: its sequences' keys and values
        # once, their query rows in and out
        pre_kv = sum(int(w.seq_lens[s]) for s in range(S) if ql[s] > 1)
        pre_rows = int(sum(int(x) for x in ql if x > 1))
        pre_bytes = (pre_kv * 2 * w.num_kv_heads * w.head_size * e
                     + 2 * pre_rows * w.num_heads * w.head_size * w.io_bytes)
        mixed = os.environ.get("PKV_MIXED", "1") != "0" and w.dtype in ("bf16", "fp8") and ps != -1
        if mixed:
            # one launch carries the prefill tiles and the decode rows: its
            # ideal time is set by the bytes of all rows (HBM), not by the
            # prefill flops
            main_bytes = B - out_bytes - (W.algorithmic_bytes(w) - W.algorithmic_bytes(w, include_write=False))
            achieved = main_bytes / (kavg * 1e-3) / 1e9 if kavg else None
            roof = {"bound": "hbm", "achieved": round(achieved, 1) if achieved else None,
                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4) if achieved else None,
                    "traffic": load_traffic(w.name),
                    "kernel_ms": round(kavg, 5) if kavg else None, "launches": len(kern_ms),
                    "kernel_bytes": int(main_bytes), "kernel": "mixed prefill + decode launch",
                    "prefill_flops": int(pre_flops),
                    "prefill_tflops_over_kernel_time": round(pre_flops / (kavg * 1e-3) / 1e12, 2) if kavg else None}
        else:
            achieved = pre_flops / (kavg * 1e-3) / 1e12 if kavg else None
            roof = {"bound": "mfma", "achieved": round(achieved, 2) if achieved else None,
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4) if achieved else None,
                    "traffic": load_traffic(w.name),
                    "kernel_ms": round(kavg, 5) if kavg else None, "launches": len(kern_ms),
                    "kernel_flops": int(pre_flops), "kernel_bytes": int(pre_bytes),
                    "kernel": "prefill launch", "total_flops": flops}

    rec = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "step_us_p10_p50_p90": [round(float(np.percentile(per_step_us, q)), 2) for q in (10, 50, 90)],
        "graph_replay_us_per_step": round(graph_us, 2) if graph_us else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8 e4m3 cache, bf16 q/out"}[w.dtype],
        "data": "synthetic (seeded; shapes and length distributions of the workload)",
        "config": {"workload": w.name, "description": WORKLOAD_DESC[args.workload],
                   "num_seqs": S, "query_rows": T, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_size": w.head_size,
                   "block_size": w.block_size, "kv_tokens": int(w.seq_lens.sum()),
                   "algorithmic_bytes": int(B), "partition_size": ps,
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if cascade:
        rec["cascade"] = {"common_prefix_len": w.common_prefix_len,
                          "plain_form_bytes": int(W.algorithmic_bytes(w, shared_prefix=False)),
                          "plain_call_us_per_step": round(plain_us, 2) if plain_us else None,
                          "speedup_over_plain_call": round(plain_us / (ms_per_step * 1e3), 2)
                          if plain_us else None}
    del dw
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
