#!/usr/bin/env python3
"""Throughput of causal sparse attention on one MI355X.

One step = the whole DSA-style prefill hot path on the 64K workload (T = 65,536 tokens,
16 query heads on 1 KV head of dim 128, bf16; indexer of 4 heads x 64; top-2048 per query
united with a 128-token window): the fused indexer -> top-k (sa_indexer_topk) in one call
over all 65,536 rows (``--chunk`` splits it into row chunks), then sa_sparse_attn_fwd
(``--indices two-step`` builds the indices with sa_indexer_scores + sa_topk_select, in
chunks of at most 32,768 rows, instead).  Inputs are seeded synthetic tensors
(sa_synth), resident in HBM before the timed region.  ``value`` is query tokens per second
of the whole step.

The JSON line also carries the roofline of the dominant kernel (the sparse attention: its
algorithmic bytes per launch, K/V rows gathered plus Q, O and the index rows, over its
average HIP-event duration, against the aggregate L2 read bandwidth, the level that serves
the gathered rows; its HBM side from the byte counters beside it), a read probe of the
memory hierarchy (L2-, Infinity-Cache- and HBM-resident buffers), the float64 CPU oracle
timed on every workload (full runs or bounded, labelled samples), and the other hot-path
rows, each timed cold (a 1 GiB buffer rewritten before every call) with the warm figure
beside: the sparse-attention backward (64K), E4M3 indexer inputs (64K), NSA's three
branches (prefill 64K, decode 32 x 128K), fixed-graph attention (16K, 64K, 128K),
block-sparse decode (32 x 128K) and cross-layer index reuse (128K, F,S,S,S).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--chunk ROWS] [--no-extra]
       [--no-cpu] [--only attn|prefill] [--extra all|bwd,e4m3,nsa,graph,decode,reuse]
       [--bwd-rows N] [--cpu all|3]
       python bench.py --traffic-from DIR   (profiles/traffic.json from counter runs)
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
# Aggregate L2 read bandwidth: 8 XCDs x 16 L2 channels x 128 bytes per clock per channel
# (the per-XCD L2 organisation AMD documents for CDNA 3 and keeps in CDNA 4: 4 MB of L2
# per XCD) x 2.4 GHz.
L2_PEAK_GBS = 8 * 16 * 128 * 2.4

ROOT = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCES = ("k_sparse_attn.hip", "attn_tile.h", "sa_device.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def attn_sources_hash() -> str:
    """sha256 over the sources of the sparse-attention kernel."""
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, "long_context_sparse_13_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per attention launch from the committed counter runs, or None when the
    kernel sources changed since those counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != attn_sources_hash():
        return None
    return t.get("bytes_per_launch")


TRAFFIC_CMD = ("rocprofv3 --pmc {c} --kernel-include-regex 'sparse_attn|copy|elementwise|indexer|topk' "
               "--output-format csv -d {d} -o {o} -- python3 bench.py --steps 2 --warmup 1 "
               "--no-cpu --no-extra --copy-probe 1024")


def write_traffic(base: str) -> dict:
    """profiles/traffic.json from two rocprofv3 counter runs of this script (TRAFFIC_CMD
    with FETCH_SIZE into base/fetch, -o f, then WRITE_SIZE into base/write, -o w): the
    attention launch's mean FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by
    what the same counter reads for the 1 GiB device-to-device copy of --copy-probe 1024
    (1,048,576 KiB moved each way), stored with the hash of the kernel's sources."""
    import csv
    import statistics

    def per_dispatch(f):
        agg, names, grid = {}, {}, {}
        with open(f) as fh:
            for r in csv.DictReader(fh):
                d = int(r["Dispatch_Id"])
                agg[d] = agg.get(d, 0.0) + float(r["Counter_Value"])
                names[d] = r["Kernel_Name"]
                grid[d] = int(r["Grid_Size"])
        return agg, names, grid

    def vals(agg, names, grid, key, full_grid=False):
        sel = [d for d in sorted(agg) if key in names[d]]
        if full_grid:  # the whole-T launches only (not the two-stream row ranges)
            g = max(grid[d] for d in sel)
            sel = [d for d in sel if grid[d] == g]
        return [agg[d] for d in sel]

    fa, fn, fg = per_dispatch(os.path.join(base, "fetch", "f_counter_collection.csv"))
    wa, wn, wg = per_dispatch(os.path.join(base, "write", "w_counter_collection.csv"))
    ff = 1048576.0 / max(vals(fa, fn, fg, "copyBuffer"))
    wf = 1048576.0 / max(vals(wa, wn, wg, "copyBuffer"))
    # the full 64K attention launches
    af = statistics.mean(vals(fa, fn, fg, "sparse_attn_mfma<128, true>", True))
    aw = statistics.mean(vals(wa, wn, wg, "sparse_attn_mfma<128, true>", True))
    t = {"kernel": "sparse_attn_mfma<128, true>", "workload": "dsa-prefill-bf16-64k",
         "source_sha256": attn_sources_hash(), "fetch_kib_per_launch": af,
         "write_kib_per_launch": aw, "fetch_factor": ff, "write_factor": wf,
         "bytes_per_launch": af * 1024 * ff + aw * 1024 * wf,
         "commands": [TRAFFIC_CMD.format(c="FETCH_SIZE", d=os.path.join(base, "fetch"), o="f"),
                      TRAFFIC_CMD.format(c="WRITE_SIZE", d=os.path.join(base, "write"), o="w")]}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
    return t


def memory_probe(torch, dev):
    """Read bandwidth of three buffers with the probe kernel of libsa_probe.so (16-byte
    loads, 1 KB contiguous per wavefront instruction), in GB/s: 16 MiB split in eight 2 MiB
    slices, each re-read by the workgroups of one XCD (L2-resident); 128 MiB streamed by
    every XCD (larger than the L2s, inside the 256 MB Infinity Cache); 4 GiB (HBM)."""
    import ctypes
    path = os.path.join(ROOT, "long_context_sparse_13_amd", "libsa_probe.so")
    L = ctypes.CDLL(path)
    f = L.sa_probe_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    cases = (("l2", 16 << 20, 8, 2000, 2048), ("infinity_cache", 128 << 20, 1, 40, 2048),
             ("hbm", 4 << 30, 1, 1, 8192))
    out = {}
    sink = torch.empty(8192 * 256, dtype=torch.int32, device=dev)
    for name, nbytes, slices, passes, wgs in cases:
        buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
        st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        ms = []
        for it in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = f(ctypes.c_void_p(buf.data_ptr()), nbytes, slices, passes, wgs,
                   ctypes.c_void_p(sink.data_ptr()), st)
            e1.record()
            if rc != 0:
                raise RuntimeError(f"read probe launch failed ({rc})")
            torch.cuda.synchronize()
            if it:
                ms.append(e0.elapsed_time(e1))
        out[name + "_GBps"] = nbytes * passes / (min(ms) * 1e-3) / 1e9
        del buf
    torch.cuda.empty_cache()
    return out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=65536, help="indexer/top-k rows per call")
    ap.add_argument("--indices", choices=["fused", "two-step"], default="fused",
                    help="how the step builds the indices: sa_indexer_topk, or "
                         "sa_indexer_scores + sa_topk_select")
    ap.add_argument("--no-extra", action="store_true", help="skip graph/decode/reuse rows")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--traffic-from", metavar="DIR", default=None,
                    help="write profiles/traffic.json from the counter runs under DIR and exit")
    ap.add_argument("--extra", default="all",
                    help="the extra rows to run: all, or a comma list of bwd, e4m3, nsa, graph, "
                         "decode, reuse (for profiling runs)")
    ap.add_argument("--bwd-rows", type=int, default=32768,
                    help="query rows per chunk of the backward's partial-row workspace")
    ap.add_argument("--only", choices=["attn", "prefill"], default=None,
                    help="time only one part (for profiling runs)")
    ap.add_argument("--cpu", default="all", choices=["all", "3"],
                    help="the CPU oracle on every workload, or on the 64K one only")
    ap.add_argument("--no-probe", action="store_true", help="skip the memory read probe")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="first copy MB megabytes 3 times with torch (a plain copy kernel of "
                         "known size, to calibrate the HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timer:
    """HIP events on torch's current stream (the stream every sa_* call launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        self.pairs.setdefault(name, []).append((e0, e1))

    def ms(self, name):
        ps = self.pairs.get(name, [])
        return sum(a.elapsed_time(b) for a, b in ps), len(ps)


def main():
    args = parse()
    if args.traffic_from:
        t = write_traffic(args.traffic_from)
        print(json.dumps(t))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        print("bench.py: multi-GPU runs are not implemented (the path is sharded by design "
              "only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import long_context_sparse_13_amd as sa
    import sa_synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    sa.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 3 x {args.copy_probe} MiB")
        del src, dst

    def to_dev(a, dtype):
        t = torch.from_numpy(np.ascontiguousarray(a))
        t = t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)
        return t.to(dev)

    W3 = sa_synth.WORKLOADS[3]
    p = W3.params
    T, Hq, Hkv, D, HI, DI = p["T"], p["Hq"], p["Hkv"], p["D"], p["H_I"], p["D_I"]
    topk, window, scale = p["topk"], p["window"], p["scale"]
    log(f"generating the 64K prefill inputs (seed {W3.seed})")
    x = sa_synth.prefill_inputs(W3.seed, 1, T, Hq, Hkv, D, HI, DI, "bf16")
    qi, ki, w = to_dev(x["qi"], "bf16"), to_dev(x["ki"], "bf16"), to_dev(x["w"], "f32")
    q, k, v = to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16")
    chunk = min(args.chunk, T)
    chunk2 = min(chunk, 32768)  # the two-step path's row chunks (its score buffer: 8.6 GB)
    ld = ((T + 3) // 4) * 4
    fused = args.indices == "fused"
    scores = torch.empty((1, chunk2, ld), dtype=torch.float32, device=dev)
    # the last row chunk is the longest, so its workspace serves every chunk
    ws = torch.empty(sa.sa_indexer_topk_workspace(1, T, HI, DI, T - chunk, T, topk),
                     dtype=torch.uint8, device=dev)
    idx = torch.full((1, T, topk), -1, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    tm = Timer(torch)

    def two_step_indices(timer):
        for r0 in range(0, T, chunk2):
            r1 = min(T, r0 + chunk2)
            sc = scores[:, : r1 - r0]  # (the last chunk may be shorter; a prefix stays contiguous)
            timer.run("indexer", lambda: sa.sa_indexer_scores(qi, ki, w, r0, r1, sc, ld))
            timer.run("topk", lambda: sa.sa_topk_select(sc, topk, T, r0, r1, idx, ld))

    def fused_indices(timer):
        for r0 in range(0, T, chunk):
            r1 = min(T, r0 + chunk)
            timer.run("indexer_topk", lambda: sa.sa_indexer_topk(qi, ki, w, topk, r0, r1, idx, ws))

    prefill_indices = fused_indices if fused else two_step_indices

    def step(timer):
        if args.only != "attn":
            prefill_indices(timer)
        if args.only != "prefill":
            timer.run("attn", lambda: sa.sa_sparse_attn_fwd(q, k, v, idx, window, scale, out=out))

    if args.only == "attn":
        prefill_indices(Timer(torch))
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step(Timer(torch))
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step(tm)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / args.steps
    kern = {n: tm.ms(n) for n in ("indexer_topk", "indexer", "topk", "attn")}
    log("timed: " + ", ".join(f"{n} {m / max(1, args.steps):.3f} ms/step ({c} launches)"
                              for n, (m, c) in kern.items()))

    # ---- algorithmic work of the attention launch (exact |S_t| from the indices)
    tt = torch.arange(T, device=dev, dtype=torch.int32)[:, None]
    listed = ((idx[0] >= 0) & (idx[0] <= tt - window)).sum(dim=1, dtype=torch.int64)
    win = torch.clamp(torch.arange(T, device=dev) + 1, max=window)
    n_sel = int((listed + win).sum().item())
    bytes_kv = n_sel * 2 * D * 2                       # K and V rows, fetched once per group
    bytes_qo = T * Hq * D * 2 * 2                      # Q read, O written
    bytes_idx = T * topk * 4
    attn_bytes = bytes_kv + bytes_qo + bytes_idx
    attn_flops = 4.0 * Hq * D * n_sel
    attn_ms, attn_n = kern["attn"]
    attn_avg_ms = attn_ms / max(1, attn_n)
    achieved = attn_bytes / (attn_avg_ms * 1e-3) / 1e9 if attn_n else None

    # the other way of building the indices, timed beside (not part of the step)
    other = Timer(torch)
    if args.only != "attn":
        (two_step_indices if fused else fused_indices)(Timer(torch))
        for _ in range(3):
            (two_step_indices if fused else fused_indices)(other)
        torch.cuda.synchronize()
        if fused:
            prefill_indices(Timer(torch))  # leave the step's own indices in idx
            torch.cuda.synchronize()
    # the same step on two streams: the attention of a row chunk starts as soon as that
    # chunk's indices exist, beside the next chunk's index build (sa_sparse_attn_fwd_rows);
    # two chunks when the step makes one call
    two_streams = None
    pchunk = chunk if chunk < T else (T + 1) // 2
    if fused and args.only is None:
        s_idx, s_att = torch.cuda.Stream(), torch.cuda.Stream()

        def piped():
            cur = torch.cuda.current_stream()
            s_idx.wait_stream(cur)
            s_att.wait_stream(cur)
            for r0 in range(0, T, pchunk):
                r1 = min(T, r0 + pchunk)
                with torch.cuda.stream(s_idx):
                    sa.sa_indexer_topk(qi, ki, w, topk, r0, r1, idx, ws)
                    ev = torch.cuda.Event()
                    ev.record(s_idx)
                s_att.wait_event(ev)
                with torch.cuda.stream(s_att):
                    sa.sa_sparse_attn_fwd_rows(q, k, v, idx, window, scale, r0, r1, out)
            cur.wait_stream(s_idx)
            cur.wait_stream(s_att)

        out_seq = out.clone()
        for _ in range(args.warmup):
            piped()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            piped()
        e1.record()
        torch.cuda.synchronize()
        ms_p = e0.elapsed_time(e1) / args.steps
        two_streams = {"ms_per_step": ms_p, "query_tokens_per_s": T / (ms_p * 1e-3),
                       "vs_sequential_step": ms_step / ms_p, "row_chunk": pchunk,
                       "same_output": bool(torch.equal(out_seq, out))}
        log(f"two streams: {ms_p:.3f} ms/step (sequential {ms_step:.3f})")
        del out_seq
    tsrc = other if fused else tm
    nsteps_two = 3 if fused else args.steps
    idx_ms = tsrc.ms("indexer")[0] / nsteps_two
    topk_ms = tsrc.ms("topk")[0] / nsteps_two
    fsrc = tm if fused else other
    nsteps_f = args.steps if fused else 3
    fused_ms = fsrc.ms("indexer_topk")[0] / nsteps_f
    n_recomputed = int(ws[:4].view(torch.int32).item()) if fused_ms else None
    n_pairs = T * (T + 1) // 2
    probe = None if args.no_probe else memory_probe(torch, dev)
    if probe:
        log("read probe: " + ", ".join(f"{k} {v:.0f}" for k, v in probe.items()))
    traffic = measured_traffic()
    bytes_hbm = T * Hkv * D * 2 * 2 + bytes_qo + bytes_idx   # K, V once; Q, O; idx
    l2_frac = achieved / L2_PEAK_GBS if achieved else None
    res = {
        "metric": "sparse-attn fwd query-tokens/s at 64K ctx, top-k=2048; % HBM/MFMA roofline",
        "value": T / (ms_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 tensors, indexer weights U(0,1))",
        "config": {"workload": "dsa-prefill-bf16-64k: indexer(4x64) + top-2048 + window-128 "
                               "sparse attention, T=65536, Hq=16, Hkv=1, D=128, batch 1",
                   "global_batch": 1, "seq_len": T, "parallelism": "none (1 GPU)",
                   "row_chunk": chunk, "indices": args.indices, "only": args.only},
        "step_breakdown_ms": ({"indexer_topk": fused_ms} if fused else
                              {"indexer": idx_ms, "topk": topk_ms}) | {"sparse_attn": attn_avg_ms},
        "sparse_attn_query_tokens_per_s": T / (attn_avg_ms * 1e-3) if attn_n else None,
        "two_streams": two_streams,
        "roofline": {
            "kernel": "sparse_attn_mfma<128, true>",
            # the gathered K/V rows (33.5 MB of keys and values, re-read ~2,100 times) are
            # served by the L2 and the Infinity Cache, not by HBM: the bound is the
            # aggregate L2 read bandwidth
            "bound": "l2",
            "achieved": achieved,
            "peak": L2_PEAK_GBS,
            "unit": "GB/s",
            "frac": l2_frac,
            "traffic": traffic,
            "peak_source": "8 XCDs x 16 L2 channels x 128 B/clk x 2.4 GHz (CDNA 3/4 L2 "
                           "organisation); checked by the read probe (l2_probe_GBps)",
            "algorithmic_bytes_per_launch": attn_bytes,
            "selected_keys_per_launch": n_sel,
            "avg_launch_ms": attn_avg_ms,
            "l2_probe_GBps": probe["l2_GBps"] if probe else None,
            "frac_of_l2_probe": (achieved / probe["l2_GBps"]) if probe and achieved else None,
            "hbm": {
                "compulsory_bytes": bytes_hbm,
                "compulsory_GBps": bytes_hbm / (attn_avg_ms * 1e-3) / 1e9 if attn_n else None,
                "compulsory_frac": (bytes_hbm / (attn_avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
                if attn_n else None,
                "past_l2_bytes": traffic,
                "past_l2_GBps": traffic / (attn_avg_ms * 1e-3) / 1e9 if traffic and attn_n
                else None,
                "past_l2_frac": traffic / (attn_avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS
                if traffic and attn_n else None,
                "note": "past_l2 = FETCH_SIZE + WRITE_SIZE (copy-calibrated): L2 misses, "
                        "which include Infinity Cache hits; compulsory = K, V once + Q + O + idx",
            },
            "mfma": {
                "tflops": attn_flops / (attn_avg_ms * 1e-3) / 1e12 if attn_n else None,
                "frac": attn_flops / (attn_avg_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS
                if attn_n else None,
            },
        },
        "memory_probe": probe,
        "indexer_topk": {
            "avg_ms_per_step": fused_ms,
            "effective_tflops": (n_pairs * 2 * HI * DI) / (fused_ms * 1e-3) / 1e12
            if fused_ms else None,
            "mfma_frac": ((n_pairs * 2 * HI * DI) / (fused_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS)
            if fused_ms else None,
            "rows_recomputed_last_chunk": n_recomputed,
            "vs_two_step": (idx_ms + topk_ms) / fused_ms if fused_ms and idx_ms else None,
        },
        "indexer": {
            "avg_ms_per_step": idx_ms,
            "tflops": (n_pairs * 2 * HI * DI) / (idx_ms * 1e-3) / 1e12 if idx_ms else None,
            "mfma_frac": ((n_pairs * 2 * HI * DI) / (idx_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS)
            if idx_ms else None,
            "score_write_GBps": n_pairs * 4 / (idx_ms * 1e-3) / 1e9 if idx_ms else None,
        },
        "topk": {
            "avg_ms_per_step": topk_ms,
            "score_read_GBps": n_pairs * 4 / (topk_ms * 1e-3) / 1e9 if topk_ms else None,
        },
        "context_figures_from_pages": {
            "SpatialLM-Mini": "2.47x training speedup at 16,384 tokens, RTX 3050 8 GB",
            "IndexCache": "prefill 19.5 s -> 10.7 s at 200K tokens, GLM-4.7 Flash",
            "NSA": "9x forward speedup at 64K, NVIDIA GPUs",
        },
    }
    del scores, ws
    torch.cuda.empty_cache()

    keep = {}  # host inputs of the decode and reuse workloads, for the CPU oracle
    want_host = not args.no_cpu and args.cpu == "all"
    if not args.no_extra:
        res["rows"] = extra_rows(torch, np, sa, sa_synth, to_dev, args, q, k, v, idx,
                                 keep if want_host else None)
    del q, k, v, idx, qi, ki, w, out
    torch.cuda.empty_cache()

    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(np, sa_synth, x, p, args.cpu_seconds, args.cpu, keep)
    print(json.dumps(res), flush=True)


def extra_rows(torch, np, sa, sa_synth, to_dev, args, q64, k64, v64, idx64, keep=None):
    """The other hot-path rows.  ``keep`` (a dict, or None) receives the host inputs of the
    decode and index-reuse workloads for the CPU oracle."""
    dev = q64.device
    rows = {}
    reps = 20
    groups = None if args.extra == "all" else set(args.extra.split(","))

    def want(name):
        return groups is None or name in groups

    def timed(fn, n):
        """Warm: n calls back to back on the same inputs (caches keep what fits)."""
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # 1 GiB (four times the Infinity Cache, far more than the L2s) read and rewritten
    # before each cold call
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)

    def timed_cold(fn, n):
        """Cold: the median of n calls, each timed alone right after the flush."""
        fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(n):
            flush.add_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        return ts[len(ts) // 2]

    # ---- the backward of the 64K sparse attention (same q, k, v, indices; a seeded bf16
    # upstream gradient), with the forward timed beside it
    if want("bwd"):
        log("sparse attention backward (64K)")
        p3 = sa_synth.WORKLOADS[3].params
        o_f = torch.empty_like(q64)
        t_fwd = timed(lambda: sa.sa_sparse_attn_fwd(q64, k64, v64, idx64, p3["window"], p3["scale"],
                                                    out=o_f), 2)
        o_f, lse_f = sa.sa_sparse_attn_fwd(q64, k64, v64, idx64, p3["window"], p3["scale"],
                                           return_lse=True)
        g_out = torch.randn(q64.shape, generator=torch.Generator(device=dev).manual_seed(1006),
                            device=dev, dtype=torch.float32).to(torch.bfloat16)
        dq_b = torch.empty(q64.shape, dtype=torch.float32, device=dev)
        dk_b = torch.empty(k64.shape, dtype=torch.float32, device=dev)
        dv_b = torch.empty(v64.shape, dtype=torch.float32, device=dev)
        B3, T3b, Hkv3, D3 = k64.shape[0], k64.shape[1], k64.shape[2], k64.shape[3]
        topk3b = idx64.shape[2]
        ws_n = sa.sa_sparse_attn_bwd_workspace(B3, T3b, Hkv3, D3, topk3b, p3["window"], args.bwd_rows)
        ws_b = torch.empty(ws_n, dtype=torch.uint8, device=dev)
        t_bwd = timed(lambda: sa.sa_sparse_attn_bwd(q64, k64, v64, idx64, p3["window"], p3["scale"],
                                                    o_f, lse_f, g_out, dq_b, dk_b, dv_b,
                                                    workspace=ws_b), 3)
        dk_w, dv_w = dk_b.clone(), dv_b.clone()
        t_atom = timed(lambda: sa.sa_sparse_attn_bwd(q64, k64, v64, idx64, p3["window"], p3["scale"],
                                                     o_f, lse_f, g_out, dq_b, dk_b, dv_b), 1)
        # the two ways of summing dK / dV agree (the workspace path rounds each pair's
        # contribution to bf16)
        agree = max(float((a - b).abs().max() / b.abs().max()) for a, b in ((dk_w, dk_b), (dv_w, dv_b)))
        tt = torch.arange(T3b, device=dev, dtype=torch.int32)[:, None]
        pairs = int((((idx64[0] >= 0) & (idx64[0] <= tt - p3["window"])).sum(dtype=torch.int64)
                     + torch.clamp(torch.arange(T3b, device=dev) + 1, max=p3["window"]).sum()).item())
        part_bytes = pairs * 4 * D3 * 2  # each pair's bf16 [dK | dV] row written once, read once
        rows["sparse_attn_bwd_64k"] = {
            "ms": t_bwd, "forward_ms": t_fwd, "bwd_over_fwd": t_bwd / t_fwd,
            "query_tokens_per_s": q64.shape[1] / (t_bwd * 1e-3),
            "path": f"partial rows, workspace {ws_n / 2**30:.1f} GiB (chunks of {args.bwd_rows} rows)",
            "atomic_path_ms": t_atom, "max_rel_diff_vs_atomic": agree,
            "pairs": pairs, "partial_row_bytes": part_bytes,
            "atomic_float_adds": pairs * 2 * D3,
        }
        del o_f, lse_f, g_out, dq_b, dk_b, dv_b, ws_b, dk_w, dv_w
        torch.cuda.empty_cache()

    # ---- the 64K fused index path with 8-bit (E4M3) indexer inputs: the same draws as the
    # bf16 step, encoded to E4M3; bf16 timed beside on the same sizes
    if want("e4m3"):
        W3 = sa_synth.WORKLOADS[3]
        p = W3.params
        T3, topk3 = p["T"], p["topk"]
        log("fused indices with E4M3 inputs (64K)")
        x8 = sa_synth.indexer_inputs(W3.seed, 1, T3, p["H_I"], p["D_I"], "fp8")
        qi8 = torch.from_numpy(x8["qi"]).view(torch.float8_e4m3fn).to(dev)
        ki8 = torch.from_numpy(x8["ki"]).view(torch.float8_e4m3fn).to(dev)
        w8 = to_dev(x8["w"], "f32")
        xb = sa_synth.indexer_inputs(W3.seed, 1, T3, p["H_I"], p["D_I"], "bf16")
        qib, kib, wb = to_dev(xb["qi"], "bf16"), to_dev(xb["ki"], "bf16"), to_dev(xb["w"], "f32")
        del x8, xb
        chunk3 = 32768
        ws3 = torch.empty(sa.sa_indexer_topk_workspace(1, T3, p["H_I"], p["D_I"], T3 - chunk3, T3,
                                                       topk3), dtype=torch.uint8, device=dev)
        idx3 = torch.full((1, T3, topk3), -1, dtype=torch.int32, device=dev)

        def fused(qq, kk, ww):
            for r0 in range(0, T3, chunk3):
                sa.sa_indexer_topk(qq, kk, ww, topk3, r0, min(T3, r0 + chunk3), idx3, ws3)

        t8 = timed(lambda: fused(qi8, ki8, w8), 5)
        tb = timed(lambda: fused(qib, kib, wb), 5)
        flops3 = 2.0 * p["H_I"] * p["D_I"] * T3 * (T3 + 1) / 2
        rows["indexer_topk_e4m3_64k"] = {
            "ms_per_step": t8, "bf16_ms_per_step": tb, "speedup_vs_bf16": tb / t8,
            "effective_tflops": flops3 / (t8 * 1e-3) / 1e12,
            "input_bytes": qi8.numel() + ki8.numel(), "bf16_input_bytes": 2 * (qib.numel() + kib.numel()),
        }
        del qi8, ki8, w8, qib, kib, wb, ws3, idx3
        torch.cuda.empty_cache()

    # ---- NSA's three branches over the 64K prefill tensors: compressed attention over the
    # 64-token block means, the top-16 blocks per row, a 512-token window (the block-sparse
    # decode workload's parameters), gated combine
    if want("nsa"):
        log("NSA three-branch prefill (64K)")
        T3, Hq3, D3 = q64.shape[1], q64.shape[2], q64.shape[3]
        nblk, ntop, nwin = 64, 16, 512
        scale3 = D3 ** -0.5
        lens3 = torch.full((1,), T3, dtype=torch.int32, device=dev)
        kbar3 = sa.sa_block_meanpool(k64, lens3, nblk)
        vbar3 = sa.sa_block_meanpool(v64, lens3, nblk)
        ws_c = torch.empty(sa.sa_cmp_attn_workspace(1, T3, k64.shape[2], D3, nblk), dtype=torch.uint8,
                           device=dev)
        ws_s = torch.empty(sa.sa_block_select_workspace(1, T3, k64.shape[2], D3, nblk, 0, T3),
                           dtype=torch.uint8, device=dev)
        idx_n = torch.full((1, T3, ntop * nblk), -1, dtype=torch.int32, device=dev)
        oc3, os3, ow3, on3 = (torch.empty_like(q64) for _ in range(4))
        gates3 = torch.rand((1, T3, Hq3, 3), generator=torch.Generator(device=dev).manual_seed(1003),
                            device=dev, dtype=torch.float32)
        parts = {
            "meanpool_k_v": lambda: (sa.sa_block_meanpool(k64, lens3, nblk, kbar3),
                                     sa.sa_block_meanpool(v64, lens3, nblk, vbar3)),
            "compressed": lambda: sa.sa_cmp_attn_fwd(q64, kbar3, vbar3, nblk, scale3, out=oc3,
                                                     workspace=ws_c),
            "block_select": lambda: sa.sa_block_select(q64, kbar3, nblk, ntop, idx=idx_n,
                                                       workspace=ws_s),
            "selected": lambda: sa.sa_sparse_attn_fwd(q64, k64, v64, idx_n, 0, scale3, out=os3),
            "window": lambda: sa.sa_sparse_attn_fwd(q64, k64, v64, None, nwin, scale3, out=ow3),
            "combine": lambda: sa.sa_nsa_combine(oc3, os3, ow3, gates3, out=on3),
        }
        part_ms = {name: timed_cold(fn, 3) for name, fn in parts.items()}
        t_nsa = timed_cold(lambda: [fn() for fn in parts.values()], 3)
        t_nsa_warm = timed(lambda: [fn() for fn in parts.values()], 3)
        rows["nsa_prefill_64k"] = {
            "ms_per_step": t_nsa, "warm_ms_per_step": t_nsa_warm, "timing": "cold",
            "query_tokens_per_s": T3 / (t_nsa * 1e-3), "parts_ms": part_ms,
            "block": nblk, "top_blocks": ntop, "window": nwin,
            "selected_keys_per_query": ntop * nblk,
        }
        del kbar3, vbar3, ws_c, ws_s, idx_n, oc3, os3, ow3, on3, gates3
        torch.cuda.empty_cache()

    # ---- fixed-graph distance attention: the 16K workload, and the same distributions
    # at 64K and 128K (16K alone is launch/latency-bound)
    if want("graph"):
        W2 = sa_synth.WORKLOADS[2]
        p = W2.params
        H2, D2 = p["H"], p["D"]
        for T2, name in ((p["T"], "graph_attn_16k"), (65536, "graph_attn_64k"),
                         (131072, "graph_attn_128k")):
            log(f"graph attention ({T2} tokens)")
            g = sa_synth.graph_inputs(W2.seed, 1, T2, H2, D2, "bf16")
            cq, ck, vg, bias = (to_dev(g["cq"], "bf16"), to_dev(g["ck"], "bf16"),
                                to_dev(g["v"], "bf16"), to_dev(g["bias"], "f32"))
            del g
            og = torch.empty_like(vg)
            gfn = lambda: sa.sa_graph_attn_fwd(cq, ck, vg, bias, p["tau"], p["local"],  # noqa: E731
                                               p["n_pow2"], out=og)
            ms = timed_cold(gfn, reps)
            ms_warm = timed(gfn, reps)
            edges = sum(min(t, p["local"]) + 1 + sum(1 for j in range(p["n_pow2"])
                                                      if (1 << j) > p["local"] and (1 << j) <= t)
                        for t in range(T2))
            comp = T2 * H2 * (2 * D2 * 2 + 2 * 3 * 2)
            rows[name] = {
                "ms": ms, "warm_ms": ms_warm, "timing": "cold",
                "query_tokens_per_s": T2 / (ms * 1e-3),
                "compulsory_bytes": comp, "compulsory_GBps": comp / (ms * 1e-3) / 1e9,
                "edge_bytes": edges * H2 * (D2 * 2 + 6),
                "edge_GBps": edges * H2 * (D2 * 2 + 6) / (ms * 1e-3) / 1e9,
                "hbm_frac_compulsory": comp / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            }
            del cq, ck, vg, bias, og

    # ---- block-sparse decode, 32 x 128K
    if want("decode"):
        W5 = sa_synth.WORKLOADS[5]
        p = W5.params
        log("block-sparse decode (32 x 128K): generating caches")
        dx = sa_synth.decode_inputs(W5.seed, p["B"], p["L"], p["Hq"], p["Hkv"], p["D"], "bf16")
        qd = to_dev(dx["q"], "bf16")
        kc = to_dev(dx["kcache"], "bf16")
        vc = to_dev(dx["vcache"], "bf16")
        if keep is not None:
            keep["w5"] = dx
        del dx
        lens = torch.full((p["B"],), p["L"], dtype=torch.int32, device=dev)
        t_pool = timed(lambda: sa.sa_block_meanpool(kc, lens, p["block"]), 3)
        kbar = sa.sa_block_meanpool(kc, lens, p["block"])
        need = sa.sa_sparse_decode_workspace(p["B"], p["L"], p["Hq"], p["Hkv"], p["D"], p["block"],
                                             p["top_blocks"], p["window"], 0)
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        od = torch.empty_like(qd)
        dfn = lambda: sa.sa_sparse_decode(qd, kc, vc, kbar, lens, p["block"],  # noqa: E731
                                          p["top_blocks"], p["window"], p["scale"],
                                          workspace=ws, out=od)
        ms = timed_cold(dfn, 30)
        ms_warm = timed(dfn, 50)
        _, sel = sa.sa_sparse_decode(qd, kc, vc, kbar, lens, p["block"], p["top_blocks"], p["window"],
                                     p["scale"], workspace=ws, return_sel=True)
        wstart = p["L"] - p["window"]
        sel_h = sel.cpu().numpy()
        u_tok = 0
        for b in range(p["B"]):
            for j in sel_h[b, 0]:
                if j >= 0:
                    u_tok += max(0, min(p["block"], wstart - int(j) * p["block"]))
            u_tok += p["window"]
        nb = p["L"] // p["block"]
        dbytes = p["B"] * nb * p["D"] * 4 + u_tok * 2 * p["D"] * 2 + p["B"] * p["Hq"] * p["D"] * 2 * 2
        rows["sparse_decode_b32_128k"] = {
            "us_per_step": ms * 1e3, "warm_us_per_step": ms_warm * 1e3, "timing": "cold",
            "warm_hbm_frac": dbytes / (ms_warm * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "tokens_per_s": p["B"] / (ms * 1e-3),
            "algorithmic_bytes_per_step": dbytes, "achieved_GBps": dbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": dbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "n_splits": sa.sa_sparse_decode_auto_splits(p["B"], p["L"], p["Hkv"], p["block"],
                                                        p["top_blocks"], p["window"]),
            "meanpool_ms_once_per_cache": t_pool,
        }
        # NSA's three branches on the same caches: compressed (bf16 block means, pooled once per
        # cache), selected (the chosen blocks' tokens: sa_sparse_decode with window 0), window,
        # gated combine
        log("NSA three-branch decode (32 x 128K)")
        kb16 = sa.sa_block_meanpool_bf16(kc, lens, p["block"])
        vb16 = sa.sa_block_meanpool_bf16(vc, lens, p["block"])
        t_pool16 = timed(lambda: (sa.sa_block_meanpool_bf16(kc, lens, p["block"], kb16),
                                  sa.sa_block_meanpool_bf16(vc, lens, p["block"], vb16)), 3)
        ws0 = torch.zeros(sa.sa_sparse_decode_workspace(p["B"], p["L"], p["Hq"], p["Hkv"], p["D"],
                                                        p["block"], p["top_blocks"], 0, 0),
                          dtype=torch.uint8, device=dev)
        # the compressed range (L/64 = 2048 rows) split over 7 workgroups per sequence: with
        # the window's one, 32 x 8 = 256 workgroups of 8 wavefronts, one per CU (their
        # registers fill it), so the combined launch runs in one round (8 + 1 splits:
        # 37 us instead of 29)
        ns_c = 7
        ws_c = torch.zeros(sa.sa_nsa_decode_branch_workspace(p["B"], p["Hq"], p["Hkv"], p["D"], ns_c),
                           dtype=torch.uint8, device=dev)
        ocd, osd, owd, ond = (torch.empty_like(qd) for _ in range(4))
        gd = torch.rand((p["B"], 1, p["Hq"], 3), generator=torch.Generator(device=dev).manual_seed(1005),
                        device=dev, dtype=torch.float32)
        dparts = {
            "compressed": lambda: sa.sa_nsa_decode_branch(qd, kb16, vb16, lens, 1, p["block"],
                                                          p["window"], p["scale"], out=ocd,
                                                          n_splits=ns_c, workspace=ws_c),
            "selected": lambda: sa.sa_sparse_decode(qd, kc, vc, kbar, lens, p["block"], p["top_blocks"],
                                                    0, p["scale"], workspace=ws0, out=osd),
            "window": lambda: sa.sa_nsa_decode_branch(qd, kc, vc, lens, 0, p["block"], p["window"],
                                                      p["scale"], out=owd),
            "combine": lambda: sa.sa_nsa_combine(ocd[:, None], osd[:, None], owd[:, None], gd,
                                                 out=ond[:, None]),
        }
        # the step: compressed and window branches in one launch, the selected branch, the
        # combine; each branch alone and the four separate calls are timed beside
        ocw, oww = torch.empty_like(qd), torch.empty_like(qd)
        ws_cw = torch.zeros(max(256, sa.sa_nsa_decode_cmp_win_workspace(p["B"], p["Hq"], p["Hkv"],
                                                                        p["D"], ns_c, 1)),
                            dtype=torch.uint8, device=dev)
        step_fns = [
            lambda: sa.sa_nsa_decode_cmp_win(qd, kb16, vb16, kc, vc, lens, p["block"], p["window"],
                                             p["scale"], out_cmp=ocw, out_win=oww,
                                             n_splits_cmp=ns_c, workspace=ws_cw),
            dparts["selected"],
            lambda: sa.sa_nsa_combine(ocw[:, None], osd[:, None], oww[:, None], gd,
                                      out=ond[:, None]),
        ]
        dpart_us = {name: timed_cold(fn, 20) * 1e3 for name, fn in dparts.items()}
        dpart_us["compressed_and_window"] = timed_cold(step_fns[0], 20) * 1e3
        t_sep = timed_cold(lambda: [fn() for fn in dparts.values()], 20)
        t_nd = timed_cold(lambda: [fn() for fn in step_fns], 20)
        t_nd_warm = timed(lambda: [fn() for fn in step_fns], 20)
        rows["nsa_decode_b32_128k"] = {
            "us_per_step": t_nd * 1e3, "warm_us_per_step": t_nd_warm * 1e3, "timing": "cold",
            "tokens_per_s": p["B"] / (t_nd * 1e-3), "parts_us": dpart_us,
            "separate_branch_calls_us_per_step": t_sep * 1e3,
            "compressed_splits": ns_c,
            "bf16_meanpool_ms_once_per_cache": t_pool16,
        }
        del ocw, oww, ws_cw
        del kb16, vb16, ws0, ocd, osd, owd, ond, gd
        del qd, kc, vc, kbar, ws, od
        torch.cuda.empty_cache()

    # ---- cross-layer index reuse, 128K, F,S,S,S
    if want("reuse"):
        W4 = sa_synth.WORKLOADS[4]
        p = W4.params
        T = p["T"]
        log("index reuse F,S,S,S (128K): generating inputs")
        xi = sa_synth.indexer_inputs(W4.seed, 1, T, p["H_I"], p["D_I"], "bf16")
        qi, ki, w = to_dev(xi["qi"], "bf16"), to_dev(xi["ki"], "bf16"), to_dev(xi["w"], "f32")
        layers = []
        for l in range(4):
            lx = sa_synth.attn_inputs(sa_synth.layer_seed(l), 1, T, p["Hq"], p["Hkv"], p["D"], "bf16")
            layers.append(tuple(to_dev(lx[n], "bf16") for n in ("q", "k", "v")))
            if keep is not None:
                keep.setdefault("w4_layers", []).append(lx)
            del lx
        if keep is not None:
            keep["w4_index"] = xi
        chunk = 32768
        ws = torch.empty(sa.sa_indexer_topk_workspace(1, T, p["H_I"], p["D_I"], T - chunk, T,
                                                      p["topk"]), dtype=torch.uint8, device=dev)
        idx = torch.full((1, T, p["topk"]), -1, dtype=torch.int32, device=dev)
        o4 = torch.empty_like(layers[0][0])

        def index_once():
            for r0 in range(0, T, chunk):
                r1 = min(T, r0 + chunk)
                sa.sa_indexer_topk(qi, ki, w, p["topk"], r0, r1, idx, ws)

        def attn(l):
            qq, kk, vv = layers[l]
            sa.sa_sparse_attn_fwd(qq, kk, vv, idx, p["window"], p["scale"], out=o4)

        t_index = timed_cold(index_once, 3)
        t_attn = [timed_cold(lambda l=l: attn(l), 3) for l in range(4)]
        reuse = t_index + sum(t_attn)
        no_reuse = 4 * t_index + sum(t_attn)
        rows["indexcache_FSSS_128k"] = {
            "timing": "cold", "index_ms": t_index, "attn_ms_per_layer": t_attn,
            "four_layers_ms_with_reuse": reuse, "four_layers_ms_indexing_every_layer": no_reuse,
            "indexer_time_saved_ms": 3 * t_index, "saved_frac": 3 * t_index / no_reuse,
            "attn_query_tokens_per_s": T / (sum(t_attn) / 4 * 1e-3),
        }
        del ws, idx, layers, qi, ki, w, o4
        torch.cuda.empty_cache()
    del flush
    torch.cuda.empty_cache()
    return rows


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count()


def cpu_baseline(np, sa_synth, x, p, seconds, which="all", host=None):
    """The float64 oracle, as it stands, on the machine's host cores.  The headline entry is
    the 64K workload on rows drawn uniformly from [0, T) (each through indexer scores,
    exact top-k and dense-masked attention), for about ``seconds`` s, scaled to query
    tokens per second.  ``workloads`` holds every workload: the 2K top-k prefill and the
    32 x 128K decode run in full; the 16K graph attention and the 128K index reuse
    (indexer + top-k once, four attention layers) on uniformly sampled rows, their
    whole-workload seconds extrapolated from the rate and labelled so.  ``host`` may
    hold the host inputs of workloads 4 and 5 already drawn for the GPU rows."""
    import oracle.reference as orc
    host = host or {}
    threads = _blas_threads()
    T, k, W = p["T"], p["topk"], p["window"]

    def entry(name, n, el, unit_n, unit, total, extrapolated, sample):
        rate = unit_n / el
        return {"workload": name, "value": rate, "unit": unit, "seconds": el, "units_timed": unit_n,
                "whole_workload_seconds": total / rate, "extrapolated": extrapolated,
                "sample": sample}

    g = sa_synth.rng(4242)
    done = 0
    idx = np.full((1, T, k), -1, np.int32)
    t0 = time.perf_counter()
    while True:
        rows = sorted(g.integers(0, T, size=8).tolist())
        for t in rows:
            idx[0, t] = orc.topk_select_row(orc.indexer_scores_row(x["qi"], x["ki"], x["w"], 0, t), k)
        orc.sparse_attn(x["q"], x["k"], x["v"], idx, W, p["scale"], rows)
        done += len(rows)
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    del idx
    w3 = entry(sa_synth.WORKLOADS[3].name, done, el, done, "query-tokens/s", T, True,
               f"{done} rows drawn uniformly from [0, T) of the 64K prefill workload "
               f"(indexer row + exact top-k + dense-masked float64 attention), {el:.1f} s")
    res = {"value": w3["value"], "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
           "sample": w3["sample"], "cpu_model": _cpu_model(), "blas_threads": threads,
           "workloads": {"3": w3}}
    if which != "all":
        return res

    log("CPU oracle: workload 1 (all 2048 rows)")
    W1 = sa_synth.WORKLOADS[1]
    p1 = W1.params
    x1 = sa_synth.prefill_inputs(W1.seed, 1, p1["T"], p1["Hq"], p1["Hkv"], p1["D"], p1["H_I"],
                                 p1["D_I"], "f32")
    t0 = time.perf_counter()
    sc = orc.indexer_scores(x1["qi"], x1["ki"], x1["w"])
    idx1 = orc.topk_select(sc, p1["topk"], 1, p1["T"])
    orc.sparse_attn(x1["q"], x1["k"], x1["v"], idx1, p1["window"], p1["scale"])
    el = time.perf_counter() - t0
    res["workloads"]["1"] = entry(W1.name, p1["T"], el, p1["T"], "query-tokens/s", p1["T"], False,
                                  "every row: indexer scores, exact top-k, dense-masked attention")
    del x1, sc, idx1

    log("CPU oracle: workload 2 (sampled rows)")
    W2 = sa_synth.WORKLOADS[2]
    p2 = W2.params
    x2 = sa_synth.graph_inputs(W2.seed, 1, p2["T"], p2["H"], p2["D"], "bf16")
    g2 = sa_synth.rng(4243)
    done, t0 = 0, time.perf_counter()
    while True:
        rows = sorted(g2.integers(0, p2["T"], size=16).tolist())
        orc.graph_attn(x2["cq"], x2["ck"], x2["v"], x2["bias"], p2["tau"], p2["local"],
                       p2["n_pow2"], rows)
        done += len(rows)
        el = time.perf_counter() - t0
        if el >= 8.0:
            break
    res["workloads"]["2"] = entry(W2.name, done, el, done, "query-tokens/s", p2["T"], True,
                                  f"{done} rows drawn uniformly from [0, T) (dense logits over "
                                  f"s <= t under the fixed-graph mask), {el:.1f} s")
    del x2

    log("CPU oracle: workload 4 (1024 sampled rows, four layers)")
    W4 = sa_synth.WORKLOADS[4]
    p4 = W4.params
    T4 = p4["T"]
    xi = host.get("w4_index") or sa_synth.indexer_inputs(W4.seed, 1, T4, p4["H_I"], p4["D_I"],
                                                         "bf16")
    layers = host.get("w4_layers") or [
        sa_synth.attn_inputs(sa_synth.layer_seed(l), 1, T4, p4["Hq"], p4["Hkv"], p4["D"], "bf16")
        for l in range(4)]
    g4 = sa_synth.rng(4244)
    rows4 = sorted(g4.integers(0, T4, size=1024).tolist())
    idx4 = np.full((1, T4, p4["topk"]), -1, np.int32)
    t0 = time.perf_counter()
    for i in range(0, len(rows4), 128):
        rows = rows4[i:i + 128]
        for t in rows:
            idx4[0, t] = orc.topk_select_row(orc.indexer_scores_row(xi["qi"], xi["ki"], xi["w"], 0, t),
                                             p4["topk"])
        for lay in layers:
            orc.sparse_attn(lay["q"], lay["k"], lay["v"], idx4, p4["window"], p4["scale"], rows)
        log(f"  workload 4: {i + len(rows)} rows, {time.perf_counter() - t0:.1f} s")
    el = time.perf_counter() - t0
    res["workloads"]["4"] = entry(W4.name, len(rows4), el, len(rows4), "query-tokens/s", T4, True,
                                  f"{len(rows4)} rows drawn uniformly from [0, T): indexer row + "
                                  f"exact top-k once, then dense-masked attention in each of the "
                                  f"4 layers (F,S,S,S), {el:.1f} s; whole-workload seconds "
                                  f"extrapolated as T / rate")
    del xi, layers, idx4

    log("CPU oracle: workload 5 (all 32 sequences)")
    W5 = sa_synth.WORKLOADS[5]
    p5 = W5.params
    dx = host.get("w5") or sa_synth.decode_inputs(W5.seed, p5["B"], p5["L"], p5["Hq"], p5["Hkv"],
                                                  p5["D"], "bf16")
    t0 = time.perf_counter()
    orc.sparse_decode(dx["q"], dx["kcache"], dx["vcache"], dx["lens"], p5["block"],
                      p5["top_blocks"], p5["window"], p5["scale"])
    el = time.perf_counter() - t0
    res["workloads"]["5"] = entry(W5.name, p5["B"], el, p5["B"], "tokens/s", p5["B"], False,
                                  "all 32 sequences: block means, block scores and top-16, "
                                  "dense-masked attention over the 131,072-token cache")
    return res


if __name__ == "__main__":
    main()
