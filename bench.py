"""Benchmark of the sparse latent attention hot path on one MI355X.

A step is one pass of the whole path over one batch: sparse_attn with its window index
lists generated inside the kernel from the query positions (the fused form of
sa_window_topk_idxs; --explicit-window launches that first and reads the whole list), the
compressed columns read from the index lists, and the inverse-RoPE epilogue. Inputs are
seeded and synthetic and already resident in HBM.

The default run reports the long-context prefill with compression (1 sequence of 8192
queries, 128 heads, d 512, 128 window + 2048 compressed columns, bf16 storage) as the
headline line, and in the same JSON line, under "workloads", the other workloads: the
window-only decode (32 x 1 query, 64 heads, 128-slot ring), the window-only prefill (4096
queries, 64 heads, window 128) and the window + compressed decode (64 x 1 query, 128
heads, 640 columns), each with bf16 and with fp8 storage, and the long prefill with fp8
storage. Each record carries its own roofline and CPU baseline.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|NAME] [--kv bf16|fp8]

Timing:
  * value / ms_per_step: exactly K steps replayed from one captured HIP graph, bracketed by
    device synchronisations, after W warm-up steps. The steps walk through enough distinct
    input sets (each its own q, kv, index and output buffers) that together they exceed
    twice the 256 MB Infinity Cache, and a pass over every set runs before the warm-up, so
    the timed steps read their inputs from HBM. For the prefill records, ~20 ms of plain
    device copies stream through HBM ahead of that pass (hbm_prewarm): after the idle set-up
    the first ~40 steps of the window prefill ran up to 11% slower than its steady state (200
    against 179 us per step), and a GPU spin that moves no memory did not change that, while
    the copies did; with the pre-warm, W = 5 gives the step times that 50 warm-up steps of the
    workload itself give. The decode records are short launches that 50 warm-up steps leave
    unchanged and that such traffic slows (the 64-row KV write 3.0 -> 3.4 us), so they run
    without it.
  * roofline: the attention kernel's own duration, from HIP events recorded on the launch
    stream around batches of back-to-back calls, after a GPU spin that lets the host enqueue
    every launch first (no host gaps inside the intervals), then, for the prefill records,
    the same HBM pre-warm (the spin itself moves no memory). achieved = algorithmic bytes
    (HBM-bound workloads: both decodes and the window-only prefill) or flops (the long
    prefill) per call / average duration. traffic = HBM bytes per call from the committed
    FETCH_SIZE / WRITE_SIZE counter summary of the same kernel sources
    (profiles/traffic_*.json), null when the sources have changed since.
  * cpu_baseline: the CPU oracle (window lists, sparse_attn, inverse RoPE) on a bounded
    sample of the same workload's queries, scaled to one step.
One JSON line goes to stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sa_workloads as W  # noqa: E402
import sparse_latent_attention_attn_amd as sa  # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6        # dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
MALL_BYTES = 256 << 20
PREWARM_S = 0.02                 # HBM streaming ahead of measured launches, seconds

DECODE = {"decode_window", "decode_compress"}
# The window lists are generated inside sparse_attn from the query positions (its fused
# window mode), so a step is one kernel; --explicit-window runs sa_window_topk_idxs first
# and has sparse_attn read the whole list from idx.
FUSED_WINDOW = True
# the roofline that bounds each workload's kernel (arithmetic intensity against the ridge
# of 2516.6 TFLOP/s / 8 TB/s = 315 flop/B): the window-only prefill does 126 flop/B
HBM_BOUND = {"decode_window", "decode_compress", "prefill_window"}
HEADLINE = ("prefill_compress", "bf16")
SUB_RECORDS = [("prefill_compress", "fp8"), ("decode_window", "bf16"), ("decode_window", "fp8"),
               ("prefill_window", "bf16"), ("prefill_window", "fp8"), ("decode_compress", "bf16"),
               ("decode_compress", "fp8")]


# ------------------------------------------------------------------ algorithmic work
def algorithmic(w: W.Workload, idx: np.ndarray, kv_format: str, epilogue: bool = True):
    """Bytes the method must move and flops it must do for one step: q, out, the index
    lists, the sink, and every distinct KV row a sequence's lists name, once, in its storage
    format (1024 B per bf16 row at d 512, 528 B per fp8 row with its scales); with the
    epilogue also the positions and their (cos, sin) rows. Flops: 4 h d per valid (query,
    index) pair."""
    row_bytes = w.d * 2 if kv_format == "bf16" else w.d + w.d // 32
    distinct = 0
    valid_pairs = 0
    for sq in range(w.b):
        v = idx[sq][idx[sq] >= 0]
        distinct += np.unique(v).size
        valid_pairs += v.size
    kv_bytes = distinct * row_bytes
    nq = w.b * w.s
    qo_bytes = 2 * nq * w.h * w.d * 2
    # with fused window lists only the compressed columns of idx are read
    idx_bytes = nq * (w.topk - (w.win_cols if FUSED_WINDOW else 0)) * 4
    small = w.h * 4 + (nq * 4 + nq * (w.rd // 2) * 8 if epilogue else 0)   # sink, positions, rope rows
    attn_bytes = kv_bytes + qo_bytes + idx_bytes + small
    flops = 4.0 * w.h * w.d * valid_pairs
    return dict(kv_bytes=kv_bytes, attn_bytes=attn_bytes, flops=flops, valid_pairs=valid_pairs,
                distinct_rows=distinct)


# ------------------------------------------------------------------ device input sets
class Step:
    """One input set on the device and the library calls of one step."""

    def __init__(self, w, q, kv, kv_scale, sink, idx, pos, table, start_pos, ws, epilogue=True):
        self.epilogue = epilogue
        self.w, self.q, self.kv, self.kv_scale, self.sink = w, q, kv, kv_scale, sink
        self.idx, self.pos, self.table, self.start_pos, self.ws = idx, pos, table, start_pos, ws
        self.out = torch.empty_like(q)
        self.idx_view = idx.view(w.win_nseq, w.win_seqlen, w.topk)

    def window(self):
        w = self.w
        sa.window_topk_idxs(w.window, w.win_seqlen, w.win_nseq, start_pos=self.start_pos,
                            out=self.idx_view)

    def attend(self):
        w = self.w
        fused = (w.window, "chunk" if w.win_start_pos is None else "ring", self.pos) if FUSED_WINDOW else None
        sa.sparse_attn(self.q, self.kv, self.sink, self.idx, w.scale, out=self.out,
                       kv_scale=self.kv_scale, rope=(self.table, self.pos) if self.epilogue else None,
                       workspace=self.ws, window=fused)

    def run(self):
        if not FUSED_WINDOW:
            self.window()
        self.attend()


def make_sets(w: W.Workload, kv_format: str, touched_bytes: int, dev, epilogue: bool = True):
    """Set 0 from the seeded draws; the other sets are device copies of it at distinct
    addresses (same values, so every set computes the same result)."""
    q0 = w.q.to(dev)
    kv_raw = w.kv.to(dev)
    scales0 = None
    if kv_format == "fp8":
        kv0, scales0 = sa.quant_kv_fp8(kv_raw, want=("codes", "scales"))
    else:
        (kv0,) = sa.quant_kv_fp8(kv_raw, want=("roundtrip",)) if w.kv_roundtrip else (kv_raw,)
    del kv_raw
    sink = w.sink.to(dev)
    idx0 = torch.empty(w.b, w.s, w.topk, dtype=torch.int32, device=dev)
    if w.comp_idx is not None:
        idx0[:, :, w.win_cols:] = w.comp_idx.to(dev)
    pos0 = w.pos.to(dev)
    sp0 = None if w.win_start_pos is None else w.win_start_pos.to(dev)
    table = sa.rope_table(w.rd, w.max_pos, w.rope_base, dev)
    probe = sa.make_args(q0, kv0, sink, idx0, w.scale, torch.empty_like(q0), kv_scale=scales0,
                         rope=(table, pos0),
                         window=(w.window, "chunk" if w.win_start_pos is None else "ring", pos0) if FUSED_WINDOW else None)
    ws_bytes = sa.sparse_attn_workspace_bytes(probe)
    nsets = max(2, min(64, math.ceil(2 * MALL_BYTES / max(touched_bytes, 1))))
    sets = []
    for k in range(nsets):
        c = (lambda t: t) if k == 0 else (lambda t: None if t is None else t.clone())
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev) if ws_bytes else None
        sets.append(Step(w, c(q0), c(kv0), c(scales0), sink, c(idx0), c(pos0), table, c(sp0), ws, epilogue))
    return sets


# ------------------------------------------------------------------ timing
def _capture(stream, calls):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    return g


_PREWARM_BUFS = []


def hbm_prewarm(seconds: float = PREWARM_S):
    """Copies between two 256 MiB device buffers, about `seconds` of HBM streaming at ~5 TB/s,
    enqueued on the current stream ahead of measured launches: the memory clocks are then in
    their loaded state, as in a serving loop, rather than ramping up during the measurement.
    No step's input or output is touched."""
    if not _PREWARM_BUFS:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        _PREWARM_BUFS.extend([a, torch.empty_like(a)])
    a, b = _PREWARM_BUFS
    for i in range(max(1, int(seconds / 1e-4))):        # 512 MiB of traffic per copy
        (b if i % 2 == 0 else a).copy_(a if i % 2 == 0 else b)


def time_steps(sets, steps: int, warmup: int, prewarm: bool = False):
    """Exactly `steps` timed steps, replayed from one captured HIP graph. Before them: the HBM
    pre-warm (if asked for), one pass over every input set (so each timed step's set was last touched more
    than twice the Infinity Cache ago), then `warmup` steps on the sets the timed steps use
    last. Returns ms per step."""
    n = len(sets)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for s in sets:              # eager pass (also loads the kernels)
            s.run()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g_all = _capture(stream, [s.run for s in sets])
    g_warm = _capture(stream, [sets[(n - 1 - i) % n].run for i in range(warmup)]) if warmup > 0 else None
    g_timed = _capture(stream, [sets[i % n].run for i in range(steps)])
    torch.cuda.synchronize()
    if prewarm:
        hbm_prewarm()
    g_all.replay()
    if g_warm is not None:
        g_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_timed.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    return dt * 1e3 / steps


def time_kernel(sets, calls: int, prewarm: bool = False):
    """Average duration of one sparse_attn call: events on its stream around `calls`
    back-to-back calls over the input sets, after a GPU spin that lets the host enqueue them
    all first (so no host gap lands inside the interval) and, if asked for, the HBM pre-warm. Returns (mean ms, mean ms of the
    fastest of 5 such batches)."""
    st = torch.cuda.current_stream()
    # the spin must outlast the host's enqueueing of the whole batch (slower under a kernel
    # tracer): time one batch's enqueueing first and spin for twice that, at least 5 ms
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(calls):
        sets[i % len(sets)].attend()
    enqueue_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    spin_s = max(0.005, 2.0 * enqueue_s)
    per = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * spin_s))       # GPU spin while the host enqueues
        if prewarm:
            hbm_prewarm()
        e0.record(st)
        for i in range(calls):
            sets[i % len(sets)].attend()
        e1.record(st)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / calls)
    return float(np.mean(per)), float(np.min(per))


_CPU_CACHE = {}


def cpu_step_seconds(w: W.Workload, budget_s: float, rope: bool = True):
    """Seconds one step takes the oracle (plain C, OpenMP over queries) on the host: window
    lists, sparse_attn and the inverse RoPE of a bounded sample of queries, scaled to all
    queries. The kv rows are stored round-tripped before the timed region, as on the GPU.
    Cached per workload (the storage format does not change the oracle's work)."""
    key = (w.name, rope)
    if key in _CPU_CACHE:
        return _CPU_CACHE[key]
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from sa_harness import oracle_kv, u16
    nq = w.b * w.s
    threads = oracle.max_threads()
    sp = None if w.win_start_pos is None else w.win_start_pos.numpy()
    win = oracle.window_topk_idxs(w.window, w.win_seqlen, sp, nseq=w.win_nseq).reshape(w.b, w.s, -1)
    idx = win if w.comp_idx is None else np.ascontiguousarray(np.concatenate([win, w.comp_idx.numpy()], -1))

    def sample(n):
        return np.unique(np.linspace(0, nq - 1, n).round().astype(np.int64))

    q16, sink = u16(w.q), w.sink.numpy()
    cs = oracle.freqs_cis(w.rd, w.max_pos, w.rope_base) if rope else None
    pos = w.pos.numpy().reshape(-1)

    def run(sel, kv):
        sp_ = None if w.win_start_pos is None else w.win_start_pos.numpy()
        oracle.window_topk_idxs(w.window, w.win_seqlen, sp_, nseq=w.win_nseq)
        out = oracle.sparse_attn(q16, kv, sink, idx, w.scale, qsel=sel, nthreads=threads)
        if rope:
            oracle.apply_rotary(out, w.rd, cs, pos[sel], inverse=True)

    # per-query cost from one query, then a sample sized to the budget
    one_sel = np.array([nq - 1])
    kv1 = oracle_kv(w, w.kv_roundtrip, [int(nq - 1) // w.s], idx, one_sel)
    t0 = time.perf_counter()
    run(one_sel, kv1)
    one = time.perf_counter() - t0
    sel = sample(int(max(1, min(nq, budget_s * threads / max(one, 1e-6)))))
    kv = oracle_kv(w, w.kv_roundtrip, sorted({int(i) // w.s for i in sel}), idx, sel)
    reps = 1
    t0 = time.perf_counter()
    while True:                      # a step cheaper than the budget is repeated (>= 2 s of work)
        run(sel, kv)
        dt = time.perf_counter() - t0
        if sel.size < nq or dt >= 2.0 or reps >= 100:
            break
        reps += 1
    per_step = dt / reps * nq / sel.size
    _CPU_CACHE[key] = (per_step, sel.size, nq, reps, dt, threads)
    return _CPU_CACHE[key]


def cpu_baseline(w: W.Workload, alg, budget_s: float, rope: bool = True):
    per_step, n, nq, reps, dt, threads = cpu_step_seconds(w, budget_s, rope)
    if w.name in DECODE:
        value, unit = alg["kv_bytes"] / per_step / 1e9, "GB/s"
    else:
        value, unit = alg["flops"] / per_step / 1e12, "TFLOP/s"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{n} of {nq} queries (all heads) x {reps} run(s): window lists, "
                      f"sparse_attn{' and inverse RoPE' if rope else ''}; {dt:.1f} s wall, "
                      f"scaled to one step"}


# ------------------------------------------------------------------ HBM traffic counters
CAL_BYTES = 1 << 30              # calibration copy: 1 GiB read, 1 GiB written
# per family of workloads: the sources its kernels are built from, and the kernel names
# (substrings) of one call
FAMILY_SOURCES = {
    "attn": ["attn_fwd_kernel.hpp", "attn_fwd.hip", "attn_fwd_wide.hip", "sa_api.cpp", "sa_internal.hpp",
             "sa_device.hpp", "lds_dma.hpp"],
    "kv_write": ["aux_kernels.hip", "sa_device.hpp"],
    "indexer": ["indexer.hip", "lds_dma.hpp", "sa_device.hpp"],
    "proj": ["wo_proj.hip", "lds_dma.hpp", "sa_device.hpp"],
}
FAMILY_KERNELS = {
    "attn": ["attn_fwd_kernel", "attn_combine_kernel", "dequant_kv_kernel"],
    "kv_write": ["kv_write_kernel"],
    "indexer": ["index_scores", "index_topk"],
    "proj": ["proj_stream_kernel", "proj_skinny_kernel", "proj_wide_kernel", "proj_tiled_kernel"],
}


def family(workload: str) -> str:
    if workload.startswith("kv_write"):
        return "kv_write"
    if workload.startswith("indexer"):
        return "indexer"
    if workload.startswith("wo_proj"):
        return "proj"
    return "attn"


def kernel_source_hash(fam: str = "attn") -> str:
    """Hash of the kernel sources' code: line and block comments and whitespace are left
    out (the sources hold no comment markers inside string literals), so that an edit of a
    comment does not orphan counters taken on identical code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in FAMILY_SOURCES[fam]:
        with open(os.path.join(ROOT, "sparse_latent_attention_attn_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_path(workload: str, kv: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}_{kv}.json")


def stored_traffic(workload: str, kv: str):
    """HBM bytes per sparse_attn call from the committed counter summary, or None when it is
    missing or was taken on other kernel sources."""
    path = traffic_path(workload, kv)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    return rec["traffic_bytes_per_call"] if rec.get("kernel_source_sha") == kernel_source_hash(family(workload)) else None


def profile_pass(sets, calls: int, dev):
    """Eager steps for a counter run, then the calibration copy (a plain device copy)."""
    for i in range(calls):
        sets[i % len(sets)].run()
    torch.cuda.synchronize()
    src = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"profile pass: {calls} steps over {len(sets)} input sets, 3 copies of {CAL_BYTES} B",
          file=sys.stderr)


def pmc_summary(workload: str, kv: str, fetch_csv: str, write_csv: str):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the kernels of one call, each
    scaled by the ratio of the known size of the calibration copy to what the counter read
    for it."""
    import csv
    pats = FAMILY_KERNELS[family(workload)]

    def read(path, counter):
        per = {p: [] for p in pats}
        cal = []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                name, v = r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0
                hit = [p for p in pats if p in name]
                if hit:
                    per[hit[0]].append(v)
                elif "copyBuffer" in name or "elementwise" in name:
                    cal.append(v)
        if not any(per.values()) or not cal:
            raise SystemExit(f"{path}: no {counter} rows for {' / '.join(pats)} or the copy kernel")
        # the calibration copies are the three largest copy dispatches (input-set clones
        # before them are far smaller)
        cal = sorted(cal)[-3:]
        return {p: (float(np.mean(v)) if v else 0.0) for p, v in per.items()}, float(np.median(cal))

    fk, fcal = read(fetch_csv, "FETCH_SIZE")
    wk, wcal = read(write_csv, "WRITE_SIZE")
    kf, kw = CAL_BYTES / fcal, CAL_BYTES / wcal
    rec = {
        "workload": workload, "kv": kv, "kernel_source_sha": kernel_source_hash(family(workload)),
        "fetch_bytes_raw": fk, "write_bytes_raw": wk,
        "copy_fetch_bytes_raw": fcal, "copy_write_bytes_raw": wcal, "copy_bytes": CAL_BYTES,
        "fetch_scale": kf, "write_scale": kw,
        "traffic_bytes_per_call": sum(fk.values()) * kf + sum(wk.values()) * kw,
    }
    os.makedirs(os.path.dirname(traffic_path(workload, kv)), exist_ok=True)
    with open(traffic_path(workload, kv), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def trace_summary(stats_csv: str):
    """The kernel table of a rocprofv3 --kernel-trace --stats run (its kernel_stats.csv)."""
    import csv
    print(f"{'kernel':70s} {'calls':>7s} {'avg us':>10s} {'min us':>10s} {'max us':>10s}")
    with open(stats_csv) as fh:
        for r in csv.DictReader(fh):
            print(f"{r['Name'][:70]:70s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} "
                  f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f}")


def counter_summary(workload: str, csvs):
    """Per-call averages of the counters of one family's kernels over rocprofv3 --pmc runs,
    with derived ratios: L2 hit rate, mean L1-to-L2 read latency, texture-unit stall share,
    wait shares, MFMA busy share."""
    import csv
    import collections
    pats = FAMILY_KERNELS[family(workload)]
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in csvs:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                hit = [p for p in pats if p in r["Kernel_Name"]]
                if hit:
                    vals[r["Kernel_Name"][:80]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    for kern, cs in vals.items():
        print(kern)
        avg = {c: float(np.mean(v)) for c, v in cs.items()}
        for c in sorted(avg):
            print(f"  {c:36s} {avg[c]:14.4g}   (calls {len(cs[c])})")

        def ratio(a, b):
            return avg[a] / avg[b] if a in avg and b in avg and avg[b] else None
        derived = [
            ("L2 hit rate, TCC_HIT / (TCC_HIT + TCC_MISS)",
             avg["TCC_HIT"] / (avg["TCC_HIT"] + avg["TCC_MISS"]) if "TCC_HIT" in avg and "TCC_MISS" in avg else None),
            ("mean L1->L2 read latency (clocks), TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ",
             ratio("TCP_TCC_READ_REQ_LATENCY", "TCP_TCC_READ_REQ")),
            ("texture unit stalled by the L1, TA_ADDR_STALLED_BY_TC_CYCLES / TA_TA_BUSY",
             ratio("TA_ADDR_STALLED_BY_TC_CYCLES", "TA_TA_BUSY")),
            ("LDS-DMA gather wavefronts per call, TA_BUFFER_READ_LDS_WAVEFRONTS",
             avg.get("TA_BUFFER_READ_LDS_WAVEFRONTS")),
            ("waves waiting to issue, SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES", ratio("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")),
            ("waves waiting on a counter, SQ_WAIT_ANY / SQ_WAVE_CYCLES", ratio("SQ_WAIT_ANY", "SQ_WAVE_CYCLES")),
            ("LDS bank-conflict share, SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS",
             ratio("SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS")),
        ]
        print("  derived:")
        for name, v in derived:
            if v is not None:
                print(f"    {name}: {v:.4g}")


def prepare(w: W.Workload, kv: str, dev, epilogue: bool):
    """The algorithmic counts of one step (from the library's own index lists) and the
    device input sets."""
    probe_idx = torch.empty(w.b, w.s, w.topk, dtype=torch.int32, device=dev)
    view = probe_idx.view(w.win_nseq, w.win_seqlen, w.topk)
    sa.window_topk_idxs(w.window, w.win_seqlen, w.win_nseq,
                        start_pos=None if w.win_start_pos is None else w.win_start_pos.to(dev), out=view)
    if w.comp_idx is not None:
        probe_idx[:, :, w.win_cols:] = w.comp_idx.to(dev)
    alg = algorithmic(w, probe_idx.cpu().numpy(), kv, epilogue=epilogue)
    del probe_idx
    return alg, make_sets(w, kv, alg["attn_bytes"], dev, epilogue=epilogue)


def measure(w: W.Workload, kv: str, dev, steps: int, warmup: int, epilogue: bool,
            cpu_budget_s: float | None):
    """One record: step rate, kernel roofline and CPU baseline of workload w with storage kv."""
    alg, sets = prepare(w, kv, dev, epilogue)
    pw = w.name not in DECODE
    ms_step = time_steps(sets, steps, warmup, prewarm=pw)
    k_mean, k_best = time_kernel(sets, calls=min(400, max(50, steps * 5 if w.name in DECODE else steps)), prewarm=pw)
    if w.name in DECODE:
        value = alg["kv_bytes"] / (ms_step * 1e-3) / 1e9
        metric, unit = "sparse_attn KV GB/s (decode)", "GB/s"
    else:
        value = alg["flops"] / (ms_step * 1e-3) / 1e12
        metric, unit = "sparse_attn TFLOP/s (prefill)", "TFLOP/s"
    if w.name in HBM_BOUND:
        achieved = alg["attn_bytes"] / (k_mean * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = alg["flops"] / (k_mean * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_PEAK_TFLOPS}
    roof["traffic"] = stored_traffic(w.name, kv) if epilogue else None
    roof["kernel"] = "sparse_attn (attn_fwd_kernel [+ attn_combine_kernel] [+ dequant_kv_kernel])"
    roof["kernel_ms_mean"] = k_mean
    roof["kernel_ms_best_batch"] = k_best
    roof["algorithmic_bytes_per_launch"] = alg["attn_bytes"]
    roof["algorithmic_flops_per_launch"] = alg["flops"]
    if w.name == "prefill_window":
        roof["mfma_frac"] = alg["flops"] / (k_mean * 1e-3) / 1e12 / BF16_PEAK_TFLOPS
    cpu = cpu_baseline(w, alg, cpu_budget_s, rope=epilogue) if cpu_budget_s else None
    del sets
    torch.cuda.empty_cache()
    return {
        "metric": metric, "value": value, "unit": unit, "ms_per_step": ms_step, "steps": steps,
        "dtype": "bf16" if kv == "bf16" else "fp8-e4m3 storage, bf16 compute",
        "config": {"workload": w.name, "sequences": w.b, "queries_per_sequence": w.s, "heads": w.h,
                   "head_dim": w.d, "rope_dim": w.rd, "topk": w.topk, "kv_rows_per_sequence": w.kv_rows,
                   "kv_storage": kv, "epilogue": "inverse RoPE" if epilogue else "none",
                   "window_lists": "generated inside sparse_attn" if FUSED_WINDOW else "sa_window_topk_idxs",
                   "kv_bytes_per_step": alg["kv_bytes"], "distinct_kv_rows": alg["distinct_rows"],
                   "valid_pairs": alg["valid_pairs"]},
        "roofline": roof,
        "cpu_baseline": cpu,
    }


# ------------------------------------------------------------------ other steps of the path
def time_launches(fns, calls: int, prewarm: bool = False):
    """Average duration of one launch of fns[i % len(fns)]: HIP events on the current stream
    around `calls` back-to-back launches after a GPU spin and, if asked for, the HBM
    pre-warm (as time_kernel). Returns (mean ms,
    best-batch ms)."""
    st = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(calls):
        fns[i % len(fns)]()
    spin_s = max(0.005, 2.0 * (time.perf_counter() - t0))
    torch.cuda.synchronize()
    per = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.4e9 * spin_s))
        if prewarm:
            hbm_prewarm()
        e0.record(st)
        for i in range(calls):
            fns[i % len(fns)]()
        e1.record(st)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / calls)
    return float(np.mean(per)), float(np.min(per))


def time_graph_steps(fns, steps: int, warmup: int, prewarm: bool = False):
    """Exactly `steps` launches replayed from one captured graph after the HBM pre-warm (if asked
    for), a pass over every input set and `warmup` launches; ms per launch."""
    n = len(fns)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g_all = _capture(stream, fns)
    g_warm = _capture(stream, [fns[(n - 1 - i) % n] for i in range(warmup)]) if warmup > 0 else None
    g_timed = _capture(stream, [fns[i % n] for i in range(steps)])
    torch.cuda.synchronize()
    if prewarm:
        hbm_prewarm()
    g_all.replay()
    if g_warm is not None:
        g_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_timed.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def _oracle_seconds(fn, min_s: float = 1.0):
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_s or reps >= 1000:
            return dt / reps, reps, dt


KV_WRITE = {   # name: (sequences, rows per sequence, ring positions start)
    "kv_write_prefill": (1, 8192, 0),        # the long prefill's chunk: 8192 tokens, ring of 128
    "kv_write_decode": (64, 1, 65535),       # one token for each of 64 sequences
}


def run_eager(fns, calls: int):
    """Counter-collection mode: `calls` eager launches over the input sets."""
    for i in range(calls):
        fns[i % len(fns)]()
    torch.cuda.synchronize()


def measure_kv_write(name: str, dev, steps: int, warmup: int, cpu: bool, profile_calls: int = 0):
    """The KV write path (sa_kv_write): normalised rows -> forward RoPE -> fp8 round trip ->
    ring slot, bf16 storage, with the rows returned for the prefill. HBM-bound: bytes = rows
    read + positions + (cos, sin) rows + rows returned + rows stored."""
    b, s, p0 = KV_WRITE[name]
    d, rd, window = 512, 64, 128
    g = torch.Generator().manual_seed(31)
    x0 = torch.randn(b, s, d, generator=g).to(torch.bfloat16)
    pos0 = (torch.arange(s, dtype=torch.int32)[None] + p0).repeat(b, 1)
    max_pos = int(pos0.max()) + 1
    table = sa.rope_table(rd, max_pos, 10000.0, dev)
    want_rows = s > 1
    stored = b * min(s, window)
    alg_bytes = b * s * (2 * d + 4 + rd // 2 * 8) + (b * s * 2 * d if want_rows else 0) + stored * 2 * d
    nsets = max(2, min(64, math.ceil(2 * MALL_BYTES / alg_bytes)))
    sets = []
    for _ in range(nsets):
        x, pos = x0.to(dev), pos0.to(dev)
        ring = torch.zeros(b, window, d, dtype=torch.bfloat16, device=dev)
        rows = torch.empty(b, s, d, dtype=torch.bfloat16, device=dev) if want_rows else None
        sets.append((x, pos, ring, rows))
    fns = [(lambda x=x, pos=pos, ring=ring, rows=rows:
            sa.kv_write(x, pos, ring, rope=table, window=window, rows_out=rows)) for x, pos, ring, rows in sets]
    if profile_calls:
        run_eager(fns, profile_calls)
        return None
    ms_step = time_graph_steps(fns, steps, warmup, prewarm=want_rows)
    k_mean, k_best = time_launches(fns, calls=min(400, max(50, 5 * steps)), prewarm=want_rows)
    achieved = alg_bytes / (k_mean * 1e-3) / 1e9
    rec = {
        "metric": "kv_write GB/s", "value": alg_bytes / (ms_step * 1e-3) / 1e9, "unit": "GB/s",
        "ms_per_step": ms_step, "steps": steps, "dtype": "bf16 rows, f32 rotation, fp8 round trip",
        "config": {"workload": name, "sequences": b, "rows_per_sequence": s, "head_dim": d,
                   "rope_dim": rd, "window": window, "kv_storage": "bf16", "rows_returned": want_rows},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": stored_traffic(name, "bf16"), "kernel": "kv_write_kernel",
                     "kernel_ms_mean": k_mean, "kernel_ms_best_batch": k_best,
                     "algorithmic_bytes_per_launch": alg_bytes},
        "cpu_baseline": None,
    }
    if cpu:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        import oracle
        from sa_harness import u16
        xo, po = u16(x0), pos0.numpy()
        cs = oracle.freqs_cis(rd, max_pos, 10000.0)
        ring_o = np.zeros((b, window, d), np.uint16)
        per, reps, dt = _oracle_seconds(lambda: oracle.kv_write(xo, po, rd, cs, window, window,
                                                                cache_bf16=ring_o, want_rows=want_rows))
        rec["cpu_baseline"] = {"value": alg_bytes / per / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"the whole step x {reps} run(s), {dt:.1f} s wall (single-threaded)"}
    del sets, fns
    torch.cuda.empty_cache()
    return rec


INDEXER = {   # name: (sequences, queries per sequence, compressed positions, query positions)
    "indexer_decode": (64, 1, 16384, "decode"),     # the window + compressed decode's lists
    "indexer_prefill": (1, 8192, 2048, "prefill"),  # the long prefill's lists
}


def measure_indexer(name: str, dev, steps: int, warmup: int, cpu: bool, profile_calls: int = 0):
    """The indexer (sa_indexer_topk: MFMA scores, then the radix-select top-k lists) with 32
    index heads of 128, ratio 4, 512 picks, and select_candidate_blocks (sa_candidate_blocks,
    2048 blocks of 8) on its scores. Decode reads 4 MB of index keys per sequence and is
    HBM-bound; the prefill does 2 h d flops per visible (query, position) pair and is bound by
    the MFMA roofline. Bytes: keys, q, w, positions, the lists, and the f32 scores (an output
    of the call, written by the score kernel and read back by the top-k)."""
    b, s, n_pos, kind = INDEXER[name]
    h, d, ratio, topk = 32, 128, 4, 512
    g = torch.Generator().manual_seed(41)
    q0 = torch.randn(b, s, h, d, generator=g).to(torch.bfloat16)
    k0 = torch.randn(b, n_pos, d, generator=g).to(torch.bfloat16)
    w0 = torch.randn(b, s, h, generator=g) * (d ** -0.5 * h ** -0.5)
    pos0 = (torch.full((b, s), 65535, dtype=torch.int32) if kind == "decode"
            else torch.arange(s, dtype=torch.int32)[None].repeat(b, 1))
    vis = torch.clamp((pos0.long() + 1) // ratio, max=n_pos)
    pairs = int(vis.sum())
    flops = 2.0 * h * d * pairs
    key_bytes = b * n_pos * d * 2
    alg_bytes = key_bytes + b * s * (h * d * 2 + h * 4 + 4 + topk * 4) + b * s * n_pos * 4 * 2
    nsets = max(2, min(64, math.ceil(2 * MALL_BYTES / alg_bytes)))
    sets = []
    for _ in range(nsets):
        sets.append(dict(q=q0.to(dev), k=k0.to(dev), w=w0.to(dev), pos=pos0.to(dev),
                         sc=torch.empty(b, s, n_pos, dtype=torch.float32, device=dev),
                         idx=torch.empty(b, s, topk, dtype=torch.int32, device=dev),
                         mask=torch.empty(b, s, n_pos, dtype=torch.uint8, device=dev)))
    fns = [(lambda x=x: sa.indexer_topk(x["q"], x["k"], x["w"], x["pos"], ratio, topk=topk, offset=128,
                                        scores=x["sc"], idx=x["idx"])) for x in sets]
    cand_fns = [(lambda x=x: sa.candidate_blocks(x["sc"], x["pos"], ratio, 2048, 8, mask=x["mask"])) for x in sets]
    if profile_calls:
        run_eager(fns, profile_calls)
        run_eager(cand_fns, profile_calls)
        return None
    pw = kind == "prefill"
    ms_step = time_graph_steps(fns, steps, warmup, prewarm=pw)
    k_mean, k_best = time_launches(fns, calls=min(400, max(50, 5 * steps)), prewarm=pw)
    c_mean, _ = time_launches(cand_fns, calls=min(400, max(50, 5 * steps)), prewarm=pw)
    if kind == "decode":
        achieved = alg_bytes / (k_mean * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
        value, unit, metric = key_bytes / (ms_step * 1e-3) / 1e9, "GB/s", "indexer key GB/s (decode)"
    else:
        achieved = flops / (k_mean * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_PEAK_TFLOPS}
        value, unit, metric = flops / (ms_step * 1e-3) / 1e12, "TFLOP/s", "indexer TFLOP/s (prefill)"
    roof.update({"traffic": stored_traffic(name, "bf16"), "kernel": "sa_indexer_topk (index_scores_kernel + index_topk_kernel)",
                 "kernel_ms_mean": k_mean, "kernel_ms_best_batch": k_best,
                 "algorithmic_bytes_per_launch": alg_bytes, "algorithmic_flops_per_launch": flops})
    cand_bytes = b * s * n_pos * 5
    rec = {
        "metric": metric, "value": value, "unit": unit, "ms_per_step": ms_step, "steps": steps,
        "dtype": "bf16 inputs, f32 scores",
        "config": {"workload": name, "sequences": b, "queries_per_sequence": s, "index_heads": h,
                   "index_head_dim": d, "compressed_positions": n_pos, "ratio": ratio, "topk": topk,
                   "visible_pairs": pairs},
        "roofline": roof,
        "candidate_blocks": {"kernel_ms_mean": c_mean, "topk_blocks": 2048, "block_size": 8,
                             "bytes_per_launch": cand_bytes,
                             "hbm_frac": cand_bytes / (c_mean * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "cpu_baseline": None,
    }
    if cpu:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        import oracle
        from sa_harness import u16
        nq = b * s
        sel = np.unique(np.linspace(0, nq - 1, 4 if kind == "decode" else 32).round().astype(np.int64))
        bs_, ss_ = sel // s, sel % s
        qs, ws, ps = u16(q0[bs_, ss_].reshape(-1, 1, h, d)), w0[bs_, ss_].reshape(-1, 1, h).numpy(), pos0[bs_, ss_].view(-1, 1).numpy()
        ks = u16((k0[bs_] if b > 1 else k0.expand(sel.size, -1, -1)).contiguous())
        threads = oracle.max_threads()
        per, reps, dt = _oracle_seconds(lambda: oracle.index_topk(
            oracle.index_scores(qs, ks, ws, ps, ratio, nthreads=threads), topk, 128), 2.0)
        sel_pairs = int(vis[bs_, ss_].sum())
        per_step = per * pairs / max(sel_pairs, 1)
        val = (key_bytes / per_step / 1e9, "GB/s") if kind == "decode" else (flops / per_step / 1e12, "TFLOP/s")
        rec["cpu_baseline"] = {"value": val[0], "unit": val[1], "cores": threads, "kind": "oracle",
                               "sample": f"{sel.size} of {nq} queries x {reps} run(s), {dt:.1f} s wall, "
                                         f"scaled by visible pairs to one step"}
    del sets, fns, cand_fns
    torch.cuda.empty_cache()
    return rec


PROJ = {   # name: (tokens, weight storage)
    "wo_proj_decode": (64, "bf16"),         # the 64 decode queries of the window + compressed decode
    "wo_proj_decode_fp8": (64, "fp8"),
    "wo_proj_prefill": (8192, "bf16"),      # the long prefill's 8192 queries
}


def measure_proj(name: str, dev, steps: int, warmup: int, cpu: bool, profile_calls: int = 0):
    """The grouped output projection (sa_grouped_proj) at the model config's 8 groups of
    o_lora_rank 1024 on 128 heads of 512 (k 8192 per group). Decode streams the weights once
    (HBM-bound); the prefill is a dense bf16 contraction (MFMA-bound)."""
    m, wfmt = PROJ[name]
    g, r, kg = 8, 1024, 8192
    gen = torch.Generator().manual_seed(51)
    o0 = torch.randn(m, g * kg, generator=gen).to(torch.bfloat16)
    w0 = (torch.randn(g, r, kg, generator=gen) * kg ** -0.5).to(torch.bfloat16)
    flops = 2.0 * m * g * r * kg
    w_bytes = g * r * kg * (2 if wfmt == "bf16" else 1) + (g * r * kg // 32 if wfmt == "fp8" else 0)
    alg_bytes = w_bytes + m * g * kg * 2 + m * g * r * 2
    nsets = max(2, min(64, math.ceil(2 * MALL_BYTES / alg_bytes)))
    wd = w0.to(dev)
    wsc = None
    if wfmt == "fp8":
        wd, wsc = sa.quant_kv_fp8(wd, want=("codes", "scales"))
    sets = [dict(o=o0.to(dev), w=wd if i == 0 else wd.clone(), ws=None if wsc is None else (wsc if i == 0 else wsc.clone()),
                 out=torch.empty(m, g, r, dtype=torch.bfloat16, device=dev)) for i in range(nsets)]
    fns = [(lambda x=x: sa.grouped_proj(x["o"], x["w"], w_scale=x["ws"], out=x["out"])) for x in sets]
    if profile_calls:
        run_eager(fns, profile_calls)
        return None
    ms_step = time_graph_steps(fns, steps, warmup, prewarm=m > 64)
    k_mean, k_best = time_launches(fns, calls=min(400, max(20, 5 * steps)), prewarm=m > 64)
    if m <= 64:
        achieved = alg_bytes / (k_mean * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
        value, unit, metric = alg_bytes / (ms_step * 1e-3) / 1e9, "GB/s", "grouped wo_a GB/s (decode)"
    else:
        achieved = flops / (k_mean * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_PEAK_TFLOPS}
        value, unit, metric = flops / (ms_step * 1e-3) / 1e12, "TFLOP/s", "grouped wo_a TFLOP/s (prefill)"
    roof.update({"traffic": stored_traffic(name, "bf16"), "kernel": "proj_stream_kernel" if m <= 64 else ("proj_tiled_kernel" if wfmt == "fp8" else "proj_wide_kernel"),
                 "kernel_ms_mean": k_mean, "kernel_ms_best_batch": k_best,
                 "algorithmic_bytes_per_launch": alg_bytes, "algorithmic_flops_per_launch": flops})
    rec = {"metric": metric, "value": value, "unit": unit, "ms_per_step": ms_step, "steps": steps,
           "dtype": "bf16 (f32 accumulation)" if wfmt == "bf16" else "fp8-e4m3 weights, bf16 compute",
           "config": {"workload": name, "tokens": m, "groups": g, "rank": r, "k_per_group": kg,
                      "weights": wfmt},
           "roofline": roof, "cpu_baseline": None}
    if cpu:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        import oracle
        from sa_harness import u16
        ms = 2 if m > 64 else 8
        oq, wq = u16(o0[:ms]).reshape(ms, g, kg), u16(w0)
        threads = oracle.max_threads()
        per, reps, dt = _oracle_seconds(lambda: oracle.grouped_proj(oq, wq, nthreads=threads), 2.0)
        per_step = per * m / ms
        val = (alg_bytes / per_step / 1e9, "GB/s") if m <= 64 else (flops / per_step / 1e12, "TFLOP/s")
        rec["cpu_baseline"] = {"value": val[0], "unit": val[1], "cores": threads, "kind": "oracle",
                               "sample": f"{ms} of {m} tokens (bf16 weights) x {reps} run(s), {dt:.1f} s wall, "
                                         f"scaled to one step"}
    del sets, fns
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    extra = list(KV_WRITE) + list(INDEXER) + list(PROJ)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(W.WORKLOADS) + extra)
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"],
                    help="storage of a single --workload (the default run times both)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--explicit-window", action="store_true",
                    help="run sa_window_topk_idxs before sparse_attn in every step instead of "
                         "generating the window lists inside sparse_attn")
    ap.add_argument("--no-epilogue", action="store_true",
                    help="time sparse_attn without the inverse-RoPE epilogue (plain bf16 output)")
    ap.add_argument("--profile-calls", type=int, default=0,
                    help="counter-collection mode (single --workload): N eager steps over the "
                         "input sets, then the copy kernel of known size that calibrates the "
                         "byte counters; no timing, no JSON line")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "--profile-calls into profiles/traffic_<workload>_<kv>.json")
    ap.add_argument("--trace-summary", metavar="KERNEL_STATS_CSV",
                    help="print the kernel table of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--counter-summary", nargs="+", metavar="COUNTER_CSV",
                    help="print per-call counter averages and derived ratios of --workload's "
                         "kernels from rocprofv3 --pmc runs")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(args.workload, args.counter_summary)
        return
    if args.pmc_summary:
        if args.workload == "all":
            ap.error("--pmc-summary needs --workload")
        pmc_summary(args.workload, args.kv, *args.pmc_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(sparse_attn would shard over heads with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sa.lib()
    epilogue = not args.no_epilogue
    global FUSED_WINDOW
    FUSED_WINDOW = not args.explicit_window

    extra_fn = {**{k: measure_kv_write for k in KV_WRITE}, **{k: measure_indexer for k in INDEXER},
                **{k: measure_proj for k in PROJ}}
    if args.profile_calls:
        if args.workload == "all":
            ap.error("--profile-calls needs --workload")
        if args.workload in extra_fn:
            extra_fn[args.workload](args.workload, dev, 1, 0, False, profile_calls=args.profile_calls)
            profile_pass([], 0, dev)
        else:
            _, sets = prepare(W.make(args.workload), args.kv, dev, epilogue)
            profile_pass(sets, args.profile_calls, dev)
        return
    if args.workload in extra_fn:
        rec = extra_fn[args.workload](args.workload, dev, args.steps, args.warmup, not args.no_cpu_baseline)
        line = {"metric": rec["metric"], "value": rec["value"], "unit": rec["unit"], "n_gpus": 1,
                "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec["ms_per_step"],
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": rec["dtype"],
                "data": "synthetic", "config": rec["config"], "roofline": rec["roofline"],
                "cpu_baseline": rec["cpu_baseline"]}
        print(json.dumps(line))
        return

    cpu = not args.no_cpu_baseline
    if args.workload != "all":
        head = (args.workload, args.kv)
        subs = []
    else:
        head, subs = HEADLINE, SUB_RECORDS
    t_start = time.perf_counter()
    made = {}

    def workload(name):
        if name not in made:
            made.clear()
            made[name] = W.make(name)
        return made[name]

    records = []
    # the headline first (its CPU baseline gets the larger budget), then the sub-records
    # grouped by workload (shared draws)
    rec = measure(workload(head[0]), head[1], dev, args.steps, args.warmup, epilogue, 12.0 if cpu else None)
    head_rec = rec
    print(f"[bench] {head[0]} {head[1]}: {rec['value']:.4g} {rec['unit']} "
          f"({time.perf_counter() - t_start:.0f} s)", file=sys.stderr, flush=True)
    for name, kv in subs:
        rec = measure(workload(name), kv, dev, args.steps, args.warmup, epilogue, 4.0 if cpu else None)
        records.append(rec)
        print(f"[bench] {name} {kv}: {rec['value']:.4g} {rec['unit']}, kernel "
              f"{rec['roofline']['kernel_ms_mean'] * 1e3:.2f} us, {rec['roofline']['frac']:.3f} of "
              f"{rec['roofline']['bound']} ({time.perf_counter() - t_start:.0f} s)", file=sys.stderr, flush=True)
    if args.workload == "all":
        made.clear()
        for name in INDEXER:
            r = measure_indexer(name, dev, args.steps, args.warmup, cpu)
            records.append(r)
            print(f"[bench] {name}: {r['value']:.4g} {r['unit']}, kernel "
                  f"{r['roofline']['kernel_ms_mean'] * 1e3:.2f} us, {r['roofline']['frac']:.3f} of "
                  f"{r['roofline']['bound']}; candidate blocks {r['candidate_blocks']['kernel_ms_mean'] * 1e3:.2f} us "
                  f"({time.perf_counter() - t_start:.0f} s)", file=sys.stderr, flush=True)
        for name in PROJ:
            r = measure_proj(name, dev, args.steps, args.warmup, cpu)
            records.append(r)
            print(f"[bench] {name}: {r['value']:.4g} {r['unit']}, kernel "
                  f"{r['roofline']['kernel_ms_mean'] * 1e3:.2f} us, {r['roofline']['frac']:.3f} of "
                  f"{r['roofline']['bound']} ({time.perf_counter() - t_start:.0f} s)", file=sys.stderr, flush=True)
        for name in KV_WRITE:
            r = measure_kv_write(name, dev, args.steps, args.warmup, cpu)
            records.append(r)
            print(f"[bench] {name}: {r['value']:.4g} {r['unit']}, kernel "
                  f"{r['roofline']['kernel_ms_mean'] * 1e3:.2f} us, {r['roofline']['frac']:.3f} of hbm "
                  f"({time.perf_counter() - t_start:.0f} s)", file=sys.stderr, flush=True)
    rec = head_rec
    line = {
        "metric": rec["metric"], "value": rec["value"], "unit": rec["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": rec["dtype"],
        "data": "synthetic", "config": rec["config"], "roofline": rec["roofline"],
        "cpu_baseline": rec["cpu_baseline"],
    }
    if records:
        line["workloads"] = records
    print(json.dumps(line))


if __name__ == "__main__":
    main()
