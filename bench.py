"""Benchmark of the sparse latent attention hot path on one MI355X.

A step is one pass of the whole path over one batch: the window index lists
(sa_window_topk_idxs) followed by sparse_attn with the inverse-RoPE epilogue, bf16 KV
storage, on the decode workload by default (32 sequences x 1 query, 64 heads, d 512,
128-slot ring). Inputs are seeded and synthetic and already resident in HBM.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--kv fp8]

Timing:
  * value / ms_per_step: K steps replayed from one captured HIP graph, bracketed by
    device synchronisations. The graph walks through enough distinct input sets (each
    its own q, kv, index and output buffers) that together they exceed twice the 256 MB
    Infinity Cache, so every step reads its inputs from HBM.
  * roofline: the attention kernel's own duration, from HIP events recorded on the
    launch stream around batches of back-to-back calls, after a GPU spin that lets the host
    enqueue every launch first (no host gaps inside the intervals). achieved = algorithmic
    bytes (decode) or flops (prefill) per call / average duration. traffic = HBM bytes per
    call from the committed FETCH_SIZE / WRITE_SIZE counter summary of the same kernel
    sources (profiles/traffic_*.json), null when the sources have changed since.
  * cpu_baseline: the CPU oracle on a bounded sample of the same workload.
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

DECODE = {"decode_window", "decode_compress"}


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
    idx_bytes = nq * w.topk * 4
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
        sa.sparse_attn(self.q, self.kv, self.sink, self.idx, self.w.scale, out=self.out,
                       kv_scale=self.kv_scale, rope=(self.table, self.pos) if self.epilogue else None,
                       workspace=self.ws)

    def run(self):
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
                         rope=(table, pos0))
    ws_bytes = sa.sparse_attn_workspace_bytes(probe)
    nsets = max(2, min(64, math.ceil(2 * MALL_BYTES / max(touched_bytes, 1))))
    sets = []
    for k in range(nsets):
        c = (lambda t: t) if k == 0 else (lambda t: None if t is None else t.clone())
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev) if ws_bytes else None
        sets.append(Step(w, c(q0), c(kv0), c(scales0), sink, c(idx0), c(pos0), table, c(sp0), ws, epilogue))
    return sets


# ------------------------------------------------------------------ timing
def time_graph(sets, steps: int, warmup: int):
    """Capture one pass over all sets in a HIP graph; replay it to cover warmup and the K
    timed steps. Returns ms per step."""
    n = len(sets)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for s in sets:              # eager pass (also loads the kernels)
            s.run()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for s in sets:
            s.run()
    torch.cuda.synchronize()
    for _ in range(max(1, math.ceil(warmup / n))):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(steps / n))
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    return dt * 1e3 / (reps * n), reps * n, g


def time_kernel(sets, calls: int):
    """Average duration of one sparse_attn call: events on its stream around `calls`
    back-to-back calls over the input sets, after a GPU spin that lets the host enqueue them
    all first (so no host gap lands inside the interval). Returns (mean ms, mean ms of the
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
        e0.record(st)
        for i in range(calls):
            sets[i % len(sets)].attend()
        e1.record(st)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / calls)
    return float(np.mean(per)), float(np.min(per))


def cpu_baseline(w: W.Workload, kv_format: str, alg, budget_s: float = 12.0, rope: bool = True):
    """The oracle (plain C, OpenMP over queries) on a bounded sample of queries, scaled to
    the metric's unit."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from sa_harness import oracle_indices, oracle_run  # noqa: F401
    nq = w.b * w.s
    threads = oracle.max_threads()
    # per-query cost estimate from one query, then a sample sized to the budget
    t0 = time.perf_counter()
    oracle_run(w, qsel=np.array([nq - 1]), rope=rope, round_trip=w.kv_roundtrip, nthreads=1)
    one = time.perf_counter() - t0
    n = int(max(1, min(nq, budget_s * threads / max(one, 1e-6))))
    sel = np.linspace(0, nq - 1, n).round().astype(np.int64)
    sel = np.unique(sel)
    # when the whole step is cheaper than the budget, repeat it (at least 2 s of work)
    reps = 1
    t0 = time.perf_counter()
    while True:
        oracle_run(w, qsel=sel, rope=rope, round_trip=w.kv_roundtrip, nthreads=threads)
        dt = time.perf_counter() - t0
        if sel.size < nq or dt >= 2.0 or reps >= 100:
            break
        reps += 1
    per_step = dt / reps * nq / sel.size
    if w.name in DECODE:
        value, unit = alg["kv_bytes"] / per_step / 1e9, "GB/s"
    else:
        value, unit = alg["flops"] / per_step / 1e12, "TFLOP/s"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{sel.size} of {nq} queries (all heads) x {reps} run(s), oracle incl. "
                      f"fp8 round trip of their rows, window lists{' and inverse RoPE' if rope else ''}; {dt:.1f} s "
                      f"wall, scaled to one step"}


# ------------------------------------------------------------------ HBM traffic counters
CAL_BYTES = 1 << 30              # calibration copy: 1 GiB read, 1 GiB written
KERNEL_SOURCES = ["attn_fwd_kernel.hpp", "attn_fwd.hip", "attn_fwd_wide.hip", "sa_api.cpp", "sa_internal.hpp", "sa_device.hpp"]


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: line and block comments and whitespace are left
    out (the sources hold no comment markers inside string literals), so that an edit of a
    comment does not orphan counters taken on identical code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
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
    return rec["traffic_bytes_per_call"] if rec.get("kernel_source_sha") == kernel_source_hash() else None


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
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the attention kernel, each scaled
    by the ratio of the known size of the calibration copy to what the counter read for it."""
    import csv

    def read(path, counter):
        att, comb, cal = [], [], []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                name, v = r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0
                if "attn_fwd_kernel" in name:
                    att.append(v)
                elif "attn_combine_kernel" in name:
                    comb.append(v)
                elif "copyBuffer" in name or "elementwise" in name:
                    cal.append(v)
        if not att or not cal:
            raise SystemExit(f"{path}: no {counter} rows for the attention or the copy kernel")
        # the calibration copies are the three largest copy dispatches (input-set clones
        # before them are far smaller)
        cal = sorted(cal)[-3:]
        return float(np.mean(att)), (float(np.mean(comb)) if comb else 0.0), float(np.median(cal))

    fa, fc, fcal = read(fetch_csv, "FETCH_SIZE")
    wa, wc, wcal = read(write_csv, "WRITE_SIZE")
    kf, kw = CAL_BYTES / fcal, CAL_BYTES / wcal
    rec = {
        "workload": workload, "kv": kv, "kernel_source_sha": kernel_source_hash(),
        "fetch_bytes_raw": fa, "write_bytes_raw": wa,
        "combine_fetch_bytes_raw": fc, "combine_write_bytes_raw": wc,
        "copy_fetch_bytes_raw": fcal, "copy_write_bytes_raw": wcal, "copy_bytes": CAL_BYTES,
        "fetch_scale": kf, "write_scale": kw,
        "traffic_bytes_per_call": (fa + fc) * kf + (wa + wc) * kw,
    }
    os.makedirs(os.path.dirname(traffic_path(workload, kv)), exist_ok=True)
    with open(traffic_path(workload, kv), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode_window", choices=sorted(W.WORKLOADS))
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-epilogue", action="store_true",
                    help="time sparse_attn without the inverse-RoPE epilogue (plain bf16 output)")
    ap.add_argument("--profile-calls", type=int, default=0,
                    help="counter-collection mode: N eager steps over the input sets, then "
                         "the copy kernel of known size that calibrates the byte counters; "
                         "no timing, no JSON line")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "--profile-calls into profiles/traffic_<workload>_<kv>.json")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.workload, args.kv, *args.pmc_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sparse_attn would shard over heads with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sa.lib()

    w = W.make(args.workload)
    sets = None
    # the reference step's index lists, for the algorithmic counts
    probe_idx = torch.empty(w.b, w.s, w.topk, dtype=torch.int32, device=dev)
    view = probe_idx.view(w.win_nseq, w.win_seqlen, w.topk)
    sa.window_topk_idxs(w.window, w.win_seqlen, w.win_nseq,
                        start_pos=None if w.win_start_pos is None else w.win_start_pos.to(dev), out=view)
    if w.comp_idx is not None:
        probe_idx[:, :, w.win_cols:] = w.comp_idx.to(dev)
    alg = algorithmic(w, probe_idx.cpu().numpy(), args.kv, epilogue=not args.no_epilogue)
    del probe_idx

    sets = make_sets(w, args.kv, alg["attn_bytes"], dev, epilogue=not args.no_epilogue)
    if args.profile_calls:
        profile_pass(sets, args.profile_calls, dev)
        return
    ms_step, timed_steps, _g = time_graph(sets, args.steps, args.warmup)
    k_mean, k_best = time_kernel(sets, calls=min(400, max(50, args.steps // 5)))

    decode = w.name in DECODE
    if decode:
        value = alg["kv_bytes"] / (ms_step * 1e-3) / 1e9
        metric, unit = "sparse_attn KV GB/s (decode)", "GB/s"
        achieved = alg["attn_bytes"] / (k_mean * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None}
    else:
        value = alg["flops"] / (ms_step * 1e-3) / 1e12
        metric, unit = "sparse_attn TFLOP/s (prefill)", "TFLOP/s"
        achieved = alg["flops"] / (k_mean * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None}
    roof["traffic"] = stored_traffic(w.name, args.kv)
    roof["kernel"] = "sparse_attn (attn_fwd_kernel [+ attn_combine_kernel])"
    roof["kernel_ms_mean"] = k_mean
    roof["kernel_ms_best_batch"] = k_best
    roof["algorithmic_bytes_per_launch"] = alg["attn_bytes"]
    roof["algorithmic_flops_per_launch"] = alg["flops"]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.kv, alg, rope=not args.no_epilogue)

    rec = {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": timed_steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if args.kv == "bf16" else "fp8-e4m3 storage, bf16 compute",
        "data": "synthetic",
        "config": {"workload": w.name, "sequences": w.b, "queries_per_sequence": w.s, "heads": w.h,
                   "head_dim": w.d, "rope_dim": w.rd, "topk": w.topk, "kv_rows_per_sequence": w.kv_rows,
                   "kv_storage": args.kv, "epilogue": "none" if args.no_epilogue else "inverse RoPE", "input_sets": len(sets),
                   "kv_bytes_per_step": alg["kv_bytes"], "distinct_kv_rows": alg["distinct_rows"],
                   "valid_pairs": alg["valid_pairs"]},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
