#!/usr/bin/env python3
"""Benchmark of the q6_K x q8 decode GEMV path on one MI355X.

A step is one pass of the hot path over one batch: RMSNorm -> q8 on the
activation row(s) and the q6_K (dpl) x q8 GEMV over the 152064 x 5120 lm_head
matrix (638.67 MB of q6_K content). By default the step is the library's fused
RMSNorm -> q8 -> GEMV call (one kernel); --path split runs the producer kernel then
the GEMV kernel. Inputs are resident in HBM before timing starts. The weights
rotate over enough device copies (>= 1 GiB in total) that the 256 MB last-level
cache cannot serve them from one step to the next.

Prints one JSON line: content GB/s of the whole step (`value`), the dominant
kernel's own rate against the 8 TB/s HBM peak (`roofline`, timed with HIP events on
the stream the kernels run on), and the oracle timed on host cores (`cpu_baseline`).

    python bench.py [--gpus 1] [--steps 300] [--warmup 100] [--nt 1] [--path fused|split]
                    [--no-cpu-baseline]
    python bench.py --copy-calib    # plain device copy of known size, for counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
PAGES_LM_HEAD_GBS = 250.0       # the pages' dpl lm_head content rate (GB10; context only)
ROTATE_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mmvq_lm_head_traffic.txt")
TYPE_NAMES = {12: "q4_K", 13: "q5_K", 14: "q6_K"}
# the GEMV kernel by the plan's kind
GEMV_KERNELS = {0: "mmvq_long", 1: "mmvq_rows", 2: "mmvq_split", 3: "mmvq_pairs"}
PRODUCER_NAMES = {"rmsnorm": "fused RMSNorm->q8", "swiglu": "fused SwiGLU->q8",
                  "quant": "q8"}
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_decode_gemv_amd", "csrc", f)
                  for f in ("mmvq.hip", "q6k_unit.h", "q6k_norm.h", "kq_unit.h", "kq_format.h",
                            "bufload.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """The source without its comments, trailing blanks and empty lines, so that an
    edit of comments alone keeps the hash (the kernels are the same)."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] in "\"'":
            q, j = text[i], i + 1
            while j < n and text[j] != q:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    lines = ("".join(out)).split("\n")
    return "\n".join(l.rstrip() for l in lines if l.strip())


def kernel_hash() -> str:
    """sha256 (first 16 hex) of the kernel sources' code (comments stripped)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(key: str):
    """HBM bytes per launch of the dominant kernel (key: e.g. fused_nt1, gemv_nt4)
    from the committed counter summary, or None when the summary is absent or was
    taken on a different kernel source."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                parts = line.split()
                if len(parts) == 2 and not line.startswith("#"):
                    kv[parts[0]] = parts[1]
        if kv.get("kernel_sha") != kernel_hash():
            return None
        return float(kv[f"bytes_per_launch_{key}"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calib(steps: int) -> None:
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes_read": n, "copy_calib_bytes_written": n,
                      "launches": steps}), flush=True)


def read_ceiling(sizes_mb, steps: int) -> None:
    """The read ceiling by size: the probe library streams each size with the GEMV's
    load form and row walk (4 KB rows, no arithmetic), `steps` launches per HIP graph
    replay; the best of depths 1-4 and grids of 1-8 workgroups per CU is one JSON line
    per size. Buffers rotate over
    copies of at least 1 GiB in all, as the GEMV's weights do, so no launch reads
    what the last one left in the caches."""
    import ctypes
    import torch
    from quantized_decode_gemv_amd import build as libbuild
    if not os.path.exists(libbuild.PROBE_LIB):
        libbuild.build()
    lib = ctypes.CDLL(libbuild.PROBE_LIB)
    lib.q6k_read_probe.restype = ctypes.c_int
    lib.q6k_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p]
    dev = "cuda:0"
    num_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    for mb in sizes_mb:
        nbytes = int(mb * 1e6) // 4096 * 4096
        copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
        best = None
        for depth in (1, 2, 3, 4):
            for wpc in (1, 2, 4, 8):
                grid = num_cu * wpc

                def launch(i, st):
                    rc = lib.q6k_read_probe(bufs[i % copies].data_ptr(), nbytes, depth, grid,
                                            sink.data_ptr(), st.cuda_stream)
                    assert rc == 0, rc
                # the launches are replayed from a HIP graph: a few-microsecond kernel
                # launched from Python would measure the host's launch rate instead
                side = torch.cuda.Stream()
                with torch.cuda.stream(side):
                    for i in range(copies):
                        launch(i, side)
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=side):
                    for i in range(steps):
                        launch(i, side)
                graph.replay()
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(side):
                    e0.record(side)
                    graph.replay()
                    e1.record(side)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / steps
                del graph
                if best is None or us < best[0]:
                    best = (us, depth, grid)
        us, depth, grid = best
        print(json.dumps({"read_ceiling_bytes": nbytes, "us": round(us, 2),
                          "TB_per_s": round(nbytes / us / 1e6, 3), "depth": depth,
                          "grid": grid, "launches_per_graph": steps}), flush=True)
        del bufs
        torch.cuda.empty_cache()


def cpu_baseline(w, raw, x, g, gate, up, nt: int, budget_s: float = 20.0) -> dict:
    """The oracle chain (the workload's producer, q8, GEMV) on the host over a row
    sample of the same matrix, single thread; the sample is sized to stay near
    budget_s and only the GEMV is timed."""
    import oracle
    import q6ksynth

    if w.producer == "rmsnorm":
        xn = oracle.rmsnorm(x, g, q6ksynth.RMS_EPS)
    elif w.producer == "swiglu":
        xn = oracle.swiglu(gate, up)
    else:
        xn = x
    qs, d = oracle.quant_q8(xn)

    def gemv(n):
        if w.qtype == q6ksynth.Q6_K:
            oracle.mmvq(oracle.RAW, raw[:n], n, w.K, qs, d, nthreads=1)
        else:
            oracle.kq_mmvq(w.qtype, oracle.RAW, raw[:n], n, w.K, qs, d, nthreads=1)

    probe = min(2048, w.N)
    t0 = time.perf_counter()
    gemv(probe)
    per_row = (time.perf_counter() - t0) / probe
    rows = int(min(w.N, max(probe, budget_s / 3 / per_row)))
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        gemv(rows)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    content = rows * w.nbe * q6ksynth.KQ_BLOCK_BYTES[w.qtype]
    return {"value": round(content / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {rows} of {w.N} rows of the {w.N}x{w.K} matrix, nt={nt}, "
                      f"scalar C oracle GEMV (fp64), single thread, median of 3 runs "
                      f"({t:.2f} s each); the host producer and q8 not timed",
            "us_per_gemv_equiv": round(t / rows * w.N * 1e6, 1)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--nt", type=int, default=1, help="activation rows per step (1 or 4)")
    ap.add_argument("--workload", default="lm_head")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--read-ceiling", default=None, metavar="MB,MB,...",
                    help="time the read probe at these sizes (MB) instead of the GEMV step")
    ap.add_argument("--path", choices=["fused", "split", "formb"], default="fused",
                    help="fused: one RMSNorm -> q8 -> GEMV call per step (RMSNorm workloads "
                         "only); split: the producer kernel, then the GEMV kernel; formb: "
                         "gate+up GEMV, SwiGLU and q8 in one call on a resident q8 row "
                         "(gate+up workloads, one token), against the GEMV then the SwiGLU "
                         "producer")
    ap.add_argument("--graph", type=int, default=0, metavar="G",
                    help="run the timed steps as replays of a HIP graph holding G steps")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the path is measured on one GPU's share at its "
              f"real shape); --gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import q6ksynth
    import quantized_decode_gemv_amd as q

    if args.copy_calib:
        copy_calib(args.steps)
        return 0
    if args.read_ceiling:
        read_ceiling([float(v) for v in args.read_ceiling.split(",")], args.steps)
        return 0

    dev = "cuda:0"
    w = q6ksynth.WORKLOADS[args.workload]
    N, K, nt = w.N, w.K, args.nt
    log(f"bench: {w.name} N={N} K={K} nt={nt} steps={args.steps} warmup={args.warmup}")

    raw = q6ksynth.weights(w)
    qt = w.qtype
    dpl_bytes = q.kq_dpl_bytes(qt, N, K)
    copies = max(2, math.ceil(ROTATE_BYTES / dpl_bytes)) if dpl_bytes < ROTATE_BYTES else 2
    copies = min(copies, 4096)
    raw_d = torch.from_numpy(raw.reshape(-1)).to(dev)
    W0 = torch.empty(dpl_bytes, dtype=torch.uint8, device=dev)
    q.repack_kq_dpl(qt, raw_d, W0, N, K)
    del raw_d
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]

    g = q6ksynth.gamma(K, q6ksynth.gamma_seed(w))
    g_d = torch.from_numpy(g).to(dev)
    x = gate = up = x_d = gate_d = up_d = None
    if w.producer == "swiglu":
        gate, up = q6ksynth.swiglu_pairs(w, nt)
        gate_d = torch.from_numpy(gate).to(dev)
        up_d = torch.from_numpy(up).to(dev)
    else:
        x = q6ksynth.activations(w, nt)
        x_d = torch.from_numpy(x).to(dev)
    y_norm = torch.empty((nt, K), dtype=torch.float32, device=dev)
    plane = torch.empty(q.q8_plane_bytes(K, nt), dtype=torch.uint8, device=dev)
    y = torch.empty((nt, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    # the fused call runs as one kernel only for the shapes the library fuses (one
    # token); elsewhere it would queue the same two kernels as the split step
    fused = (args.path == "fused" and w.producer == "rmsnorm"
             and q.rmsnorm_mmvq_fused(N, K, nt))

    def produce(st):
        if w.producer == "rmsnorm":
            q.rmsnorm_quant_q8(x_d, g_d, q6ksynth.RMS_EPS, y_norm, plane, K, nt, st)
        elif w.producer == "swiglu":
            q.swiglu_quant_q8(gate_d, up_d, y_norm, plane, K, nt, st)
        else:
            q.quant_q8(x_d, plane, K, nt, st)

    def gemv(i, st):
        q.mmvq_kq_q8(qt, Ws[i % copies], plane, y, N, K, nt, st)

    def fused_call(i, st):
        q.mmvq_kq_rmsnorm_q8(qt, Ws[i % copies], x_d, g_d, q6ksynth.RMS_EPS, None, plane, y,
                             N, K, nt, st)

    def split_step(i, st):
        produce(st)
        gemv(i, st)

    formb = args.path == "formb"
    if formb:
        # the matrix is [gate rows; up rows]; the activation row's q8 plane stays resident
        if nt != 1 or N % 64:
            print("--path formb takes one token and an even number of 32-row blocks",
                  file=sys.stderr)
            return 2
        Nh = N // 2
        produce(stream)
        torch.cuda.synchronize()
        gu = torch.empty(N, dtype=torch.float32, device=dev)
        y_sw = torch.empty(Nh, dtype=torch.float32, device=dev)
        plane_out = torch.empty(q.q8_plane_bytes(Nh, 1), dtype=torch.uint8, device=dev)

        def formb_call(i, st):
            q.mmvq_kq_gate_up_swiglu_q8(qt, Ws[i % copies], plane, gu, None, plane_out, Nh, K,
                                        1, st)

        def gemv_swiglu(i, st):
            q.mmvq_kq_q8(qt, Ws[i % copies], plane, gu, N, K, 1, st)
            q.swiglu_quant_q8(gu[:Nh], gu[Nh:], y_sw, plane_out, Nh, 1, st)

        fused = False
        step, split_step = formb_call, gemv_swiglu
    else:
        step = fused_call if fused else split_step

    def time_steps(fn, n):
        t0 = time.perf_counter()
        for i in range(n):
            fn(i, stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    def time_back_to_back(fn, n):
        """Launches back to back on the stream between two HIP events recorded on
        that stream; mean duration per launch."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    for i in range(args.warmup):
        step(i, stream)
        if fused or formb:
            split_step(i, stream)
    torch.cuda.synchronize()

    # The step loop: weights rotating, nothing else queued. With --graph G the same
    # launches are captured G steps at a time into one HIP graph (weights still
    # rotating inside it) and the graph is replayed.
    if args.graph > 0:
        G = args.graph
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for i in range(G):
                    step(i, side)
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup // G)):
            graph.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // G)
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / (reps * G)
    else:
        ms_per_step = time_steps(step, args.steps)
    ms_per_step_split = time_steps(split_step, args.steps) if (fused or formb) else None

    # The dominant kernel alone: the fused kernel (fused path, Form B) or the GEMV kernel.
    if formb:
        kern_us = time_back_to_back(formb_call, args.steps)
        gemv_us = time_back_to_back(lambda i, st: q.mmvq_kq_q8(qt, Ws[i % copies], plane, gu, N, K,
                                                               1, st), args.steps)
    else:
        kern_us = time_back_to_back(fused_call if fused else gemv, args.steps)
        gemv_us = time_back_to_back(gemv, args.steps) if fused else kern_us

    # Diagnostic: events around every GEMV inside producer+GEMV steps (these also
    # count each launch's dispatch latency).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(min(args.steps, 100))]
    for i, (a, b) in enumerate(evs):
        produce(stream)
        a.record(stream)
        gemv(i, stream)
        b.record(stream)
    torch.cuda.synchronize()
    inline = [a.elapsed_time(b) * 1e3 for a, b in evs]
    kern_inline_us = statistics.mean(inline)
    kern_inline_med_us = statistics.median(inline)

    content = w.content_bytes
    value = content / (ms_per_step * 1e-3) / 1e9
    achieved = content / (kern_us * 1e-6) / 1e9
    traffic = (None if formb or w.name != "lm_head"
               else recorded_traffic(f"{'fused' if fused else 'gemv'}_nt{nt}"))
    plan = q.mmvq_plan(N, K, nt, torch.cuda.get_device_properties(0).multi_processor_count, qt)

    out = {
        "metric": "q6_K MMVQ content GB/s and % of HBM peak; us per GEMV at lm_head shape",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGES_LM_HEAD_GBS, 3) if (w.name == "lm_head" and nt == 1) else None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{w.name} {TYPE_NAMES[qt]} GEMV N={N} K={K} nt={nt}: "
                               + (f"RMSNorm->q8->split-plane {TYPE_NAMES[qt]} x q8 MMVQ in one "
                                  f"kernel" if fused else
                                  f"Form B: gate+up {TYPE_NAMES[qt]} GEMV, SwiGLU and q8 in one "
                                  f"kernel on a resident q8 row" if formb else
                                  f"{PRODUCER_NAMES[w.producer]} producer + split-plane "
                                  f"{TYPE_NAMES[qt]} x q8 MMVQ"),
                   "N": N, "K": K, "nt": nt, "content_bytes": content,
                   "dpl_bytes": dpl_bytes, "weight_copies": copies},
        "dominant_kernel": ("mmvq_rmsnorm_rows (fused)" if fused else
                            "gate_up_swiglu_rows (Form B)" if formb else
                            GEMV_KERNELS[plan["kind"]]),
        "us_per_dominant_kernel": round(kern_us, 2),
        "us_per_gemv": round(gemv_us, 2),
        "ms_per_step_split": round(ms_per_step_split, 5) if ms_per_step_split else None,
        "us_per_gemv_inline_events": {"mean": round(kern_inline_us, 2),
                                      "median": round(kern_inline_med_us, 2)},
        "pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "mmvq_plan": plan,
        "step_launch": f"hip graph of {args.graph} steps" if args.graph > 0 else "eager",
        "kernel_sha": kernel_hash(),
        "baseline_note": "vs_baseline divides by the pages' 250.0 GB/s dpl lm_head content "
                         "rate, measured on an NVIDIA GB10: context, not a target",
    }
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(w, raw, x, g, gate, up, nt)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
