#!/usr/bin/env python3
"""Benchmark of the q6_K x q8 decode GEMV path on one MI355X.

A step is one pass of the hot path over one batch: RMSNorm -> q8 on the
activation row(s) and the q6_K (dpl) x q8 GEMV over the 152064 x 5120 lm_head
matrix (638.67 MB of q6_K content). By default the step is the library's fused
RMSNorm -> q8 -> GEMV call (one kernel); --path split runs the producer kernel then
the GEMV kernel. Inputs are resident in HBM before timing starts. The weights
rotate over enough device copies (>= 1 GiB in total) that the 256 MB last-level
cache cannot serve them from one step to the next.

Timing protocol:
  - warm-up: the requested --warmup steps, continued until at least WARMUP_MIN_MS of
    GPU work and WARMUP_MIN_LAUNCHES launches have run (a fresh process runs its first
    milliseconds of launches slower); the effective count is reported;
  - steps: TRIALS trials of exactly --steps steps, each bracketed by
    torch.cuda.synchronize(); ms_per_step is the median trial;
  - kernels: TRIALS trials of max(--steps, MIN_KERNEL_LAUNCHES) back-to-back launches
    of the dominant kernel, the GEMV alone and the GEMV on one resident buffer ("hot",
    cache-resident for small matrices), interleaved, each bracketed by HIP events
    recorded on the launch stream; each figure is the median trial;
  - the dominant kernel's time must not exceed the step time (it is part of the step);
    if it does the measurement is repeated, and a run that stays inconsistent fails.

Prints one JSON line: content GB/s of the whole step (`value`), the dominant
kernel's own rate against the 8 TB/s HBM peak (`roofline`), the read ceiling measured
live at the same size (`read_ceiling`, best of the probe's load forms) and the oracle
timed on host cores, one thread and all cores (`cpu_baseline`).

    python bench.py [--gpus 1] [--steps 300] [--warmup 100] [--nt 1] [--path fused|split]
                    [--no-cpu-baseline] [--no-read-ceiling]
    python bench.py --copy-calib    # plain device copy of known size, for counter scaling
    python bench.py --read-ceiling MB,MB,...   # read ceiling by size, every probe form
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
TRIALS = 5
MIN_KERNEL_LAUNCHES = 200
WARMUP_MIN_MS = 200.0
WARMUP_MIN_LAUNCHES = 100
# workloads whose content takes under this long at the HBM peak are bound by launch
# latency, not by HBM: their GB/s says little about the memory system
LAUNCH_BOUND_US = 2.0
# plain-stream probe forms (q6k_read_probe_stream)
PROBE_FORMS = {0: "buffer_nt", 1: "buffer_default", 2: "global_nt", 3: "global_default"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mmvq_lm_head_traffic.txt")
TYPE_NAMES = {12: "q4_K", 13: "q5_K", 14: "q6_K"}
# the GEMV kernel by the plan's kind
GEMV_KERNELS = {0: "mmvq_long", 1: "mmvq_rows", 2: "mmvq_split", 3: "mmvq_pairs",
                4: "mmvq_tiles"}
PRODUCER_NAMES = {"rmsnorm": "fused RMSNorm->q8", "swiglu": "fused SwiGLU->q8",
                  "quant": "q8"}
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_decode_gemv_amd", "csrc", f)
                  for f in ("mmvq.hip", "tiles.hip", "q6k_unit.h", "q6k_norm.h", "kq_unit.h",
                            "kq_format.h", "bufload.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """The source without its comments, every run of blanks and line breaks outside
    string literals made one space, so that an edit of comments or layout alone keeps
    the hash (the kernels are the same)."""
    parts, buf, i, n = [], [], 0, len(text)

    def flush():
        code = " ".join("".join(buf).split())
        if code:
            parts.append(code)
        buf.clear()

    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            buf.append(" ")
        elif text[i] in "\"'":
            q, j = text[i], i + 1
            while j < n and text[j] != q:
                j += 2 if text[j] == "\\" else 1
            flush()
            parts.append(text[i:j + 1])
            i = j + 1
        else:
            buf.append(text[i])
            i += 1
    flush()
    return " ".join(parts)


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


class ReadProbe:
    """The read-bandwidth probe library (csrc/read_probe.hip): the GEMV's row walk and
    plain streams of several load forms, timed from HIP-graph replays (a kernel of a
    few microseconds launched from Python would measure the host's launch rate)."""

    def __init__(self):
        import ctypes
        import torch
        from quantized_decode_gemv_amd import build as libbuild
        if not os.path.exists(libbuild.PROBE_LIB):
            raise RuntimeError(f"{libbuild.PROBE_LIB} is not built (run __graft_entry__.build())")
        self.torch = torch
        lib = ctypes.CDLL(libbuild.PROBE_LIB)
        lib.q6k_read_probe.restype = ctypes.c_int
        lib.q6k_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.q6k_read_probe_stream.restype = ctypes.c_int
        lib.q6k_read_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p]
        self.lib = lib
        self.num_cu = torch.cuda.get_device_properties(0).multi_processor_count
        self.sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")

    def configs(self, full: bool):
        """(name, config) pairs: the row walk over depths and workgroups per CU, and the
        plain streams over forms, bytes per lane, loads in flight and workgroups per CU.
        full=False is the short list the default bench measures live."""
        out = []
        for depth in ((1, 2, 3, 4) if full else (1, 2, 3)):
            for wpc in ((1, 2, 4, 8) if full else (1, 2)):
                out.append(("row_walk", dict(kind="rows", depth=depth, wpc=wpc)))
        # the short list: the shapes that won the full sweep at 4-640 MB (non-temporal
        # loads, 8 B x 4 or 4 B x 8 per lane, 2-8 workgroups per CU)
        shapes = ([(w, u) for w in (16, 8, 4) for u in (4, 8, 16)] if full
                  else [(16, 4), (8, 4), (4, 8), (16, 8)])
        for form in ((0, 1, 2, 3) if full else (0, 2)):
            for width, unroll in shapes:
                for wpc in ((1, 2, 4, 8) if full else (2, 4, 8)):
                    out.append((PROBE_FORMS[form],
                                dict(kind="stream", form=form, width=width, unroll=unroll,
                                     wpc=wpc)))
        return out

    def time(self, nbytes: int, cfg: dict, steps: int) -> float:
        """Microseconds per launch over copies of >= 1 GiB in all (rotating, so no launch
        reads what the last one left in the caches)."""
        torch = self.torch
        copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
        buf = torch.empty(copies * nbytes, dtype=torch.uint8, device="cuda:0")
        base = buf.data_ptr()
        grid = self.num_cu * cfg["wpc"]

        def launch(i, st):
            ptr = base + (i % copies) * nbytes
            if cfg["kind"] == "rows":
                rc = self.lib.q6k_read_probe(ptr, nbytes, cfg["depth"], grid,
                                             self.sink.data_ptr(), st.cuda_stream)
            else:
                rc = self.lib.q6k_read_probe_stream(ptr, nbytes, cfg["form"], cfg["width"],
                                                    cfg["unroll"], grid, self.sink.data_ptr(),
                                                    st.cuda_stream)
            assert rc == 0, (rc, cfg)
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
        del graph, buf
        return e0.elapsed_time(e1) * 1e3 / steps

    def ceiling(self, nbytes: int, steps: int, full: bool):
        """Best time for nbytes (rounded down to whole 64 KB tiles) over the configs:
        (best record, {form: best record of that form})."""
        nbytes = nbytes // 65536 * 65536
        best, by_form = None, {}
        for name, cfg in self.configs(full):
            us = self.time(nbytes, cfg, steps)
            rec = dict(form=name, us=round(us, 3), GB_per_s=round(nbytes / us / 1e3, 1),
                       grid=self.num_cu * cfg["wpc"],
                       **{k: v for k, v in cfg.items() if k not in ("kind", "form", "wpc")})
            if name not in by_form or us < by_form[name]["us"]:
                by_form[name] = rec
            if best is None or us < best["us"]:
                best = rec
        best = dict(best, bytes=nbytes)
        return best, by_form


def read_ceiling(sizes_mb, steps: int) -> None:
    """The read ceiling by size: every probe form and launch shape, `steps` launches per
    HIP graph replay; one JSON line per size with the best overall and per form."""
    probe = ReadProbe()
    for mb in sizes_mb:
        best, by_form = probe.ceiling(int(mb * 1e6), steps, full=True)
        print(json.dumps({"read_ceiling_bytes": best["bytes"], "us": best["us"],
                          "TB_per_s": round(best["GB_per_s"] / 1e3, 3), "best": best,
                          "best_by_form": by_form, "launches_per_graph": steps}), flush=True)


def host_cpu() -> dict:
    """The host's core count (nproc), the cores this process may run on, and the CPU
    model from /proc/cpuinfo."""
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
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"nproc": os.cpu_count(), "usable": usable, "model": model}


def cpu_baseline(w, raw, x, g, gate, up, nt: int, budget_s: float = 12.0) -> dict:
    """The oracle chain (the workload's producer, q8, GEMV) on the host over a row
    sample of the same matrix; only the GEMV is timed, on one thread (the canonical
    baseline, `value`) and on all the cores the process may use, at most 16 (the
    oracle's OpenMP rows-parallel loop; `all_cores`). Each leg's sample is sized to
    stay near budget_s over its 3 runs; each figure is the median run."""
    import oracle
    import q6ksynth

    if w.producer == "rmsnorm":
        xn = oracle.rmsnorm(x, g, q6ksynth.RMS_EPS)
    elif w.producer == "swiglu":
        xn = oracle.swiglu(gate, up)
    else:
        xn = x
    qs, d = oracle.quant_q8(xn)

    def gemv(n, threads):
        if w.qtype == q6ksynth.Q6_K:
            oracle.mmvq(oracle.RAW, raw[:n], n, w.K, qs, d, nthreads=threads)
        else:
            oracle.kq_mmvq(w.qtype, oracle.RAW, raw[:n], n, w.K, qs, d, nthreads=threads)

    def leg(threads):
        probe = min(2048 * threads, w.N)
        t0 = time.perf_counter()
        gemv(probe, threads)
        per_row = (time.perf_counter() - t0) / probe
        rows = int(min(w.N, max(probe, budget_s / 3 / per_row)))
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            gemv(rows, threads)
            times.append(time.perf_counter() - t0)
        t = statistics.median(times)
        content = rows * w.nbe * q6ksynth.KQ_BLOCK_BYTES[w.qtype]
        return rows, t, content / t / 1e9

    host = host_cpu()
    threads = max(1, min(16, host["usable"]))
    rows1, t1, gbs1 = leg(1)
    rowsn, tn, gbsn = leg(threads)
    return {"value": round(gbs1, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {rows1} of {w.N} rows of the {w.N}x{w.K} matrix, nt={nt}, "
                      f"scalar C oracle GEMV (fp64), single thread, median of 3 runs "
                      f"({t1:.2f} s each); the host producer and q8 not timed",
            "us_per_gemv_equiv": round(t1 / rows1 * w.N * 1e6, 1),
            "all_cores": {"value": round(gbsn, 4), "unit": "GB/s", "cores": threads,
                          "sample": f"first {rowsn} of {w.N} rows, the same oracle GEMV split "
                                    f"by rows over {threads} OpenMP threads, median of 3 runs "
                                    f"({tn:.2f} s each)",
                          "us_per_gemv_equiv": round(tn / rowsn * w.N * 1e6, 1)},
            "host": host}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--nt", type=int, default=1, help="activation rows per step (1 or 4)")
    ap.add_argument("--workload", default="lm_head")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the live read-ceiling measurement at the workload's size")
    ap.add_argument("--under-counters", action="store_true",
                    help="the run is under a counter-collecting profiler (rocprofv3 --pmc), "
                         "which serialises dispatches: timings are not meaningful, so the "
                         "kernel <= step consistency check is skipped")
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
    # enough copies that the rotation spans >= 1 GiB (4x the last-level cache), in one
    # allocation: copy i at byte i * dpl_bytes (a multiple of 16)
    copies = max(2, math.ceil(ROTATE_BYTES / dpl_bytes))
    raw_d = torch.from_numpy(raw.reshape(-1)).to(dev)
    W_all = torch.empty(copies * dpl_bytes, dtype=torch.uint8, device=dev)
    W0 = W_all[:dpl_bytes]
    q.repack_kq_dpl(qt, raw_d, W0, N, K)
    del raw_d
    W_all.view(copies, dpl_bytes)[1:].copy_(W0.view(1, dpl_bytes).expand(copies - 1, dpl_bytes))
    Ws = [W_all[i * dpl_bytes:(i + 1) * dpl_bytes] for i in range(copies)]

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

    def gemv_hot(i, st):
        q.mmvq_kq_q8(qt, W0, plane, y, N, K, nt, st)

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

        def gemv(i, st):
            q.mmvq_kq_q8(qt, Ws[i % copies], plane, gu, N, K, 1, st)

        def gemv_hot(i, st):
            q.mmvq_kq_q8(qt, W0, plane, gu, N, K, 1, st)

        fused = False
        step, split_step = formb_call, gemv_swiglu
        dominant = formb_call
    else:
        step = fused_call if fused else split_step
        dominant = fused_call if fused else gemv
    produce(stream)                     # the GEMV-only timings read a valid q8 plane

    def events_over(fn, n):
        """n launches back to back between two HIP events recorded on the launch
        stream; us per launch."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    # Warm-up: the requested steps, then on until WARMUP_MIN_MS of GPU time and
    # WARMUP_MIN_LAUNCHES launches have run.
    torch.cuda.synchronize()
    t_w = time.perf_counter()
    warm_launches = 0
    for i in range(args.warmup):
        step(i, stream)
        warm_launches += 1
    torch.cuda.synchronize()
    while ((time.perf_counter() - t_w) * 1e3 < WARMUP_MIN_MS
           or warm_launches < WARMUP_MIN_LAUNCHES):
        for i in range(20):
            step(i, stream)
            if fused or formb:
                split_step(i, stream)
        warm_launches += 20
        torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t_w) * 1e3

    graph = None
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

    def step_trial():
        """One trial of exactly --steps steps (graph: replays of G steps), bracketed by
        synchronisations; (host ms per step, event ms per step)."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        if graph is not None:
            reps = max(1, args.steps // args.graph)
            for _ in range(reps):
                graph.replay()
            n = reps * args.graph
        else:
            for i in range(args.steps):
                step(i, stream)
            n = args.steps
        e1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n, e0.elapsed_time(e1) / n

    R = max(args.steps, MIN_KERNEL_LAUNCHES)

    def measure():
        steps_host, steps_ev, kern, gem, hot, split = [], [], [], [], [], []
        for _ in range(TRIALS):
            h, e = step_trial()
            steps_host.append(h)
            steps_ev.append(e)
            kern.append(events_over(dominant, R))
            if fused or formb:
                gem.append(events_over(gemv, R))
            hot.append(events_over(gemv_hot, R))
            if fused or formb:
                t0 = time.perf_counter()
                for i in range(args.steps):
                    split_step(i, stream)
                torch.cuda.synchronize()
                split.append((time.perf_counter() - t0) * 1e3 / args.steps)
        return dict(step=steps_host, step_ev=steps_ev, kern=kern, gemv=gem or kern, hot=hot,
                    split=split)

    med = statistics.median
    for attempt in range(3):
        m = measure()
        ms_per_step, kern_us = med(m["step"]), med(m["kern"])
        if kern_us <= 1000.0 * ms_per_step * 1.01 or args.under_counters:
            break
        log(f"bench: dominant kernel {kern_us:.2f} us > step {1000 * ms_per_step:.2f} us; "
            f"measuring again")
    else:
        raise AssertionError(f"dominant kernel time {kern_us:.2f} us exceeds the step time "
                             f"{1000 * ms_per_step:.2f} us in three measurements")
    gemv_us, hot_us = med(m["gemv"]), med(m["hot"])
    ms_per_step_split = med(m["split"]) if m["split"] else None

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

    content = w.content_bytes
    value = content / (ms_per_step * 1e-3) / 1e9
    achieved = content / (kern_us * 1e-6) / 1e9
    traffic = (None if formb or w.name != "lm_head"
               else recorded_traffic(f"{'fused' if fused else 'gemv'}_nt{nt}"))
    plan = q.mmvq_plan(N, K, nt, torch.cuda.get_device_properties(0).multi_processor_count, qt)
    launch_bound = content / (HBM_PEAK_GBS * 1e3) < LAUNCH_BOUND_US

    ceiling = None
    if not args.no_read_ceiling:
        log("bench: read ceiling at the workload's size")
        del W_all, Ws, W0
        torch.cuda.empty_cache()
        best, by_form = ReadProbe().ceiling(content, 100, full=False)
        ceiling = dict(best, best_by_form=by_form)

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
                   "dpl_bytes": dpl_bytes, "weight_copies": copies,
                   "rotation_bytes": copies * dpl_bytes},
        "timing": {"warmup_effective_launches": warm_launches,
                   "warmup_ms": round(warm_ms, 1), "trials": TRIALS,
                   "steps_per_trial": args.steps, "kernel_launches_per_trial": R,
                   "step_ms_trials": [round(v, 5) for v in m["step"]],
                   "step_ms_trials_events": [round(v, 5) for v in m["step_ev"]],
                   "dominant_us_trials": [round(v, 2) for v in m["kern"]],
                   "statistic": "median of trials"},
        "dominant_kernel": ("mmvq_rmsnorm_rows (fused)" if fused else
                            "gate_up_swiglu_rows (Form B)" if formb else
                            GEMV_KERNELS[plan["kind"]]),
        "us_per_dominant_kernel": round(kern_us, 2),
        "us_per_gemv": round(gemv_us, 2),
        "us_per_gemv_hot": round(hot_us, 2),
        "hot_note": "the GEMV on one resident weight buffer, no rotation: cache-resident "
                    "when the matrix fits the 256 MB last-level cache",
        "ms_per_step_split": round(ms_per_step_split, 5) if ms_per_step_split else None,
        "us_per_gemv_inline_events": {"mean": round(statistics.mean(inline), 2),
                                      "median": round(med(inline), 2)},
        "pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "launch_bound": launch_bound,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "fetch_over_content": round(traffic / content, 4) if traffic else None,
        "read_ceiling": ceiling,
        "pct_of_read_ceiling": (round(100 * achieved / ceiling["GB_per_s"], 2)
                                if ceiling else None),
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
