#!/usr/bin/env python3
"""Benchmark of the fused affine-quantized matmul on one MI355X.

Headline (one JSON line on stdout): fused 4-bit qGEMV HBM GB/s at M=1 on the
Llama-3.2-1B-shaped decode projections (q/o 2048x2048, k/v 512x2048,
gate/up 8192x2048, down 2048x8192, lm_head 128256x2048; N x K, g64, f16
scales/biases, f16 x ~ N(0,1)).  One step = every projection once, launched
as a decoder layer allows: projections reading the same activation share one
mxq_qmv_grouped launch -- {q,k,v}, {o}, {gate,up}, {down}, {lm_head}, 5
launches (the 8-launch and 1-launch plans are reported too).  The projection
set is replicated REPLICAS times with distinct seeded weights (~1.1 GB in total) and the steps cycle through the replicas,
so every step streams its weights from HBM, not from the 256 MB Infinity
Cache.  value = algorithmic bytes per step / time per step.

Extra objects on the same line:
  roofline      the dominant kernel (most time per step), timed per launch with
                HIP events on the launch stream: algorithmic bytes / duration,
                against the 8 TB/s HBM peak;  traffic from committed rocprofv3
                PMC counters when they match the current kernel source;
  cpu_baseline  the f64 CPU oracle on a bounded sample (layer 0 and a slice
                of lm_head), all cores and one pinned core, with the host's
                CPU model and thread counts;
  read_probe    GB/s of a plain 16-byte streaming read at the per-launch byte
                counts (the floor small launches are judged against);
  configs       the small single problem (N=512) and the 48-case edge sweep,
                GB/s per launch;
  decode_step   16 layers x {q,k,v,o,gate,up,down} + lm_head, ~697 MB of
                distinct weights, as 113 separate launches and as 65 grouped
                launches (eager and graph replay): bytes/step, GB/s, steps/s;
  qmm           M=512 prefill on gate/up (8192x2048) and down (2048x8192),
                f16 and bf16 scales, after a 200 ms warm-up the median of three
                rounds of 20 calls back to back per projection:
                TFLOP/s and MFMA utilisation (of the 2.5 PFLOP/s dense f16
                peak); the same projections with int8 activations
                (mxq_linear_a8, integer matrix cores): TOP/s against the
                5.0 POP/s dense int8 peak;
  bf16_activations  the lm_head decode launch (GB/s) and the M=512 prefill
                projections (TFLOP/s) with bf16 x and y;
  few_rows      the lm_head launch at M = 1, 2, 4, 8 and 16: the f16 route of
                mxq_qmv (decode kernel at M = 1, the K-split matrix-core kernel
                from M = 2; kernel named) against the int8-activation route
                (mxq_linear_a8), GB/s;
  dequant       standalone dequant of the lm_head weights to f32, GB/s.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused 4-bit qGEMV HBM GB/s (% of peak) at M=1; qGEMM TFLOP/s at M=512"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
MFMA_I8_PEAK_TOPS = 5000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qmv_traffic.json")
SETTLE_MS = 200.0  # untimed run of the step before the warm-up steps (see the headline timing)
KERNEL_SOURCES = [os.path.join(ROOT, "dequant_matmul_qmv_amd", "csrc", f)
                  for f in ("qmv.hip", "mxq_device.h")]


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def call_bytes(M, N, K, bits=4, group_size=64):
    """Algorithmic bytes of one fused call: codes + scales + biases + x + y."""
    G = K // group_size
    return N * K * bits // 8 + 2 * N * G * 2 + M * K * 2 + M * N * 2


class Call:
    """One pre-marshalled mxq_qmv / mxq_qmm launch (raw pointers only)."""

    def __init__(self, lib, fn, x, w, s, b, y, M, N, K, bits, gs, sb_code, name):
        self.fn = getattr(lib, fn)
        self.tensors = (x, w, s, b, y)  # keep alive
        self.args = (x.data_ptr(), w.data_ptr(), s.data_ptr(), b.data_ptr(), y.data_ptr(),
                     M, N, K, bits, gs, sb_code)
        self.name = name
        self.M, self.N, self.K = M, N, K
        self.bytes = call_bytes(M, N, K, bits, gs)

    def __call__(self, stream_handle):
        st = self.fn(*self.args, stream_handle)
        if st != 0:
            raise RuntimeError(f"{self.name}: libmxq status {st}")


class GroupCall:
    """One pre-marshalled mxq_qmv_grouped launch over a list of Call problems."""

    def __init__(self, lib, mxq, calls):
        self.fn = lib.mxq_qmv_grouped
        self.arr = (mxq.QmvProblem * len(calls))(*[
            mxq.QmvProblem(c.args[0], c.args[1], c.args[2], c.args[3], c.args[4], c.N, c.K) for c in calls])
        self.calls = calls
        self.bytes = sum(c.bytes for c in calls)

    def __call__(self, stream_handle):
        st = self.fn(self.arr, len(self.calls), 1, 4, 64, 0, stream_handle)
        if st != 0:
            raise RuntimeError(f"grouped launch: libmxq status {st}")


class A8Call:
    """One pre-marshalled mxq_linear_a8 launch (f16 x quantized per row to int8; no output bias)."""

    def __init__(self, lib, x, w, s, b, y, M, N, K, name, bits=4, gs=64, sb_code=0):
        self.fn = lib.mxq_linear_a8
        self.tensors = (x, w, s, b, y)  # keep alive
        self.args = (x.data_ptr(), w.data_ptr(), s.data_ptr(), b.data_ptr(), None, y.data_ptr(),
                     M, N, K, bits, gs, sb_code)
        self.name = name
        self.M, self.N, self.K = M, N, K

    def __call__(self, stream_handle):
        st = self.fn(*self.args, stream_handle)
        if st != 0:
            raise RuntimeError(f"{self.name}: libmxq status {st}")


class ActCall:
    """One pre-marshalled mxq_linear_act launch with bf16 activations (no output bias)."""

    def __init__(self, lib, x, w, s, b, y, M, N, K, name, bits=4, gs=64):
        self.fn = lib.mxq_linear_act
        self.tensors = (x, w, s, b, y)  # keep alive
        self.args = (x.data_ptr(), w.data_ptr(), s.data_ptr(), b.data_ptr(), None, y.data_ptr(),
                     M, N, K, bits, gs, 0, 1)
        self.name = name
        self.M, self.N, self.K = M, N, K

    def __call__(self, stream_handle):
        st = self.fn(*self.args, stream_handle)
        if st != 0:
            raise RuntimeError(f"{self.name}: libmxq status {st}")


def make_qmv_set(mxq, lib, synth, torch, config, replica, shapes, dev, sb="f16"):
    import numpy as np
    calls = []
    sbt = torch.float16 if sb == "f16" else torch.bfloat16
    for idx, (name, N, K) in enumerate(shapes):
        w, s, b = synth.make_weights(N, K, 4, 64, sb, seed=synth.proj_seed(config, replica, idx))
        x = synth.make_x(1, K, seed=synth.proj_seed(config, replica, idx) + 500)
        tw = torch.from_numpy(w.view(np.int32)).to(dev)
        ts = torch.from_numpy(s.view(np.int16)).view(sbt).to(dev)
        tb = torch.from_numpy(b.view(np.int16)).view(sbt).to(dev)
        tx = torch.from_numpy(x).to(dev)
        ty = torch.empty((1, N), dtype=torch.float16, device=dev)
        calls.append(Call(lib, "mxq_qmv", tx, tw, ts, tb, ty, 1, N, K, 4, 64,
                          0 if sb == "f16" else 1, name))
    return calls


def time_steps(torch, steps_fns, warmup, steps):
    """Run warmup then exactly `steps` steps; returns seconds per step."""
    n = len(steps_fns)
    for i in range(warmup):
        steps_fns[i % n]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        steps_fns[i % n]()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # one eager run on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def cur_stream(torch):
    import ctypes
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def timed_rounds(torch, launches, st, n=20, rounds=3, warm_ms=200.0):
    """{name: ms per call} for a list of (name, launch) pairs: the launches run
    in turn until warm_ms of GPU time has passed (the part settles into its
    sustained clocks under matrix-core load), then `rounds` rounds over all of
    them, n calls back to back per launch and round between one event pair;
    the median round per launch."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    while True:
        for _, f in launches:
            for _ in range(10):
                f(st)
        e1.record()
        torch.cuda.synchronize()
        if e0.elapsed_time(e1) >= warm_ms:
            break
    res = {}
    for _ in range(rounds):
        for name, f in launches:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                f(st)
            b.record()
            torch.cuda.synchronize()
            res.setdefault(name, []).append(a.elapsed_time(b) / n)
    return {k: sorted(v)[len(v) // 2] for k, v in res.items()}


def per_launch_times(torch, sets, reps):
    """Eager launches with an event pair around each; returns {name: [ms, ...]}."""
    out = {}
    pairs = []
    st = cur_stream(torch)
    for r in range(reps):
        for c in sets[r % len(sets)]:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            c(st)
            e1.record()
            pairs.append((c, e0, e1))
    torch.cuda.synchronize()
    for c, e0, e1 in pairs:
        out.setdefault(c.name, []).append(e0.elapsed_time(e1))
    return out


def read_traffic(kernel_desc: str, per_launch_alg_bytes: float):
    """HBM bytes per launch from committed rocprofv3 PMC counters, if current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != kernel_source_sha() or t.get("kernel") != kernel_desc:
        return None
    return t.get("hbm_bytes_per_launch")


COPY_BYTES = 256 << 20


def traffic_pass():
    """Workload for the rocprofv3 --pmc passes: a copy of known size (calibration),
    then the dominant kernel's launches (lm_head qmv, rotating two weight sets)."""
    import torch

    import dequant_matmul_qmv_amd as mxq
    import synth
    lib = mxq.load()
    dev = "cuda:0"
    src = torch.randint(0, 1 << 30, (COPY_BYTES // 4,), dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    sets = [make_qmv_set(mxq, lib, synth, torch, 1, r, [synth.LLAMA_1B_LM_HEAD], dev) for r in range(2)]
    for i in range(6):
        sets[i % 2][0](cur_stream(torch))
    torch.cuda.synchronize()
    N, K = synth.LLAMA_1B_LM_HEAD[1:]
    meta = {"kernel": mxq.mxq_describe("qmv", 1, N, K, 4, 64, "f16"), "source_sha": kernel_source_sha(),
            "alg_bytes_per_launch": call_bytes(1, N, K)}
    print(json.dumps(meta), flush=True)


def qmm_pass():
    """Workload for rocprofv3 --pmc passes over the prefill kernel: the M=512
    gate (8192x2048) and down (2048x8192) projections, 4-bit g64, f16
    scales, five calls each."""
    import numpy as np
    import torch

    import dequant_matmul_qmv_amd as mxq
    import synth
    mxq.load()
    dev = "cuda:0"
    # calibration: a copy of known size, as in the decode kernel's traffic pass
    src = torch.randint(0, 1 << 30, (COPY_BYTES // 4,), dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for N, K in ((8192, 2048), (2048, 8192)):
        p = synth.make_problem(512, N, K, 4, 64, "f16", seed=3)
        x = torch.from_numpy(p.x).to(dev)
        w = torch.from_numpy(p.w.view(np.int32)).to(dev)
        s = torch.from_numpy(p.scales.view(np.int16)).view(torch.float16).to(dev)
        b = torch.from_numpy(p.biases.view(np.int16)).view(torch.float16).to(dev)
        y = torch.empty((512, N), dtype=torch.float16, device=dev)
        for _ in range(5):
            mxq.mxq_qmm(x, w, s, b, y, bits=4)
        torch.cuda.synchronize()
        print(json.dumps({"kernel": mxq.mxq_describe("qmm", 512, N, K), "N": N, "K": K, "calls": 5}), flush=True)


def step_pass(replays=20):
    """Workload for the decode-step kernel trace: the 16-layer step (q,k,v,o,
    gate,up,down per layer, then lm_head) as 65 launches -- {q,k,v}, {o},
    {gate,up}, {down} per layer, lm_head last -- captured in one HIP graph and
    replayed `replays` times."""
    import torch

    import dequant_matmul_qmv_amd as mxq
    import synth
    lib = mxq.load()
    dev = "cuda:0"
    layers = [make_qmv_set(mxq, lib, synth, torch, 3, layer, list(synth.LLAMA_1B_PROJ), dev)
              for layer in range(synth.LLAMA_1B_LAYERS)]
    head = make_qmv_set(mxq, lib, synth, torch, 3, 99, [synth.LLAMA_1B_LM_HEAD], dev)
    launches = []
    for lay in layers:
        by = {c.name: c for c in lay}
        launches += [GroupCall(lib, mxq, [by["q"], by["k"], by["v"]]), by["o"],
                     GroupCall(lib, mxq, [by["gate"], by["up"]]), by["down"]]
    launches += head

    def fn():
        st = cur_stream(torch)
        for c in launches:
            c(st)
    g = capture(torch, fn)
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    print(json.dumps({"launches_per_step": len(launches), "replays": replays}), flush=True)


STEP_KINDS = ("q+k+v", "o", "gate+up", "down")


def summarize_step_trace(trace_csv: str, launches=65, replays=20):
    """Markdown summary of a rocprofv3 kernel trace of --step-pass: the last
    `replays` x `launches` dispatches are the graph replays; per launch kind,
    the mean kernel duration and the mean idle gap from the end of the
    previous kernel to the start of this one (first launch of a replay
    excluded from the gaps)."""
    import csv
    import statistics
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    rows = rows[-launches * replays:]
    kinds = {}
    spans, busy = [], []
    for i in range(replays):
        rep = rows[i * launches:(i + 1) * launches]
        spans.append((rep[-1][1] - rep[0][0]) / 1e3)
        busy.append(sum(e - s for s, e, _ in rep) / 1e3)
        for j, (s, e, name) in enumerate(rep):
            kind = "lm_head" if j == launches - 1 else STEP_KINDS[j % 4]
            d = kinds.setdefault(kind, {"dur": [], "gap": [], "name": name.split("(")[0]})
            d["dur"].append((e - s) / 1e3)
            if j:
                d["gap"].append((s - rep[j - 1][1]) / 1e3)
    out = ["| launch | kernel | per step | mean duration (us) | mean gap before it (us) |", "|---|---|---|---|---|"]
    for kind in STEP_KINDS + ("lm_head",):
        d = kinds[kind]
        out.append(f"| {kind} | `{d['name']}` | {len(d['dur']) // replays} | {statistics.mean(d['dur']):.2f} | "
                   f"{statistics.mean(d['gap']):.2f} |")
    span, b = statistics.median(spans), statistics.median(busy)
    out.append("")
    out.append(f"Step span (first kernel start to last kernel end), median of {replays} replays: {span:.1f} us; "
               f"sum of kernel durations: {b:.1f} us; idle between kernels: {span - b:.1f} us "
               f"({100 * (span - b) / span:.1f} %).")
    print("\n".join(out))


def few_pass():
    """Workload for rocprofv3 passes over the few-row kernels: lm_head
    (128256 x 2048, 4-bit g64, f16 scales) at M = 2, 4, 8 and 16 through
    mxq_qmv (the K-split matrix-core kernel), then M = 16 at K = 2304 (not a
    multiple of 512, so the 16-row-block kernel), five calls each on two
    rotating weight sets, after the copy calibration."""
    import numpy as np
    import torch

    import dequant_matmul_qmv_amd as mxq
    import synth
    mxq.load()
    dev = "cuda:0"
    src = torch.randint(0, 1 << 30, (COPY_BYTES // 4,), dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    N = synth.LLAMA_1B_LM_HEAD[1]
    for K, Ms in ((2048, (2, 4, 8, 16)), (2304, (16,))):
        sets = []
        for r in range(2):
            w, s, b = synth.make_weights(N, K, 4, 64, "f16", seed=900 + r)
            sets.append((torch.from_numpy(w.view(np.int32)).to(dev),
                         torch.from_numpy(s.view(np.int16)).view(torch.float16).to(dev),
                         torch.from_numpy(b.view(np.int16)).view(torch.float16).to(dev)))
        for M in Ms:
            x = torch.from_numpy(synth.make_x(M, K, seed=910 + M)).to(dev)
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            for i in range(5):
                w, s, b = sets[i % 2]
                mxq.mxq_qmv(x, w, s, b, y, bits=4)
            torch.cuda.synchronize()
            print(json.dumps({"kernel": mxq.mxq_describe("qmv", M, N, K), "M": M, "N": N, "K": K,
                              "alg_bytes": call_bytes(M, N, K), "calls": 5}), flush=True)
        del sets


def write_traffic(fetch_csv: str, write_csv: str, meta_json: str):
    """Turn two rocprofv3 counter CSVs into profiles/qmv_traffic.json.

    FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch; each is scaled by the
    factor that makes the calibration copy (COPY_BYTES read, COPY_BYTES written)
    come out exact."""
    import csv
    import statistics
    meta = json.loads(open(meta_json).read().strip().splitlines()[-1])

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    def calib(vals):
        # the copy kernel's large dispatches (the COPY_BYTES calibration copies)
        big = [x for k, v in vals.items() if "copy" in k.lower() for x in v if x * 1024 > COPY_BYTES / 8]
        return "copy", COPY_BYTES / (statistics.median(big) * 1024)

    fv, wv = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    qmv_name = next(k for k in fv if "qmv_kernel" in k)
    _, ff = calib(fv)
    _, fw = calib(wv)
    fetch = statistics.median(fv[qmv_name]) * 1024 * ff
    write = statistics.median(wv[qmv_name]) * 1024 * fw
    out = dict(meta, kernel_symbol=qmv_name.split("(")[0], fetch_bytes_per_launch=round(fetch),
               write_bytes_per_launch=round(write), hbm_bytes_per_launch=round(fetch + write),
               fetch_scale=round(ff, 4), write_scale=round(fw, 4),
               calibration_bytes=COPY_BYTES, launches=len(fv[qmv_name]))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


POOL_BYTES = 1536 << 20  # rotation pool of the read probe: > the 256 MiB Infinity Cache


def probe_curve(torch, lib, sizes, reps=40):
    """Our own read kernel (mxq_read_probe, the decode kernel's load form) at
    each size in bytes, reading from offsets that rotate through a 1.5 GiB pool
    so the data comes from HBM: {size: {"GB/s": back-to-back, "bracketed_GB/s":
    an event pair per launch, "us": ...}}."""
    import ctypes
    pool = torch.empty(POOL_BYTES, dtype=torch.uint8, device="cuda:0")
    pool.fill_(1)
    out = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    st = cur_stream(torch)
    base = pool.data_ptr()
    res = {}
    for size in sizes:
        size16 = (int(size) + 15) // 16 * 16
        step = (size16 + 4095) // 4096 * 4096
        nslots = max(1, (POOL_BYTES - size16) // step)

        def launch(r):
            off = (r % nslots) * step
            stt = lib.mxq_read_probe(ctypes.c_void_p(base + off), size16, ctypes.c_void_p(out.data_ptr()), st)
            if stt != 0:
                raise RuntimeError(f"read probe: libmxq status {stt}")
        for r in range(8):
            launch(r)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            launch(r)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        pairs = []
        for r in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            launch(r + reps)
            b.record()
            pairs.append((a, b))
        torch.cuda.synchronize()
        import statistics
        bms = statistics.median(a.elapsed_time(b) for a, b in pairs)
        res[int(size)] = {"us": round(ms * 1e3, 2), "GB/s": round(size16 / (ms / 1e3) / 1e9, 1),
                          "bracketed_us": round(bms * 1e3, 2),
                          "bracketed_GB/s": round(size16 / (bms / 1e3) / 1e9, 1)}
    del pool, out
    torch.cuda.empty_cache()
    return res


def rotating_launch_time(torch, make_launch, nrep, reps=30):
    """Back-to-back time (ms) per launch of make_launch(i) over i = 0, 1, ...
    (the callable picks replica i % nrep), and the median with an event pair
    around each launch."""
    import statistics
    for i in range(min(nrep, 6)):
        make_launch(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        make_launch(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    pairs = []
    for i in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        make_launch(i + reps)
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    return ms, statistics.median(a.elapsed_time(b) for a, b in pairs)


def config_legs(torch, lib, synth, dev):
    """The small single problem (M=1, N=512, K=2048, 4-bit g64, f16, seed 0)
    and the 48-case edge sweep (M in {1,2,4,8}, K=8192, N in {2048,1023,2050},
    4/8-bit, f16/bf16 scales) through mxq_qmv and mxq_qmm: GB/s per launch,
    weights replicated on the device (identical copies at distinct addresses)
    so that each leg streams at least 512 MB and the data comes from HBM."""
    import numpy as np

    def dev_problem(p, reps_min_bytes=512 << 20):
        sbt = torch.float16 if p.sb_dtype == "f16" else torch.bfloat16
        w = torch.from_numpy(p.w.view(np.int32)).to(dev)
        s = torch.from_numpy(p.scales.view(np.int16)).view(sbt).to(dev)
        b = torch.from_numpy(p.biases.view(np.int16)).view(sbt).to(dev)
        x = torch.from_numpy(p.x).to(dev)
        y = torch.empty((p.M, p.N), dtype=torch.float16, device=dev)
        per = w.numel() * 4 + s.numel() * 4
        nrep = max(2, -(-reps_min_bytes // per))
        reps = [(w, s, b)] + [(w.clone(), s.clone(), b.clone()) for _ in range(nrep - 1)]
        return x, y, reps

    def leg(fn_name, p, x, y, reps):
        fn = getattr(lib, fn_name)
        sb = 0 if p.sb_dtype == "f16" else 1
        st = cur_stream(torch)

        def launch(i):
            w, s, b = reps[i % len(reps)]
            r = fn(x.data_ptr(), w.data_ptr(), s.data_ptr(), b.data_ptr(), y.data_ptr(), p.M, p.N, p.K, p.bits,
                   p.group_size, sb, st)
            if r != 0:
                raise RuntimeError(f"{fn_name} M={p.M} N={p.N}: libmxq status {r}")
        ms, bms = rotating_launch_time(torch, launch, len(reps))
        nb = call_bytes(p.M, p.N, p.K, p.bits, p.group_size)
        return {"us": round(ms * 1e3, 2), "GB/s": round(nb / (ms / 1e3) / 1e9, 1),
                "bracketed_GB/s": round(nb / (bms / 1e3) / 1e9, 1)}

    out = {}
    p = synth.small_qmv_problem()
    x, y, reps = dev_problem(p)
    out["small_qmv_M1_N512_K2048"] = dict(leg("mxq_qmv", p, x, y, reps), bytes=call_bytes(1, 512, 2048),
                                          note="latency-bound: 0.59 MB moves in 74 ns at 8 TB/s")
    del reps
    sweep = {}
    for case in synth.edge_cases():
        p = synth.make_problem(**case)
        x, y, reps = dev_problem(p, 256 << 20)
        key = f"M{p.M}_N{p.N}_b{p.bits}_{p.sb_dtype}"
        sweep[key] = {"qmv": leg("mxq_qmv", p, x, y, reps)["GB/s"], "qmm": leg("mxq_qmm", p, x, y, reps)["GB/s"]}
        del reps
    torch.cuda.empty_cache()
    vals = [v[e] for v in sweep.values() for e in ("qmv", "qmm")]
    out["edge_sweep_K8192"] = {"GB/s": sweep, "median_GB/s": round(float(np.median(vals)), 1),
                               "min_GB/s": min(vals), "max_GB/s": max(vals),
                               "timing": "30 launches back to back per entry, replicated weights (>= 256 MB)"}
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(synth, reps=5):
    """The f64 oracle on a bounded sample, timed on the host's cores.

    Sample: all seven layer-0 projections + lm_head rows 0..16383 (M=1,
    4-bit g64, f16 scales; ~53 MB, 10-20 s for both legs).  Two legs: all available cores (numpy's BLAS with its default
    thread count; unpack and dequant are single-threaded numpy) and one core
    (affinity pinned to one CPU, one BLAS thread).  Each leg times the whole
    oracle (oracle.matmul_ref: unpack, dequant, matmul) and its two phases
    apart (oracle.dequant_f64; the f64 product of oracle.widen_act(x) with the
    dequantized weights, as matmul_ref computes it) over the sample, median
    of `reps` passes after one warm-up.  value = algorithmic bytes of the
    sample / the whole oracle's time, all cores."""
    import statistics
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    shapes = list(synth.LLAMA_1B_PROJ) + [("lm_head[0:16384]", 16384, 2048)]
    probs = []
    for idx, (name, N, K) in enumerate(shapes):
        w, s, b = synth.make_weights(N, K, 4, 64, "f16", seed=synth.proj_seed(1, 0, idx))
        x = synth.make_x(1, K, seed=synth.proj_seed(1, 0, idx) + 500)
        probs.append((x, w, s, b, N, K))
    sample_bytes = sum(call_bytes(1, N, K) for *_, N, K in probs)

    def one_pass(fn):
        t0 = time.perf_counter()
        for x, w, s, b, N, K in probs:
            fn(x, w, s, b, K)
        return time.perf_counter() - t0

    wdq = [oracle.dequant_f64(w, s, b, K, 4, 64, "f16") for x, w, s, b, N, K in probs]

    def mm_pass():
        t0 = time.perf_counter()
        for (x, *_), w in zip(probs, wdq):
            oracle.widen_act(x) @ w.T
        return time.perf_counter() - t0

    def leg(blas_threads):
        whole = lambda x, w, s, b, K: oracle.matmul_ref(x, w, s, b, K, 4, 64, "f16")  # noqa: E731
        dq = lambda x, w, s, b, K: oracle.dequant_f64(w, s, b, K, 4, 64, "f16")  # noqa: E731
        ctx = threadpool_limits(limits=blas_threads) if threadpool_limits else None
        if ctx:
            ctx.__enter__()
        try:
            one_pass(whole)
            t_whole = statistics.median(one_pass(whole) for _ in range(reps))
            t_dq = statistics.median(one_pass(dq) for _ in range(reps))
            mm_pass()
            t_mm = statistics.median(mm_pass() for _ in range(reps))
        finally:
            if ctx:
                ctx.__exit__(None, None, None)
        return {"GB/s": round(sample_bytes / t_whole / 1e9, 4), "ms_per_pass": round(t_whole * 1e3, 1),
                "unpack_dequant_ms": round(t_dq * 1e3, 1), "matmul_ms": round(t_mm * 1e3, 2)}

    cpus = sorted(os.sched_getaffinity(0))
    blas = None
    if threadpool_info:
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in threadpool_info()]
    t0 = time.perf_counter()
    all_cores = leg(None)
    os.sched_setaffinity(0, {cpus[0]})
    try:
        one_core = leg(1)
    finally:
        os.sched_setaffinity(0, set(cpus))
    el = time.perf_counter() - t0
    blas_threads = max((b["threads"] or 1 for b in blas), default=1) if blas else None
    return {"value": all_cores["GB/s"], "unit": "GB/s", "cores": blas_threads or len(cpus), "kind": "oracle",
            "sample": f"layer-0 q,k,v,o,gate,up,down + lm_head rows 0..16383 (M=1, 4-bit g64, f16 scales; "
                      f"{sample_bytes} algorithmic bytes per pass), f64 numpy oracle, median of {reps} passes "
                      f"after one warm-up per leg, {el:.1f} s in all",
            "host": {"cpu_model": _cpu_model(), "cpus_available": len(cpus), "blas": blas},
            "all_cores": dict(all_cores, blas_threads=blas_threads),
            "one_core": dict(one_core, blas_threads=1, pinned_cpu=cpus[0])}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--replicas", type=int, default=6)
    ap.add_argument("--mode", choices=["graph", "eager"], default="eager",
                    help="launch the timed steps eagerly (pre-marshalled C-ABI calls) or by "
                         "HIP-graph replay")
    ap.add_argument("--launch-plan", choices=["layer", "separate", "single"], default="layer",
                    help="layer: {q,k,v},{o},{gate,up},{down},{lm_head} (grouped where a decoder "
                         "layer shares the activation); separate: one launch per projection; "
                         "single: one grouped launch for all eight")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip decode_step, qmm and dequant legs")
    ap.add_argument("--traffic-pass", action="store_true",
                    help="only run the workload of the rocprofv3 --pmc traffic passes")
    ap.add_argument("--qmm-pass", action="store_true",
                    help="only run the M=512 prefill workload of the rocprofv3 --pmc counter passes")
    ap.add_argument("--write-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "META_JSON"),
                    help="write profiles/qmv_traffic.json from two rocprofv3 counter CSVs")
    ap.add_argument("--step-pass", action="store_true",
                    help="only run the graph-replayed 16-layer decode step (kernel-trace workload)")
    ap.add_argument("--step-trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="summarize a rocprofv3 kernel trace of --step-pass (durations and gaps)")
    ap.add_argument("--few-pass", action="store_true",
                    help="only run the few-row workload of the rocprofv3 counter passes")
    args = ap.parse_args()
    if args.step_trace_summary:
        summarize_step_trace(args.step_trace_summary)
        return
    if args.step_pass:
        step_pass()
        return
    if args.few_pass:
        few_pass()
        return
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.traffic_pass:
        traffic_pass()
        return
    if args.qmm_pass:
        qmm_pass()
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the fused quantized matmul has no multi-GPU path in this "
              "library (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import dequant_matmul_qmv_amd as mxq
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lib = mxq.load(build_if_missing=True)
    dev = "cuda:0"
    torch.cuda.set_device(0)

    # ---------------- headline: the projection set at M=1 ------------------
    shapes = list(synth.LLAMA_1B_PROJ) + [synth.LLAMA_1B_LM_HEAD]
    log(f"generating {args.replicas} replicas of the decode projection set ...")
    sets = [make_qmv_set(mxq, lib, synth, torch, 1, r, shapes, dev) for r in range(args.replicas)]
    bytes_per_step = sum(c.bytes for c in sets[0])

    def plan_launches(calls, plan):
        """The launches of one step.  `layer`: projections that read the same
        activation in a decoder layer share one grouped launch -- {q,k,v}, {o},
        {gate,up}, {down}, {lm_head}; `separate`: one mxq_qmv per projection;
        `single`: all eight projections in one grouped launch."""
        by = {c.name: c for c in calls}
        if plan == "separate":
            return list(calls)
        if plan == "single":
            return [GroupCall(lib, mxq, calls)]
        return [GroupCall(lib, mxq, [by["q"], by["k"], by["v"]]), by["o"],
                GroupCall(lib, mxq, [by["gate"], by["up"]]), by["down"], by["lm_head"]]

    st_head = cur_stream(torch)

    def step_fn(launches, st=None):
        # eager steps take the stream handle once; captured steps look it up
        # at call time (under capture it is the capturing stream)
        if st is not None:
            return lambda: [c(st) for c in launches]
        return lambda: [c(cur_stream(torch)) for c in launches]

    plans = {p: [plan_launches(s, p) for s in sets] for p in ("layer", "separate", "single")}
    fns = {p: [step_fn(l, st_head) for l in plans[p]] for p in plans}
    head_plan = args.launch_plan
    graphs = [capture(torch, step_fn(l)) for l in plans[head_plan]]
    step_fns = [g.replay for g in graphs] if args.mode == "graph" else fns[head_plan]
    log("timing headline steps ...")
    # Settle: the part runs the step for SETTLE_MS before the warm-up steps, so
    # the timed steps see its sustained clocks rather than the ramp out of
    # idle (a short timed region otherwise lands inside that ramp).
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < SETTLE_MS / 1e3:
        step_fns[i % len(step_fns)]()
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    torch.cuda.synchronize()
    sec = time_steps(torch, step_fns, args.warmup, args.steps)
    value = bytes_per_step / sec / 1e9
    other = {}
    for p in plans:
        if p != head_plan:
            other[p] = time_steps(torch, fns[p], args.warmup, args.steps)
    graph_sec = time_steps(torch, [g.replay for g in graphs], 10, min(args.steps, 200)) \
        if args.mode != "graph" else time_steps(torch, fns[head_plan], 10, min(args.steps, 200))

    # ---------------- roofline of the dominant kernel -----------------------
    # per-launch HIP events around the headline plan's launches; a launch is
    # attributed to the kernel instantiation of its largest problem
    head_launches = plans[head_plan]
    pairs = []
    st = cur_stream(torch)
    for r in range(max(2 * args.replicas, 24)):
        for li, c in enumerate(head_launches[r % len(head_launches)]):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            c(st)
            e1.record()
            pairs.append((li, e0, e1))
    torch.cuda.synchronize()
    launch_ms = {}
    for li, e0, e1 in pairs:
        launch_ms.setdefault(li, []).append(e0.elapsed_time(e1))
    by_kernel = {}
    per_launch = {}
    desc_of = {}
    for li, c in enumerate(head_launches[0]):
        probs = c.calls if isinstance(c, GroupCall) else [c]
        big = max(probs, key=lambda q: q.N)
        desc = mxq.mxq_describe("qmv", 1, big.N, big.K, 4, 64, "f16")
        desc_of[li] = desc
        ms = float(np.median(launch_ms[li]))
        d = by_kernel.setdefault(desc, {"bytes": 0, "ms": 0.0, "launches": 0, "names": []})
        d["bytes"] += c.bytes
        d["ms"] += ms
        d["launches"] += 1
        name = "+".join(q.name for q in probs)
        d["names"].append(name)
        per_launch[name] = {"us": round(ms * 1e3, 2), "GB/s": round(c.bytes / (ms / 1e3) / 1e9, 1),
                            "bytes": c.bytes}
    dom_desc, dom = max(by_kernel.items(), key=lambda kv: kv[1]["ms"])
    bracketed_ms = dom["ms"] / dom["launches"]
    avg_bytes = dom["bytes"] / dom["launches"]
    # The dominant kernel's average launch duration: its launches back to back
    # on the launch stream, rotating through the replicas (so the weights come
    # from HBM), between one event pair -- the kernel's duration in a stream of
    # launches, without the ~1.5 us that an event pair around every launch adds.
    dom_lis = [li for li, d in desc_of.items() if d == dom_desc]
    reps = max(4 * args.replicas, 24)
    for r in range(len(head_launches)):
        for li in dom_lis:
            head_launches[r][li](st)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(reps):
        for li in dom_lis:
            head_launches[r % len(head_launches)][li](st)
    e1.record()
    torch.cuda.synchronize()
    avg_ms = e0.elapsed_time(e1) / (reps * len(dom_lis))
    achieved = avg_bytes / (avg_ms / 1e3) / 1e9
    traffic = read_traffic(dom_desc, avg_bytes)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom_desc, "launches_per_step": dom["launches"], "projections": dom["names"],
                "avg_launch_us": round(avg_ms * 1e3, 3), "timing": f"{reps * len(dom_lis)} launches back to back",
                "bracketed_launch_us": round(bracketed_ms * 1e3, 3), "alg_bytes_per_launch": int(avg_bytes)}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_ms": SETTLE_MS, "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "Llama-3.2-1B-shaped decode projections q,k,v,o,gate,up,down,lm_head "
                               "(N x K: 2048x2048, 512x2048, 512x2048, 2048x2048, 8192x2048, 8192x2048, "
                               "2048x8192, 128256x2048), M=1, 4-bit codes g64, f16 scales/biases, "
                               "f16 x ~ N(0,1)",
                   "replicas": args.replicas, "launch_plan": head_plan,
                   "launches_per_step": len(plans[head_plan][0]),
                   "bytes_per_step": bytes_per_step, "launch_mode": args.mode},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "other_launch_plans_GB/s": {p: round(bytes_per_step / t / 1e9, 1) for p, t in other.items()},
        ("graph_GB/s" if args.mode != "graph" else "eager_GB/s"): round(bytes_per_step / graph_sec / 1e9, 1),
        "per_launch": per_launch,
        "roofline": roofline,
    }
    del sets, plans, fns, step_fns, graphs, head_launches
    torch.cuda.empty_cache()

    # ---------------- our own read kernel at the same sizes -----------------
    # (a fused launch is judged against what a plain read of the same bytes
    # attains: small reads cannot reach the HBM peak however they are done)
    log("read probe ...")
    launch_sizes = {name: int(v["bytes"]) for name, v in per_launch.items()}
    curve_sizes = sorted(set(launch_sizes.values()) | {1 << 20, 4 << 20, 16 << 20, 64 << 20, 512 << 20})
    curve = probe_curve(torch, lib, curve_sizes)
    for name, v in per_launch.items():
        pr = curve[launch_sizes[name]]
        v["probe_bracketed_GB/s"] = pr["bracketed_GB/s"]
        v["frac_of_probe"] = round(v["GB/s"] / pr["bracketed_GB/s"], 3)
    dom_probe = curve[int(avg_bytes)] if int(avg_bytes) in curve else None
    if dom_probe:
        roofline["probe_GB/s_same_size"] = dom_probe["GB/s"]
        roofline["frac_of_probe"] = round(achieved / dom_probe["GB/s"], 3)
    result["read_probe"] = {"kernel": "mxq_read_probe (16-byte non-temporal loads, 2 workgroups of 256 per CU)",
                            "timing": "40 launches back to back (GB/s) and an event pair per launch "
                                      "(bracketed), offsets rotating through a 1.5 GiB pool",
                            "curve": {str(k): v for k, v in curve.items()}}

    # ---------------- extras ------------------------------------------------
    if not args.no_extras:
        log("small problem and edge sweep ...")
        result["configs"] = config_legs(torch, lib, synth, dev)

        log("decode step (16 layers + lm_head) ...")
        layers = []
        for layer in range(synth.LLAMA_1B_LAYERS):
            layers.append(make_qmv_set(mxq, lib, synth, torch, 3, layer, list(synth.LLAMA_1B_PROJ), dev))
        head = make_qmv_set(mxq, lib, synth, torch, 3, 99, [synth.LLAMA_1B_LM_HEAD], dev)
        flat = [c for lay in layers for c in lay] + head
        dbytes = sum(c.bytes for c in flat)
        grouped = []
        for lay in layers:
            by = {c.name: c for c in lay}
            grouped += [GroupCall(lib, mxq, [by["q"], by["k"], by["v"]]), by["o"],
                        GroupCall(lib, mxq, [by["gate"], by["up"]]), by["down"]]
        grouped += head
        entry = {"bytes_per_step": dbytes,
                 "weight_bytes_per_step": sum(c.N * c.K // 2 + c.N * (c.K // 64) * 4 for c in flat)}
        for label, launches in (("separate", flat), ("layer", grouped)):
            g = capture(torch, step_fn(launches))
            gsec = time_steps(torch, [g.replay], 5, 50)
            esec = time_steps(torch, [step_fn(launches, st_head)], 3, 20)
            entry[label] = {"launches": len(launches),
                            "graph_us_per_step": round(gsec * 1e6, 1), "graph_GB/s": round(dbytes / gsec / 1e9, 1),
                            "graph_steps_per_s": round(1 / gsec, 1),
                            "eager_us_per_step": round(esec * 1e6, 1), "eager_GB/s": round(dbytes / esec / 1e9, 1)}
            del g
        result["decode_step"] = entry
        del layers, head, flat, grouped
        torch.cuda.empty_cache()

        log("qmm M=512 ...")
        qmm = {}
        for sb in ("f16", "bf16"):
            sbt = torch.float16 if sb == "f16" else torch.bfloat16
            calls = []
            for idx, (name, N, K) in enumerate([("gate", 8192, 2048), ("up", 8192, 2048), ("down", 2048, 8192)]):
                w, s, b = synth.make_weights(N, K, 4, 64, sb, seed=synth.proj_seed(4, 0, idx))
                x = synth.make_x(512, K, seed=synth.proj_seed(4, 0, idx) + 500)
                calls.append(Call(lib, "mxq_qmm", torch.from_numpy(x).to(dev),
                                  torch.from_numpy(w.view(np.int32)).to(dev),
                                  torch.from_numpy(s.view(np.int16)).view(sbt).to(dev),
                                  torch.from_numpy(b.view(np.int16)).view(sbt).to(dev),
                                  torch.empty((512, N), dtype=torch.float16, device=dev),
                                  512, N, K, 4, 64, 0 if sb == "f16" else 1, name))
            # back-to-back calls per projection (a prefill runs them in a row):
            # after a 200 ms warm-up, the median of three rounds of 20 calls
            st = cur_stream(torch)
            entry = {}
            tot_flop, tot_ms = 0, 0.0
            times = timed_rounds(torch, [(c.name, c) for c in calls], st)
            for c in calls:
                ms = times[c.name]
                flop = 2 * c.M * c.N * c.K
                entry[c.name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(flop / (ms / 1e3) / 1e12, 1)}
                tot_flop += flop
                tot_ms += ms
            tf = tot_flop / (tot_ms / 1e3) / 1e12
            entry["TFLOP/s"] = round(tf, 1)
            entry["mfma_util"] = round(tf / MFMA_F16_PEAK_TFLOPS, 4)
            entry["kernel"] = mxq.mxq_describe("qmm", 512, 8192, 2048, 4, 64, sb)
            qmm[sb] = entry
            if sb == "f16":
                # the same projections with int8 activations (mxq_linear_a8):
                # rows quantized once, then the integer matrix cores
                a8 = {}
                a8_op, a8_ms = 0, 0.0
                acs = [A8Call(lib, *c.tensors, c.M, c.N, c.K, c.name) for c in calls]
                times = timed_rounds(torch, [(ac.name, ac) for ac in acs], st)
                for c in calls:
                    ms = times[c.name]
                    op = 2 * c.M * c.N * c.K
                    a8[c.name] = {"us": round(ms * 1e3, 2), "TOP/s": round(op / (ms / 1e3) / 1e12, 1)}
                    a8_op += op
                    a8_ms += ms
                a8["TOP/s"] = round(a8_op / (a8_ms / 1e3) / 1e12, 1)
                a8["frac_of_int8_peak"] = round(a8_op / (a8_ms / 1e3) / 1e12 / MFMA_I8_PEAK_TOPS, 4)
                a8["kernel"] = mxq.mxq_describe("a8", 512, 8192, 2048, 4, 64, sb)
                a8["timing"] = ("after a 200 ms warm-up, the median of three rounds of 20 calls back to back per "
                                "projection, quantization of x included")
                qmm["int8_activations"] = a8
        result["qmm"] = qmm

        # bf16 activations (x and y bf16) through mxq_linear_act: the lm_head
        # decode launch (two weight sets alternating, 296 MB > the 256 MB
        # Infinity Cache) and the M=512 prefill projections, f16 scales.
        log("bf16 activations ...")
        act = {}
        lm_sets = []
        for r in range(2):
            w, s, b = synth.make_weights(128256, 2048, 4, 64, "f16", seed=synth.proj_seed(1, r, 7))
            xb = synth.make_x(1, 2048, seed=synth.proj_seed(1, r, 7) + 500, act_dtype="bf16")
            lm_sets.append(ActCall(lib, torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev),
                                   torch.from_numpy(w.view(np.int32)).to(dev),
                                   torch.from_numpy(s.view(np.int16)).view(torch.float16).to(dev),
                                   torch.from_numpy(b.view(np.int16)).view(torch.float16).to(dev),
                                   torch.empty((1, 128256), dtype=torch.bfloat16, device=dev),
                                   1, 128256, 2048, "lm_head"))
        st = cur_stream(torch)
        for i in range(6):
            lm_sets[i % 2](st)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(20):
            lm_sets[i % 2](st)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        act["lm_head_decode"] = {"us": round(ms * 1e3, 2),
                                 "GB/s": round(call_bytes(1, 128256, 2048) / (ms / 1e3) / 1e9, 1)}
        del lm_sets
        torch.cuda.empty_cache()
        tot_flop, tot_ms = 0, 0.0
        prefill = {}
        acalls = []
        for idx, (name, N, K) in enumerate([("gate", 8192, 2048), ("up", 8192, 2048), ("down", 2048, 8192)]):
            w, s, b = synth.make_weights(N, K, 4, 64, "f16", seed=synth.proj_seed(4, 0, idx))
            xb = synth.make_x(512, K, seed=synth.proj_seed(4, 0, idx) + 500, act_dtype="bf16")
            acalls.append(ActCall(lib, torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev),
                                  torch.from_numpy(w.view(np.int32)).to(dev),
                                  torch.from_numpy(s.view(np.int16)).view(torch.float16).to(dev),
                                  torch.from_numpy(b.view(np.int16)).view(torch.float16).to(dev),
                                  torch.empty((512, N), dtype=torch.bfloat16, device=dev), 512, N, K, name))
        times = timed_rounds(torch, [(c.name, c) for c in acalls], st)
        for c in acalls:
            name, N, K = c.name, c.N, c.K
            ms = times[name]
            flop = 2 * 512 * N * K
            prefill[name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(flop / (ms / 1e3) / 1e12, 1)}
            tot_flop += flop
            tot_ms += ms
        prefill["TFLOP/s"] = round(tot_flop / (tot_ms / 1e3) / 1e12, 1)
        act["qmm_m512"] = prefill
        result["bf16_activations"] = act

        # few activation rows on the lm_head shape: the f16 route mxq_qmv takes
        # (decode kernel at M = 1, the K-split matrix-core kernel from M = 2)
        # against the int8-activation route (mxq_linear_a8), three weight sets
        # (444 MB, more than the Infinity Cache holds) rotating
        log("few rows (f16 and int8 activations) ...")
        few = {}
        wsets = []
        for r in range(3):
            w, s, b = synth.make_weights(128256, 2048, 4, 64, "f16", seed=synth.proj_seed(1, r, 7))
            wsets.append((torch.from_numpy(w.view(np.int32)).to(dev),
                          torch.from_numpy(s.view(np.int16)).view(torch.float16).to(dev),
                          torch.from_numpy(b.view(np.int16)).view(torch.float16).to(dev)))
        sfew = cur_stream(torch)
        wptrs = [(tw.data_ptr(), ts.data_ptr(), tb.data_ptr()) for tw, ts, tb in wsets]
        cases = []
        for M in (1, 2, 4, 8, 16):
            x8 = torch.from_numpy(synth.make_x(M, 2048, seed=91 + M)).to(dev)
            y8 = torch.empty((M, 128256), dtype=torch.float16, device=dev)
            for label, fn in (("f16", lib.mxq_qmv), ("int8", lib.mxq_linear_a8)):
                cases.append((M, label, fn, x8, y8))

        def few_launch(case, i):
            # pointers and stream taken once: the launches are issued faster than
            # the ~25-35 us kernels run, so the events time the GPU
            M, label, fn, x8, y8 = case
            pw, ps, pb = wptrs[i % 3]
            if label == "f16":
                st_ = fn(x8.data_ptr(), pw, ps, pb, y8.data_ptr(), M, 128256, 2048, 4, 64, 0, sfew)
            else:
                st_ = fn(x8.data_ptr(), pw, ps, pb, None, y8.data_ptr(), M, 128256, 2048, 4, 64, 0, sfew)
            if st_ != 0:
                raise RuntimeError(f"{label} lm_head M={M}: libmxq status {st_}")

        # a 200 ms warm-up, then five rounds over all cases (so that a slow
        # spell of the part does not land on one case), 20 launches back to
        # back per case and round; the median of the five rounds
        few_ms = {}

        def few_rec(case):
            def f(st_):
                few_launch(case, f.i)
                f.i += 1
            f.i = 0
            return f
        launches = [(case[:2], few_rec(case)) for case in cases]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        while True:
            for _, f in launches:
                for _ in range(10):
                    f(sfew)
            e1.record()
            torch.cuda.synchronize()
            if e0.elapsed_time(e1) >= 200.0:
                break
        for rnd in range(5):
            for key, f in launches:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(20):
                    f(sfew)
                b.record()
                torch.cuda.synchronize()
                few_ms.setdefault(key, []).append(a.elapsed_time(b) / 20)
        for M in (1, 2, 4, 8, 16):
            row = {}
            for label in ("f16", "int8"):
                ms = sorted(few_ms[(M, label)])[2]  # median of five rounds
                row[label] = {"us": round(ms * 1e3, 2),
                              "GB/s": round(call_bytes(M, 128256, 2048) / (ms / 1e3) / 1e9, 1),
                              "rounds_us": [round(v * 1e3, 2) for v in few_ms[(M, label)]]}
            row["f16"]["kernel"] = mxq.mxq_describe("qmv", M, 128256, 2048)
            few[f"lm_head_M{M}"] = row
        del cases
        del wsets
        torch.cuda.empty_cache()
        result["few_rows"] = few

        log("dequant ...")
        w, s, b = synth.make_weights(128256, 2048, 4, 64, "f16", seed=7)
        tw = torch.from_numpy(w.view(np.int32)).to(dev)
        ts = torch.from_numpy(s.view(np.int16)).view(torch.float16).to(dev)
        tb = torch.from_numpy(b.view(np.int16)).view(torch.float16).to(dev)
        out = torch.empty((128256, 2048), dtype=torch.float32, device=dev)
        for _ in range(3):
            mxq.mxq_dequant(tw, ts, tb, out, bits=4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            mxq.mxq_dequant(tw, ts, tb, out, bits=4)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        dq_bytes = 128256 * 2048 // 2 + 128256 * 32 * 4 + 128256 * 2048 * 4
        result["dequant"] = {"shape": "128256x2048 4-bit -> f32", "us": round(ms * 1e3, 1),
                             "GB/s": round(dq_bytes / (ms / 1e3) / 1e9, 1)}
        del out, tw
        torch.cuda.empty_cache()

        # Dense f16 comparator (context, not the product): the same shapes with
        # plain f16 weights through PyTorch's GEMM (hipBLASLt).  The pages'
        # acceptance for the packed path is that it beats f16-resident weights.
        log("dense f16 comparator ...")
        gen = torch.Generator(device=dev).manual_seed(11)
        dense = []
        for name, N, K in shapes:
            wd = (torch.randn((N, K), device=dev, generator=gen) * 0.02).half()
            xd = torch.randn((1, K), device=dev, generator=gen).half()
            dense.append((name, xd, wd))
        dfn = lambda: [torch.nn.functional.linear(xd, wd) for _, xd, wd in dense]  # noqa: E731
        fsec = time_steps(torch, [dfn], 20, 200)
        f16_bytes = sum(wd.numel() * 2 + xd.numel() * 2 + wd.shape[0] * 2 for _, xd, wd in dense)
        packed_sec = bytes_per_step / (value * 1e9)
        cmp = {"decode_step_us": round(fsec * 1e6, 2), "weight_bytes_per_step": f16_bytes,
               "GB/s": round(f16_bytes / fsec / 1e9, 1),
               "packed_speedup_vs_f16": round(fsec / packed_sec, 3)}
        del dense
        prefill = {}
        # timed like the packed prefill legs: a 200 ms warm-up, then the
        # median of three rounds of 20 calls per projection
        dshapes = (("gate", 8192, 2048), ("down", 2048, 8192))
        dts = {name: ((torch.randn((N, K), device=dev, generator=gen) * 0.02).half(),
                      torch.randn((512, K), device=dev, generator=gen).half()) for name, N, K in dshapes}
        times = timed_rounds(torch, [(name, (lambda st_, w_=wd, x_=xd: torch.nn.functional.linear(x_, w_)))
                                     for name, (wd, xd) in dts.items()], cur_stream(torch))
        for name, N, K in dshapes:
            ms = times[name]
            prefill[name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(2 * 512 * N * K / (ms / 1e3) / 1e12, 1)}
        del dts
        cmp["prefill_m512"] = prefill
        result["dense_f16_comparator"] = cmp
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(synth)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
