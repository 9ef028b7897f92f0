#!/usr/bin/env python3
"""Throughput of the MiTA forward pass on one MI355X, with its roofline.

    python bench.py [--steps K] [--warmup W] [--workload deit-s] [--also hires-3136]
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR WORKLOAD   (counter summary)

A step is one full ``mita_forward`` (pooling, landmark scores + top-k +
landmark values, routing + grouping, grouped expert attention) over one batch
of synthetic, seeded inputs already resident in device memory.  Before every
timed step a 512 MiB buffer is read (summed) so that neither L2 nor the 256 MB
Infinity Cache holds the inputs (the DeiT-S inputs would otherwise fit in
it); a read leaves clean lines, so the first kernel does not share HBM with
the write-back of a flush buffer.  A step is timed by HIP events on the
caller's stream right before and after the call (the staged schedule runs
routing and grouping on a side stream, which the binding owns and passes in,
beside the landmark pass, and joins it back before attention); ms_per_step is
the mean step time (median and p10/p90 beside it).  A second cold series runs
with the library's per-kernel events (mita_forward_ex records one before its
first kernel and one after each): a kernel's time is the interval from its
start event to its end (stage_us), and that series' mean step time is
instrumented_ms_per_step.  Where a schedule forks onto the side stream, the
same cold steps are also timed with every kernel on one stream (one_stream_*).
A warm (no flush) figure is reported beside it unless --no-warm.  Defaults:
100 timed steps after 20 warm-up steps.

Prints ONE JSON line.  ``value`` is query-heads per second (B*H*N per step)
on the headline workload (DeiT-S shape); the 3136-token workload is reported
in ``secondary`` (with its own oracle baseline), and ``extras`` holds a
shorter record (20 cold steps) for every other workload and for the variants
(two experts per query; route-only with the plain pass's entry count).  ``roofline`` covers the kernel that dominates the step;
``kernel_gbs`` gives every kernel's algorithmic bytes per second and
``kernel_mfma`` the contraction kernels' algorithmic matrix flops per second
against the dense bf16 MFMA peak (2.5 PFLOP/s);
``cpu_baseline`` is the fp64 oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MiTA fwd query-heads/sec (DeiT-S, 3136-tok); fraction of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16
FLUSH_BYTES = 512 << 20


# measured HBM traffic per launch, written by --summarize-pmc from two rocprofv3
# counter runs (FETCH_SIZE, WRITE_SIZE) of this script, scaled by a plain copy
# kernel's readings; an entry is used only while its kernel's sources still
# hash to the value recorded with it
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
CSRC = os.path.join(ROOT, "efficient_attention_avg_amd", "csrc")
SHARED_SOURCES = ["common.h", "mfma.h", "select.h", "internal.h"]
KERNEL_SOURCES = {
    "bf16": {"fused": "fused.hip", "pool": "pool_bf16.hip", "landmark": "landmark_bf16.hip",
             "route": "route_bf16.hip", "group": "route_bf16.hip", "attend": "attend_bf16.hip"},
    "f32": {"pool": "pool.hip", "landmark": "landmark.hip", "route": "route.hip",
            "group": "route.hip", "attend": "attend.hip"},
}
# rocprofv3 kernel names -> the names mita_kernel_names uses
PROFILE_NAMES = [("mita_fused_kernel", "fused"), ("pool_bf16_kernel", "pool"),
                 ("pool_kernel", "pool"), ("landmark_kernel", "landmark"),
                 ("route_bf16_kernel", "route"), ("route_kernel", "route"),
                 ("group_bf16_kernel", "group"), ("group_kernel", "group"),
                 ("attend_bf16_kernel", "attend"), ("attend_kernel", "attend")]


def source_hash(dtype, kernel):
    import hashlib
    h = hashlib.sha256()
    for f in [KERNEL_SOURCES[dtype][kernel]] + SHARED_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, dtype, kernel):
    """HBM bytes per launch from the committed counter summary, or None when absent or
    taken on other sources."""
    if not os.path.exists(TRAFFIC_FILE) or kernel not in KERNEL_SOURCES.get(dtype, {}):
        return None
    want = source_hash(dtype, kernel)
    for line in open(TRAFFIC_FILE):
        f = line.split()
        if len(f) == 5 and not line.startswith("#") and f[0] == kernel and f[1] == workload \
                and f[4] == want:
            return int(f[2]) + int(f[3])
    return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def describe(w, s=1, route_only=False):
    return (f"{w['name']}: B={w['B']} H={w['H']} grid {w['grid_h']}x{w['grid_w']} "
            f"(N={w['grid_h'] * w['grid_w']}) d={w['d']} m={w['m_h'] * w['m_w']} "
            f"({w['m_h']}x{w['m_w']} pool) k={w['k']} s={s}"
            + (", route-only" if route_only else "") + f", {w['dtype']} in, fp32 out")


def variant_flops_per_qh(w, s=1, route_only=False):
    """Matrix flops per query-head of a variant: S and routing (2md each), with the
    shared expert V_L and the shared logits and P V_L (2md each), and 4d per routed
    entry (q.k and p v) for s*k entries."""
    d, m, k = w["d"], w["m_h"] * w["m_w"], w["k"]
    return 2 * m * d * 2 + (0 if route_only else 2 * m * d * 2) + 4 * d * s * k


def algorithmic(w):
    """Bytes and flops the method itself must move / do, per query-head and per kernel."""
    N, d, m, k = w["grid_h"] * w["grid_w"], w["d"], w["m_h"] * w["m_w"], w["k"]
    s_in = 2 if w["dtype"] == "bf16" else 4
    BH = w["B"] * w["H"]
    per_qh = 3 * d * s_in + d * 4
    kern = {
        # the whole pass in one kernel: read Q, K, V once, write out
        "fused": BH * N * per_qh,
        # pooling: read Q, write Q_L
        "pool": BH * (N * d * s_in + m * d * 4),
        # landmark pass: read Q_L, K, V; write idx and V_L
        "landmark": BH * (m * d * 4 + 2 * N * d * s_in + m * k * 4 + m * d * 4),
        # routing: read Q and Q_L, write routes
        "route": BH * (N * d * s_in + m * d * 4 + N * 4),
        # grouping: read routes, write perm, counts and offsets
        "group": BH * (2 * N * 4 + (2 * m + 1) * 4),
        # attention: read Q, each expert's K/V rows once, Q_L, V_L, idx, perm; write out
        "attend": BH * (N * d * s_in + 2 * m * k * d * s_in + 2 * m * d * 4 + m * k * 4
                        + N * 4 + N * d * 4),
    }
    # matrix flops each kernel must do (multiply-adds x 2; no hi/lo duplicates)
    flops = {
        "fused": BH * N * 4 * d * (2 * m + k),
        "pool": 0,
        # S = Q_L K^T and V_L = P V
        "landmark": BH * 4 * m * N * d,
        # R = Q Q_L^T
        "route": BH * 2 * N * m * d,
        "group": 0,
        # shared logits and P V_L, routed logits and P V_e
        "attend": BH * 4 * N * d * (m + k),
    }
    return dict(bytes_per_qh=per_qh, flops_per_qh=4 * d * (2 * m + k), kernel_bytes=kern,
                kernel_flops=flops, qh=BH * N)


class Runner:
    def __init__(self, name, path="auto", s=1, route_only=False, k=None):
        import torch

        import efficient_attention_avg_amd as mita
        import synth
        self.torch, self.mita = torch, mita
        self.w = w = synth.workload(name)
        if k is not None:
            w["k"] = k
        self.path = path
        self.s, self.route_only = s, route_only
        t0 = time.time()
        Q, K, V = synth.workload_inputs(name)
        self.host = (Q, K, V)
        log(f"{name}: inputs generated in {time.time() - t0:.1f}s")
        dt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float32
        self.q, self.k, self.v = (torch.from_numpy(x).to(dt).cuda() for x in (Q, K, V))
        self.args = (w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], w["k"])
        self.out = torch.empty(self.q.shape, dtype=torch.float32, device="cuda")
        code = mita.MITA_BF16 if w["dtype"] == "bf16" else mita.MITA_F32
        nb = mita.mita_workspace_bytes(w["B"], w["H"], w["grid_h"], w["grid_w"], w["d"],
                                       w["m_h"], w["m_w"], w["k"], code, path=path, s=s,
                                       route_only=route_only)
        self.ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
        self.flush_buf = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.flush_f32 = self.flush_buf.view(torch.float32)
        self.flush_sink = torch.zeros((), dtype=torch.float32, device="cuda")
        self.sched = mita.mita_kernel_schedule(w["B"], w["H"], w["grid_h"], w["grid_w"], w["d"],
                                              w["m_h"], w["m_w"], w["k"], code, path=path,
                                              overlap=True, s=s, route_only=route_only)
        self.kernels = [nm for nm, _ in self.sched]

        self.overlap = True

    def step(self, events=None):
        self.mita.mita_forward_ex(self.q, self.k, self.v, *self.args, out=self.out,
                                  workspace=self.ws, path=self.path, events=events,
                                  overlap=self.overlap, s=self.s, route_only=self.route_only)

    def flush(self):
        # a read of 512 MiB evicts L2 and the Infinity Cache with clean lines; a write
        # would leave them full of dirty lines whose write-back then competes with
        # the first kernel's reads
        self.flush_sink += self.flush_f32.sum()

    def timed_calls(self, n, flush=True, overlap=True):
        """n steps, optionally flushing the caches before each, timed by HIP events on the
        caller's stream right before and after each call (nothing recorded between the
        kernels).  Returns the mean step time (ms) and every step's time."""
        torch = self.torch
        self.overlap = overlap
        try:
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]
            for e0, e1 in evs:
                e0.record()  # creates the HIP events before the timed steps
                e1.record()
            torch.cuda.synchronize()
            for e0, e1 in evs:
                if flush:
                    self.flush()
                e0.record()
                self.step()
                e1.record()
            torch.cuda.synchronize()
        finally:
            self.overlap = True
        ms = [e0.elapsed_time(e1) for e0, e1 in evs]
        return sum(ms) / n, ms

    def timed(self, n, flush=True):
        """n steps, optionally flushing the caches before each, with the library's per-kernel
        events: it records one before its first kernel and one after each kernel (the staged
        schedule's routing and grouping on its side stream); each kernel's time is the
        interval from its start event (mita_kernel_schedule) to its own end.  Returns the
        mean instrumented step time (ms), every step's time, and each kernel's mean time (ms)."""
        torch = self.torch
        kevs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(self.kernels) + 1)]
                for _ in range(n)]
        for kev in kevs:
            for e in kev:
                e.record()  # creates the HIP event before the timed steps
        torch.cuda.synchronize()
        for kev in kevs:
            if flush:
                self.flush()
            self.step(events=kev)
        torch.cuda.synchronize()
        ms = [kev[0].elapsed_time(kev[-1]) for kev in kevs]
        per = {name: sum(kev[st].elapsed_time(kev[i + 1]) for kev in kevs) / n
               for i, (name, st) in enumerate(self.sched)}
        return sum(ms) / len(ms), ms, per


def measure(name, steps, warmup, path="auto", warm=True):
    import torch
    r = Runner(name, path)
    w = r.w
    alg = algorithmic(w)
    for _ in range(warmup):
        r.flush()
        r.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cold_ms, cold_all = r.timed_calls(steps, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the per-kernel breakdown comes from a second cold series with the library's
    # per-kernel events (which add a little time of their own)
    inst_ms, _, stages = r.timed(steps, flush=True)
    warm_ms = None
    if warm:
        warm_ms, _ = r.timed_calls(steps, flush=False)
    one_stream = None
    if any(st != i for i, (_, st) in enumerate(r.sched)):
        # the staged schedule forks routing and grouping onto a side stream: time the
        # single-stream form too
        os_ms, os_all = r.timed_calls(steps, flush=True, overlap=False)
        one_stream = (os_ms, sorted(os_all)[steps // 2])
        log(f"{name}: one stream {one_stream[0] * 1e3:.1f} us/step (median {one_stream[1] * 1e3:.1f})")
    log(f"{name}: with per-kernel events {inst_ms * 1e3:.1f} us/step")
    log(f"{name}: cold {cold_ms * 1e3:.1f} us/step"
        + (f", warm {warm_ms * 1e3:.1f} us/step" if warm_ms else ""))
    qh = alg["qh"]
    sched = "fused" if r.kernels == ["fused"] else "staged"
    log(f"{name}: {sched} schedule, kernel event times (us) "
        + ", ".join(f"{k}={v * 1e3:.1f}" for k, v in stages.items()))
    dom = max(stages, key=stages.get)
    dom_bytes = alg["kernel_bytes"][dom]
    dom_gbs = dom_bytes / (stages[dom] * 1e-3) / 1e9
    pass_gbs = alg["bytes_per_qh"] * qh / (cold_ms * 1e-3) / 1e9
    res = dict(
        workload=w, value=qh / (cold_ms * 1e-3), ms_per_step=cold_ms,
        ms_p10=sorted(cold_all)[len(cold_all) // 10], ms_p90=sorted(cold_all)[(9 * len(cold_all)) // 10],
        ms_median=sorted(cold_all)[len(cold_all) // 2],
        warm_ms_per_step=warm_ms, warm_value=qh / (warm_ms * 1e-3) if warm_ms else None,
        wall_s=wall,
        roofline=dict(bound="hbm", kernel=dom, achieved=dom_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=dom_gbs / HBM_PEAK_GBS,
                      traffic=measured_traffic(w["name"], w["dtype"], dom),
                      algorithmic_bytes_per_launch=dom_bytes, avg_launch_us=stages[dom] * 1e3),
        pass_roofline=dict(bound="hbm", achieved=pass_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                           frac=pass_gbs / HBM_PEAK_GBS, bytes_per_qh=alg["bytes_per_qh"],
                           flops_per_qh=alg["flops_per_qh"]),
        stage_us={k: v * 1e3 for k, v in stages.items()},
        kernel_gbs={k: alg["kernel_bytes"][k] / (v * 1e-3) / 1e9 for k, v in stages.items()},
        # MFMA utilisation of the contraction kernels: algorithmic flops / time against
        # the dense bf16 peak
        kernel_mfma={k: dict(tflops=alg["kernel_flops"][k] / (v * 1e-3) / 1e12,
                             frac=alg["kernel_flops"][k] / (v * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS)
                     for k, v in stages.items() if alg["kernel_flops"].get(k)},
        schedule=sched, dtype=w["dtype"],
        one_stream_ms=one_stream, instrumented_ms_per_step=inst_ms,
    )
    return r, res


def measure_light(name, steps, warmup, s=1, route_only=False, k=None):
    """A shorter record for the other workloads and the variants: warm-up, then cold
    steps timed by events around each call and a cold series with per-kernel events."""
    import torch
    r = Runner(name, "auto", s=s, route_only=route_only, k=k)
    w = r.w
    alg = algorithmic(w)
    for _ in range(warmup):
        r.flush()
        r.step()
    torch.cuda.synchronize()
    cold_ms, cold_all = r.timed_calls(steps, flush=True)
    inst_ms, _, stages = r.timed(steps, flush=True)
    qh = alg["qh"]
    pass_gbs = alg["bytes_per_qh"] * qh / (cold_ms * 1e-3) / 1e9
    fl = variant_flops_per_qh(w, s, route_only)
    res = dict(workload=describe(w, s, route_only), value=qh / (cold_ms * 1e-3),
               unit="query-heads/s", ms_per_step=cold_ms,
               ms_median=sorted(cold_all)[len(cold_all) // 2],
               schedule="fused" if r.kernels == ["fused"] else "staged",
               pass_roofline=dict(bound="hbm", achieved=pass_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                                  frac=pass_gbs / HBM_PEAK_GBS, bytes_per_qh=alg["bytes_per_qh"],
                                  flops_per_qh=fl,
                                  mfma_frac=fl * qh / (cold_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS),
               stage_us={kk: v * 1e3 for kk, v in stages.items()},
               instrumented_ms_per_step=inst_ms)
    log(f"{res['workload']}: {cold_ms * 1e3:.1f} us/step, kernels (us) "
        + ", ".join(f"{kk}={v * 1e3:.1f}" for kk, v in stages.items()))
    del r
    torch.cuda.empty_cache()
    return res


def measure_backward(name, steps, warmup):
    """The backward (mita_backward: the forward's choices recomputed, then dQ, dK, dV) on a
    workload: cold steps timed by events around each call.  Algorithmic bytes per
    query-head: Q, K, V and dOut read once, dQ, dK, dV written once."""
    import torch

    import efficient_attention_avg_amd as mita
    import synth
    w = synth.workload(name)
    Q, K, V = synth.workload_inputs(name)
    dt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).to(dt).cuda() for x in (Q, K, V))
    g = torch.randn(q.shape, dtype=torch.float32, device="cuda",
                    generator=torch.Generator(device="cuda").manual_seed(0))
    args = (w["grid_h"], w["grid_w"], w["m_h"], w["m_w"], w["k"])
    code = mita.MITA_BF16 if w["dtype"] == "bf16" else mita.MITA_F32
    ex = mita._Extras()
    import ctypes
    nb = int(mita.lib().mita_backward_workspace_bytes(w["B"], w["H"], *args[:2], w["d"],
                                                     *args[2:], code, ctypes.byref(ex)))
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        mita.mita_backward(q, k, v, g, *args, workspace=ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        sink += flush.sum()
        e0.record()
        mita.mita_backward(q, k, v, g, *args, workspace=ws)
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    mean = sum(ms) / len(ms)
    qh = w["B"] * w["H"] * w["grid_h"] * w["grid_w"]
    s_in = 2 if w["dtype"] == "bf16" else 4
    per_qh = 3 * w["d"] * s_in + w["d"] * 4 + 3 * w["d"] * 4
    gbs = per_qh * qh / (mean * 1e-3) / 1e9
    log(f"{name} backward: {mean * 1e3:.1f} us/step")
    del q, k, v, g, ws, flush
    torch.cuda.empty_cache()
    return dict(workload=describe(w) + ", backward (dQ, dK, dV)", value=qh / (mean * 1e-3),
                unit="query-heads/s", ms_per_step=mean, ms_median=ms[len(ms) // 2],
                pass_roofline=dict(bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                                   frac=gbs / HBM_PEAK_GBS, bytes_per_qh=per_qh))


# the other workloads and the variants, one light record each
EXTRA_LINES = [
    ("deit-t", 1, False, None), ("long-16k", 1, False, None), ("ade-1024", 1, False, None),
    ("ade-1600", 1, False, None), ("seq-64k", 1, False, None), ("seq-256k", 1, False, None),
    ("deit-s", 2, False, None), ("hires-3136", 2, False, None),
    # route-only with the plain pass's m + k entries per query
    ("deit-s", 1, True, 50), ("hires-3136", 1, True, 113),
]


def cpu_baseline(runner, seconds):
    """The fp64 oracle, as it stands, on the first heads of the same inputs (bounded time)."""
    from threadpoolctl import threadpool_limits

    import oracle
    w = runner.w
    Q, K, V = runner.host
    N = w["grid_h"] * w["grid_w"]
    heads = 0
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for b in range(w["B"]):
            for h in range(w["H"]):
                oracle.mita_head(Q[b, h], K[b, h], V[b, h], w["grid_h"], w["grid_w"], w["m_h"],
                                 w["m_w"], w["k"])
                heads += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            if time.perf_counter() - t0 >= seconds:
                break
        el = time.perf_counter() - t0
    return dict(value=heads * N / el, unit="query-heads/s", cores=cores, kind="oracle",
                sample=f"first {heads} of {w['B'] * w['H']} (b,h) heads of {w['name']}, "
                       f"{el:.1f}s, numpy fp64, BLAS threads = the {cores} cores this process "
                       f"may run on")


COPY_MIB = 256


def copy_calibration():
    """One plain copy kernel of known size (reads and writes COPY_MIB MiB), for scaling the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    a = torch.ones(COPY_MIB << 18, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.neg(a, out=b)
    torch.cuda.synchronize()


def summarize_pmc(fetch_dir, write_dir, workload):
    """Per-launch HBM bytes of each MiTA kernel from two rocprofv3 counter runs of this script
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), scaled by the copy kernel's readings.
    Prints lines for profiles/hbm_traffic.txt."""
    import csv
    import glob

    def read(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                key = "copy" if "neg" in name.lower() else next(
                    (k for pat, k in PROFILE_NAMES if pat in name), None)
                if key:
                    vals.setdefault(key, []).append(float(row["Counter_Value"]) * 1024.0)
        return {k: sum(v) / len(v) for k, v in vals.items()}

    fetch, write = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")
    copy_bytes = float(COPY_MIB << 20)
    sf, sw = copy_bytes / fetch["copy"], copy_bytes / write["copy"]
    print(f"# copy kernel of {COPY_MIB} MiB: FETCH_SIZE reads {fetch['copy'] / 1024:.0f} KiB "
          f"(x{sf:.4f}), WRITE_SIZE reads {write['copy'] / 1024:.0f} KiB (x{sw:.4f})")
    import synth
    dtype = synth.workload(workload)["dtype"]
    for k in sorted(set(fetch) & set(write) - {"copy"}):
        print(f"{k} {workload} {int(fetch[k] * sf)} {int(write[k] * sw)} {source_hash(dtype, k)}")


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        summarize_pmc(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="deit-s")
    ap.add_argument("--also", default="hires-3136", help="second workload ('' to skip)")
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "staged"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm (no flush) figure, e.g. under a profiler")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain copy kernel of known size (counter scaling)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the light records of the other workloads and the variants")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward on --workload (and --also), one JSON line of "
                         "backward records (for profiling the backward kernels)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this MiTA build runs on exactly one GPU; every (batch, head) is "
              "independent, so N GPUs would each run the same kernels on B*H/N heads with no "
              "communication. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import efficient_attention_avg_amd as mita
    if not os.path.exists(mita.LIB_PATH):
        from efficient_attention_avg_amd import build as _b
        _b.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.backward_only:
        recs = [measure_backward(n, args.steps, args.warmup) for n in (args.workload, args.also) if n]
        print(json.dumps({"backward": recs}))
        return
    if args.copy_calibration:
        copy_calibration()
    runner, main_res = measure(args.workload, args.steps, args.warmup, args.path,
                               warm=not args.no_warm)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        cpu = cpu_baseline(runner, args.cpu_seconds)
        log(f"oracle: {cpu['value']:.3g} qh/s ({cpu['sample']})")
    del runner
    torch.cuda.empty_cache()
    secondary = None
    if args.also:
        r2, res2 = measure(args.also, args.steps, args.warmup, args.path, warm=not args.no_warm)
        cpu2 = None
        if not args.no_cpu_baseline:
            cpu2 = cpu_baseline(r2, args.cpu_seconds)
            log(f"oracle ({args.also}): {cpu2['value']:.3g} qh/s ({cpu2['sample']})")
        del r2
        torch.cuda.empty_cache()
        secondary = {
            "workload": describe(res2["workload"]), "value": res2["value"], "unit": "query-heads/s",
            "ms_per_step": res2["ms_per_step"], "ms_median": res2["ms_median"],
            "ms_p10": res2["ms_p10"], "ms_p90": res2["ms_p90"],
            "warm_ms_per_step": res2["warm_ms_per_step"],
            "streams": "routing and grouping on a side stream beside the landmark pass",
            "instrumented_ms_per_step": res2["instrumented_ms_per_step"],
            "one_stream_ms_per_step": res2["one_stream_ms"][0] if res2["one_stream_ms"] else None,
            "one_stream_ms_median": res2["one_stream_ms"][1] if res2["one_stream_ms"] else None,
            "roofline": res2["roofline"], "pass_roofline": res2["pass_roofline"],
            "stage_us": res2["stage_us"], "kernel_gbs": res2["kernel_gbs"],
            "kernel_mfma": res2["kernel_mfma"],
            "schedule": res2["schedule"], "dtype": res2["dtype"], "cpu_baseline": cpu2,
        }
    extras = []
    if not args.no_extras:
        for name, s_, ro, k in EXTRA_LINES:
            extras.append(measure_light(name, args.extra_steps, 5, s=s_, route_only=ro, k=k))
        for name in ("deit-s", "hires-3136"):
            extras.append(measure_backward(name, args.extra_steps, 3))
    w = main_res["workload"]
    line = {
        "metric": METRIC, "value": main_res["value"], "unit": "query-heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": main_res["dtype"], "data": "synthetic",
        "config": {"workload": describe(w), "B": w["B"], "H": w["H"], "seq_len": w["grid_h"] * w["grid_w"],
                   "m": w["m_h"] * w["m_w"], "k": w["k"], "path": args.path,
                   "schedule": main_res["schedule"],
                   "timing": "HIP events on the caller's stream around each call, mean over the "
                             "timed steps (median and p10/p90 beside it), L2 + Infinity Cache "
                             "flushed (512 MiB read) before each step; per-kernel times from a "
                             "second cold series with the library's per-kernel events"},
        "ms_median": main_res["ms_median"], "ms_p10": main_res["ms_p10"], "ms_p90": main_res["ms_p90"],
        "warm_ms_per_step": main_res["warm_ms_per_step"], "warm_value": main_res["warm_value"],
        "instrumented_ms_per_step": main_res["instrumented_ms_per_step"],
        "roofline": main_res["roofline"], "pass_roofline": main_res["pass_roofline"],
        "stage_us": main_res["stage_us"], "kernel_gbs": main_res["kernel_gbs"],
        "kernel_mfma": main_res["kernel_mfma"],
        "cpu_baseline": cpu, "secondary": secondary, "extras": extras,
        "library": mita.lib().mita_version().decode(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
