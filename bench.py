#!/usr/bin/env python3
"""Throughput of the MiTA forward pass on one MI355X, with its roofline.

    python bench.py [--steps K] [--warmup W] [--workload deit-s] [--also hires-3136]

A step is one full ``mita_forward`` (pooling, landmark scores + top-k +
landmark values, routing + grouping, grouped expert attention) over one batch
of synthetic, seeded inputs already resident in device memory.  Before every
timed step a 512 MiB buffer is overwritten so that neither L2 nor the 256 MB
Infinity Cache holds the inputs (the DeiT-S inputs would otherwise fit in
it); each step is bracketed by HIP events on the stream the library launches
on, and ms_per_step is the mean of those event times.  A warm (no flush)
back-to-back figure is reported beside it.

Prints ONE JSON line.  ``value`` is query-heads per second (B*H*N per step)
on the headline workload (DeiT-S shape); the 3136-token workload is reported
in ``secondary``.  ``roofline`` covers the kernel that dominates the step;
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
FLUSH_BYTES = 512 << 20


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def describe(w):
    return (f"{w['name']}: B={w['B']} H={w['H']} grid {w['grid_h']}x{w['grid_w']} "
            f"(N={w['grid_h'] * w['grid_w']}) d={w['d']} m={w['m_h'] * w['m_w']} "
            f"({w['m_h']}x{w['m_w']} pool) k={w['k']} s=1, {w['dtype']} in, fp32 out")


def algorithmic(w):
    """Bytes and flops the method itself must move / do, per query-head and per kernel."""
    N, d, m, k = w["grid_h"] * w["grid_w"], w["d"], w["m_h"] * w["m_w"], w["k"]
    s_in = 2 if w["dtype"] == "bf16" else 4
    BH = w["B"] * w["H"]
    per_qh = 3 * d * s_in + d * 4
    kern = {
        # pooling: read Q, write Q_L
        "pool": BH * (N * d * s_in + m * d * 4),
        # landmark pass: read Q_L, K, V; write idx and V_L
        "landmark": BH * (m * d * 4 + 2 * N * d * s_in + m * k * 4 + m * d * 4),
        # routing + grouping: read Q, Q_L; write route, counts, offsets, perm
        "route": BH * (N * d * s_in + m * d * 4 + 2 * N * 4 + (2 * m + 1) * 4),
        # attention: read Q, each expert's K/V rows once, Q_L, V_L, idx, route, perm; write out
        "attend": BH * (N * d * s_in + 2 * m * k * d * s_in + 2 * m * d * 4 + m * k * 4
                        + 2 * N * 4 + N * d * 4),
    }
    return dict(bytes_per_qh=per_qh, flops_per_qh=4 * d * (2 * m + k), kernel_bytes=kern,
                qh=BH * N)


class Runner:
    def __init__(self, name, path="auto"):
        import torch

        import efficient_attention_avg_amd as mita
        import synth
        self.torch, self.mita = torch, mita
        self.w = w = synth.workload(name)
        self.path = path
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
                                       w["m_h"], w["m_w"], w["k"], code)
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        self.flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")

    def step(self):
        self.mita.mita_forward_ex(self.q, self.k, self.v, *self.args, out=self.out,
                                  workspace=self.ws, path=self.path)

    def flush(self):
        self.flush_buf.fill_(1)

    def timed(self, fn, n, flush=True):
        """Mean event time (ms) of fn over n calls, optionally flushing caches before each."""
        torch = self.torch
        ev = []
        for _ in range(n):
            if flush:
                self.flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev.append((a, b))
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        return sum(ms) / len(ms), ms

    def stage_times(self, n):
        """Per-step-kernel event times through the stage entry points (same kernels)."""
        mita, torch = self.mita, self.torch
        gh, gw, mh, mw, k = self.args
        ql = mita.mita_pool(self.q, gh, gw, mh, mw)
        idx, vl = mita.mita_landmark(ql, self.k, self.v, k)
        route, counts, offsets, perm = mita.mita_route(self.q, ql)
        torch.cuda.synchronize()
        return {
            "pool": self.timed(lambda: mita.mita_pool(self.q, gh, gw, mh, mw, ql=ql), n)[0],
            "landmark": self.timed(lambda: mita.mita_landmark(ql, self.k, self.v, k), n)[0],
            "route": self.timed(lambda: mita.mita_route(self.q, ql), n)[0],
            "attend": self.timed(lambda: mita.mita_attend(self.q, self.k, self.v, ql, vl, idx,
                                                          route, offsets, perm), n)[0],
        }


def measure(name, steps, warmup, path="auto"):
    import torch
    r = Runner(name, path)
    w = r.w
    alg = algorithmic(w)
    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cold_ms, cold_all = r.timed(r.step, steps, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    warm_ms, _ = r.timed(r.step, steps, flush=False)
    log(f"{name}: cold {cold_ms * 1e3:.1f} us/step, warm {warm_ms * 1e3:.1f} us/step")
    qh = alg["qh"]
    code = r.mita.MITA_BF16 if w["dtype"] == "bf16" else r.mita.MITA_F32
    sched = r.mita.mita_schedule(w["B"], w["H"], w["grid_h"], w["grid_w"], w["d"], w["m_h"],
                                 w["m_w"], w["k"], code) if path == "auto" else path
    if sched == "fused":
        # one kernel is the whole pass: its algorithmic bytes are the pass's
        stages = {"fused": cold_ms}
        alg["kernel_bytes"]["fused"] = alg["bytes_per_qh"] * qh
    else:
        stages = r.stage_times(max(5, min(steps, 20)))
    log(f"{name}: {sched} schedule, kernel event times (us) "
        + ", ".join(f"{k}={v * 1e3:.1f}" for k, v in stages.items()))
    dom = max(stages, key=stages.get)
    dom_bytes = alg["kernel_bytes"][dom]
    dom_gbs = dom_bytes / (stages[dom] * 1e-3) / 1e9
    pass_gbs = alg["bytes_per_qh"] * qh / (cold_ms * 1e-3) / 1e9
    res = dict(
        workload=w, value=qh / (cold_ms * 1e-3), ms_per_step=cold_ms,
        ms_p10=sorted(cold_all)[len(cold_all) // 10], ms_p90=sorted(cold_all)[(9 * len(cold_all)) // 10],
        warm_ms_per_step=warm_ms, warm_value=qh / (warm_ms * 1e-3), wall_s=wall,
        roofline=dict(bound="hbm", kernel=dom, achieved=dom_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=dom_gbs / HBM_PEAK_GBS, traffic=None,
                      algorithmic_bytes_per_launch=dom_bytes, avg_launch_us=stages[dom] * 1e3),
        pass_roofline=dict(bound="hbm", achieved=pass_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                           frac=pass_gbs / HBM_PEAK_GBS, bytes_per_qh=alg["bytes_per_qh"],
                           flops_per_qh=alg["flops_per_qh"]),
        stage_us={k: v * 1e3 for k, v in stages.items()}, schedule=sched,
        dtype=w["dtype"],
    )
    return r, res


def cpu_baseline(runner, seconds):
    """The fp64 oracle, as it stands, on the first heads of the same inputs (bounded time)."""
    from threadpoolctl import threadpool_limits

    import oracle
    w = runner.w
    Q, K, V = runner.host
    N = w["grid_h"] * w["grid_w"]
    heads = 0
    with threadpool_limits(limits=1):
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
    return dict(value=heads * N / el, unit="query-heads/s", cores=1, kind="oracle",
                sample=f"first {heads} of {w['B'] * w['H']} (b,h) heads of {w['name']}, "
                       f"{el:.1f}s, numpy fp64 with BLAS limited to 1 thread")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="deit-s")
    ap.add_argument("--also", default="hires-3136", help="second workload ('' to skip)")
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "staged"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    runner, main_res = measure(args.workload, args.steps, args.warmup, args.path)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        cpu = cpu_baseline(runner, args.cpu_seconds)
        log(f"oracle: {cpu['value']:.3g} qh/s ({cpu['sample']})")
    del runner
    torch.cuda.empty_cache()
    secondary = None
    if args.also:
        r2, res2 = measure(args.also, args.steps, args.warmup, args.path)
        del r2
        secondary = {
            "workload": describe(res2["workload"]), "value": res2["value"], "unit": "query-heads/s",
            "ms_per_step": res2["ms_per_step"], "warm_ms_per_step": res2["warm_ms_per_step"],
            "roofline": res2["roofline"], "pass_roofline": res2["pass_roofline"],
            "stage_us": res2["stage_us"], "schedule": res2["schedule"], "dtype": res2["dtype"],
        }
    w = main_res["workload"]
    line = {
        "metric": METRIC, "value": main_res["value"], "unit": "query-heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": main_res["dtype"], "data": "synthetic",
        "config": {"workload": describe(w), "B": w["B"], "H": w["H"], "seq_len": w["grid_h"] * w["grid_w"],
                   "m": w["m_h"] * w["m_w"], "k": w["k"], "path": args.path,
                   "schedule": main_res["schedule"],
                   "timing": "HIP events per step, L2 + Infinity Cache flushed before each step"},
        "ms_p10": main_res["ms_p10"], "ms_p90": main_res["ms_p90"],
        "warm_ms_per_step": main_res["warm_ms_per_step"], "warm_value": main_res["warm_value"],
        "roofline": main_res["roofline"], "pass_roofline": main_res["pass_roofline"],
        "stage_us": main_res["stage_us"], "cpu_baseline": cpu, "secondary": secondary,
        "library": mita.lib().mita_version().decode(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
