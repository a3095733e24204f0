#!/usr/bin/env python3
"""Throughput of exact tiled attention (forward + backward) on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
attn_fwd (O, L) then attn_bwd (dQ, dK, dV) through the C ABI.  Inputs are
generated from the workload's seed and are resident in HBM before timing.

Prints one JSON line.  ``value`` is the algorithmic forward+backward
TFLOP/s, F = 2 #A (d + v) + 2 #A (3d + 2v) per step with #A the number of
allowed (query, key) pairs; ``roofline`` reports the dominant kernel's
algorithmic FLOPs per launch over its average launch duration (HIP events
recorded by the library on the launch stream) against the dense MFMA peak
of the dtype; ``cpu_baseline`` times the float64 oracle on the host cores on
a bounded sample (one (batch, head) unit, sub-sized if needed);
``sclk`` holds the engine clock and board power sampled over a separate run
of the same steps, and ``gemm_ceiling`` the vendor GEMM's throughput on
random operands of the same dtype on the same board (the practical ceiling
under its power limit), against which ``roofline.frac_of_gemm`` is taken.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # published dense MFMA peaks
HEADLINE = "bf16_causal_h32_n16384_d128"
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "exact_tiled_attention_attn_amd", "csrc")
# Source files each kernel class is built from (a recorded HBM byte count is
# reported only while these are unchanged).
KERNEL_SOURCES = {
    "fwd": ["attn_fwd.hip", "kern_common.h"],
    "bwd": ["attn_bwd.hip", "attn_bwd_kv.hip", "attn_bwd_kv2.hip", "kern_common.h"],
    "bwd_dq": ["attn_bwd_dq.hip", "attn_bwd_dq_pipe.hip", "kern_common.h"],
    "bwd_pre": ["attn_aux.hip"],
    "bwd_post": ["attn_aux.hip"],
    "tile_map": ["attn_aux.hip"],
}


def source_sha(kernel: str) -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, deterministic: int, kernel: str):
    """HBM bytes per launch of `kernel` from profiles/traffic_*.txt (rocprofv3
    FETCH_SIZE/WRITE_SIZE scaled by a 1 GiB copy), or None if absent or stale."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}{'' if deterministic else '_atomic'}.txt")
    if not os.path.exists(path):
        return None
    kv = dict(line.strip().split("=", 1) for line in open(path) if "=" in line)
    if kv.get(f"{kernel}.source_sha256") != source_sha(kernel):
        return None
    b = kv.get(f"{kernel}.bytes")
    return float(b) if b is not None else None


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip the engine-clock sampling run")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the vendor-GEMM ceiling measurement")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache pass (512 MiB scrub before each step)")
    ap.add_argument("--cpu-budget-s", type=float, default=25.0)
    ap.add_argument("--deterministic", type=int, default=1, choices=(0, 1),
                    help="backward dQ path: 1 = query-tile-outer kernel (default), 0 = fp32 atomics")
    ap.add_argument("--queries", type=int, default=0,
                    help="rectangular run: only the last QUERIES query rows against all n keys, causal "
                         "offset n - QUERIES (the last shard of a query-sharded sequence); 0 = square")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout probability on the attention weights (seed 1234); 0 = none")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    return ap.parse_args()


def calibrate_copy():
    """A copy kernel of known size: 1 GiB read + 1 GiB written per launch, 3 launches."""
    import torch

    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "launches": 3}), flush=True)


def host_info() -> dict:
    """CPU model, usable cores and the BLAS library numpy runs on."""
    import threadpoolctl

    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    return {"cpu": model, "usable_cores": len(os.sched_getaffinity(0)),
            "blas": ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in blas) or "unknown",
            "blas_threads": max((p.get("num_threads", 1) for p in blas), default=1)}


def _time_route(prob, route: str, budget_s: float):
    """Time one oracle route on growing leading sub-problems of unit (0, 0).

    Starts at 2048 query rows and keys (the same recipe, cut to its leading
    block; rows left without an allowed key get their diagonal key) and
    doubles while the predicted time stays within the budget, up to the full
    unit.  Returns (rows, pairs, seconds, flops) of the last size timed.
    """
    import workloads as W
    from oracle import dense, tiled

    w = prob.w
    n = w.n
    Q, K, V, G = (getattr(prob, x)[0, 0].astype(np.float64) for x in "QKVG")
    ns, spent, result = min(2048, n), 0.0, None
    while True:
        A = None if w.mask == W.MASK_NONE else prob.allowed(0)[:ns, :ns]
        if A is not None and not A.any(axis=1).all():
            A = A.copy()
            A[np.arange(ns), np.arange(ns)] = True
        pairs = ns * ns if A is None else int(A.sum())
        t0 = time.perf_counter()
        if route == "dense":
            dense.forward(Q[:ns], K[:ns], V[:ns], w.scale, A)
            dense.vjp(Q[:ns], K[:ns], V[:ns], w.scale, A, G[:ns])
        else:
            b = w.oracle_blocks[0]
            Y, m, ell, _ = tiled.forward(Q[:ns], K[:ns], V[:ns], w.scale, A, b)
            tiled.reverse(Q[:ns], K[:ns], V[:ns], w.scale, A, b, Y, m, ell, G[:ns])
        dt = time.perf_counter() - t0
        spent += dt
        result = (ns, pairs, dt, 2.0 * pairs * (w.d + w.v) + 2.0 * pairs * (3 * w.d + 2 * w.v))
        if ns >= n or spent + 4.2 * dt > budget_s:
            return result
        ns = min(n, 2 * ns)


def cpu_baseline(prob, budget_s: float) -> dict:
    """The oracle as it stands, timed on the host cores: the dense definition
    (forward + VJP, oracle/dense.py) as ``value``, the key-block procedure
    (forward + reverse, oracle/tiled.py, at the workload's oracle block size)
    beside it; half the budget each."""
    w = prob.w
    host = host_info()
    out = {}
    for route in ("dense", "tiled"):
        ns, pairs, dt, flops = _time_route(prob, route, budget_s / 2)
        what = ("dense float64 forward + VJP" if route == "dense"
                else f"key-block float64 forward + reverse, block {w.oracle_blocks[0]}")
        out[route] = {"value": flops / dt / 1e12, "seconds": round(dt, 3),
                      "sample": f"unit (b=0, h=0), query rows and keys 0..{ns - 1} of {w.n} ({pairs} allowed pairs): "
                                f"{what}"}
    d = out["dense"]
    return {
        "value": d["value"],
        "unit": "TFLOP/s",
        "cores": int(host["blas_threads"]),
        "kind": "oracle",
        "sample": d["sample"] + f", {d['seconds']:.2f} s",
        "tiled": {"value": out["tiled"]["value"], "unit": "TFLOP/s",
                  "sample": out["tiled"]["sample"] + f", {out['tiled']['seconds']:.2f} s"},
        "host": host,
    }


class ClockSampler:
    """Samples the GPU engine clock and the board power on a host thread: the
    mean over the XCDs of amdsmi's current GFX clocks and the socket power of
    the firmware's metrics table.  The table refreshes slowly, so the bench
    samples a separate run of the same work lasting a second or more, after
    the timed steps, and keeps the samples past its first half second.  A
    missing or failing amdsmi gives no samples, not an error."""

    def __init__(self, period_s: float = 0.01, settle_s: float = 0.5):
        import threading

        self.period, self.settle = period_s, settle_s
        self.samples = []  # (clock MHz, power W or None)
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._handle = None
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._handle = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception:
            self._amdsmi = None

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = [float(x) for x in m.get("current_gfxclks", []) if isinstance(x, (int, float))]
        if clks:
            clk = sum(clks) / len(clks)
        else:
            clk = float(self._amdsmi.amdsmi_get_clock_info(self._handle, self._amdsmi.AmdSmiClkType.GFX)["clk"])
        pw = None
        for key in ("current_socket_power", "average_socket_power"):
            x = m.get(key)
            if isinstance(x, (int, float)) and 0 < x < 65535:
                pw = float(x)
                break
        return clk, pw

    def _run(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            try:
                x = self._read()
            except Exception:
                return
            if time.perf_counter() - t0 >= self.settle:
                self.samples.append(x)
            self._stop.wait(self.period)

    def __enter__(self):
        if self._handle is not None:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()
        if self._amdsmi is not None:
            try:
                self._amdsmi.amdsmi_shut_down()
            except Exception:
                pass

    def summary(self, what="the same steps"):
        if not self.samples:
            return None
        x = sorted(c for c, _ in self.samples)
        out = {"median_mhz": round(x[len(x) // 2], 1), "min_mhz": round(x[0], 1), "max_mhz": round(x[-1], 1),
               "samples": len(x),
               "source": "amdsmi current GFX clocks (mean over XCDs), sampled every 10 ms past the first 0.5 s "
                         f"of a separate >= 1.5 s run of {what} after the timed ones"}
        pw = sorted(p for _, p in self.samples if p is not None)
        if pw:
            out["power_w"] = {"median": round(pw[len(pw) // 2], 1), "max": round(pw[-1], 1),
                              "source": "amdsmi socket power, same samples"}
        return out


def gemm_ceiling(torch, dtype_name: str, seconds: float = 1.5, size: int = 8192):
    """A practical MFMA ceiling on this board: torch.matmul (the vendor GEMM
    library) on N(0,1) operands of the workload's dtype, size^3, run for a
    second or more with the same clock and power sampling.  The published
    peak assumes the 2.4 GHz clock; with random operands the board's power
    limit holds every MFMA-dense kernel below it."""
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    g = torch.Generator(device="cuda:0").manual_seed(0)
    a = torch.randn(size, size, device="cuda:0", dtype=torch.float32, generator=g).to(dt)
    b = torch.randn(size, size, device="cuda:0", dtype=torch.float32, generator=g).to(dt)
    c = torch.empty(size, size, device="cuda:0", dtype=dt)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with ClockSampler() as clock:
        n, start = 0, time.perf_counter()
        t0.record()
        while time.perf_counter() - start < seconds:
            torch.matmul(a, b, out=c)
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        t1.record()
        torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / n
    del a, b, c
    out = {"kind": f"torch.matmul {dtype_name} {size}x{size}x{size}, N(0,1) operands",
           "tflops": round(2.0 * size ** 3 / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 4)}
    s = clock.summary("the same products")
    if s:
        out["sclk_mhz"] = s["median_mhz"]
        if "power_w" in s:
            out["power_w"] = s["power_w"]["median"]
    return out


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_tiled_attention_attn_amd as E
    import workloads as W

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    E.load_library()  # fail loudly if the HIP library is missing
    prob = W.generate(args.workload)
    w = prob.w
    nq, coff = w.n, 0
    if args.queries:
        if w.mask == W.MASK_BITMASK or not 0 < args.queries <= w.n:
            print("--queries needs a none/causal workload and 0 < QUERIES <= n", file=sys.stderr)
            sys.exit(2)
        nq = args.queries
        coff = w.n - nq if w.mask == W.MASK_CAUSAL else 0
        # Pairs per unit: row i (of the last nq) allows min(n, i + coff + 1) keys.
        per_unit = nq * w.n if w.mask == W.MASK_NONE else sum(min(w.n, i + coff + 1) for i in range(nq))
        pairs = w.B * w.H * per_unit
    else:
        pairs = W.allowed_pairs(w, prob)
    f_fwd, f_bwd = W.flops(w, pairs)
    dev = "cuda:0"

    def up(name):
        if w.dtype == "bf16":
            return torch.from_numpy(prob.bits[name].view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(getattr(prob, name)).to(dev)

    q, k, v, g = (up(x) for x in "QKVG")
    if nq != w.n:
        q, g = q[:, :, w.n - nq:].contiguous(), g[:, :, w.n - nq:].contiguous()
    mask = None
    if prob.mask_words is not None:
        mask = torch.from_numpy(prob.mask_words.view(np.int32)).to(dev)
    o = torch.empty((w.B, w.H, nq, w.v), dtype=q.dtype, device=dev)
    lse = torch.empty((w.B, w.H, nq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    drop = dict(dropout_p=args.dropout, dropout_seed=1234)
    pf = E.make_problem(q, k, v, o, w.scale, w.mask, mask, causal_offset=coff, **drop)
    ws_f = torch.empty(max(E.workspace_size(pf, False), 256), dtype=torch.uint8, device=dev)
    pf_b = E.make_problem(q, k, v, o, w.scale, w.mask, mask, bool(args.deterministic), coff, **drop)
    ws_b = torch.empty(max(E.workspace_size(pf_b, True), 256), dtype=torch.uint8, device=dev)

    def step():
        E.fwd(q, k, v, w.scale, w.mask, mask, out=o, lse=lse, workspace=ws_f, causal_offset=coff, **drop)
        E.bwd(q, k, v, o, g, lse, w.scale, w.mask, mask, dq=dq, dk=dk, dv=dv, workspace=ws_b,
              deterministic=bool(args.deterministic), causal_offset=coff, **drop)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    E.timing_enable(True)
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # Per-step events on the same stream give the median and spread; the
    # value is the whole timed region over K steps.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0.record(stream)
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    kern = E.timing_read()
    E.timing_enable(False)
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    # Cold-cache pass (outside the timed region): a 512 MiB buffer is
    # rewritten before each step, so that L2 and the memory-side cache hold
    # none of the inputs when the step starts; each step timed on its own.
    cold = None
    if not args.no_cold:
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold_ms = []
        for _ in range(args.steps):
            scrub.fill_(1)
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b_.record(stream)
            b_.synchronize()
            cold_ms.append(a.elapsed_time(b_))
        del scrub
        cold_ms.sort()
        med = cold_ms[len(cold_ms) // 2]
        cold = {"ms_per_step_median": round(med, 4), "ms_per_step_min": round(cold_ms[0], 4),
                "value": round((f_fwd + f_bwd) / (med * 1e-3) / 1e12, 2), "steps": args.steps,
                "scrub": "512 MiB device buffer rewritten before each step"}
    # Engine clock under this load (outside the timed region).
    sclk = None
    if not args.no_clock:
        reps = max(1, int(1500.0 / max(total_ms / args.steps, 1e-3)) + 1)
        with ClockSampler() as clock:
            for i in range(reps):
                step()
                if i % 16 == 15:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
        sclk = clock.summary()
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t.float()).all(), "non-finite output"

    ms_step = total_ms / args.steps
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    avg = {kname: (ms / cnt if cnt else 0.0) for kname, (ms, cnt) in kern.items()}
    fwd_ms = avg["fwd"] + avg["fwd_merge"] + (avg["tile_map"] if w.mask == W.MASK_BITMASK else 0.0)
    n_maps_bwd = (2 if args.deterministic else 1) if w.mask == W.MASK_BITMASK else 0
    bwd_ms = (avg["bwd_pre"] + avg["bwd"] + avg["bwd_post"] + avg["bwd_dq"] + avg["bwd_dq_merge"]
              + n_maps_bwd * avg["tile_map"])
    peak = PEAK_TFLOPS[w.dtype]
    # Algorithmic FLOPs each main kernel performs per launch: the forward
    # 2#A(d+v); the key-tile-outer backward 2#A(2d+2v) (S, dP, dV, dK) plus
    # 2#A d for dQ when fused; the query-tile-outer dQ kernel 2#A(2d+v).
    pairs_f = float(pairs)
    kflops = {"fwd": f_fwd,
              "bwd": 2 * pairs_f * (2 * w.d + 2 * w.v) + (0 if args.deterministic else 2 * pairs_f * w.d),
              "bwd_dq": 2 * pairs_f * (2 * w.d + w.v)}
    dominant = max(("fwd", "bwd", "bwd_dq"), key=lambda kname: kern[kname][0])
    achieved = kflops[dominant] / (avg[dominant] * 1e-3) / 1e12
    out = {
        "metric": "attention fwd+bwd TFLOP/s on 1 MI355X (algorithmic FLOPs over allowed pairs)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) recipe of the workload; no dataset)",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "n": w.n, "d": w.d, "v": w.v,
                   "mask": w.mask, "allowed_pairs": pairs, "scale": w.scale},
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
                "pct_peak": round(100 * f_fwd / (fwd_ms * 1e-3) / 1e12 / peak, 2)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2),
                "pct_peak": round(100 * f_bwd / (bwd_ms * 1e-3) / 1e12 / peak, 2)},
        "kernels_avg_ms": {kname: round(x, 4) for kname, x in avg.items() if kern[kname][1]},
        "backward_dq_path": "query-tile-outer kernel" if args.deterministic else "fp32 atomics",
        "roofline": {"kernel": dominant, "flops_per_launch": kflops[dominant], "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": (recorded_traffic(w.name, args.deterministic, dominant)
                                 if nq == w.n and not args.dropout else None)},
        "sclk": sclk,
        "step_ms": {"median": round(per_step[len(per_step) // 2], 4), "min": round(per_step[0], 4),
                    "max": round(per_step[-1], 4), "source": "HIP events between the timed steps"},
        "cold": cold,
    }
    if sclk:
        # The published peak assumes the 2.4 GHz engine clock; against the
        # clock measured during the steps:
        at = peak * sclk["median_mhz"] / 2400.0
        out["roofline"].update(peak_at_sclk=round(at, 1), frac_at_sclk=round(achieved / at, 4))
    if not args.no_ceiling:
        # The vendor GEMM on random operands, on the same board under the same
        # power limit: the practical ceiling for MFMA-dense work here.
        ceil = gemm_ceiling(torch, w.dtype)
        out["gemm_ceiling"] = ceil
        out["roofline"]["frac_of_gemm"] = round(achieved / ceil["tflops"], 4)
    if args.dropout:
        out["config"].update(dropout_p=args.dropout, dropout_seed=1234)
    if nq != w.n:
        out["config"].update(queries=nq, keys=w.n, causal_offset=coff,
                             workload=f"{w.name}, last {nq} query rows against all {w.n} keys")
    if not args.no_cpu_baseline and nq == w.n and not args.dropout:
        out["cpu_baseline"] = cpu_baseline(prob, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
