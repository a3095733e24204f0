"""Host-side behaviour of bench.py that needs no GPU: the one-GPU contract
and the recorded-traffic lookup that feeds the roofline's traffic field."""

from __future__ import annotations

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, env=e, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2 and "one GPU" in r.stderr
    r = _run([], env={"WORLD_SIZE": "2"})
    assert r.returncode == 2 and "WORLD_SIZE=2" in r.stderr


def test_recorded_traffic_follows_the_kernel_sources():
    b = _bench()
    # The committed summary of the headline workload was taken with the
    # current dK/dV kernel source: its bytes are reported ...
    got = b.recorded_traffic("bf16_causal_h32_n16384_d128", 1, "bwd")
    assert got is not None and got > 0
    # ... and a summary whose hash does not match is ignored.
    path = os.path.join(ROOT, "profiles", "traffic_bf16_causal_h32_n16384_d128.txt")
    lines = open(path).read().splitlines()
    assert any(line.startswith("bwd.source_sha256=") for line in lines)
    assert b.recorded_traffic("no_such_workload", 1, "bwd") is None
    assert len(b.source_sha("bwd")) == 16 and b.source_sha("bwd") != b.source_sha("fwd")


def test_clock_and_power_summary():
    b = _bench()
    s = b.ClockSampler.__new__(b.ClockSampler)  # no amdsmi needed for the summary
    s.samples = []
    assert s.summary() is None
    s.samples = [(1900.0, 1350.0), (2000.0, None), (1800.0, 1370.0)]
    out = s.summary("the same products")
    assert out["median_mhz"] == 1900.0 and out["min_mhz"] == 1800.0 and out["max_mhz"] == 2000.0
    assert out["samples"] == 3 and "the same products" in out["source"]
    # power: the median over the samples that carry one
    assert out["power_w"]["median"] == 1370.0 and out["power_w"]["max"] == 1370.0
    s.samples = [(1900.0, None)]
    assert "power_w" not in s.summary()
