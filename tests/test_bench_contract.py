"""bench.py's contract on the CPU: it refuses more than one GPU, its algorithmic work
(the numerator of roofline.achieved) equals what the oracle's routing of a call makes
the experts do, and roofline.traffic is reported only for the kernel sources the
committed counter summary was taken from."""

import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from moe_layer_scheduling_amd import synth
from oracle import moe as om

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_work_matches_the_oracle_routing():
    """Count the work of a two-layer call directly: every (token, slot) the oracle routes to
    expert e multiplies one row by that expert's gate, up and down matrices (2 flops per
    multiply-add, sizes read off the weight arrays); the bytes are the arrays of every
    expert with at least one row, the router matrices, and x in and out of each layer."""
    cfg = synth.MoEConfig("acct", (40,), 256, 8, 3, 192, layers=2, zipf_s=0.8)
    T = 40
    layers = synth.layers_as_numpy(synth.make_layers(cfg))
    x = synth.as_numpy(synth.make_x(cfg, T))
    routings, _ = om.moe_forward(x, layers, cfg.top_k, cfg.eps)
    flops = nbytes = 0
    es = 2  # bfloat16 storage
    for lay, r in zip(layers, routings):
        for e in range(cfg.experts):
            rows = int(np.sum(r.idx == e))
            mats = (lay["w_gate"][e], lay["w_up"][e], lay["w_down"][e])
            flops += rows * sum(2 * m.size for m in mats)
            if rows:
                nbytes += sum(m.size for m in mats) * es
        nbytes += lay["w_router"].size * es + 2 * x.size * es
    got = bench.algorithmic_work(cfg, T, [r.counts for r in routings])
    assert got[0] == flops
    assert got[1] == sum(2 * T * lay["w_router"].size for lay in layers)
    assert got[2] == nbytes
    assert got[3] == sum(int((r.counts > 0).sum()) for r in routings)


def test_traffic_only_for_the_measured_sources(monkeypatch):
    text = open(bench.TRAFFIC_FILE).read()
    measured = text.split('"source_sha256": "')[1].split('"')[0]
    monkeypatch.setattr(bench, "source_hash", lambda: measured)
    t = bench.measured_traffic("prefill_T4096")
    assert isinstance(t, int) and t > 4e9  # at least the algorithmic 4.56 GB
    assert bench.measured_traffic("no_such_workload") is None
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 64)
    assert bench.measured_traffic("prefill_T4096") is None


def test_source_hash_covers_the_kernel_sources(tmp_path, monkeypatch):
    h = bench.source_hash()
    assert len(h) == 64 and int(h, 16) >= 0
    # a different source tree hashes differently
    d = tmp_path / "moe_layer_scheduling_amd" / "csrc"
    d.mkdir(parents=True)
    (d / "moe.hip").write_text("// empty\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.source_hash() != h


@pytest.mark.gpu
def test_bench_line_on_the_gpu():
    """One short bench.py run of the tiny workload prints the one JSON line with the
    fields the contract names, a positive throughput and a roofline object."""
    import json

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--steps", "3", "--warmup", "1", "--no-secondary", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 3 and line["value"] > 0
    roof = line["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    assert line["config"]["workload"].startswith("tiny")
