"""bench.py's host-side logic, on the CPU: the one-GPU refusal, the sweep
options' checks, the traffic figure tied to the kernel source it was measured
on, the CPU baseline's fields, the buffer rotation and the fixed-cost fit."""
import json
import os
import subprocess
import sys
import types

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle  # noqa: E402
from residual_add_rmsnorm_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                           env=dict(os.environ, **env), capture_output=True, text=True,
                           timeout=120)
        assert r.returncode == 2 and "one GPU only" in r.stderr
        assert r.stdout == ""


def test_sweep_arguments_are_checked_before_any_gpu_work():
    for args in (["--sweep", "no_such_workload"], ["--sweep-tokens", "0,1024"],
                 ["--sweep-tokens", "many"], ["--sweep", ""]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2 and "--sweep needs" in r.stderr, (args, r.stderr[-500:])
        assert r.stdout == ""


def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    src = tmp_path / "kernels.hip"
    src.write_text("// kernel source\n")
    traffic = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    assert bench.measured_traffic() is None                      # no file
    traffic.write_text(json.dumps({"kernel_source_sha256": bench.source_digest(),
                                   "bytes_per_launch": 123}))
    assert bench.measured_traffic() == 123
    src.write_text("// changed\n")
    assert bench.measured_traffic() is None                      # stale after a change


def test_cpu_baseline_fields():
    runners = {}
    for name in bench.STEP + bench.LATENCY:
        w = wl.WORKLOADS[name].with_tokens(16)
        c = wl.make_inputs(w)
        var = None
        if w.tp_world > 1:
            rows = [wl.bits(c.qkv)] + [wl.bits(s) for s in c.shards]
            var = torch.from_numpy(sum(oracle.qk_means(r, w.q_size, w.kv_size)
                                       for r in rows).astype(np.float32))
        runners[name] = types.SimpleNamespace(name=name, w=w, cpu=c, var_in=var,
                                              bytes=w.algorithmic_bytes())
    threads = oracle.max_threads()
    cb = bench.cpu_baseline(runners, min_seconds=0.0, max_reps=2)
    assert set(cb) == {"value", "unit", "cores", "kind", "sample", "per_config"}
    assert cb["unit"] == "GB/s" and cb["kind"] == "oracle" and cb["value"] > 0
    assert cb["cores"] == threads
    assert set(cb["per_config"]) == set(bench.STEP + bench.LATENCY)
    for name, rec in cb["per_config"].items():
        assert rec["GB/s"] > 0 and rec["tokens/s"] > 0 and rec["threads"] == threads
        assert ("one_thread" in rec) == (name in bench.LATENCY)
    # the step figure is the step's bytes over the sum of its launches' times
    step_s = sum(cb["per_config"][n]["s_per_launch"] for n in bench.STEP)
    step_bytes = sum(runners[n].bytes for n in bench.STEP)
    assert abs(cb["value"] - step_bytes / step_s / 1e9) <= 0.01 * cb["value"] + 1e-3
    assert oracle.max_threads() == threads      # the one-thread leg restores the thread count


def test_rotation_keeps_each_launch_out_of_the_last_level_cache():
    for name in bench.STEP + bench.LATENCY + bench.NEXT:
        w = wl.WORKLOADS[name]
        k = bench.sets_for(w.algorithmic_bytes())
        assert k * w.algorithmic_bytes() >= (1 << 30) or k == 128
    assert bench.sets_for(wl.WORKLOADS["decode"].algorithmic_bytes()) == 84
    assert bench.sets_for(wl.WORKLOADS["qk_local"].algorithmic_bytes()) == 10
    assert bench.sets_for(wl.WORKLOADS["prefill_fp8_token"].algorithmic_bytes()) == 1


def test_fixed_cost_fit_recovers_a_known_line():
    nbytes = [29e6, 59e6, 117e6, 235e6, 470e6, 940e6]
    us = [2.4 + b / 6.2e6 for b in nbytes]       # 2.4 us + bytes at 6.2 TB/s (6.2e6 B per us)
    fixed, rate = bench.fit_fixed_and_rate(nbytes, us)
    assert abs(fixed - 2.4) < 1e-9 and abs(rate - 6200.0) < 1e-6
