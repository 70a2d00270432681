#!/usr/bin/env python3
"""Throughput of the fused TP epilogue and the QK RMSNorm on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
  1. fused_add_rmsnorm_quant_fp8        prefill, T=8192 H=8192 P=8, per-token e4m3
  2. qk_rmsnorm (local means)           MiniMax QK, T=4096, row 8192 = q 6144 | k 1024 | v
  3. fused_add_rmsnorm_quant_fp8_block  T=16384 H=7168 P=2, 1x128 e4m3 groups
  4. qk_rmsnorm (sum of 4 shard means)  as 2, tp_world=4
The launches alternate between the large FP8 passes (>= 1 GB each) and the QK
passes, so no launch finds its inputs in the 256 MB last-level cache.

Prints ONE JSON line. ``value`` is the step's algorithmic bytes (each input
read once, each output written once, weights once per launch) divided by the
wall time of a step, in GB/s, with the step's four launches captured once in a
HIP graph and replayed K times (``eager_*`` gives the same step launched from
Python). ``per_launch`` and ``roofline`` come from a separate eager pass of K
steps in which every launch is bracketed by HIP events on its stream; the
roofline is the dominant kernel's (the per-token FP8 epilogue).
``cpu_baseline`` times the CPU oracle on full steps of the same inputs (about
10 s of host time).
``next_rows`` times the further entry points (sharded-hidden RMSNorm post
stage, static-scale FP8, reduce-scatter epilogue, MLA all-gather epilogue) one
launch at a time, each right after a prefill launch that evicts the last-level
cache, so every timed launch reads its inputs from HBM. ``hbm_ceiling`` is the
library's plain streaming read and copy on the same GPU; ``latency_shapes`` the
per-call time of the two cache-resident shapes (16 x 1024, 128 x 7168).

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-cpu-baseline] [--no-next]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
KERNEL_SRC = os.path.join(ROOT, "residual_add_rmsnorm_amd", "csrc", "fusednorm_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill_fp8_token.json")
STEP = ["prefill_fp8_token", "qk_local", "fp8_block", "qk_sharded"]
DOMINANT = "prefill_fp8_token"
# Entry points beyond the step, each timed alone on its own workload.
NEXT = ["sharded_post", "static_fp8", "rs_fp8_block", "mla_ag_fp8"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (for profiler runs)")
    ap.add_argument("--no-next", action="store_true",
                    help="skip timing the entry points beyond the step")
    ap.add_argument("--out", default=None, help="also write the JSON line to this file")
    return ap.parse_args()


def source_digest() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when it is missing or was taken on other kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != source_digest():
        return None
    return t.get("bytes_per_launch")


class Part:
    """One launch of the step: inputs resident on the GPU, outputs allocated."""

    def __init__(self, name, fn, wl, torch, dev):
        self.name = name
        self.w = w = wl.WORKLOADS[name]
        t0 = time.perf_counter()
        self.cpu = wl.make_inputs(w)
        if w.kind == "qk":
            self.qkv = self.cpu.qkv.to(dev)
            self.wq = self.cpu.q_weight.to(dev)
            self.wk = self.cpu.k_weight.to(dev)
            self.q_out = torch.empty(w.T, w.q_size, dtype=torch.bfloat16, device=dev)
            self.k_out = torch.empty(w.T, w.kv_size, dtype=torch.bfloat16, device=dev)
            self.var_in = None
            if w.tp_world > 1:
                # Each shard's local means (the pre stage), summed as the
                # all-reduce between the two stages would; prepared once, untimed.
                shards = [self.qkv] + [s.to(dev) for s in self.cpu.shards]
                self.var_in = sum(fn.qk_rmsnorm_var(s, w.q_size, w.kv_size) for s in shards)
                del shards
            self.call = lambda: fn.qk_rmsnorm(self.qkv, w.q_size, w.kv_size, self.wq, self.wk,
                                              w.eps, tp_world=w.tp_world, var_in=self.var_in,
                                              q_out=self.q_out, k_out=self.k_out)
        elif w.kind == "sharded":
            self.x = self.cpu.qkv.to(dev)
            self.weight = self.cpu.q_weight.to(dev)
            self.out = torch.empty(w.T, w.q_size, dtype=torch.bfloat16, device=dev)
            shards = [self.x] + [s.to(dev) for s in self.cpu.shards]
            self.var_in = sum(fn.sharded_rmsnorm_var(s, H=w.q_size) for s in shards)
            del shards
            self.call = lambda: fn.sharded_rmsnorm(self.x, self.weight, w.eps, w.tp_world,
                                                   self.var_in, out=self.out, H=w.q_size)
        elif w.kind == "mla":
            self.rows = self.cpu.qkv.to(dev)
            self.gx, self.gy = self.cpu.q_weight.to(dev), self.cpu.k_weight.to(dev)
            self.y = torch.empty(w.T, w.kv_size, dtype=torch.bfloat16, device=dev)
            self.quant = torch.empty(w.T, w.q_size, dtype=torch.float8_e4m3fn, device=dev)
            self.scale = torch.empty(w.T, w.q_size // w.group_size, dtype=torch.float32,
                                     device=dev)
            self.call = lambda: fn.ag_dual_rmsnorm(self.rows, w.q_size, w.kv_size, self.gx,
                                                   self.gy, w.eps, w.eps, quant=True,
                                                   want_x=False, y_norm_out=self.y,
                                                   quant_out=self.quant, scale_out=self.scale)
        else:
            self.parts = [p.to(dev) for p in self.cpu.partials]
            self.res = self.cpu.residual.to(dev)
            self.weight = self.cpu.weight.to(dev)
            self.res_out = torch.empty_like(self.res)
            self.quant = torch.empty(w.T, w.H, dtype=torch.float8_e4m3fn, device=dev)
            if w.kind == "quant_token":
                self.scale = torch.empty(w.T, dtype=torch.float32, device=dev)
                f = fn.fused_add_rmsnorm_quant_fp8
            elif w.kind in ("quant_block", "rs"):
                self.scale = torch.empty(w.T, w.H // w.group_size, dtype=torch.float32,
                                         device=dev)
                f = fn.fused_add_rmsnorm_quant_fp8_block
            if w.kind == "quant_static":
                self.factor = torch.tensor([w.static_scale], dtype=torch.float32, device=dev)
                self.call = lambda: fn.fused_add_rmsnorm_quant_fp8_static(
                    self.parts, self.res, self.weight, self.factor, w.eps, norm_out=None,
                    residual_out=self.res_out, quant_out=self.quant)
            elif w.kind == "rs":
                self.add_in = self.cpu.add_in.to(dev)
                self.call = lambda: fn.fused_rs_epilogue(
                    w.pattern, self.parts, w.token_offset, self.res, self.weight, w.eps,
                    add_in=self.add_in, residual_out=self.res_out, quant_out=self.quant,
                    scale_out=self.scale)
            else:
                self.call = lambda: f(self.parts, self.res, self.weight, w.eps, norm_out=None,
                                      residual_out=self.res_out, quant_out=self.quant,
                                      scale_out=self.scale)
        self.bytes = w.algorithmic_bytes()
        log(f"[bench] {name}: {w.description}; {self.bytes / 1e6:.1f} MB per launch "
            f"(inputs drawn in {time.perf_counter() - t0:.1f} s)")


def cpu_baseline(parts, min_seconds=10.0, max_reps=8):
    """The oracle, untuned, on full steps of the same host-resident inputs,
    repeated until about min_seconds of host time have been spent."""
    import numpy as np

    import oracle
    from residual_add_rmsnorm_amd import workloads as wl

    calls = []
    for p in parts:
        w = p.w
        if w.kind == "qk":
            rows, wq, wk = wl.bits(p.cpu.qkv), wl.bits(p.cpu.q_weight), wl.bits(p.cpu.k_weight)
            var = None if p.var_in is None else p.var_in.cpu().numpy().astype(np.float32)
            calls.append((p, lambda w=w, rows=rows, wq=wq, wk=wk, var=var: oracle.qk_rmsnorm(
                rows, w.q_size, w.kv_size, wq, wk, w.eps, w.tp_world, var)))
        else:
            args = ([wl.bits(x) for x in p.cpu.partials], wl.bits(p.cpu.residual),
                    wl.bits(p.cpu.weight), w.eps)
            quant = "token" if w.kind == "quant_token" else "block"
            calls.append((p, lambda args=args, quant=quant: oracle.fused_add_rmsnorm(
                *args, quant=quant, want_norm=False)))
    step_bytes = sum(p.bytes for p in parts)
    total_s, reps = 0.0, 0
    while reps < max_reps and (reps == 0 or total_s < min_seconds):
        for p, f in calls:
            t0 = time.perf_counter()
            f()
            dt = time.perf_counter() - t0
            total_s += dt
            if reps == 0:
                log(f"[bench] cpu oracle {p.name}: {dt:.2f} s")
        reps += 1
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": round(reps * step_bytes / total_s / 1e9, 3), "unit": "GB/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{reps} full steps (all four launches, every token) on the host, "
                      f"{total_s:.1f} s in all; {model}, {os.cpu_count()} logical CPUs visible"}


def ceilings(fn, torch, dev, reps=10):
    """GB/s of the library's plain streaming kernels on this GPU: a 2 GiB read
    and a 1 GiB copy (read + write counted), inputs out of cache. They are the
    achievable ceiling next to the published 8 TB/s; the copy, of known size,
    also calibrates the FETCH_SIZE / WRITE_SIZE counters under rocprofv3."""
    out = {}
    src = torch.ones(1 << 30, dtype=torch.bfloat16, device=dev)      # 2 GiB
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    cs, cd = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev), \
        torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)       # 1 GiB each
    for name, f, nbytes in (("read_GBs", lambda: fn.stream_read(src, sink), src.nbytes),
                            ("copy_GBs", lambda: fn.stream_copy(cs, cd), 2 * cs.nbytes)):
        for _ in range(2):
            f()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            f()
        b.record()
        torch.cuda.synchronize()
        sec = a.elapsed_time(b) / 1e3 / reps
        out[name] = round(nbytes / sec / 1e9, 1)
    del src, cs, cd
    log(f"[bench] streaming ceilings: read {out['read_GBs']} GB/s, copy {out['copy_GBs']} GB/s")
    return out


def capture(torch, fn_step):
    """Captures fn_step() in a HIP graph (after one run on the capture stream to
    warm the library's launch-shape cache). No memset nodes: the kernels write
    every output element themselves."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn_step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn_step()
    return g


def latency_shapes(fn, wl, torch, dev, calls=50, reps=20):
    """GPU time per call of the two small workloads (16 x 1024 with P=1;
    128 x 7168 with P=4): `calls` back-to-back calls captured in one graph and
    replayed. Their inputs fit in the last-level cache, so these are latency
    figures, not HBM bandwidth."""
    out = {}
    for name in ("tiny", "decode"):
        w = wl.WORKLOADS[name]
        inp = wl.make_inputs(w)
        parts = [p.to(dev) for p in inp.partials]
        res, weight = inp.residual.to(dev), inp.weight.to(dev)
        norm, rout = torch.empty_like(res), torch.empty_like(res)

        def many():
            for _ in range(calls):
                fn.fused_add_rmsnorm(parts, res, weight, w.eps, norm_out=norm, residual_out=rout)
        g = capture(torch, many)
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (reps * calls)
        out[name] = {"T": w.T, "H": w.H, "P": w.P, "us_per_call": round(us, 2),
                     "GB/s": round(w.algorithmic_bytes() / us / 1e3, 1), "cache_resident": True}
        log(f"[bench] {name}: {us:.2f} us per call (graph replay, cache-resident)")
    return out


def next_rows(parts, flush, torch, K):
    """Each further entry point timed alone: K launches, each preceded by an
    untimed launch of `flush` (over 1 GB) so that its inputs are not in the
    last-level cache, and bracketed by HIP events on the launch stream."""
    out = {}
    for p in parts:
        for _ in range(2):
            p.call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        for s, e in ev:
            flush.call()
            s.record()
            p.call()
            e.record()
        torch.cuda.synchronize()
        us = sum(s.elapsed_time(e) for s, e in ev) / K * 1e3
        gbs = p.bytes / us / 1e3
        out[p.name] = {"workload": p.w.description, "us": round(us, 2), "GB/s": round(gbs, 1),
                       "frac": round(gbs / HBM_PEAK_GBS, 4),
                       "tokens/s": round(p.w.T / us * 1e6),
                       "algorithmic_bytes_per_launch": p.bytes}
        log(f"[bench] next {p.name}: {us:.1f} us, {gbs:.1f} GB/s "
            f"({100 * gbs / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f})")
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: libfusednorm runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); the multi-GPU exchange is not implemented, so there is "
              "no figure at more than one GPU.", file=sys.stderr)
        sys.exit(2)

    import torch

    from residual_add_rmsnorm_amd import fusednorm as fn
    from residual_add_rmsnorm_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] {torch.cuda.get_device_name(dev)}; library {fn.library_path()}")
    parts = [Part(n, fn, wl, torch, dev) for n in STEP]
    torch.cuda.synchronize()

    def step():
        for p in parts:
            p.call()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps

    # Pass 1, eager: each launch bracketed by HIP events on the launch stream;
    # gives the per-launch times and the dominant kernel's roofline.
    ev = {p.name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(K)] for p in parts}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        for p in parts:
            s, e = ev[p.name][k]
            s.record()
            p.call()
            e.record()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) / K * 1e3

    # Pass 2, the reported throughput: the step captured once in a HIP graph,
    # K replays bracketed by synchronisation.
    g = capture(torch, step)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    step_bytes = sum(p.bytes for p in parts)
    step_tokens = sum(p.w.T for p in parts)
    ms_per_step = wall / K * 1e3
    per = {}
    for p in parts:
        us = sum(s.elapsed_time(e) for s, e in ev[p.name]) / K * 1e3
        per[p.name] = {"us": round(us, 2), "GB/s": round(p.bytes / us / 1e3, 1),
                       "frac": round(p.bytes / us / 1e3 / HBM_PEAK_GBS, 4),
                       "tokens/s": round(p.w.T / us * 1e6)}
        log(f"[bench] {p.name}: {us:.1f} us, {per[p.name]['GB/s']} GB/s "
            f"({100 * per[p.name]['frac']:.1f}% of {HBM_PEAK_GBS:.0f})")
    dom = next(p for p in parts if p.name == DOMINANT)
    dom_gbs = per[DOMINANT]["GB/s"]
    traffic = measured_traffic()

    result = {
        "metric": "achieved HBM GB/s (% of MI355X peak) and tokens/s, fused add+RMSNorm(+FP8)",
        "value": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded CPU draws, bf16 inputs resident in HBM)",
        "config": {
            "workload": "fused TP epilogue step: prefill per-token e4m3 T=8192 H=8192 P=8 + "
                        "MiniMax QK T=4096 local means + block e4m3 T=16384 H=7168 P=2 + "
                        "MiniMax QK T=4096 with 4 shard means",
            "launches": STEP,
            "bytes_per_step": step_bytes,
            "tokens_per_step": step_tokens,
            "storage": "bf16 in; bf16 and OCP e4m3 out",
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100 * step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(step_tokens / (ms_per_step / 1e3)),
        "per_launch": per,
        "roofline": {
            "bound": "hbm", "kernel": "fused_epilogue_kernel (per-token e4m3)",
            "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dom.bytes,
        },
        "eager_ms_per_step": round(eager_ms, 4),
        "eager_GBs": round(step_bytes / (eager_ms / 1e3) / 1e9, 1),
        "hbm_ceiling": ceilings(fn, torch, dev),
        "latency_shapes": latency_shapes(fn, wl, torch, dev),
    }
    if not args.no_next:
        del g
        extra = [Part(n, fn, wl, torch, dev) for n in NEXT]
        result["next_rows"] = next_rows(extra, dom, torch, K)
        del extra
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(parts)
    line = json.dumps(result)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")
    print(line, flush=True)


if __name__ == "__main__":
    main()
