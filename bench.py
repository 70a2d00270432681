#!/usr/bin/env python3
"""Throughput of the fused TP epilogue and the QK RMSNorm on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
  1. fused_add_rmsnorm_quant_fp8        prefill, T=8192 H=8192 P=8, per-token e4m3
  2. qk_rmsnorm (local means)           MiniMax QK, T=4096, row 8192 = q 6144 | k 1024 | v
  3. fused_add_rmsnorm_quant_fp8_block  T=16384 H=7168 P=2, 1x128 e4m3 groups
  4. qk_rmsnorm (sum of 4 shard means)  as 2, tp_world=4
The launches alternate between the large FP8 passes (>= 1 GB each) and the QK
passes, so no launch of the step finds its inputs in the 256 MB last-level
cache.

Prints ONE JSON line:
  value, ms_per_step  the step's algorithmic bytes (each input read once, each
                      output written once, weights once per launch) over the
                      wall time of a step: the four launches captured once in a
                      HIP graph and replayed K times between synchronisations.
  per_config          every workload alone (the four of the step and the two
                      latency shapes, 16 x 1024 and 128 x 7168): its launches
                      rotate over enough resident copies of its buffers that
                      each launch reads and writes HBM, not the last-level
                      cache (the 16 x 1024 shape fits in the cache whatever the
                      rotation and is labelled so); N launches captured in one
                      graph, HIP events on the launch stream around the
                      replays; us per launch, GB/s, fraction of 8 TB/s,
                      tokens/s; and the same bytes moved on the same buffers
                      by the library's mixed-stream kernel (no arithmetic), the
                      measured ceiling at that read/write mix, with the
                      launch's fraction of it.
  roofline            the dominant kernel (the per-token FP8 prefill) from its
                      per_config timing; traffic from the committed counter
                      summary when it was taken on the current kernel source.
  hbm_ceiling         plain streaming read (2 GiB) and copy (1 GiB) GB/s.
  cpu_baseline        the oracle, as it stands, on every workload of the step
                      and the latency shapes (all host threads), plus the two
                      latency shapes on one thread.
  next_rows           the further entry points, each timed alone like
                      per_config.
  token_sweep         the QK norm (local means) and the MLA epilogue at 1024 to
                      32768 tokens (--sweep, --sweep-tokens choose others),
                      timed like per_config (with the mixed-stream ceiling at
                      every count), with the least-squares fit
                      us = fixed_us + bytes / (stream_GBs * 1e3): the fixed
                      cost of a launch and its streaming rate.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-cpu-baseline] [--no-next]
                    [--no-sweep] [--sweep NAME,...] [--sweep-tokens T,...] [--sweep-only]

--sweep-only prints just {"token_sweep": ...} (a measurement run, not the
benchmark line).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
LLC_BYTES = 256 << 20          # MI355X last-level (Infinity) cache
KERNEL_SRC = os.path.join(ROOT, "residual_add_rmsnorm_amd", "csrc", "fusednorm_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill_fp8_token.json")
STEP = ["prefill_fp8_token", "qk_local", "fp8_block", "qk_sharded"]
LATENCY = ["tiny", "decode"]
DOMINANT = "prefill_fp8_token"
# Entry points beyond the step, each timed alone on its own workload.
NEXT = ["sharded_post", "static_fp8", "rs_fp8_block", "mla_ag_fp8"]
# Workloads timed over token counts for the fixed-cost fit.
SWEEP = ["qk_local", "mla_ag_fp8"]
SWEEP_TOKENS = [1024, 2048, 4096, 8192, 16384, 32768]


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
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the token-count sweep of the QK norm and the MLA epilogue")
    ap.add_argument("--sweep", default=",".join(SWEEP),
                    help="workloads of the token-count sweep (comma-separated)")
    ap.add_argument("--sweep-tokens", default=",".join(map(str, SWEEP_TOKENS)),
                    help="token counts of the sweep (comma-separated)")
    ap.add_argument("--sweep-only", action="store_true",
                    help="run only the token-count sweep and print its JSON (for profiler runs)")
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


def sets_for(working_set: int, min_total: int = 1 << 30, cap: int = 128) -> int:
    """Resident copies of a launch's buffers so that a rotation over them
    touches at least `min_total` bytes (>= 4x the last-level cache)."""
    return max(1, min(cap, math.ceil(min_total / working_set)))


class Runner:
    """One workload's launches: `sets` copies of its buffers resident in HBM,
    launch i using copy i % sets; `call(i)` is the entry point, `mix(i)` the
    library's mixed-stream kernel over the same sources and destinations."""

    def __init__(self, name, fn, wl, torch, dev, T=None, quiet=False):
        self.name = name
        self.w = w = wl.WORKLOADS[name] if T is None else wl.WORKLOADS[name].with_tokens(T)
        t0 = time.perf_counter()
        self.cpu = wl.make_inputs(w)
        self.bytes = w.algorithmic_bytes()
        self.sets = sets_for(self.bytes)
        self.cache_resident = self.bytes * self.sets <= LLC_BYTES
        self.var_in = None
        S = []
        if w.kind == "qk":
            qkv = self.cpu.qkv.to(dev)
            wq, wk = self.cpu.q_weight.to(dev), self.cpu.k_weight.to(dev)
            if w.tp_world > 1:
                # each shard's local means (the pre stage), summed as the
                # all-reduce between the two stages would; prepared once, untimed
                shards = [qkv] + [s.to(dev) for s in self.cpu.shards]
                self.var_in = sum(fn.qk_rmsnorm_var(s, w.q_size, w.kv_size) for s in shards)
                del shards
            for k in range(self.sets):
                src = qkv if k == 0 else qkv.clone()
                S.append(dict(qkv=src, q=torch.empty(w.T, w.q_size, dtype=torch.bfloat16,
                                                     device=dev),
                              k=torch.empty(w.T, w.kv_size, dtype=torch.bfloat16, device=dev)))
            self._call = lambda s: fn.qk_rmsnorm(s["qkv"], w.q_size, w.kv_size, wq, wk, w.eps,
                                                 tp_world=w.tp_world, var_in=self.var_in,
                                                 q_out=s["q"], k_out=s["k"])
            self._mix = lambda s: ([s["qkv"]], [s["q"], s["k"]], (w.q_size + w.kv_size) * 2,
                                   w.row_stride * 2)
        elif w.kind == "sharded":
            x = self.cpu.qkv.to(dev)
            weight = self.cpu.q_weight.to(dev)
            shards = [x] + [s.to(dev) for s in self.cpu.shards]
            self.var_in = sum(fn.sharded_rmsnorm_var(s, H=w.q_size) for s in shards)
            del shards
            for k in range(self.sets):
                S.append(dict(x=x if k == 0 else x.clone(),
                              out=torch.empty(w.T, w.q_size, dtype=torch.bfloat16, device=dev)))
            self._call = lambda s: fn.sharded_rmsnorm(s["x"], weight, w.eps, w.tp_world,
                                                      self.var_in, out=s["out"], H=w.q_size)
            self._mix = lambda s: ([s["x"]], [s["out"]], w.q_size * 2, w.row_stride * 2)
        elif w.kind == "mla":
            rows = self.cpu.qkv.to(dev)
            gx, gy = self.cpu.q_weight.to(dev), self.cpu.k_weight.to(dev)
            for k in range(self.sets):
                S.append(dict(rows=rows if k == 0 else rows.clone(),
                              y=torch.empty(w.T, w.kv_size, dtype=torch.bfloat16, device=dev),
                              q=torch.empty(w.T, w.q_size, dtype=torch.float8_e4m3fn, device=dev),
                              s=torch.empty(w.T, w.q_size // w.group_size, dtype=torch.float32,
                                            device=dev)))
            self._call = lambda s: fn.ag_dual_rmsnorm(
                s["rows"], w.q_size, w.kv_size, gx, gy, w.eps, w.eps, quant=True, want_x=False,
                y_norm_out=s["y"], quant_out=s["q"], scale_out=s["s"])
            # the 48-byte scale rows are not a whole number of 16-byte vectors:
            # the ceiling moves everything else
            self._mix = lambda s: ([s["rows"]], [s["y"], s["q"]], (w.q_size + w.kv_size) * 2,
                                   w.row_stride * 2)
        else:
            parts0 = [p.to(dev) for p in self.cpu.partials]
            res0 = self.cpu.residual.to(dev)
            weight = self.cpu.weight.to(dev)
            add0 = self.cpu.add_in.to(dev) if w.kind == "rs" else None
            for k in range(self.sets):
                s = dict(parts=parts0 if k == 0 else [p.clone() for p in parts0],
                         res=res0 if k == 0 else res0.clone(),
                         add=add0 if k == 0 or add0 is None else add0.clone(),
                         rout=torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev))
                if w.kind == "norm":
                    s["norm"] = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev)
                else:
                    s["q"] = torch.empty(w.T, w.H, dtype=torch.float8_e4m3fn, device=dev)
                    if w.kind == "quant_token":
                        s["s"] = torch.empty(w.T, dtype=torch.float32, device=dev)
                    elif w.kind in ("quant_block", "rs"):
                        s["s"] = torch.empty(w.T, w.H // w.group_size, dtype=torch.float32,
                                             device=dev)
                S.append(s)
            if w.kind == "norm":
                self._call = lambda s: fn.fused_add_rmsnorm(s["parts"], s["res"], weight, w.eps,
                                                            norm_out=s["norm"],
                                                            residual_out=s["rout"])
                dsts = lambda s: [s["norm"], s["rout"]]
            elif w.kind == "quant_token":
                self._call = lambda s: fn.fused_add_rmsnorm_quant_fp8(
                    s["parts"], s["res"], weight, w.eps, norm_out=None, residual_out=s["rout"],
                    quant_out=s["q"], scale_out=s["s"])
                dsts = lambda s: [s["rout"], s["q"]]          # 4-byte scale rows not moved
            elif w.kind == "quant_block":
                self._call = lambda s: fn.fused_add_rmsnorm_quant_fp8_block(
                    s["parts"], s["res"], weight, w.eps, norm_out=None, residual_out=s["rout"],
                    quant_out=s["q"], scale_out=s["s"])
                dsts = lambda s: [s["rout"], s["q"], s["s"]]
            elif w.kind == "quant_static":
                factor = torch.tensor([w.static_scale], dtype=torch.float32, device=dev)
                self._call = lambda s: fn.fused_add_rmsnorm_quant_fp8_static(
                    s["parts"], s["res"], weight, factor, w.eps, norm_out=None,
                    residual_out=s["rout"], quant_out=s["q"])
                dsts = lambda s: [s["rout"], s["q"]]
            else:  # reduce-scatter epilogue on this GPU's token slice
                self._call = lambda s: fn.fused_rs_epilogue(
                    w.pattern, s["parts"], w.token_offset, s["res"], weight, w.eps,
                    add_in=s["add"], residual_out=s["rout"], quant_out=s["q"], scale_out=s["s"])
                dsts = lambda s: [s["rout"], s["q"], s["s"]]
            if w.kind == "rs":
                lo, hi = w.token_offset, w.token_offset + w.T
                self._mix = lambda s: ([p[lo:hi] for p in s["parts"]] + [s["add"], s["res"]],
                                       dsts(s), w.H * 2, w.H * 2)
            else:
                self._mix = lambda s: (list(s["parts"]) + [s["res"]], dsts(s), w.H * 2, w.H * 2)
        self.S = S
        srcs, dsts_, row, _ = self._mix(S[0])
        self.mix_bytes = w.T * (len(srcs) * row + sum(d.nbytes // w.T for d in dsts_))
        self.fn = fn
        if not quiet:
            log(f"[bench] {name}: {w.description}; {self.bytes / 1e6:.1f} MB per launch, "
                f"{self.sets} resident cop{'y' if self.sets == 1 else 'ies'} "
                f"(inputs drawn in {time.perf_counter() - t0:.1f} s)")

    def call(self, i=0):
        return self._call(self.S[i % self.sets])

    def mix(self, i=0):
        srcs, dsts, row, stride = self._mix(self.S[i % self.sets])
        self.fn.stream_mix(srcs, dsts, self.w.T, row, stride)


def capture(torch, fn_body):
    """Captures fn_body() in a HIP graph (after one run on the capture stream to
    warm the library's launch-shape cache). No memset nodes: the kernels write
    every output element themselves."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn_body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn_body()
    return g


def time_launches(torch, launch, n, reps, warm=1):
    """us per launch: `n` launches launch(0..n-1) captured in one graph, the
    graph replayed `reps` times between two HIP events on the stream the
    launches run on (the figure includes the graph's gaps between kernels)."""
    g = capture(torch, lambda: [launch(i) for i in range(n)])
    for _ in range(warm):
        g.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * n)


def measure(r, torch, launches=50):
    """One workload alone, and the mixed-stream ceiling on its buffers."""
    n = r.sets * math.ceil(10 / r.sets)          # whole rotations, at least 10 launches
    reps = math.ceil(launches / n)
    us = time_launches(torch, r.call, n, reps)
    mix_us = time_launches(torch, r.mix, n, reps)
    gbs = r.bytes / us / 1e3
    mix_gbs = r.mix_bytes / mix_us / 1e3
    out = {"workload": r.w.description, "T": r.w.T, "algorithmic_bytes_per_launch": r.bytes,
           "resident_copies": r.sets, "launches_timed": n * reps, "cache_resident": r.cache_resident,
           "us": round(us, 2), "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
           "tokens/s": round(r.w.T / us * 1e6),
           "mixed_ceiling": {"bytes_per_launch": r.mix_bytes, "us": round(mix_us, 2),
                             "GB/s": round(mix_gbs, 1)},
           "frac_of_achievable": round(gbs / mix_gbs, 4)}
    log(f"[bench] {r.name}: {us:.2f} us, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of "
        f"{HBM_PEAK_GBS:.0f}); same bytes, no arithmetic: {mix_us:.2f} us, {mix_gbs:.1f} GB/s; "
        f"{100 * gbs / mix_gbs:.1f}% of that{' (cache-resident)' if r.cache_resident else ''}")
    return out


def token_sweep(fn, wl, torch, dev, names=SWEEP, tokens=SWEEP_TOKENS):
    """Each workload of `names` at every count of `tokens`, timed like
    per_config (rotating resident copies, N launches in a graph) beside its
    mixed-stream ceiling on the same buffers, and the least-squares line
    through (bytes, us): the intercept is the launch's fixed cost, the slope
    the rate at which it streams its bytes."""
    out = {}
    for name in names:
        pts = []
        for T in tokens:
            r = Runner(name, fn, wl, torch, dev, T=T, quiet=True)
            n = r.sets * math.ceil(10 / r.sets)
            us = time_launches(torch, r.call, n, math.ceil(50 / n))
            mix_us = time_launches(torch, r.mix, n, math.ceil(50 / n))
            pts.append({"T": T, "bytes": r.bytes, "resident_copies": r.sets, "us": round(us, 2),
                        "GB/s": round(r.bytes / us / 1e3, 1),
                        "mixed_ceiling_us": round(mix_us, 2),
                        "mixed_ceiling_GBs": round(r.mix_bytes / mix_us / 1e3, 1)})
            log(f"[bench] {name} at {T} tokens: {us:.2f} us; same bytes, no arithmetic: "
                f"{mix_us:.2f} us")
            del r
            torch.cuda.empty_cache()
        fixed, rate = fit_fixed_and_rate([p["bytes"] for p in pts], [p["us"] for p in pts])
        out[name] = {"points": pts, "fixed_us": round(fixed, 2), "stream_GBs": round(rate, 1)}
        log(f"[bench] {name} over {tokens[0]}..{tokens[-1]} tokens: "
            f"{fixed:.2f} us fixed + bytes at {rate:.1f} GB/s")
    return out


def fit_fixed_and_rate(nbytes, us):
    """Least-squares line us = fixed + nbytes / (rate * 1e3): returns (fixed
    in us, rate in GB/s)."""
    n = len(nbytes)
    mx, my = sum(nbytes) / n, sum(us) / n
    slope = sum((x - mx) * (y - my) for x, y in zip(nbytes, us)) / \
        sum((x - mx) ** 2 for x in nbytes)
    return my - slope * mx, 1.0 / slope / 1e3


def ceilings(fn, torch, dev, reps=10):
    """GB/s of the library's plain streaming kernels on this GPU: a 2 GiB read
    and a 1 GiB copy (read + write counted), inputs out of cache. The copy, of
    known size, also calibrates the FETCH_SIZE / WRITE_SIZE counters under
    rocprofv3."""
    out = {}
    src = torch.ones(1 << 30, dtype=torch.bfloat16, device=dev)      # 2 GiB
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    cs, cd = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev), \
        torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)       # 1 GiB each
    for name, f, nbytes in (("read_GBs", lambda i: fn.stream_read(src, sink), src.nbytes),
                            ("copy_GBs", lambda i: fn.stream_copy(cs, cd), 2 * cs.nbytes)):
        us = time_launches(torch, f, reps, 1)
        out[name] = round(nbytes / us / 1e3, 1)
    del src, cs, cd
    log(f"[bench] streaming ceilings: read {out['read_GBs']} GB/s, copy {out['copy_GBs']} GB/s")
    return out


def _oracle_call(r, wl, oracle, np):
    w = r.w
    if w.kind == "qk":
        rows, wq, wk = wl.bits(r.cpu.qkv), wl.bits(r.cpu.q_weight), wl.bits(r.cpu.k_weight)
        var = None if r.var_in is None else r.var_in.cpu().numpy().astype(np.float32)
        return lambda: oracle.qk_rmsnorm(rows, w.q_size, w.kv_size, wq, wk, w.eps, w.tp_world,
                                         var)
    args = ([wl.bits(x) for x in r.cpu.partials], wl.bits(r.cpu.residual),
            wl.bits(r.cpu.weight), w.eps)
    if w.kind == "norm":
        return lambda: oracle.fused_add_rmsnorm(*args, quant=None, want_norm=True)
    quant = "token" if w.kind == "quant_token" else "block"
    return lambda: oracle.fused_add_rmsnorm(*args, quant=quant, want_norm=False)


def _time_cpu(f, min_seconds, max_reps):
    total, reps = 0.0, 0
    while reps < max_reps and (reps == 0 or total < min_seconds):
        t0 = time.perf_counter()
        f()
        total += time.perf_counter() - t0
        reps += 1
    return total, reps


def cpu_baseline(runners, min_seconds=2.0, max_reps=50):
    """The oracle, untuned, on the same host-resident inputs: each workload of
    the step and the two latency shapes with all host threads (OpenMP over
    tokens), repeated for about min_seconds each; the latency shapes also on
    one thread."""
    import ctypes

    import numpy as np

    import oracle
    from residual_add_rmsnorm_amd import workloads as wl

    per = {}
    step_s = 0.0
    threads = oracle.max_threads()
    for name, r in runners.items():
        f = _oracle_call(r, wl, oracle, np)
        total, reps = _time_cpu(f, min_seconds, max_reps)
        s = total / reps
        per[name] = {"s_per_launch": round(s, 5), "GB/s": round(r.bytes / s / 1e9, 3),
                     "tokens/s": round(r.w.T / s), "runs": reps, "threads": threads}
        if name in STEP:
            step_s += s
        log(f"[bench] cpu oracle {name}: {s * 1e3:.2f} ms per launch ({reps} runs, "
            f"{threads} threads), {r.bytes / s / 1e9:.3f} GB/s")
    gomp = ctypes.CDLL("libgomp.so.1")       # the OpenMP runtime the oracle runs on
    gomp.omp_set_num_threads(1)
    try:
        assert oracle.max_threads() == 1
        for name in LATENCY:
            r = runners[name]
            total, reps = _time_cpu(_oracle_call(r, wl, oracle, np), min_seconds / 2, max_reps)
            s = total / reps
            per[name]["one_thread"] = {"s_per_launch": round(s, 6),
                                       "GB/s": round(r.bytes / s / 1e9, 3),
                                       "tokens/s": round(r.w.T / s), "runs": reps}
            log(f"[bench] cpu oracle {name}, one thread: {s * 1e3:.3f} ms per launch")
    finally:
        gomp.omp_set_num_threads(threads)
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name"))
    except (OSError, StopIteration):
        pass
    step_bytes = sum(runners[n].bytes for n in STEP)
    return {"value": round(step_bytes / step_s / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"every workload of the step run whole on the host (all tokens), each "
                      f"repeated for about {min_seconds:.0f} s; value = the step's bytes over "
                      f"the sum of its launches' mean times; {model}, {os.cpu_count()} logical "
                      f"CPUs visible, {threads} OpenMP threads",
            "per_config": per}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: libfusednorm runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); the multi-GPU exchange is not implemented, so there is "
              "no figure at more than one GPU.", file=sys.stderr)
        sys.exit(2)

    from residual_add_rmsnorm_amd import workloads as wl

    names = [n for n in args.sweep.split(",") if n]
    bad = [n for n in names if n not in wl.WORKLOADS]
    try:
        tokens = [int(t) for t in args.sweep_tokens.split(",") if t]
    except ValueError:
        tokens = []
    if bad or not names or not tokens or min(tokens) < 1:
        print(f"bench.py: --sweep needs known workloads ({', '.join(wl.WORKLOADS)}) and "
              f"--sweep-tokens positive counts (got {args.sweep!r}, {args.sweep_tokens!r})",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from residual_add_rmsnorm_amd import fusednorm as fn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] {torch.cuda.get_device_name(dev)}; library {fn.library_path()}")
    if args.sweep_only:
        line = json.dumps({"token_sweep": token_sweep(fn, wl, torch, dev, names, tokens)})
        if args.out:
            with open(args.out, "w") as f:
                f.write(line + "\n")
        print(line, flush=True)
        return
    runners = {n: Runner(n, fn, wl, torch, dev) for n in STEP + LATENCY}
    torch.cuda.synchronize()
    parts = [runners[n] for n in STEP]

    def step():
        for p in parts:
            p.call()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps

    # The reported throughput: the step captured once in a HIP graph, K replays
    # bracketed by synchronisation.
    g = capture(torch, step)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del g
    step_bytes = sum(p.bytes for p in parts)
    ms_per_step = wall / K * 1e3
    log(f"[bench] step: {ms_per_step:.4f} ms, {step_bytes / (ms_per_step / 1e3) / 1e9:.1f} GB/s")

    per = {n: measure(runners[n], torch) for n in STEP + LATENCY}
    dom = per[DOMINANT]
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
        "dtype": "bf16",
        "data": "synthetic (seeded CPU draws, bf16 inputs resident in HBM)",
        "config": {
            "workload": "fused TP epilogue step: prefill per-token e4m3 T=8192 H=8192 P=8 + "
                        "MiniMax QK T=4096 local means + block e4m3 T=16384 H=7168 P=2 + "
                        "MiniMax QK T=4096 with 4 shard means",
            "launches": STEP,
            "bytes_per_step": step_bytes,
            "storage": "bf16 in; bf16 and OCP e4m3 out; fp32 arithmetic",
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100 * step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 2),
        "per_config": per,
        "roofline": {
            "bound": "hbm", "kernel": "fused_epilogue_kernel (per-token e4m3 prefill)",
            "achieved": dom["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": dom["frac"], "traffic": traffic,
            "algorithmic_bytes_per_launch": dom["algorithmic_bytes_per_launch"],
            "us_per_launch": dom["us"],
            "timing": f"{dom['launches_timed']} back-to-back launches in a HIP graph, events on "
                      "the launch stream around the replays",
            "mixed_ceiling_GBs": dom["mixed_ceiling"]["GB/s"],
            "frac_of_achievable": dom["frac_of_achievable"],
        },
        "hbm_ceiling": ceilings(fn, torch, dev),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(runners)
    del parts, runners
    torch.cuda.empty_cache()
    if not args.no_next:
        result["next_rows"] = {}
        for n in NEXT:
            r = Runner(n, fn, wl, torch, dev)
            result["next_rows"][n] = measure(r, torch)
            del r
            torch.cuda.empty_cache()
    if not args.no_sweep:
        result["token_sweep"] = token_sweep(fn, wl, torch, dev, names, tokens)
    line = json.dumps(result)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")
    print(line, flush=True)


if __name__ == "__main__":
    main()
