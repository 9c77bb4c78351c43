"""Benchmark: shifted local-window attention TFLOP/s on one MI355X.

One step = one pass of the hot path over the workload's block cycle: one
basa_window_attn_fwd call per shift of the cycle, on the same q, k, v resident in HBM.
The dense baseline (basa_full_attn_fwd, same kernel, window = whole grid) is timed
beside it for the measured-vs-theoretical speedup. Timing follows the paper's latency
protocol (§4 / App. A.2 "Implementation and latency measurement"): warm-up first, device
events around the timed region, synchronisation before reading them.

Prints ONE JSON line (rank 0). Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--cold] [--pool P] [--route]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_attention_dit_amd.build import kernel_hash  # noqa: E402
from sparse_attention_dit_amd.configs import BY_NAME  # noqa: E402
from sparse_attention_dit_amd.profiling import traffic_json_name  # noqa: E402

# MI355X published peaks: dense bf16 MFMA 2.5 PFLOP/s (256 CU x 2.4 GHz x 4096 flop/clk),
# dense fp32 MFMA 157.3 TFLOP/s (256 CU x 2.4 GHz x 256 flop/clk; the fp32 kernel's products
# run on v_mfma_f32_32x32x2_f32), HBM3E 8 TB/s.
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "flux-4096-256x256-w32"


class ClockSampler:
    """Samples the GPU core clock (the current level of the amdgpu driver's pp_dpm_sclk file)
    every `period` seconds on a background thread. Only used when exactly one card is
    visible; otherwise reports nothing. Reading the file does not touch the GPU queues."""

    def __init__(self, period: float = 0.01):
        import glob
        import threading
        files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = files[0] if len(files) == 1 else None
        self.period = period
        self.samples = []  # (perf_counter time, MHz)
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True) if self.path else None

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            mhz = self._read()
            if mhz is not None:
                self.samples.append((time.perf_counter(), mhz))
            time.sleep(self.period)

    def start(self):
        if self._thread:
            self._thread.start()
        return self

    def stop(self):
        if self._thread:
            self._stop.set()
            self._thread.join()

    def median(self, t0: float, t1: float):
        vals = sorted(m for t, m in self.samples if t0 <= t <= t1)
        return None if not vals else vals[len(vals) // 2], len(vals)


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this
    workload, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", traffic_json_name(workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def host_info():
    """CPU model, logical CPUs available to this process, physical cores, NumPy version and
    the BLAS library NumPy calls (with its thread count)."""
    import numpy as np
    model, phys = None, set()
    try:
        with open("/proc/cpuinfo") as f:
            cur = {}
            for line in f:
                if ":" in line:
                    key, val = (x.strip() for x in line.split(":", 1))
                    cur[key] = val
                    if key == "model name" and model is None:
                        model = val
                elif cur:
                    phys.add((cur.get("physical id"), cur.get("core id")))
                    cur = {}
            if cur:
                phys.add((cur.get("physical id"), cur.get("core id")))
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = {"library": libs[0].get("internal_api"), "version": libs[0].get("version"),
                    "threads": libs[0].get("num_threads")}
    except Exception:  # pragma: no cover - informational only
        pass
    return {"cpu_model": model, "logical_cpus_available": len(os.sched_getaffinity(0)),
            "physical_cores": len(phys) if phys and None not in next(iter(phys)) else None,
            "numpy": np.__version__, "blas": blas}


def cpu_baseline(w, min_s: float, pool: int = 0, route: bool = False):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload: whole
    (shift, head) slices of the windowed attention (with pooled memory when pool > 0; the
    pooling itself is done once, untimed), in step order and cycling, until at least min_s
    of CPU work."""
    from oracle import basa_oracle as O
    from oracle import memory_oracle as MO
    from oracle import routing_oracle as RO
    from sparse_attention_dit_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - informational only
        threads = None
    t = inputs.draw_qkv((w.batch, 1, w.tokens, w.head_dim), w.dtype, seed=w.seed)
    q, k, v = (t.exact[n] for n in "qkv")
    n_mem = 0
    km = vm = None
    if pool:
        km, vm = MO.pool_kv(k, w.grid, (pool, pool)), MO.pool_kv(v, w.grid, (pool, pool))
        n_mem = km.shape[2]
    routes = {}
    if route:  # routing decisions per shift, outside the timed region
        for s in w.shifts:
            routes[s] = RO.route_top1(RO.window_means(q, w.grid, w.window, s), RO.window_means(k, w.grid, w.window, s),
                                      w.grid, w.window)
    slices, elapsed, keys = 0, 0.0, 0.0
    while elapsed < min_s:
        shift = w.shifts[(slices // w.heads) % len(w.shifts)]
        t0 = time.perf_counter()
        if route:
            RO.routed_attention(q, k, v, routes[shift], w.grid, w.window, shift, km, vm)
        elif pool:
            MO.window_attention_memory(q, k, v, km, vm, w.grid, w.window, shift)
        else:
            O.window_attention(q, k, v, w.grid, w.window, shift)
        elapsed += time.perf_counter() - t0
        slices += 1
        keys += w.window_tokens * (1.0 + (float((routes[shift] >= 0).mean()) if route else 0.0)) + n_mem
    flops = 4 * w.batch * w.tokens * keys * w.head_dim
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": threads if threads is not None else len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "host": host_info(),
        "sample": f"{slices} (shift, head) slices of {w.num_windows} windows each (one step = "
                  f"{len(w.shifts) * w.heads}), fp64 numpy, one head's q/k/v drawn with the workload seed "
                  f"({flops / 1e9:.1f} GFLOP in {elapsed:.1f} s)",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=0.5, help="seconds of untimed steps before the warm-up")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(BY_NAME))
    ap.add_argument("--full-iters", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline leg")
    ap.add_argument("--cold", action="store_true", help="also time HBM-cold launches (L2/MALL flushed between)")
    ap.add_argument("--pool", type=int, default=0,
                    help="with pooled global memory of p x p regions (0: plain windowed attention)")
    ap.add_argument("--route", action="store_true", help="with top-1 true-window routing (radius one)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum CPU work timed for cpu_baseline")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (sharding by head is described, "
              "not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from sparse_attention_dit_amd import _lib, inputs

    w = BY_NAME[args.workload]
    t = inputs.draw_qkv(w.shape, w.dtype, seed=w.seed)
    dev = {}
    for n in "qkv":
        a = t.dev[n]
        if w.dtype == "bf16":
            dev[n] = torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
        else:
            dev[n] = torch.from_numpy(a).to("cuda")
    del t
    out = torch.empty_like(dev["q"])
    stream = torch.cuda.current_stream()
    n_mem = 0
    routed_frac = 0.0
    if args.route:
        # true-window routing (§3.3): per shift, window descriptors, top-1 routing within
        # radius one, then attention over window + routed window (+ memory with --pool)
        n_win = w.num_windows
        qbar = torch.empty((w.batch, w.heads, n_win, w.head_dim), dtype=torch.float32, device="cuda")
        kbar = torch.empty_like(qbar)
        routes = [torch.empty((w.batch, w.heads, n_win), dtype=torch.int32, device="cuda") for _ in w.shifts]
    if args.pool:
        # K/V-pooled global memory (§3.2): pooled once per step (it does not depend on the
        # shift), then every shift's windows attend to window + memory keys
        pool = (args.pool, args.pool)
        n_mem = _lib.pooled_count(w.grid, pool)
        kmem = torch.empty((w.batch, w.heads, n_mem, w.head_dim), dtype=dev["k"].dtype, device="cuda")
        vmem = torch.empty_like(kmem)

    if args.pool or args.route:
        km_ = kmem if args.pool else None
        vm_ = vmem if args.pool else None

        def attend(i, s):
            if args.route:
                _lib.window_means(dev["q"], dev["k"], qbar, kbar, w.grid, w.window, s, stream)
                _lib.route_top1(qbar, kbar, routes[i], w.grid, w.window, 1, stream)
            _lib.window_attn_routed_fwd(dev["q"], dev["k"], dev["v"], routes[i] if args.route else None, km_, vm_,
                                        out, w.grid, w.window, s, stream=stream)

        def step():
            if args.pool:
                _lib.pool_kv(dev["k"], dev["v"], kmem, vmem, w.grid, pool, stream)
            for i, s in enumerate(w.shifts):
                attend(i, s)
    else:
        def step():
            for s in w.shifts:
                _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, w.grid, w.window, s, stream)

    # The GPU's clocks need tens of milliseconds of sustained work to ramp up: before the W
    # warm-up steps, run untimed steps for ~0.5 s (sized from one step), reported as
    # "clock_settle_steps".
    clock = ClockSampler().start()
    settle = 0
    if args.settle_s > 0:
        step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step()
        torch.cuda.synchronize()
        settle = 2 + int(args.settle_s / max(time.perf_counter() - t0, 1e-6))
        for _ in range(settle - 2):
            step()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_timed = time.perf_counter()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    clock.stop()
    # the timed region is short; the clock is taken over it and the last 0.25 s before it,
    # spent on the same steps
    sclk_mhz, sclk_samples = clock.median(t_timed - 0.25, time.perf_counter())
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps
    launches = args.steps * len(w.shifts)
    ms_per_launch = ms_total / launches

    # Sustained rate: the same steps again, one event pair around every launch (or, with
    # --pool/--route, every shift's group of launches), for at least 20 steps and 200 ms of
    # GPU time; reported as the median launch time overall and per shift, with the clock
    # held over that span.
    def launch(i, s):
        if args.pool or args.route:
            attend(i, s)
        else:
            _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, w.grid, w.window, s, stream)

    sus_steps = max(20, int(200.0 / max(ms_per_step, 1e-3)) + 1)
    sus_clock = ClockSampler().start()
    pairs = []
    torch.cuda.synchronize()
    t_sus0 = time.perf_counter()
    for _ in range(sus_steps):
        for i, s in enumerate(w.shifts):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch(i, s)
            e1.record(stream)
            pairs.append((i, e0, e1))
    torch.cuda.synchronize()
    t_sus1 = time.perf_counter()
    sus_clock.stop()
    per_launch = [(i, e0.elapsed_time(e1)) for i, e0, e1 in pairs]
    span_ms = pairs[0][1].elapsed_time(pairs[-1][2])

    def median(xs):
        xs = sorted(xs)
        n = len(xs)
        return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])

    sus_med = median([ms for _, ms in per_launch])
    per_shift_ms = [round(median([ms for j, ms in per_launch if j == i]), 4) for i in range(len(w.shifts))]
    sus_sclk, sus_samples = sus_clock.median(t_sus0, t_sus1)
    pool_ms = None
    if args.pool:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            _lib.pool_kv(dev["k"], dev["v"], kmem, vmem, w.grid, pool, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        pool_ms = e0.elapsed_time(e1) / args.steps

    cold = None
    if args.cold:
        # HBM-cold launches: a 1 GiB write between launches (outside the events) evicts
        # q/k/v from the L2s and the MALL; median over the launches
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        times = []
        for i in range(args.steps):
            flush.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, w.grid, w.window, w.shifts[i % len(w.shifts)],
                                 stream)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        del flush
        med = sorted(times)[len(times) // 2]
        cold = {"window_attn_ms_median": round(med, 4),
                "tflops": round(w.window_flops() / (med * 1e-3) / 1e12, 2),
                "io_gbs": round(w.io_bytes() / (med * 1e-3) / 1e9, 1)}

    # dense baseline: same kernel, window = whole grid
    full_out = torch.empty_like(dev["q"])
    for _ in range(2):
        _lib.full_attn_fwd(dev["q"], dev["k"], dev["v"], full_out, stream)
    torch.cuda.synchronize()
    fs, fe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fs.record(stream)
    for _ in range(args.full_iters):
        _lib.full_attn_fwd(dev["q"], dev["k"], dev["v"], full_out, stream)
    fe.record(stream)
    torch.cuda.synchronize()
    ms_full = fs.elapsed_time(fe) / args.full_iters

    # attention FLOPs per launch: 4*B*h*N*(W*(1 + r) + M)*d, M = memory tokens (0 without
    # --pool), r = fraction of windows with a routed window (0 without --route); with
    # --pool/--route a "launch" is one shift's attention plus its share of the pooling and
    # its routing
    if args.route:
        routed_frac = float(sum((r >= 0).float().mean().item() for r in routes) / len(routes))
    keys_per_query = w.window_tokens * (1.0 + routed_frac) + n_mem
    flops_launch = 4 * w.batch * w.heads * w.tokens * keys_per_query * w.head_dim
    tflops = flops_launch / (ms_per_launch * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    theoretical = w.tokens / keys_per_query
    measured = ms_full / ms_per_launch
    io_gbs = w.io_bytes() / (ms_per_launch * 1e-3) / 1e9

    rec = {
        "metric": "windowed-attn TFLOP/s (frac of bf16 MFMA peak) + measured/theoretical speedup",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_steps": settle,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic N(0,1) q/k/v, seeded",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "grid": list(w.grid), "window": list(w.window), "shifts": [list(s) for s in w.shifts],
                   "tokens": w.tokens, "window_tokens": w.window_tokens, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": measured_traffic(w.name)},
        "speedup": {"full_attn_ms": round(ms_full, 4), "window_attn_ms": round(ms_per_launch, 4),
                    "measured": round(measured, 3), "theoretical": theoretical,
                    "ratio": round(measured / theoretical, 4),
                    "full_attn_tflops": round(w.full_flops() / (ms_full * 1e-3) / 1e12, 2)},
        "per_shift_ms": per_shift_ms,
        "sustained": {
            "steps": sus_steps, "launches": len(per_launch), "span_ms": round(span_ms, 2),
            "median_ms_per_launch": round(sus_med, 4), "mean_ms_per_launch": round(span_ms / len(per_launch), 4),
            "tflops_median": round(flops_launch / (sus_med * 1e-3) / 1e12, 2),
            "frac_median": round(flops_launch / (sus_med * 1e-3) / 1e12 / peak, 4),
            "vs_value": round((flops_launch / (sus_med * 1e-3) / 1e12) / tflops, 4),
            "sclk_mhz_median": sus_sclk, "sclk_samples": sus_samples},
        "io_gbs": round(io_gbs, 1),
        # The core clock under this load: the chip is power-limited, so it runs below the
        # 2.4 GHz the peak assumes; frac_at_clock is achieved / (peak * sclk / 2400).
        "sclk_mhz": None if sclk_mhz is None else {
            "median": sclk_mhz, "samples": sclk_samples, "source": "pp_dpm_sclk",
            "frac_at_clock": round(tflops / (peak * sclk_mhz / 2400.0), 4)},
        "kernel_hash": kernel_hash(),
        "library": _lib.library_info(),
    }
    if args.pool:
        G_bytes = 2 * w.batch * w.heads * n_mem * w.head_dim * (2 if w.dtype == "bf16" else 4)
        rec["config"]["pool"] = [args.pool, args.pool]
        rec["config"]["memory_tokens"] = n_mem
        rec["pool"] = {"pool_ms": round(pool_ms, 4),
                       "pool_gbs": round((w.io_bytes() // 2 + G_bytes) / (pool_ms * 1e-3) / 1e9, 1)}
    if args.route:
        rec["config"]["route"] = {"k": 1, "radius": 1, "routed_fraction": round(routed_frac, 4)}
    if args.pool or args.route:
        rec["roofline"]["traffic"] = None  # counters are taken on the plain windowed launch
    if cold is not None:
        rec["cold"] = cold
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, args.pool, args.route)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
