"""rocprofv3 helpers behind the text summaries kept in ``profiles/``.

``run``: the program a counter pass profiles. It launches one kernel of the hot path
(windowed or dense attention on a workload's seeded inputs) or, as the calibration, a
plain device-to-device copy of known size, a fixed number of times.

``kernel-stats``: turns the CSV of a ``rocprofv3 --kernel-trace --stats`` run of bench.py
into a markdown summary: per-launch durations of the attention kernel, split into the
windowed launches and the dense baseline launches by their order (bench.py makes the
dense launches last: 2 untimed + --full-iters timed).

``traffic``: turns four ``rocprofv3 --pmc`` passes (FETCH_SIZE and WRITE_SIZE over the
windowed kernel, the same two over the copy) into HBM bytes per launch. Each counter is
scaled by what it reads for the copy, whose true traffic is known: factor = bytes moved
/ (counter KiB * 1024). Writes ``<kernel>.<workload>.traffic.json`` (read by bench.py,
keyed by the kernel-source digest) and a markdown summary beside it.

Usage (inside the profiler, then on the CSV it wrote):
  python3 -m sparse_attention_dit_amd.profiling run --what window --workload NAME --iters 4
  python3 -m sparse_attention_dit_amd.profiling kernel-stats --dir D --dense 7 --cmd "..." --out F
  python3 -m sparse_attention_dit_amd.profiling traffic --fetch D1 --write D2 --copy-fetch D3 \\
      --copy-write D4 --workload NAME --cmd "..." --out-dir profiles
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

ATTN_KERNEL = "win_attn_bf16_kernel"
COPY_BYTES = 256 << 20  # calibration copy: 256 MiB read + 256 MiB written per launch


def traffic_json_name(workload: str) -> str:
    return f"{ATTN_KERNEL}.{workload}.traffic.json"


# ------------------------------------------------------------------ profiled program
def _run(what: str, workload: str, iters: int) -> None:
    import numpy as np
    import torch

    from sparse_attention_dit_amd import _lib, inputs
    from sparse_attention_dit_amd.configs import BY_NAME

    if what == "copy":
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(iters):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy: {iters} x {COPY_BYTES} bytes", flush=True)
        return
    w = BY_NAME[workload]
    t = inputs.draw_qkv(w.shape, w.dtype, seed=w.seed)
    if w.dtype == "bf16":
        dev = {n: torch.from_numpy(t.dev[n].view(np.int16)).to("cuda").view(torch.bfloat16) for n in "qkv"}
    else:
        dev = {n: torch.from_numpy(t.dev[n]).to("cuda") for n in "qkv"}
    out = torch.empty_like(dev["q"])
    for _ in range(iters):
        if what == "window":
            for s in w.shifts:
                _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, w.grid, w.window, s)
        else:
            _lib.full_attn_fwd(dev["q"], dev["k"], dev["v"], out)
    torch.cuda.synchronize()
    print(f"{what}: {workload}, {iters} iterations", flush=True)


# ------------------------------------------------------------------ CSV readers
def _find_csv(directory: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    return hits[0]


def _kernel_rows(directory: str):
    """Dispatches of the attention kernel from a kernel-trace CSV, in dispatch order."""
    rows = []
    with open(_find_csv(directory, "kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            if ATTN_KERNEL in r["Kernel_Name"]:
                rows.append(r)
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def _counter_per_dispatch(directory: str, counter: str, kernel_substr: str, grid: int | None = None):
    """Mean and count of a counter's per-dispatch value over the matching dispatches."""
    vals = []
    with open(_find_csv(directory, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or kernel_substr not in r["Kernel_Name"]:
                continue
            if grid is not None and int(r["Grid_Size"]) != grid:
                continue
            vals.append(float(r["Counter_Value"]))
    if not vals:
        raise ValueError(f"no {counter} rows for kernels matching {kernel_substr!r} in {directory}")
    return statistics.fmean(vals), len(vals)


def _stats_table(durations_ns):
    d = sorted(durations_ns)
    return {"calls": len(d), "avg_us": statistics.fmean(d) / 1e3, "median_us": statistics.median(d) / 1e3,
            "min_us": d[0] / 1e3, "max_us": d[-1] / 1e3}


# ------------------------------------------------------------------ summaries
def _kernel_stats(directory: str, dense: int, cmd: str, out: str, bench_json: str | None) -> None:
    rows = _kernel_rows(directory)
    if len(rows) <= dense:
        raise ValueError(f"{len(rows)} attention dispatches, expected more than {dense}")
    dur = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]
    win, full = _stats_table(dur[:-dense]), _stats_table(dur[-dense:])
    name = rows[0]["Kernel_Name"]
    lines = [f"# Kernel trace: {ATTN_KERNEL}", "", "Command (from the repository root):", "", "```", cmd, "```", "",
             f"Kernel: `{name[:120]}`", "",
             "| launches | calls | avg µs | median µs | min µs | max µs |", "|---|---|---|---|---|---|"]
    for label, s in (("windowed (all of bench.py's windowed launches)", win), ("dense baseline", full)):
        lines.append(f"| {label} | {s['calls']} | {s['avg_us']:.2f} | {s['median_us']:.2f} | {s['min_us']:.2f} | "
                     f"{s['max_us']:.2f} |")
    if bench_json:
        with open(bench_json) as f:
            b = json.loads(f.read().strip().splitlines()[-1])
        # bench.py's windowed launches, in order: clock settle, warm-up, the timed steps, ...
        per_step = len(b["config"]["shifts"])
        first = (b["clock_settle_steps"] + b["warmup"]) * per_step
        timed = _stats_table(dur[first:first + b["steps"] * per_step])
        lines.append(f"| windowed, bench.py's timed steps only | {timed['calls']} | {timed['avg_us']:.2f} | "
                     f"{timed['median_us']:.2f} | {timed['min_us']:.2f} | {timed['max_us']:.2f} |")
        lines += ["", "bench.py's own line for the same run (HIP events around the timed steps):", "",
                  f"- windowed: {b['speedup']['window_attn_ms'] * 1e3:.2f} µs per launch "
                  f"({b['value']} TFLOP/s); rocprofv3 average over the same launches: {timed['avg_us']:.2f} µs",
                  f"- dense: {b['speedup']['full_attn_ms'] * 1e3:.2f} µs per launch"]
    stats_csv = glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
    if stats_csv:
        lines += ["", "rocprofv3 --stats (all kernels of the run):", "", "| kernel | calls | avg µs | share % |",
                  "|---|---|---|---|"]
        with open(stats_csv[0]) as f:
            for r in csv.DictReader(f):
                lines.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                             f"{float(r['Percentage']):.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}: windowed avg {win['avg_us']:.2f} µs, dense avg {full['avg_us']:.2f} µs")


def _traffic(a) -> None:
    from sparse_attention_dit_amd.build import kernel_hash
    from sparse_attention_dit_amd.configs import BY_NAME

    w = BY_NAME[a.workload]
    fetch_kib, n_f = _counter_per_dispatch(a.fetch, "FETCH_SIZE", ATTN_KERNEL)
    write_kib, n_w = _counter_per_dispatch(a.write, "WRITE_SIZE", ATTN_KERNEL)
    # the copy program's device-to-device copy runs as the runtime's copy kernel
    cf_kib, n_cf = _counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cw_kib, n_cw = _counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    f_scale = COPY_BYTES / (cf_kib * 1024.0)
    w_scale = COPY_BYTES / (cw_kib * 1024.0)
    fetch_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    algo = w.io_bytes()
    rec = {
        "workload": w.name,
        "kernel": ATTN_KERNEL,
        "kernel_hash": kernel_hash(),
        "hbm_bytes_per_launch": round(fetch_b + write_b),
        "fetch_bytes_per_launch": round(fetch_b),
        "write_bytes_per_launch": round(write_b),
        "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": round((fetch_b + write_b) / algo, 4),
        "raw_kib_per_dispatch": {"FETCH_SIZE": fetch_kib, "WRITE_SIZE": write_kib,
                                 "copy_FETCH_SIZE": cf_kib, "copy_WRITE_SIZE": cw_kib},
        "dispatches": {"fetch": n_f, "write": n_w, "copy_fetch": n_cf, "copy_write": n_cw},
        "copy_bytes": COPY_BYTES,
        "scale": {"fetch": round(f_scale, 5), "write": round(w_scale, 5)},
        "commands": a.cmd,
    }
    os.makedirs(a.out_dir, exist_ok=True)
    jpath = os.path.join(a.out_dir, traffic_json_name(w.name))
    with open(jpath, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    md = [f"# HBM traffic of {ATTN_KERNEL}, workload {w.name}", "",
          "Commands (from the repository root; one rocprofv3 counter pass each):", "", "```", *a.cmd, "```", "",
          "| quantity | value |", "|---|---|",
          f"| FETCH_SIZE per dispatch (KiB, mean of {n_f}) | {fetch_kib:.1f} |",
          f"| WRITE_SIZE per dispatch (KiB, mean of {n_w}) | {write_kib:.1f} |",
          f"| copy of {COPY_BYTES >> 20} MiB: FETCH_SIZE / WRITE_SIZE (KiB) | {cf_kib:.1f} / {cw_kib:.1f} |",
          f"| scale applied (fetch / write) | {f_scale:.4f} / {w_scale:.4f} |",
          f"| HBM bytes per launch (fetch + write) | {fetch_b / 1e6:.2f} MB + {write_b / 1e6:.2f} MB "
          f"= {(fetch_b + write_b) / 1e6:.2f} MB |",
          f"| algorithmic bytes per launch (q, k, v read once, out written once) | {algo / 1e6:.2f} MB |",
          f"| traffic / algorithmic | {(fetch_b + write_b) / algo:.3f} |",
          "", f"Kernel source digest: `{rec['kernel_hash']}`"]
    mpath = os.path.join(a.out_dir, f"{ATTN_KERNEL}.{w.name}.traffic.md")
    with open(mpath, "w") as f:
        f.write("\n".join(md) + "\n")
    print(f"wrote {jpath} and {mpath}: {(fetch_b + write_b) / 1e6:.2f} MB per launch "
          f"({(fetch_b + write_b) / algo:.3f} x algorithmic)")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(prog="python -m sparse_attention_dit_amd.profiling")
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    r = sub.add_parser("run")
    r.add_argument("--what", choices=("window", "full", "copy"), required=True)
    r.add_argument("--workload", default="flux-2048-128x128-w32")
    r.add_argument("--iters", type=int, default=4)
    k = sub.add_parser("kernel-stats")
    k.add_argument("--dir", required=True)
    k.add_argument("--dense", type=int, default=7, help="number of trailing dense launches bench.py made")
    k.add_argument("--cmd", required=True)
    k.add_argument("--out", required=True)
    k.add_argument("--bench-json", default=None)
    t = sub.add_parser("traffic")
    for n in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + n.replace("_", "-"), dest=n, required=True)
    t.add_argument("--copy-kernel", default="copyBuffer", help="substring naming the copy kernel")
    t.add_argument("--workload", required=True)
    t.add_argument("--cmd", action="append", required=True)
    t.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args(argv)
    if a.cmd_name == "run":
        _run(a.what, a.workload, a.iters)
    elif a.cmd_name == "kernel-stats":
        _kernel_stats(a.dir, a.dense, a.cmd, a.out, a.bench_json)
    else:
        _traffic(a)


if __name__ == "__main__":
    main()
