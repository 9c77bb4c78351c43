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
STREAM_KERNEL = "win_attn_bf16_stream_kernel"
F32_KERNEL = "win_attn_f32_kernel"
COPY_BYTES = 256 << 20  # calibration copy: 256 MiB read + 256 MiB written per launch


def kernel_name(dtype: str, window_tokens: int) -> str:
    """The kernel the library launches for plain windowed attention over windows of
    `window_tokens` (the dense baseline: the whole sequence). Mirrors the launcher: fp32
    inputs run the fp32 kernel; bf16 windows of 2 to 15 key tiles of 64 run the stream
    kernel, all others the per-item kernel."""
    if dtype != "bf16":
        return F32_KERNEL
    tiles = -(-window_tokens // 64)
    return STREAM_KERNEL if 3 <= tiles <= 16 else ATTN_KERNEL


def traffic_json_name(workload: str, tag: str = "") -> str:
    """File name of the traffic record of a workload's windowed kernel; `tag` (e.g. "cold")
    names a record taken under other cache conditions."""
    from sparse_attention_dit_amd.configs import BY_NAME
    w = BY_NAME[workload]
    return f"{kernel_name(w.dtype, w.window_tokens)}.{workload}.{tag + '.' if tag else ''}traffic.json"


def _matches(kernel_field: str, kernel: str) -> bool:
    """rocprofv3 kernel names are demangled signatures; match the function name exactly
    (the per-item kernel's name is a prefix of neither of the others)."""
    return f"::{kernel}<" in kernel_field or kernel_field.startswith(kernel + "<") or f" {kernel}<" in kernel_field


# ------------------------------------------------------------------ profiled program
def _run(what: str, workload: str, iters: int, cold: bool = False) -> None:
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
    # cold: a 1 GiB write before every launch evicts q, k and v from the L2s and the MALL
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if cold else None
    n = 0
    for _ in range(iters):
        for s in (w.shifts if what == "window" else [None]):
            if flush is not None:
                flush.fill_(n & 0xFF)
            n += 1
            if what == "window":
                _lib.window_attn_fwd(dev["q"], dev["k"], dev["v"], out, w.grid, w.window, s)
            else:
                _lib.full_attn_fwd(dev["q"], dev["k"], dev["v"], out)
    torch.cuda.synchronize()
    print(f"{what}: {workload}, {iters} iterations{' (cold)' if cold else ''}", flush=True)


# ------------------------------------------------------------------ CSV readers
def _find_csv(directory: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    return hits[0]


def _kernel_rows(directory: str, kernels=(ATTN_KERNEL,)):
    """Dispatches of the given attention kernels from a kernel-trace CSV, in dispatch order."""
    rows = []
    with open(_find_csv(directory, "kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            if any(_matches(r["Kernel_Name"], k) for k in kernels):
                rows.append(r)
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def _counter_per_dispatch(directory: str, counter: str, kernel_substr: str, grid: int | None = None,
                          exact: bool = True):
    """Mean and count of a counter's per-dispatch value over the matching dispatches (kernel
    function named exactly, or with exact=False any kernel whose name contains the text)."""
    vals = []
    with open(_find_csv(directory, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            name_ok = _matches(r["Kernel_Name"], kernel_substr) if exact else kernel_substr in r["Kernel_Name"]
            if r["Counter_Name"] != counter or not name_ok:
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
    win_kernel = dense_kernel = ATTN_KERNEL
    if bench_json:
        from sparse_attention_dit_amd.configs import BY_NAME
        with open(bench_json) as f:
            wl = BY_NAME[json.loads(f.read().strip().splitlines()[-1])["config"]["workload"]]
        win_kernel, dense_kernel = kernel_name(wl.dtype, wl.window_tokens), kernel_name(wl.dtype, wl.tokens)
    if win_kernel == dense_kernel:
        # one kernel: bench.py's dense launches come last (2 untimed + --full-iters timed)
        rows = _kernel_rows(directory, (win_kernel,))
        if len(rows) <= dense:
            raise ValueError(f"{len(rows)} attention dispatches, expected more than {dense}")
        win_rows, dense_rows = rows[:-dense], rows[-dense:]
    else:
        win_rows, dense_rows = _kernel_rows(directory, (win_kernel,)), _kernel_rows(directory, (dense_kernel,))
    dur = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in win_rows]
    win = _stats_table(dur)
    full = _stats_table([int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in dense_rows])
    name = win_rows[0]["Kernel_Name"]
    lines = [f"# Kernel trace: {win_kernel}", "", "Command (from the repository root):", "", "```", cmd, "```", "",
             f"Kernel: `{name[:120]}`" + ("" if win_kernel == dense_kernel else
                                          f"; dense baseline: `{dense_rows[0]['Kernel_Name'][:120]}`"), "",
             "| launches | calls | avg µs | median µs | min µs | max µs |", "|---|---|---|---|---|---|"]
    for label, s in (("windowed (all of bench.py's windowed launches)", win), ("dense baseline", full)):
        lines.append(f"| {label} | {s['calls']} | {s['avg_us']:.2f} | {s['median_us']:.2f} | {s['min_us']:.2f} | "
                     f"{s['max_us']:.2f} |")
    if bench_json:
        from sparse_attention_dit_amd.configs import BY_NAME
        with open(bench_json) as f:
            b = json.loads(f.read().strip().splitlines()[-1])
        w = BY_NAME[b["config"]["workload"]]
        # bench.py's windowed launches, in order: clock settle, warm-up, the timed steps,
        # the sustained steps, ...
        per_step = len(b["config"]["shifts"])
        first = (b["clock_settle_steps"] + b["warmup"]) * per_step
        timed = _stats_table(dur[first:first + b["steps"] * per_step])
        lines.append(f"| windowed, bench.py's timed steps only | {timed['calls']} | {timed['avg_us']:.2f} | "
                     f"{timed['median_us']:.2f} | {timed['min_us']:.2f} | {timed['max_us']:.2f} |")
        sus = None
        if "sustained" in b:
            s0 = first + b["steps"] * per_step
            sus = _stats_table(dur[s0:s0 + b["sustained"]["launches"]])
            lines.append(f"| windowed, bench.py's sustained steps | {sus['calls']} | {sus['avg_us']:.2f} | "
                         f"{sus['median_us']:.2f} | {sus['min_us']:.2f} | {sus['max_us']:.2f} |")
        peak = 2516.6 if w.dtype == "bf16" else 157.3
        flops = w.window_flops()
        sclk = (b.get("sclk_mhz") or {}).get("median")
        frac = flops / (timed["avg_us"] * 1e-6) / 1e12 / peak
        lines += ["", "bench.py's own line for the same run (HIP events around the timed steps):", "",
                  f"- windowed: {b['speedup']['window_attn_ms'] * 1e3:.2f} µs per launch "
                  f"({b['value']} TFLOP/s, frac {b['roofline']['frac']}); rocprofv3 average over the same "
                  f"launches: {timed['avg_us']:.2f} µs, i.e. {flops / 1e9:.2f} GFLOP / {timed['avg_us']:.2f} µs = "
                  f"{flops / (timed['avg_us'] * 1e-6) / 1e12:.1f} TFLOP/s = {frac:.4f} of {peak} TFLOP/s",
                  f"- kernel time per step from the trace: {timed['avg_us'] * per_step / 1e3:.4f} ms; bench.py's "
                  f"ms_per_step: {b['ms_per_step']}",
                  f"- dense: {b['speedup']['full_attn_ms'] * 1e3:.2f} µs per launch"]
        if sclk:
            lines.append(f"- core clock held over the timed steps (pp_dpm_sclk median): {sclk:.0f} MHz; fraction of "
                         f"the peak at that clock (peak x sclk / 2400): {frac * 2400.0 / sclk:.4f}")
        if sus is not None:
            sb = b["sustained"]
            lines.append(f"- sustained: bench.py median {sb['median_ms_per_launch'] * 1e3:.2f} µs per launch over "
                         f"{sb['launches']} launches ({sb['span_ms']:.0f} ms, clock {sb['sclk_mhz_median']} MHz); "
                         f"rocprofv3 median over the same launches {sus['median_us']:.2f} µs")
        lines.append(f"- library: `{b.get('library', {}).get('path')}` sha256 {b.get('library', {}).get('sha256_16')}, "
                     f"kernel source digest `{b.get('kernel_hash')}`")
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
    kernel = kernel_name(w.dtype, w.window_tokens)
    fetch_kib, n_f = _counter_per_dispatch(a.fetch, "FETCH_SIZE", kernel)
    write_kib, n_w = _counter_per_dispatch(a.write, "WRITE_SIZE", kernel)
    # the copy program's device-to-device copy runs as the runtime's copy kernel
    cf_kib, n_cf = _counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel, exact=False)
    cw_kib, n_cw = _counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel, exact=False)
    f_scale = COPY_BYTES / (cf_kib * 1024.0)
    w_scale = COPY_BYTES / (cw_kib * 1024.0)
    fetch_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    algo = w.io_bytes()
    rec = {
        "workload": w.name,
        "kernel": kernel,
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
        "caches": "cold: 1 GiB written before each launch" if a.tag == "cold" else "as left by the previous launch",
        "tag": a.tag,
        "commands": a.cmd,
    }
    os.makedirs(a.out_dir, exist_ok=True)
    jpath = os.path.join(a.out_dir, traffic_json_name(w.name, a.tag))
    with open(jpath, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    md = [f"# HBM traffic of {kernel}, workload {w.name}{' (' + a.tag + ')' if a.tag else ''}", "",
          f"Caches: {rec['caches']}.", "",
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
    mpath = os.path.join(a.out_dir, traffic_json_name(w.name, a.tag)[:-len("json")] + "md")
    with open(mpath, "w") as f:
        f.write("\n".join(md) + "\n")
    print(f"wrote {jpath} and {mpath}: {(fetch_b + write_b) / 1e6:.2f} MB per launch "
          f"({(fetch_b + write_b) / algo:.3f} x algorithmic)")


# Counter passes of the MFMA/LDS record. Each pass stays within one collection's hardware
# limits (at most 8 SQ and 2 GRBM counters); MfmaUtil and LDSBankConflict are rocprofv3's
# derived metrics over SQ_VALU_MFMA_BUSY_CYCLES / SQ_LDS_BANK_CONFLICT and GRBM_GUI_ACTIVE.
COUNTER_PASSES = {
    "mfma": ("MfmaUtil", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
             "SQ_INSTS_MFMA", "SQ_VALU_MFMA_COEXEC_CYCLES"),
    "valu": ("LDSBankConflict", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_VALU",
             "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS"),
}
SIMDS = 1024  # 256 CUs x 4 SIMDs
MFMA_FLOP = {"bf16": 32 * 32 * 16 * 2, "f32": 32 * 32 * 2 * 2}  # v_mfma_f32_32x32x16_bf16 / 32x32x2_f32


def _counters(a) -> None:
    from sparse_attention_dit_amd.build import kernel_hash
    from sparse_attention_dit_amd.configs import BY_NAME

    w = BY_NAME[a.workload]
    if a.kernel is None:
        a.kernel = kernel_name(w.dtype, w.window_tokens if a.what == "window" else w.tokens)
    vals = {}
    for directory, names in ((a.mfma, COUNTER_PASSES["mfma"]), (a.valu, COUNTER_PASSES["valu"])):
        for n in names:
            vals[n], count = _counter_per_dispatch(directory, n, a.kernel)
            vals[n + "#dispatches"] = count
    flops = w.window_flops() if a.what == "window" else w.full_flops()
    mfma_alg = flops / MFMA_FLOP[w.dtype]
    mops_flop = vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    rec = {
        "workload": w.name, "launch": a.what, "kernel": a.kernel, "kernel_hash": kernel_hash(),
        "raw_per_dispatch": {k: v for k, v in vals.items() if not k.endswith("#dispatches")},
        "dispatches": {k[:-11]: v for k, v in vals.items() if k.endswith("#dispatches")},
        "algorithmic_flop_per_launch": flops,
        "mfma_flop_counted_over_algorithmic": round(mops_flop / flops, 4) if w.dtype == "bf16" else None,
        "mfma_instructions_over_algorithmic": round(vals["SQ_INSTS_MFMA"] / mfma_alg, 4),
        "mfma_util_pct": round(vals["MfmaUtil"], 2),
        "coexec_cycles_per_simd": round(vals["SQ_VALU_MFMA_COEXEC_CYCLES"] / SIMDS),
        "lds_bank_conflict_pct_of_time": round(vals["LDSBankConflict"], 2),
        "lds_bank_conflict_over_lds_active": round(vals["SQ_LDS_BANK_CONFLICT"] / vals["SQ_LDS_IDX_ACTIVE"], 4),
        # MfmaUtil divides the summed busy cycles by the largest GUI-active count of one
        # instance; the raw GRBM_GUI_ACTIVE row is the sum over instances
        "gui_active_cycles_one_instance": round(vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (vals["MfmaUtil"] / 100.0) / SIMDS),
        "mfma_busy_cycles_per_simd": round(vals["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS),
        "valu_per_mfma": round(vals["SQ_INSTS_VALU"] / vals["SQ_INSTS_MFMA"], 3),
        "trans_f32_per_mfma": round(vals["SQ_INSTS_VALU_TRANS_F32"] / vals["SQ_INSTS_MFMA"], 3),
        "lds_instr_per_mfma": round(vals["SQ_INSTS_LDS"] / vals["SQ_INSTS_MFMA"], 3),
        "commands": a.cmd,
    }
    os.makedirs(a.out_dir, exist_ok=True)
    stem = f"{a.kernel}.{w.name}.{a.what}.counters"
    with open(os.path.join(a.out_dir, stem + ".json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    md = [f"# MFMA, VALU and LDS counters of {a.kernel}, workload {w.name} ({a.what} launch)", "",
          "Commands (from the repository root; one rocprofv3 counter pass each):", "", "```", *a.cmd, "```", "",
          "| quantity | value |", "|---|---|",
          f"| algorithmic FLOP per launch | {flops / 1e9:.2f} GFLOP |",
          f"| MFMA FLOP counted (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) / algorithmic | "
          f"{rec['mfma_flop_counted_over_algorithmic']} |",
          f"| MFMA instructions (SQ_INSTS_MFMA) / algorithmic count | {rec['mfma_instructions_over_algorithmic']} |",
          f"| MFMA utilisation (MfmaUtil: busy cycles / (GUI-active cycles x SIMDs)) | {rec['mfma_util_pct']} % |",
          f"| MFMA-busy cycles per SIMD / GUI-active cycles of one instance | {rec['mfma_busy_cycles_per_simd']} / "
          f"{rec['gui_active_cycles_one_instance']} |",
          f"| MFMA-busy cycles with a VALU instruction co-issued, per SIMD | {rec['coexec_cycles_per_simd']} |",
          f"| LDS stalled by bank conflicts (LDSBankConflict, % of time per CU) | "
          f"{rec['lds_bank_conflict_pct_of_time']} % |",
          f"| SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE | {rec['lds_bank_conflict_over_lds_active']} |",
          f"| VALU instructions per MFMA | {rec['valu_per_mfma']} |",
          f"| fp32 transcendental instructions per MFMA | {rec['trans_f32_per_mfma']} |",
          f"| LDS instructions per MFMA | {rec['lds_instr_per_mfma']} |",
          "", "Raw values per dispatch (mean over the profiled dispatches):", "",
          "| counter | value |", "|---|---|"]
    md += [f"| {k} | {v:.6g} |" for k, v in rec["raw_per_dispatch"].items()]
    md += ["", f"Kernel source digest: `{rec['kernel_hash']}`"]
    with open(os.path.join(a.out_dir, stem + ".md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(f"wrote {stem}: MfmaUtil {rec['mfma_util_pct']} %, MFMA/alg {rec['mfma_instructions_over_algorithmic']}, "
          f"LDS conflict {rec['lds_bank_conflict_over_lds_active']}")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(prog="python -m sparse_attention_dit_amd.profiling")
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    r = sub.add_parser("run")
    r.add_argument("--what", choices=("window", "full", "copy"), required=True)
    r.add_argument("--workload", default="flux-2048-128x128-w32")
    r.add_argument("--iters", type=int, default=4)
    r.add_argument("--cold", action="store_true", help="write 1 GiB before each launch (HBM-cold caches)")
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
    t.add_argument("--tag", default="", choices=("", "cold"), help="cache conditions of the counted launches")
    t.add_argument("--cmd", action="append", required=True)
    t.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    c = sub.add_parser("counters")
    c.add_argument("--mfma", required=True, help="output directory of the 'mfma' counter pass")
    c.add_argument("--valu", required=True, help="output directory of the 'valu' counter pass")
    c.add_argument("--workload", required=True)
    c.add_argument("--what", choices=("window", "full"), default="window")
    c.add_argument("--kernel", default=None, help="profiled kernel (default: the one the library launches)")
    c.add_argument("--cmd", action="append", required=True)
    c.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args(argv)
    if a.cmd_name == "counters":
        _counters(a)
        return
    if a.cmd_name == "run":
        _run(a.what, a.workload, a.iters, a.cold)
    elif a.cmd_name == "kernel-stats":
        _kernel_stats(a.dir, a.dense, a.cmd, a.out, a.bench_json)
    else:
        _traffic(a)


if __name__ == "__main__":
    main()
