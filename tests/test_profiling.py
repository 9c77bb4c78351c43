"""Host logic of the profile summaries: counter scaling and launch splitting, on small
hand-made CSV files shaped like rocprofv3's output."""
import csv
import json
import os

import pytest

from sparse_attention_dit_amd import profiling
from sparse_attention_dit_amd.build import kernel_hash
from sparse_attention_dit_amd.configs import BY_NAME

COUNTER_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
                "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
                "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
                "End_Timestamp"]


def _counters(path, rows):
    os.makedirs(path)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, COUNTER_COLS)
        wr.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            r = dict.fromkeys(COUNTER_COLS, "0")
            r.update(Dispatch_Id=str(i + 1), Kernel_Name=kernel, Counter_Name=counter, Counter_Value=str(value))
            wr.writerow(r)


def test_traffic_scaling(tmp_path):
    wl = "flux-2048-128x128-w32"
    k = f"void basa::{profiling.kernel_name('bf16', BY_NAME[wl].window_tokens)}<128, 8>(...)"
    c = "__amd_rocclr_copyBuffer"
    _counters(tmp_path / "f", [(k, "FETCH_SIZE", 100.0), (k, "FETCH_SIZE", 102.0), ("other", "FETCH_SIZE", 1e9)])
    _counters(tmp_path / "w", [(k, "WRITE_SIZE", 50.0)])
    half = profiling.COPY_BYTES / 1024 / 2
    _counters(tmp_path / "cf", [(c, "FETCH_SIZE", half)])                  # counter reads half the bytes
    _counters(tmp_path / "cw", [(c, "WRITE_SIZE", profiling.COPY_BYTES / 1024)])
    out = tmp_path / "out"
    profiling.main(["traffic", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"),
                    "--copy-fetch", str(tmp_path / "cf"), "--copy-write", str(tmp_path / "cw"),
                    "--workload", wl, "--cmd", "cmd", "--out-dir", str(out)])
    rec = json.load(open(out / profiling.traffic_json_name(wl)))
    assert rec["tag"] == "" and not (out / profiling.traffic_json_name(wl, "cold")).exists()
    assert rec["fetch_bytes_per_launch"] == round(101.0 * 1024 * 2)
    assert rec["write_bytes_per_launch"] == 50 * 1024
    assert rec["hbm_bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["algorithmic_bytes_per_launch"] == BY_NAME[wl].io_bytes()
    assert rec["kernel_hash"] == kernel_hash()
    profiling.main(["traffic", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"),
                    "--copy-fetch", str(tmp_path / "cf"), "--copy-write", str(tmp_path / "cw"),
                    "--workload", wl, "--tag", "cold", "--cmd", "cmd", "--out-dir", str(out)])
    cold = json.load(open(out / profiling.traffic_json_name(wl, "cold")))
    assert cold["tag"] == "cold" and cold["hbm_bytes_per_launch"] == rec["hbm_bytes_per_launch"]
    assert (out / profiling.traffic_json_name(wl, "cold").replace(".json", ".md")).exists()


def test_kernel_stats_split(tmp_path):
    d = tmp_path / "t"
    os.makedirs(d)
    cols = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    with open(d / "b_kernel_trace.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, cols)
        wr.writeheader()
        rows = [(3, 1000), (1, 2000), (2, 4000), (5, 30000), (4, 50000)]   # (dispatch, ns), unordered
        for did, ns in rows:
            wr.writerow({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": did,
                         "Kernel_Name": "void basa::win_attn_bf16_kernel<128, 8>(x)",
                         "Start_Timestamp": 10, "End_Timestamp": 10 + ns})
        wr.writerow({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": 6, "Kernel_Name": "other",
                     "Start_Timestamp": 0, "End_Timestamp": 10 ** 9})
    out = tmp_path / "s.md"
    profiling.main(["kernel-stats", "--dir", str(d), "--dense", "2", "--cmd", "c", "--out", str(out)])
    text = out.read_text()
    # dispatches 1..3 are the windowed launches (2000, 1000, 4000 ns), 4..5 the dense ones
    assert "| windowed (all of bench.py's windowed launches) | 3 | 2.33 | 2.00 | 1.00 | 4.00 |" in text
    assert "| dense baseline | 2 | 40.00 | 40.00 | 30.00 | 50.00 |" in text


def test_committed_traffic_records_are_consistent():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pdir = os.path.join(root, "profiles")
    found = [f for f in os.listdir(pdir) if f.endswith(".traffic.json")] if os.path.isdir(pdir) else []
    if not found:
        pytest.skip("no committed traffic record")
    for name in found:
        rec = json.load(open(os.path.join(pdir, name)))
        wl = BY_NAME[rec["workload"]]
        assert name == profiling.traffic_json_name(wl.name, rec.get("tag", ""))
        assert rec["kernel"] == profiling.kernel_name(wl.dtype, wl.window_tokens)
        assert rec["algorithmic_bytes_per_launch"] == wl.io_bytes()
        assert rec["hbm_bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def test_clock_sampler_reads_the_marked_level(tmp_path):
    """bench.py's clock sampler takes the level marked '*' in the amdgpu kernel driver's pp_dpm_sclk text
    (idle: the sleep level; under load: the current frequency between min and max)."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    s = bench.ClockSampler()
    f = tmp_path / "pp_dpm_sclk"
    s.path = str(f)
    f.write_text("0: 500Mhz\n1: 1916Mhz *\n2: 2400Mhz\n")
    assert s._read() == 1916.0
    f.write_text("S: 111Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    assert s._read() == 111.0
    f.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert s._read() is None
    s.samples = [(0.0, 1900.0), (1.0, 1950.0), (2.0, 1920.0), (3.0, 2400.0)]
    assert s.median(0.5, 2.5) == (1950.0, 2)
    assert s.median(5.0, 6.0) == (None, 0)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 (or a multi-rank launch) exits with status 2
    and says why, before touching torch or the GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""


def test_counter_summary(tmp_path):
    """MFMA/VALU/LDS record: counters are averaged over the kernel's dispatches and related
    to the algorithmic MFMA count of the workload."""
    wl = BY_NAME["flux-2048-128x128-w32"]
    kname = profiling.kernel_name("bf16", wl.window_tokens)
    k = f"void basa::{kname}<128, 8>(...)"
    n_mfma = wl.window_flops() / (32 * 32 * 16 * 2)
    mfma = [(k, "MfmaUtil", 50.0), (k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1000.0), (k, "GRBM_GUI_ACTIVE", 16000.0),
            (k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", wl.window_flops() / 512), (k, "SQ_INSTS_MFMA", n_mfma),
            (k, "SQ_VALU_MFMA_COEXEC_CYCLES", 1024 * 300.0), ("other", "SQ_INSTS_MFMA", 1.0)]
    valu = [(k, "LDSBankConflict", 3.0), (k, "SQ_LDS_BANK_CONFLICT", 250.0), (k, "SQ_LDS_IDX_ACTIVE", 1000.0),
            (k, "SQ_INSTS_VALU", 4 * n_mfma), (k, "SQ_INSTS_VALU_TRANS_F32", n_mfma), (k, "SQ_INSTS_LDS", n_mfma / 2)]
    _counters(tmp_path / "m", mfma)
    _counters(tmp_path / "v", valu)
    out = tmp_path / "out"
    profiling.main(["counters", "--mfma", str(tmp_path / "m"), "--valu", str(tmp_path / "v"), "--workload", wl.name,
                    "--cmd", "c1", "--cmd", "c2", "--out-dir", str(out)])
    rec = json.load(open(out / f"{kname}.{wl.name}.window.counters.json"))
    assert rec["mfma_flop_counted_over_algorithmic"] == 1.0
    assert rec["mfma_instructions_over_algorithmic"] == 1.0
    assert rec["mfma_util_pct"] == 50.0
    assert rec["mfma_busy_cycles_per_simd"] == 1000
    assert rec["gui_active_cycles_one_instance"] == 2000
    assert rec["lds_bank_conflict_over_lds_active"] == 0.25
    assert rec["valu_per_mfma"] == 4.0 and rec["trans_f32_per_mfma"] == 1.0 and rec["lds_instr_per_mfma"] == 0.5
    assert rec["kernel_hash"] == kernel_hash()
    assert (out / f"{kname}.{wl.name}.window.counters.md").exists()


def test_host_info_fields():
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    info = bench.host_info()
    assert info["logical_cpus_available"] >= 1
    assert info["numpy"]
    assert set(info) == {"cpu_model", "logical_cpus_available", "physical_cores", "numpy", "blas"}


def test_kernel_choice_mirrors_the_launcher():
    """The profile summaries name the kernel the library launches for a workload: fp32 inputs
    the fp32 kernel, bf16 windows of 3-16 key tiles of 64 the stream kernel, else the per-item
    kernel (the launcher's rule in attn_kernels.hip)."""
    assert profiling.kernel_name("f32", 64) == "win_attn_f32_kernel"
    assert profiling.kernel_name("bf16", 64) == "win_attn_bf16_kernel"
    assert profiling.kernel_name("bf16", 128) == "win_attn_bf16_kernel"
    assert profiling.kernel_name("bf16", 129) == "win_attn_bf16_stream_kernel"
    assert profiling.kernel_name("bf16", 256) == "win_attn_bf16_stream_kernel"
    assert profiling.kernel_name("bf16", 960) == "win_attn_bf16_stream_kernel"
    assert profiling.kernel_name("bf16", 1024) == "win_attn_bf16_stream_kernel"
    assert profiling.kernel_name("bf16", 1025) == "win_attn_bf16_kernel"
    assert profiling.kernel_name("bf16", 2730) == "win_attn_bf16_kernel"
    assert profiling._matches("void basa::win_attn_bf16_stream_kernel<128, 8>(basa::Bf16KernelArgs)",
                              "win_attn_bf16_stream_kernel")
    assert not profiling._matches("void basa::win_attn_bf16_stream_kernel<128, 8>(basa::Bf16KernelArgs)",
                                  "win_attn_bf16_kernel")
    assert profiling._matches("void basa::win_attn_bf16_kernel<128, 8>(basa::Bf16KernelArgs)", "win_attn_bf16_kernel")
