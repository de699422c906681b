"""CPU tests of bench.py's host logic: the one-GPU contract, the roofline
choice and the summaries it writes from rocprofv3 output (synthetic rocpd
databases with the tables those summaries read)."""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _db(path, counters=(), kernels=()):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real, "
                "dispatch_id int)")
    con.execute("create table kernels (name text, dispatch_id int, duration int)")
    con.executemany("insert into counters_collection values (?,?,?,?)", counters)
    con.executemany("insert into kernels values (?,?,?)", kernels)
    con.commit()
    con.close()


G1 = "_ZN12_GLOBAL__N_116gemm_pipe_kernelILi0ELi0EDF16bEEv"
G2 = "_ZN12_GLOBAL__N_116gemm_pipe_kernelILi1ELi0EDF16bEEv"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


def test_roofline_picks_the_bound_by_arithmetic_intensity():
    ridge = bench.MFMA_BF16_PEAK_TFS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    # below the ridge: HBM-bound, MFMA fraction rides along
    r = {"gemm1_flops": 200e9, "gemm1_bytes": 1e9, "gemm1_alg_gbs": 4000.0, "gemm1_tflops": 800.0}
    lo = bench.gemm1_roofline(r)
    assert lo["bound"] == "hbm" and lo["frac"] == pytest.approx(0.5)
    assert lo["other_bound"]["bound"] == "mfma" and lo["other_bound"]["frac"] == pytest.approx(0.32)
    assert lo["ridge_flop_per_byte"] == pytest.approx(ridge) and lo["flop_per_byte"] == pytest.approx(200)
    r = {"gemm1_flops": 500e9, "gemm1_bytes": 1e9, "gemm1_alg_gbs": 2000.0, "gemm1_tflops": 1000.0}
    hi = bench.gemm1_roofline(r)
    assert hi["bound"] == "mfma" and hi["frac"] == pytest.approx(0.4)
    assert hi["unit"] == "TFLOP/s" and hi["peak"] == bench.MFMA_BF16_PEAK_TFS


def test_counter_summary_sums_instances_and_averages_dispatches(tmp_path, capsys):
    # two dispatches of gemm1 (counter read from two instances each), one of
    # gemm2, one unrelated kernel; durations of the same dispatches
    c = [(G1, "SQ_BUSY_CYCLES", 10.0, 1), (G1, "SQ_BUSY_CYCLES", 5.0, 1),
         (G1, "SQ_BUSY_CYCLES", 7.0, 3), (G1, "GRBM_GUI_ACTIVE", 80.0, 1),
         (G1, "GRBM_GUI_ACTIVE", 40.0, 3), (G2, "SQ_BUSY_CYCLES", 2.0, 2),
         ("other_kernel", "SQ_BUSY_CYCLES", 99.0, 4)]
    k = [(G1, 1, 1000), (G1, 3, 3000), (G2, 2, 500), ("other_kernel", 4, 7)]
    _db(str(tmp_path / "run" / "x" / "k_results.db"), c, k)
    out = bench.summarize_counters(str(tmp_path / "run"), "753b_a40b_bf16")
    assert out["gemm1"]["SQ_BUSY_CYCLES"] == pytest.approx(11.0)   # (15 + 7) / 2
    assert out["gemm1"]["GRBM_GUI_ACTIVE"] == pytest.approx(60.0)
    assert out["gemm2"]["SQ_BUSY_CYCLES"] == pytest.approx(2.0)
    assert out["dispatches"] == {"gemm1": 2, "gemm2": 1}
    assert out["duration_ns"]["gemm1"] == {"mean": pytest.approx(2000.0), "n": 2}
    assert json.loads(capsys.readouterr().out.strip().splitlines()[-1])["dispatches"]["gemm1"] == 2


def test_kernel_stats_summary_from_a_rocpd_database(tmp_path):
    k = [(G1, i, d) for i, d in enumerate((7000, 7010, 7030, 7040))] + \
        [("combine_kernel", 10 + i, 300) for i in range(8)]
    db = str(tmp_path / "prof" / "c5_results.db")
    _db(db, (), k)
    md = str(tmp_path / "stats.md")
    bench.summarize_stats(db, "rocprofv3 --kernel-trace --stats -- python bench.py", md)
    text = open(md).read()
    lines = [l for l in text.splitlines() if l.startswith("| `")]
    assert lines[0].startswith(f"| `{G1}` | 4 | 7.02 | 7.00 | 7.04 |")   # most time first, in us
    assert lines[1].startswith("| `combine_kernel` | 8 | 0.30 |")
    assert "rocprofv3 --kernel-trace --stats -- python bench.py" in text


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    # the 1 GiB copy reads 0.5 GiB as FETCH_SIZE (KiB) and writes 1 GiB as WRITE_SIZE
    cal = ("__amd_rocclr_copyBuffer", bench.CAL_BYTES / 2048.0, bench.CAL_BYTES / 1024.0)
    fetch = [(cal[0], "FETCH_SIZE", cal[1], 0), (G1, "FETCH_SIZE", 1000.0, 1), (G1, "FETCH_SIZE", 3000.0, 2),
             (G2, "FETCH_SIZE", 99999.0, 3)]
    write = [(cal[0], "WRITE_SIZE", cal[2], 0), (G1, "WRITE_SIZE", 50.0, 1), (G1, "WRITE_SIZE", 70.0, 2)]
    _db(str(tmp_path / "f" / "f_results.db"), fetch)
    _db(str(tmp_path / "w" / "w_results.db"), write)
    out_json = str(tmp_path / "traffic.json")
    monkeypatch.setattr(bench, "traffic_json", lambda workload, T: out_json)
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "753b_a40b_bf16", "16384")
    t = json.load(open(out_json))
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert t["fetch_bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2.0)
    assert t["write_bytes_per_launch"] == pytest.approx(60.0 * 1024)
    assert t["launches"] == [2, 2] and t["T"] == 16384
    # the stored figure is used only while the kernel source is the one measured
    assert bench.stored_traffic("753b_a40b_bf16", 16384) == pytest.approx(2000.0 * 2048 + 60.0 * 1024)
    t["source_sha256"] = "0" * 64
    json.dump(t, open(out_json, "w"))
    assert bench.stored_traffic("753b_a40b_bf16", 16384) is None
