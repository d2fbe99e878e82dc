"""Host logic of bench.py, on the CPU: the profile summarizer on small
synthetic rocprofv3 CSV files, the byte model behind its roofline, and the
refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _trace_row(kernel, t0, us, grid, wg=256):
    return {"Kernel_Name": f"void {kernel}(qig::MmqArgs)", "Start_Timestamp": t0,
            "End_Timestamp": t0 + int(us * 1000), "Grid_Size_X": grid * wg, "Workgroup_Size_X": wg}


def _pmc_rows(values):
    return [{"Kernel_Name": f"void {k}(int)", "Counter_Name": c, "Counter_Value": v} for k, c, v in values]


def test_algorithmic_bytes_model():
    alg = bench._algorithmic_bytes()
    nsb = bench.ID // 256
    q8 = bench.NT * bench.ID // 32 * 40
    y = bench.NT * bench.OD * 4
    assert alg["mmq_q4k_q8t"] == (bench.OD * nsb * 144 + q8, y)
    assert alg["mmq_q6k_raw_q8t"] == (bench.OD * nsb * 224 + q8, y)
    # limb buffer: two int8 planes and one fp32 d per super-block
    assert alg["mmq_q6k_limbs_q8t"] == (2 * bench.OD * bench.ID + bench.OD * nsb * 4 + q8, y)
    down = bench._algorithmic_bytes(2630, 3584, 18944)
    assert down["quantize_q8_tiled"] == (2630 * 18944 * 4, 2630 * 18944 // 32 * 40)


def test_summarize_profiles_proj(tmp_path):
    src = tmp_path / "prof"
    out = tmp_path / "out"
    out.mkdir()
    limb = "qig::mmq_limbs_kernel<2>"
    q4 = "qig::mmq_kernel<4, 0, 0, 1>"
    _write_csv(str(src / "trace" / "t_kernel_trace.csv"),
               [_trace_row(limb, 1000 * i, 30 + i, 3136) for i in range(5)]
               + [_trace_row(q4, 10 ** 6 + 1000 * i, 25, 3136) for i in range(3)])
    copy = "__amd_rocclr_copyBuffer"
    mib256 = 256 * 1024
    _write_csv(str(src / "fetch" / "p_counter_collection.csv"),
               _pmc_rows([(copy, "FETCH_SIZE", mib256 / 2), (limb, "FETCH_SIZE", 20000), (q4, "FETCH_SIZE", 10000)]))
    _write_csv(str(src / "write" / "p_counter_collection.csv"),
               _pmc_rows([(copy, "WRITE_SIZE", mib256), (limb, "WRITE_SIZE", 7168), (q4, "WRITE_SIZE", 7168)]))
    bench.summarize_profiles(str(src), "proj", out_dir=str(out))
    trace = (out / "mmq_3584x3584_nt512_kernel_trace.md").read_text()
    # median of 30..34 us is 32; grouped with its workgroup count
    assert "| mmq_q6k_limbs_q8t | 3136 | 5 | 32.00 |" in trace
    assert "| mmq_q4k_q8t | 3136 | 3 | 25.00 |" in trace
    counters = (out / "mmq_3584x3584_nt512_counters.md").read_text()
    assert "mmq_q6k_limbs_q8t" in counters
    rec = json.loads((out / "mmq_traffic.json").read_text())
    # FETCH_SIZE scaled by the copy's 0.5 read factor, WRITE_SIZE by 1.0
    assert rec["fetch_scale"] == pytest.approx(0.5)
    assert rec["bytes_per_launch"]["mmq_q6k_limbs_q8t"] == (20000 * 1024) * 2 + 7168 * 1024
    assert rec["bytes_per_launch"]["mmq_q4k_q8t"] == (10000 * 1024) * 2 + 7168 * 1024


def test_summarize_profiles_layer_trace_only(tmp_path):
    src = tmp_path / "prof"
    out = tmp_path / "out"
    out.mkdir()
    q4 = "qig::mmq_kernel<4, 0, 0, 1>"
    _write_csv(str(src / "trace" / "t_kernel_trace.csv"),
               [_trace_row(q4, 0, 600, 12432), _trace_row(q4, 10 ** 6, 40, 336)])
    bench.summarize_profiles(str(src), "layer", out_dir=str(out))
    trace = (out / "mmq_layer_nt2630_kernel_trace.md").read_text()
    assert "| mmq_q4k_q8t | 12432 | 1 |" in trace and "| mmq_q4k_q8t | 336 | 1 |" in trace
    assert not (out / "mmq_layer_nt2630_counters.md").exists()


def test_valu_roofline(monkeypatch):
    """insts x 64 lanes / duration against 256 CUs x 4 SIMDs x 32 lanes x
    2.4 GHz, and against 0.74 of that (the two-wave ceiling); None without
    recorded counters."""
    monkeypatch.setattr(bench, "recorded_counter", lambda k, f="bytes_per_launch": 10_000_000)
    r = bench.valu_roofline("mmq_q6k_limbs_q8t", 32.0, 2000)
    achieved = 10_000_000 * 64 / 32e-6 / 1e12
    peak = 256 * 4 * 32 * 2.4e9 / 1e12
    assert r["peak"] == pytest.approx(78.6432)
    assert r["achieved"] == pytest.approx(achieved, abs=0.01)
    assert r["frac"] == pytest.approx(achieved / peak, abs=1e-4)
    assert r["frac_of_2wave_ceiling"] == pytest.approx(achieved / (0.74 * peak), abs=1e-4)
    assert r["frac_at_clock"] == pytest.approx(achieved / (peak * 2000 / 2400), abs=1e-4)
    monkeypatch.setattr(bench, "recorded_counter", lambda k, f="bytes_per_launch": None)
    assert bench.valu_roofline("mmq_q6k_limbs_q8t", 32.0, 2000) is None


def test_recorded_counter_guard(tmp_path, monkeypatch):
    """A recorded figure is returned only while the kernel sources hash to
    the digest it was taken on."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"kernel_code_sha256": bench.kernel_source_digest(), "valu_insts_per_launch": {"k": 7}}
    (prof / "mmq_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: rec["kernel_code_sha256"])
    assert bench.recorded_counter("k", "valu_insts_per_launch") == 7
    assert bench.recorded_counter("other", "valu_insts_per_launch") is None
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 64)
    assert bench.recorded_counter("k", "valu_insts_per_launch") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
