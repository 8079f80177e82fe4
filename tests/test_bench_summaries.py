"""bench.py's profile summaries, on small hand-made counter and trace files (no GPU).

The profiles/ summaries turn rocprofv3 CSVs into per-forward figures; these tests check
that arithmetic on inputs whose answers are known: the copy calibration of FETCH_SIZE /
WRITE_SIZE, the division by the number of forwards, the exclusion of set-up and torch
kernels, the MFMA rate / clock / busy share, the per-forward kernel table, and the source
hash that decides whether a recorded traffic figure still applies.
"""
import csv
import json
import os

import pytest

import bench

KIB = 1024.0


def write_counter_csv(path, rows):
    """rows: (dispatch_id, kernel name, counter, value, start_ns, end_ns)."""
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                    "End_Timestamp"])
        for r in rows:
            w.writerow(r)


def test_hbm_traffic_calibrated_per_forward(tmp_path, monkeypatch):
    calib_kib = bench.CALIB_BYTES / KIB
    # FETCH_SIZE reads half the true bytes (as measured on the chip), WRITE_SIZE all of them.
    fetch = [(1, "void smoe::(anonymous namespace)::gg_up_kernel<false, 0>(UpArgs)", "FETCH_SIZE", 500.0 / 2, 0, 1),
             (2, "void smoe::(anonymous namespace)::gg_up_kernel<false, 0>(UpArgs)", "FETCH_SIZE", 700.0 / 2, 0, 1),
             (3, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 9e9, 0, 1),
             (4, "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel(...)", "FETCH_SIZE",
              calib_kib / 2, 0, 1)]
    write = [(1, "void smoe::(anonymous namespace)::gg_up_kernel<false, 0>(UpArgs)", "WRITE_SIZE", 100.0, 0, 1),
             (2, "void smoe::(anonymous namespace)::gg_up_kernel<false, 0>(UpArgs)", "WRITE_SIZE", 300.0, 0, 1),
             (4, "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel(...)", "WRITE_SIZE",
              calib_kib, 0, 1)]
    fcsv, wcsv, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.md"
    write_counter_csv(fcsv, fetch)
    write_counter_csv(wcsv, write)
    bench.summarize_pmc(str(fcsv), str(wcsv), "qwen_prefill_t8192", str(out), "cmd", forwards=2)
    text = out.read_text()
    rec = json.loads(text.split("traffic_json: ")[1])
    # (500 + 700 + 100 + 300) KiB over 2 forwards; the runtime copy and the calibration
    # kernel are not the layer's.
    assert rec["bytes_per_forward"] == pytest.approx(1600 * KIB / 2)
    assert "rocclr" not in text
    assert rec["csrc_hash"] == bench.kernel_source_hash()


def test_mfma_summary_rate_clock_and_busy(tmp_path):
    name = "void smoe::(anonymous namespace)::gg_up_kernel<false, 0>(smoe::(anonymous namespace)::UpArgs)"
    t_ns = 400_000  # 400 us per dispatch
    grbm = 8 * 2.0e9 * t_ns * 1e-9  # 8 XCDs at 2.0 GHz
    mops = 1.0e15 * t_ns * 1e-9 / 512  # 1 PFLOP/s
    busy = 0.5 * (grbm / 8) * bench.N_SIMD
    rows = []
    for disp in (1, 2):
        rows += [(disp, name, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops, 0, t_ns),
                 (disp, name, "SQ_VALU_MFMA_BUSY_CYCLES", busy, 0, t_ns),
                 (disp, name, "GRBM_GUI_ACTIVE", grbm, 0, t_ns)]
    path, out = tmp_path / "m.csv", tmp_path / "m.md"
    write_counter_csv(path, rows)
    bench.summarize_mfma(str(path), "qwen_prefill_t8192", str(out), "cmd")
    line = [l for l in out.read_text().splitlines() if "gg_up_kernel" in l][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    # kernel | dispatches | avg us | GFLOP | PFLOP/s | of peak | clock | busy
    assert cells[1] == "2" and float(cells[2]) == pytest.approx(400.0)
    assert float(cells[3]) == pytest.approx(400.0, rel=1e-3)   # 1 PFLOP/s x 400 us
    assert float(cells[4]) == pytest.approx(1.0, rel=1e-3)
    assert float(cells[5]) == pytest.approx(1.0e15 / bench.MFMA_BF16_PEAK, abs=1e-3)
    assert float(cells[6]) == pytest.approx(2.0, abs=0.01)
    assert float(cells[7]) == pytest.approx(0.5, abs=1e-3)


def test_kernel_stats_per_forward(tmp_path):
    stats = tmp_path / "s.csv"
    with open(stats, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"])
        w.writerow(["void smoe::(anonymous namespace)::expert_up_gemv_kernel<4>(GemvUp)", 10, 1_000_000, 100_000,
                    50, 90_000, 110_000])
        w.writerow(["void smoe::(anonymous namespace)::expert_down_gemv_kernel<1>(GemvDown)", 10, 500_000, 50_000,
                    25, 40_000, 60_000])
        w.writerow(["__amd_rocclr_copyBuffer", 3, 9_000_000, 3_000_000, 25, 1, 1])
    log = tmp_path / "run.log"
    log.write_text('noise\n{"forward_only": {"workload": "qwen_decode_t64", "ms_per_step": 0.16, '
                   '"steps": 8, "warmup": 2}}\n')
    bj = tmp_path / "bench.json"
    bj.write_text(json.dumps({"config": {"workload": "qwen_decode_t64"}, "ms_per_step": 0.15, "sweep": []}) + "\n")
    out = tmp_path / "k.md"
    bench.summarize_stats(str(stats), str(log), "qwen_decode_t64", str(out), "cmd", str(bj))
    text = out.read_text()
    # (1 ms + 0.5 ms) over 10 forwards = 150 us per forward; the copy is left out.
    assert "150.0 us per forward" in text
    assert "copyBuffer" not in text
    assert "kernels / step = 93.8%" in text    # 150 / 160 under the profiler
    assert "kernels / step = 100.0%" in text   # 150 / 150 without it


def test_recorded_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_file", lambda w: str(tmp_path / f"{w}.md"))
    good = {"workload": "x", "bytes_per_forward": 123.0, "csrc_hash": bench.kernel_source_hash()}
    (tmp_path / "x.md").write_text("# t\n\ntraffic_json: " + json.dumps(good) + "\n")
    assert bench.recorded_traffic("x") == 123.0
    stale = dict(good, csrc_hash="0" * 16)
    (tmp_path / "y.md").write_text("traffic_json: " + json.dumps(stale) + "\n")
    assert bench.recorded_traffic("y") is None
    assert bench.recorded_traffic("absent") is None


def test_every_default_sweep_workload_has_profiles():
    root = os.path.dirname(os.path.abspath(bench.__file__))
    for w in [bench.DEFAULT] + bench.DEFAULT_SWEEP:
        assert w in bench.WORKLOADS
        assert os.path.exists(os.path.join(root, "profiles", f"{w}_kernel_stats.md")), w
        assert os.path.exists(os.path.join(root, "profiles", f"{w}_hbm_traffic.md")), w
