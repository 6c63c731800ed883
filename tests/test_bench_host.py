"""Host-side logic of bench.py, no GPU: which verify kernel a profiler row
belongs to, and how the byte counters of a calibration copy turn the raw
FETCH_SIZE / WRITE_SIZE readings into HBM bytes per launch."""
import csv
import json
import os

import bench

COPY = "__amd_rocclr_copyBuffer.kd"


def test_layout_of_kernel_names():
    f = bench._layout_of
    assert f("void vq::walk_kernel<2, false, 2, 8, 4, true>(vq::KGroup)") == "panel"
    assert f("void vq::walk_kernel<1, false, 1, 8, 4, false>(vq::KGroup)") == "row_major"
    assert f("void vq::walk_kernel<2, true, 1, 8, 8, true>(vq::KGroup)") == "fp8_panel"
    assert f("void vq::walk_kernel<2, true, 1, 8, 8, false>(vq::KGroup)") == "fp8_row_major"
    assert f("void vq::oneshot_kernel<2, false, 1, 8, 4>(vq::KGroup)") is None
    assert f("vq::fp8_panel_pack_kernel(unsigned int __vector(4) const*, int, int, int, long)") is None
    assert f(COPY) is None


def _counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_from_scales_by_the_calibration_copy(tmp_path):
    panel = "void vq::walk_kernel<2, false, 2, 8, 4, true>(vq::KGroup)"
    rm = "void vq::walk_kernel<2, false, 1, 8, 4, false>(vq::KGroup)"
    f8p = "void vq::walk_kernel<2, true, 1, 8, 8, true>(vq::KGroup)"
    copy_kib = bench.COPY_BYTES // 1024
    # FETCH_SIZE reads half of the copy's bytes (scale 2); a small copy is not
    # a calibration copy; panel dispatches average 101 KiB
    _counters(str(tmp_path / "f"), "FETCH_SIZE",
              [(COPY, copy_kib / 2), (COPY, copy_kib / 2), (COPY, 1000.0), (panel, 100.0), (panel, 102.0),
               (rm, 110.0), (f8p, 200.0)])
    _counters(str(tmp_path / "w"), "WRITE_SIZE",
              [(COPY, copy_kib), (panel, 6.0), (rm, 4.0), (f8p, 8.0), (panel, 6.0)])
    out = str(tmp_path / "traffic.json")
    rec = bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"), out_path=out)
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["panel"]["read_bytes_per_launch"] == 101 * 1024 * 2
    assert rec["panel"]["write_bytes_per_launch"] == 6 * 1024
    assert rec["panel"]["hbm_bytes_per_launch"] == 101 * 2048 + 6 * 1024
    assert rec["row_major"]["hbm_bytes_per_launch"] == 110 * 2048 + 4 * 1024
    assert rec["fp8_panel"]["hbm_bytes_per_launch"] == 200 * 2048 + 8 * 1024
    assert "fp8_row_major" not in rec          # no dispatches of it in the run
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()
    with open(out) as fh:
        assert json.load(fh) == rec


def test_stored_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    path = tmp_path / "t.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.stored_traffic("panel") is None
    path.write_text(json.dumps({"kernel_source_hash": "0" * 16, "panel": {"hbm_bytes_per_launch": 5}}))
    assert bench.stored_traffic("panel") is None
    path.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(),
                                "panel": {"hbm_bytes_per_launch": 5}}))
    assert bench.stored_traffic("panel") == 5
    assert bench.stored_traffic("fp8_panel") is None


def test_gpu_state_parsing():
    clocks = {"card0": {"fclk clock speed:": "(1600Mhz)", "mclk clock speed:": "(1300Mhz)",
                        "sclk clock speed:": "(2400Mhz)", "sclk clock level:": "1", "Card Series": "x"},
              "system": {"note": 1}}
    assert bench.smi_clocks(clocks) == {"card0": {"fclk": "(1600Mhz)", "mclk": "(1300Mhz)", "sclk": "(2400Mhz)"}}
    pids = {"system": {"PID77": "python3, 1, 1024, 0, 0", "PID5": "other, 1, 0, 0, 0", "Note": "x"}}
    assert bench.smi_other_processes(pids, 77) == [(5, "other")]
    assert bench.smi_other_processes({"system": {}}, 1) == []
    assert bench.smi_clocks(None) is None and bench.smi_other_processes(None, 1) is None


def test_mhz():
    assert bench.mhz("(2100Mhz)") == 2100.0
    assert bench.mhz("n/a") is None
