"""Host logic of bench.py's roofline traffic: per-launch HBM bytes of a
kernel from two rocprofv3 counter-collection CSVs (FETCH_SIZE, WRITE_SIZE in
KiB per dispatch), scaled by the calibration copy's reading, and the check
that drops the figure once the kernel's sources change."""
import csv
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

FIELDS = ["Kernel_Name", "Counter_Name", "Counter_Value"]


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, kib in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def test_summary_scales_by_the_copy_and_tracks_the_sources(tmp_path, monkeypatch):
    gib_kib = (1 << 30) / 1024
    # the counters read half the copy's fetched bytes and all of its writes
    write_csv(tmp_path / "f.csv", "FETCH_SIZE",
              [("prism::k_bwd_dkdv(...)", 1000.0), ("other_kernel", 5.0),
               ("void at::native::bitwise_not_kernel(...)", gib_kib / 2)])
    write_csv(tmp_path / "w.csv", "WRITE_SIZE",
              [("prism::k_bwd_dkdv(...)", 30.0),
               ("void at::native::bitwise_not_kernel(...)", gib_kib)])
    out = tmp_path / "summary.md"
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "bwd.dkdv", "wl",
                        ["cmd one"], str(out))
    monkeypatch.setattr(bench, "traffic_file", lambda stage, workload: str(out))
    got = bench.read_traffic("bwd.dkdv", "wl")
    assert got == pytest.approx(2 * 1000 * 1024 + 30 * 1024, rel=1e-5)
    # a summary taken on other sources is not reported
    text = out.read_text().replace(bench.kernel_source_sha("bwd.dkdv"), "0" * 64)
    out.write_text(text)
    assert bench.read_traffic("bwd.dkdv", "wl") is None


def test_summary_needs_exactly_one_calibration_copy(tmp_path):
    write_csv(tmp_path / "f.csv", "FETCH_SIZE", [("prism::k_bwd_dkdv(...)", 10.0)])
    write_csv(tmp_path / "w.csv", "WRITE_SIZE", [("prism::k_bwd_dkdv(...)", 10.0)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "bwd.dkdv", "wl",
                            [], str(tmp_path / "out.md"))


def test_missing_summary_reports_none(monkeypatch, tmp_path):
    monkeypatch.setattr(bench, "traffic_file", lambda stage, workload: str(tmp_path / "none.md"))
    assert bench.read_traffic("bwd.dkdv", "wl") is None
