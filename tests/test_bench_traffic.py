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


def _write_rows(path, rows):
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(fields, r)))


def test_hbm_table_rates(tmp_path):
    gib_kib = (1 << 30) / 1024
    # a kernel fetching 1 GB (its counter reads half) and writing 1 GB in 1 s
    _write_rows(tmp_path / "f.csv", [
        ("prism::k_x(int)", "FETCH_SIZE", 1e9 / 1024 / 2, 0, 10**9),
        ("void at::native::bitwise_not_kernel", "FETCH_SIZE", gib_kib / 2, 0, 10**6)])
    _write_rows(tmp_path / "w.csv", [
        ("prism::k_x(int)", "WRITE_SIZE", 1e9 / 1024, 0, 10**9),
        ("void at::native::bitwise_not_kernel", "WRITE_SIZE", gib_kib, 0, 10**6)])
    out = tmp_path / "t.md"
    bench.summarize_hbm_table(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "wl", [], str(out))
    row = [l for l in out.read_text().splitlines() if l.startswith("| `k_x`")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    # time 1000 ms, fetch and write 1.00 GB each, 0.002 TB/s
    assert float(cells[2]) == pytest.approx(1000.0)
    assert cells[3] == "1.00" and cells[4] == "1.00" and cells[5] == "0.00"


def test_mfma_summary_uses_the_xcd_count(tmp_path):
    # 2 s at 2 GHz on 8 XCDs; half of 1024 SIMDs' cycles busy
    t = 2 * 10**9
    gui = 2.0e9 * 2 * 8
    busy = 0.5 * 2.0e9 * 2 * 1024
    _write_rows(tmp_path / "m.csv", [
        ("prism::k_attn_fwd_bf16(x)", "SQ_VALU_MFMA_BUSY_CYCLES", busy, 0, t),
        ("prism::k_attn_fwd_bf16(x)", "GRBM_GUI_ACTIVE", gui, 0, t),
        ("prism::k_attn_fwd_bf16(x)", "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e15 / 512, 0, t)])
    with open(tmp_path / "a.csv", "w") as f:
        f.write("Simd_Count,Num_Xcc\n0,0\n1024,8\n")
    out = tmp_path / "m.md"
    bench.summarize_mfma(str(tmp_path / "m.csv"), str(tmp_path / "a.csv"), "wl", [], str(out))
    row = [l for l in out.read_text().splitlines() if "k_attn_fwd_bf16" in l][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[2] == "2.00" and cells[3] == "50.0" and cells[4] == "500.0"
