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
    """rows: (kernel name, KiB[, duration ns]); dispatches run back to back"""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS + ["Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for name, kib, *dur in rows:
            d = dur[0] if dur else 1000
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib,
                        "Start_Timestamp": t, "End_Timestamp": t + d})
            t += d


def test_summary_scales_by_the_copy_and_tracks_the_sources(tmp_path, monkeypatch):
    gib_kib = (1 << 30) / 1024
    # the counters read half the copy's fetched bytes and all of its writes;
    # the kernel's short first dispatch (a small warm-up grid) is not the launch
    write_csv(tmp_path / "f.csv", "FETCH_SIZE",
              [("prism::k_bwd_dkdv(...)", 7.0, 50), ("prism::k_bwd_dkdv(...)", 1000.0, 9000),
               ("other_kernel", 5.0),
               ("void at::native::bitwise_not_kernel(...)", gib_kib / 2)])
    write_csv(tmp_path / "w.csv", "WRITE_SIZE",
              [("prism::k_bwd_dkdv(...)", 3.0, 50), ("prism::k_bwd_dkdv(...)", 30.0, 9000),
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
    # the copy moves 2 GiB in 1 ms: 2.15 TB/s, of which 0.002 TB/s is 0.1 %
    assert "2.15 TB/s" in out.read_text() and cells[7] == "0.1"


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


def test_stall_summary_takes_each_kernels_longest_dispatch(tmp_path):
    """The stall table reads the full-size dispatch (the longest) of each
    attention kernel and gives fractions of the resident wave-cycles."""
    rows_a, rows_b = [], []
    for dur, scale in ((100, 1.0), (10**6, 10.0)):   # a warm-up dispatch, then the launch
        for n, v in zip(bench.STALL_COUNTERS_A, (1000, 300, 200, 10, 500, 250, 40, 100)):
            rows_a.append(("prism::k_bwd_dkdv<true>(int)", n, v * scale, 0, dur))
        for n, v in zip(bench.STALL_COUNTERS_B, (5, 0, 500, 150, 500, 100, 1000, 0)):
            rows_b.append(("prism::k_bwd_dkdv<true>(int)", n, v * scale, 0, dur))
    for path, rows in (("a.csv", rows_a), ("b.csv", rows_b)):
        with open(tmp_path / path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value",
                                              "Start_Timestamp", "End_Timestamp", "Dispatch_Id"])
            w.writeheader()
            for i, r in enumerate(rows):
                w.writerow({"Kernel_Name": r[0], "Counter_Name": r[1], "Counter_Value": r[2],
                            "Start_Timestamp": r[3], "End_Timestamp": r[4],
                            "Dispatch_Id": 1 if r[4] == 100 else 2})
    out = tmp_path / "s.md"
    bench.summarize_stalls(str(tmp_path / "a.csv"), str(tmp_path / "b.csv"), "wl", [], str(out))
    row = [l for l in out.read_text().splitlines() if l.startswith("| `k_bwd_dkdv")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1:4] == ["30.0 %", "20.0 %", "50.0 %"]
    assert cells[7] == "1.00 %"          # 5 of 500 LDS-active cycles
    assert cells[8] == "4.00"            # (500 - 100) VALU per 100 MFMA


def test_wave_utilisation_counts_idle_waves():
    """One 256-row unit of four 64-token query blocks whose lists are {0, 1},
    {0}, {} and {1} (64-token key blocks): the unit steps through 2 tiles with
    8 waves (16 wave-steps) and its waves compute 4 + 2 + 0 + 2 of them."""
    import numpy as np

    class FakePlan:
        arrays = {"blk_off": np.array([0, 4]), "row_ptr": np.array([0, 2, 3, 3, 4]),
                  "col_idx": np.array([0, 1, 0, 1]), "blk_start": np.array([0, 64, 128, 192]),
                  "shape_id": np.array([0], dtype=np.uint8)}

        def export(self, name):
            return self.arrays[name]

    class Wl:
        N = 512
        heads = 1

    assert bench.wave_utilisation(FakePlan(), Wl(), (0,)) == {0: 0.5}


def test_trace_summary_groups_the_librarys_kernels(tmp_path):
    """The kernel-trace summary reads the rocpd database's kernels view:
    the library's kernels by name (templates kept), their totals, average
    and longest dispatch with its launch shape; everything else counted
    apart; the header says what the traced command ran."""
    import sqlite3
    db = tmp_path / "run_results.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, duration integer, grid_x integer, "
                "grid_y integer, workgroup_x integer, vgpr_count integer, "
                "accum_vgpr_count integer, lds_size integer)")
    rows = [("void prism::k_frame_energy<1>(void const*, long)", 3_000_000, 18176, 40, 256, 28,
             0, 2048),
            ("void prism::k_frame_energy<1>(void const*, long)", 5_000_000, 18176, 40, 256, 28,
             0, 2048),
            ("prism::k_cuts(double const*, int)", 20_000, 256, 1, 256, 8, 0, 0),
            ("at::native::elementwise_kernel", 7_000_000, 1, 1, 64, 4, 0, 0)]
    con.executemany("insert into kernels values (?, ?, ?, ?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()
    out = tmp_path / "trace.md"
    bench.summarize_trace(str(db), "train2k", ["cmd one"], str(out), "upstream")
    text = out.read_text()
    assert text.startswith("# Kernel trace, train2k (upstream)")
    assert bench.TRACE_WHAT["upstream"] in text
    fe = [l for l in text.splitlines() if l.startswith("| `k_frame_energy<1>`")]
    assert len(fe) == 1
    cells = [c.strip() for c in fe[0].strip("|").split("|")]
    assert cells[1:5] == ["2", "8.000", "4.000", "5.000"]
    assert "Other (input generation, torch) kernels: 1 dispatches, 7.0 ms." in text
    # the kernels' order: by total time
    assert text.index("k_frame_energy") < text.index("k_cuts")


def test_upstream_oracle_leg_on_a_small_grid():
    """The oracle's leg beside the upstream kernels runs on host copies of
    bounded samples and reports a rate for each (CPU tensors stand in for
    the device ones here)."""
    from dynamic_block_sparse_zone_amd import synth
    wl = synth.WORKLOADS["check"]
    x = synth.make_inputs(wl, device="cpu", with_grad=False)
    a = synth.make_audio(wl, 64, device="cpu")
    res = bench.upstream_cpu(x, a, wl, threads=2, av_tokens=256, cut_heads=2)
    assert res["av_norm"]["kind"] == res["cuts"]["kind"] == "oracle"
    assert res["av_norm"]["value"] > 0 and res["cuts"]["value"] > 0
    assert "256 random tokens" in res["av_norm"]["sample"]
    assert "2 of 3 heads" in res["cuts"]["sample"]
