"""The decision report (integer-grid block scores and fp32 shape arithmetic
against plain fp64 decisions) runs and stays near the fp64 decisions on the
small workloads.  The numbers are reported, not a parity gate: the bounds
below only catch a report, or a reading, that has gone badly wrong."""
from dynamic_block_sparse_zone_amd import synth
from tests import decision_report as R


def test_decision_report_tiny_and_check(orc):
    for name in ("tiny", "check"):
        r = R.report(orc, synth.WORKLOADS[name])
        assert r["rows"] > 0 and r["zones"] > 0
        assert r["shape_differs"] <= r["zones"] // 20, r
        assert r["jaccard_mean"] > 0.99 and r["jaccard_min"] > 0.8, r
        assert abs(r["mass_grid_mean"] - r["mass_fp64_mean"]) < 1e-3, r
