"""C-ABI checks that need no GPU: the library loads, exports every entry
point declared in include/prism.h, validates configurations on the host and
carries the same candidate table as the oracle (two independent listings)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def nat():
    from dynamic_block_sparse_zone_amd import _native
    if not os.path.exists(_native.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    _native.lib()
    return _native


def declared_functions():
    src = open(os.path.join(ROOT, "include", "prism.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(prism_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(nat):
    decl = declared_functions()
    assert len(decl) >= 12
    L = nat.lib()
    for name in decl:
        assert hasattr(L, name), name
    assert sorted(nat.EXPORTED) == decl


def _cfg(nat, **kw):
    c = nat.PrismConfig()
    nat.lib().prism_config_default(ctypes.byref(c))
    c.T, c.H, c.W, c.heads, c.head_dim = 16, 16, 16, 2, 128
    for k, v in kw.items():
        if k == "fixed_shape":
            for i in range(3):
                c.fixed_shape[i] = v[i]
        else:
            setattr(c, k, v)
    return c


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    ({"T": 12}, 1), ({"H": 0}, 1), ({"heads": 0}, 1), ({"head_dim": 96}, 2),
    ({"dtype": 5}, 1), ({"top_k": -1}, 1), ({"top_p": float("nan")}, 1), ({"top_p": -0.1}, 1),
    ({"volume_mask": 0}, 1), ({"volume_mask": 9}, 1), ({"fixed_shape": (4, 4, 4)}, 0),
    ({"fixed_shape": (4, 4, 3)}, 1), ({"fixed_shape": (8, 8, 8)}, 1), ({"eps": 0.0}, 1),
    ({"tau128": 0.2, "tau256": 0.3}, 1), ({"top_k_frac": -1.0}, 1), ({"top_p": 1.5}, 0),
    # one head's rows are addressed with 32-bit byte offsets: fewer than 2^24 tokens
    ({"T": 256, "H": 256, "W": 256}, 2), ({"T": 248, "H": 256, "W": 256}, 0),
])
def test_config_validation(nat, kw, status):
    c = _cfg(nat, **kw)
    assert nat.lib().prism_config_check(ctypes.byref(c)) == status


def test_null_and_size_errors(nat):
    L = nat.lib()
    c = _cfg(nat)
    n = ctypes.c_size_t()
    assert L.prism_plan_workspace_size(None, 0, ctypes.byref(n)) == nat.PRISM_EINVAL
    assert L.prism_plan_workspace_size(ctypes.byref(c), 0, None) == nat.PRISM_EINVAL
    assert L.prism_plan_workspace_size(ctypes.byref(c), 0, ctypes.byref(n)) == 0
    small = n.value
    assert L.prism_plan_workspace_size(ctypes.byref(c), 1000, ctypes.byref(n)) == 0
    assert n.value >= small + 1000 * 8
    h = ctypes.c_void_p()
    nn = ctypes.c_int64()
    assert L.prism_plan_create(ctypes.byref(c), None, None, None, None, None, 0, None,
                               ctypes.byref(h), ctypes.byref(nn)) == nat.PRISM_EINVAL
    assert L.prism_attn_fwd(None, None, None, None, None, None, None) == nat.PRISM_EINVAL
    assert L.prism_attn_bwd(None, *([None] * 10), 0, None) == nat.PRISM_EINVAL
    assert L.prism_plan_export(None, 0, None, 0, None) == nat.PRISM_EINVAL
    assert L.prism_block_scores(None, 0, None, None) == nat.PRISM_EINVAL
    assert L.prism_candidate(16, (ctypes.c_int32 * 4)()) == nat.PRISM_EINVAL
    for s in range(6):
        assert len(nat.status_str(s)) > 0


def test_candidate_table_matches_oracle(nat, orc):
    a = (ctypes.c_int32 * 4)()
    for i, row in enumerate(orc.candidates()):
        assert nat.lib().prism_candidate(i, a) == 0
        assert tuple(a) == tuple(int(x) for x in row)


def test_sparsity_schedules(nat):
    """paper.rainbus.top "独立分析的弱点" (4): schedules of a sparsity
    hyper-parameter over steps, against their closed forms."""
    import math
    from dynamic_block_sparse_zone_amd import api
    f32 = lambda x: float(ctypes.c_float(x).value)
    for kind in ("constant", "linear", "cosine"):
        assert api.schedule_value(kind, 0, 10, 0.9, 0.2) == f32(0.9)
        assert api.schedule_value(kind, 0, 1, 0.9, 0.2) == f32(0.9)
    assert api.schedule_value("constant", 9, 10, 0.9, 0.2) == f32(0.9)
    for kind in ("linear", "cosine"):
        assert api.schedule_value(kind, 9, 10, 0.9, 0.2) == f32(0.2)
        assert api.schedule_value(kind, 99, 10, 0.9, 0.2) == f32(0.2)      # clamped
        vals = [api.schedule_value(kind, s, 21, 0.9, 0.2) for s in range(21)]
        assert all(a >= b for a, b in zip(vals, vals[1:]))                 # monotone
    assert api.schedule_value("linear", 5, 11, 0.0, 1.0) == f32(0.5)
    assert abs(api.schedule_value("cosine", 5, 11, 0.0, 1.0) - 0.5) < 1e-7
    s = 3 / 10
    assert abs(api.schedule_value("cosine", 3, 11, 1.0, 0.0) -
               (0.5 * (1 + math.cos(math.pi * s)))) < 1e-7
    out = ctypes.c_float()
    L = nat.lib()
    assert L.prism_schedule_value(7, 0, 10, 0.1, 0.2, ctypes.byref(out)) == 1
    assert L.prism_schedule_value(1, 0, 0, 0.1, 0.2, ctypes.byref(out)) == 1
    assert L.prism_schedule_value(1, 0, 10, float("nan"), 0.2, ctypes.byref(out)) == 1
