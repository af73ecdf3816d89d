"""Parity of the plan stages on the GPU with the CPU oracle: zone statistics,
shapes, block table, permutation, pooled means and their integer grid, block
scores and the selected key-block lists must match bit for bit."""
import numpy as np
import pytest
import torch

from dynamic_block_sparse_zone_amd import synth
from tests.helpers import csr_rows, gpu_plan, host_bits, oracle_config, to_dev

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def prism():
    import dynamic_block_sparse_zone_amd as p
    return p


def _case(prism, orc, name, use_audio=True, **over):
    wl = synth.WORKLOADS[name]
    x = synth.make_inputs(wl, device="cpu", with_grad=False)
    print(f"[plan parity] workload={name} over={over} audio={use_audio}", flush=True)
    dx = to_dev(x, DEV)
    pl = gpu_plan(prism, wl, dx, use_audio=use_audio, **over)
    torch.cuda.synchronize()
    hb = host_bits(x)
    cfg = oracle_config(orc, wl, **over)
    opl = orc.plan(hb["q"], hb["k"], hb["v"], x["av"].numpy() if use_audio else None, cfg)
    return wl, pl, opl


def _check_plan_arrays(pl, opl, cfg):
    H, Z = cfg.heads, cfg.Z
    np.testing.assert_array_equal(pl.export("zone_stats").reshape(H, Z, 5), opl.vstats)
    if opl.astats is not None:
        np.testing.assert_array_equal(pl.export("audio_stats").reshape(Z, 4), opl.astats)
    np.testing.assert_array_equal(pl.export("shape_id").reshape(H, Z), opl.shape_id)
    np.testing.assert_array_equal(pl.export("blk_off"), opl.blk_off)
    G = int(opl.blk_off[-1])
    start = pl.export("blk_start")
    np.testing.assert_array_equal(start[:G], opl.blk_start)
    np.testing.assert_array_equal(pl.export("perm").reshape(H, -1), opl.perm)
    # each block's first token: where the attention kernels start the
    # block -> token map of its rows
    heads_of = np.repeat(np.arange(H), np.diff(opl.blk_off))
    np.testing.assert_array_equal(pl.export("blk_org")[:G], opl.perm[heads_of, opl.blk_start])
    D = cfg.head_dim
    np.testing.assert_array_equal(pl.export("qbar").reshape(G, D), opl.qbar)
    np.testing.assert_array_equal(pl.export("kbar").reshape(G, D), opl.kbar)
    np.testing.assert_array_equal(pl.export("qexp"), opl.qexp)
    np.testing.assert_array_equal(pl.export("kexp"), opl.kexp)
    qg = pl.export("qgrid").reshape(G, D)
    kg = pl.export("kgrid").reshape(G, D)
    to_f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(to_f(qg), opl.qgrid)
    np.testing.assert_array_equal(to_f(kg), opl.kgrid)
    np.testing.assert_array_equal(to_f(pl.export("qlo").reshape(G, D)), opl.qlo)
    np.testing.assert_array_equal(to_f(pl.export("klo").reshape(G, D)), opl.klo)


def _check_csr(pl, opl, orc, rows_per_head=None, seed=0):
    cfg = opl.cfg
    row_ptr = pl.export("row_ptr")
    col = pl.export("col_idx")
    assert row_ptr[-1] == pl.nnz == len(col)
    rng = np.random.default_rng(seed)
    checked = 0
    for h in range(cfg.heads):
        n = opl.nblk(h)
        rows = range(n) if rows_per_head is None else rng.choice(n, min(n, rows_per_head),
                                                                replace=False)
        for i in rows:
            g = int(opl.blk_off[h]) + int(i)
            got = csr_rows(row_ptr, col, g)
            want = orc.select_row(opl, h, int(i))
            assert np.array_equal(got, want), (h, i, got[:10], want[:10])
            checked += 1
        # every row, any size: ascending, in range, at least k long
        k = cfg.k_for(n)
        for i in range(n):
            r = csr_rows(row_ptr, col, int(opl.blk_off[h]) + i)
            assert len(r) >= k and (len(r) == 0 or (r[0] >= 0 and r[-1] < n))
            assert np.all(np.diff(r) > 0)
    return checked


def _check_transpose(pl, opl):
    cfg = opl.cfg
    row_ptr, col = pl.export("row_ptr"), pl.export("col_idx")
    tp, tc = pl.export("colt_ptr"), pl.export("colt_idx")
    assert tp[-1] == len(col) == len(tc)
    for h in range(cfg.heads):
        o, n = int(opl.blk_off[h]), opl.nblk(h)
        lists = [[] for _ in range(n)]
        for i in range(n):
            for j in csr_rows(row_ptr, col, o + i):
                lists[j].append(i)
        for j in range(n):
            assert np.array_equal(csr_rows(tp, tc, o + j), np.array(lists[j], np.int32)), (h, j)


@pytest.mark.parametrize("name", ["tiny", "check", "small"])
def test_plan_bit_exact(prism, orc, name):
    wl, pl, opl = _case(prism, orc, name)
    _check_plan_arrays(pl, opl, opl.cfg)
    _check_csr(pl, opl, orc)
    _check_transpose(pl, opl)
    info = pl.info()
    assert info["nnz"] == pl.nnz and info["total_blocks"] == int(opl.blk_off[-1])
    hist = np.bincount(opl.shape_id.reshape(-1), minlength=16)
    assert info["shape_hist"] == hist.tolist()


def test_plan_first_layer_without_audio(prism, orc):
    wl, pl, opl = _case(prism, orc, "check", use_audio=False)
    _check_plan_arrays(pl, opl, opl.cfg)
    _check_csr(pl, opl, orc)


@pytest.mark.parametrize("over", [
    {"top_p": 1.0},                    # every block
    {"top_p": 0.0, "top_k": 5},        # Top-k only
    {"top_p": 0.0, "top_k": 0},        # empty selection
    {"top_k": 1000, "top_p": 0.5},     # k larger than the block count
    {"top_k_frac": 0.05, "top_p": 0.2},  # the pages' operating point
    {"fixed_shape": (4, 4, 8)},
    {"volume_mask": 5},
    {"tau128": 0.9, "tau256": 0.6},
])
def test_plan_variants(prism, orc, over):
    wl, pl, opl = _case(prism, orc, "check", **over)
    _check_plan_arrays(pl, opl, opl.cfg)
    _check_csr(pl, opl, orc)


@pytest.mark.parametrize("shape_map,alpha", [(0, 1 / 3), (0, 2.0), (1, 0.5), (2, 0.5),
                                             (3, 0.5), (4, 0.5)])
def test_shape_map_variants(prism, orc, shape_map, alpha):
    """The shape-mapping ablations (power alpha = 1/3 and 2, isotropic,
    softmax, rank, entropy) give the oracle's shapes, block table and lists
    bit for bit."""
    for name in ("check", "small"):
        wl, pl, opl = _case(prism, orc, name, shape_map=shape_map, alpha=alpha)
        _check_plan_arrays(pl, opl, opl.cfg)
        _check_csr(pl, opl, orc, rows_per_head=None if name == "check" else 40)
        pl.close()


def test_block_scores_bit_exact(prism, orc):
    wl, pl, opl = _case(prism, orc, "small")
    rng = np.random.default_rng(3)
    for h in (0, wl.heads - 1):
        s = prism.block_scores(pl, h).cpu().numpy()
        for i in rng.choice(opl.nblk(h), 12, replace=False):
            np.testing.assert_array_equal(s[i], orc.score_row(opl, h, int(i)))


@pytest.mark.parametrize("name", ["check", "small"])
def test_block_scores_every_row(prism, orc, name):
    """Every score of one head (a block count that is not a multiple of the
    kernel's 128 x 128 tiles, so the ragged last tiles are covered) equals
    the oracle's row bit for bit."""
    wl, pl, opl = _case(prism, orc, name)
    h = wl.heads - 1
    s = prism.block_scores(pl, h).cpu().numpy()
    n = opl.nblk(h)
    assert s.shape == (n, n)
    if name == "small":
        assert n % 128 != 0, n
    for i in range(n):
        np.testing.assert_array_equal(s[i], orc.score_row(opl, h, i))


def test_plan_deterministic(prism):
    wl = synth.WORKLOADS["small"]
    dx = to_dev(synth.make_inputs(wl, device="cpu", with_grad=False), DEV)
    a = gpu_plan(prism, wl, dx)
    b = gpu_plan(prism, wl, dx)
    for name in ("shape_id", "row_ptr", "col_idx", "colt_idx", "qbar", "zone_stats"):
        assert np.array_equal(a.export(name), b.export(name)), name


@pytest.mark.parametrize("over", [{}, {"fixed_shape": (4, 4, 8)}, {"top_p": 1.0}])
def test_kv_order(prism, over):
    """The dK/dV kernel's unit order: per head a permutation of the 128-row
    units, longest walk first (the longest key-major list among the unit's
    key blocks, counted in 64-row tiles of the query blocks it names), ties
    by unit index.  Recomputed here from the exported lists."""
    wl = synth.WORKLOADS["small"]
    print(f"[kv order] over={over}", flush=True)
    dx = to_dev(synth.make_inputs(wl, device="cpu", with_grad=False), DEV)
    pl = gpu_plan(prism, wl, dx, **over)
    N = wl.T * wl.H * wl.W
    upH = N // 128
    order = pl.export("kv_order").reshape(wl.heads, upH)
    off, start = pl.export("blk_off"), pl.export("blk_start")
    cptr, cidx = pl.export("colt_ptr"), pl.export("colt_idx")
    for h in range(wl.heads):
        b0, b1 = int(off[h]), int(off[h + 1])
        st = start[b0:b1].astype(np.int64)
        tiles = np.diff(np.append(st, N)) // 64
        work = np.array([tiles[cidx[cptr[b0 + j]:cptr[b0 + j + 1]]].sum() for j in range(b1 - b0)])
        unit_work = np.zeros(upH, np.int64)
        for u in range(upH):
            r0 = u * 128
            first = np.searchsorted(st, r0, side="right") - 1
            last = np.searchsorted(st, r0 + 128, side="left")
            unit_work[u] = work[first:max(last, first + 1)].max()
        want = sorted(range(upH), key=lambda u: (-min(int(unit_work[u]), 16383), u))
        np.testing.assert_array_equal(order[h], np.array(want, np.int32))


def test_shot_cut_zones(prism, orc):
    """Shot-cut-aware temporal zones: the GPU finds the oracle's cuts (the
    two spliced shots of the cuts workload; the energies of every frame are
    far from the threshold) and gives its shapes, block table and lists bit
    for bit."""
    wl = synth.WORKLOADS["cuts"]
    wl_, pl, opl = _case(prism, orc, "cuts", cut_threshold=4.0)
    got = pl.export("cuts")
    _, energy = orc.detect_cuts(synth.to_numpy_bits(
        synth.make_inputs(wl, device="cpu", with_grad=False)["v"]), opl.cfg)
    thr = 4.0 * energy[1:].mean()
    assert np.all(np.abs(energy[1:] - thr) > 1e-6 * thr)      # no decision near the threshold
    np.testing.assert_array_equal(got, opl.cuts)
    assert np.nonzero(got)[0].tolist() == list(wl.cut_frames)
    _check_plan_arrays(pl, opl, opl.cfg)
    _check_csr(pl, opl, orc)


def test_schedule_gives_nested_selections(prism, orc):
    """A Top-p schedule loosening from 0.2 to 0.9 over the steps: each step's
    selection holds the previous one (both are prefixes of one order), and
    each is the oracle's for its p."""
    wl = synth.WORKLOADS["check"]
    x = synth.make_inputs(wl, device="cpu", with_grad=False)
    dx = to_dev(x, DEV)
    hb = host_bits(x)
    prev = None
    for step in range(4):
        p = prism.schedule_value("cosine", step, 4, 0.2, 0.9)
        pl = gpu_plan(prism, wl, dx, top_p=p)
        rp, col = pl.export("row_ptr"), pl.export("col_idx")
        rows = [set(col[rp[g]:rp[g + 1]].tolist()) for g in range(len(rp) - 1)]
        if prev is not None:
            assert all(a <= b for a, b in zip(prev, rows))
        prev = rows
        opl = orc.plan(hb["q"], hb["k"], hb["v"], x["av"].numpy(),
                       oracle_config(orc, wl, top_p=p))
        _check_csr(pl, opl, orc, rows_per_head=30, seed=step)
        pl.close()
