"""Selection over block-score rows longer than the 16,384 entries the
register selection holds: one head of 64 x 128 x 136 tokens with 64-token
blocks only, 17,408 key blocks per row, where the rows are selected from
global memory by the exact radix select (xyznot.com/id "Metode" 3:
S_i = TopK(P_i, k) U TopP(P_i, p)) and their masks are built from the lists.
Every CSR row is compared bit for bit with the oracle, the key-major
transpose (built from those masks) is checked to be exactly its transpose,
and two sampled query blocks go through the forward."""
import os

import numpy as np
import pytest
import torch

from dynamic_block_sparse_zone_amd import synth
from tests.helpers import compare_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
THREADS = max(1, min(16, int(os.environ.get("OMP_NUM_THREADS", 0) or os.cpu_count() or 1)))
WL = synth.Workload("longrow", 64, 128, 136, 1, 128, "bf16", top_k=16, top_p=0.9,
                    volume_mask=1, seed=1008)


@pytest.fixture(scope="module")
def run(orc):
    import dynamic_block_sparse_zone_amd as prism
    x = synth.make_inputs(WL, device="cpu", with_grad=False)
    print(f"[longrow] {WL.T}x{WL.H}x{WL.W}, {WL.Z * 8} blocks per head", flush=True)
    dx = {n: x[n].to(DEV) for n in ("q", "k", "v", "av")}
    pl = prism.plan(dx["q"], dx["k"], dx["v"], dx["av"], T=WL.T, H=WL.H, W=WL.W,
                    top_k=WL.top_k, top_p=WL.top_p, volume_mask=WL.volume_mask)
    o, lse = prism.attn_fwd(pl, dx["q"], dx["k"], dx["v"])
    torch.cuda.synchronize()
    got = {n: pl.export(n) for n in ("blk_off", "row_ptr", "col_idx", "colt_ptr", "colt_idx")}
    got["o"], got["lse"] = o[0].float().cpu().numpy(), lse[0].cpu().numpy()
    pl.close()
    bits = {n: synth.to_numpy_bits(x[n]) for n in ("q", "k", "v")}
    cfg = orc.Config(WL.T, WL.H, WL.W, 1, WL.head_dim, top_k=WL.top_k, top_p=WL.top_p,
                     volume_mask=WL.volume_mask)
    opl = orc.plan(bits["q"], bits["k"], bits["v"], x["av"].numpy(), cfg)
    row_ptr, col = orc.select_all(opl, threads=THREADS)
    return got, opl, row_ptr, col, bits


def test_rows_longer_than_lds(run):
    got, opl, row_ptr, col, _ = run
    assert opl.nblk(0) == WL.Z * 8 > 16384
    assert np.array_equal(got["blk_off"], opl.blk_off)
    assert np.array_equal(got["row_ptr"], row_ptr)
    assert np.array_equal(got["col_idx"], col)


def test_transpose_of_long_rows(run):
    got, opl, row_ptr, col, _ = run
    n = opl.nblk(0)
    rows = np.repeat(np.arange(n, dtype=np.int64), np.diff(row_ptr))
    order = np.lexsort((rows, col))
    assert np.array_equal(got["colt_ptr"],
                          np.concatenate([[0], np.cumsum(np.bincount(col, minlength=n))]))
    assert np.array_equal(got["colt_idx"], rows[order].astype(np.int32))


def test_forward_sampled(run, orc):
    got, opl, _, _, bits = run
    items = [(0, 0), (0, opl.nblk(0) - 1)]
    o_ref, lse_ref = orc.attn_fwd(bits["q"], bits["k"], bits["v"], opl, items)
    for it, (_, b) in enumerate(items):
        toks = orc.tokens_of_block(opl, 0, b)
        compare_bf16(got["o"][toks], o_ref[it, :len(toks)], what=f"O b{b}")
        assert np.abs(got["lse"][toks] - lse_ref[it, :len(toks)]).max() < 2e-3
