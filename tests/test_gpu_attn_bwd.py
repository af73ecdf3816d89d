"""Parity of the sparse attention backward on the GPU with the fp64 oracle:
dQ, dK, dV element by element, plus the invariants the pages fix (plan
detached: unselected key blocks get no gradient; softmax rows sum to one, so
the dK of a head sums to zero over keys)."""
import numpy as np
import pytest
import torch

from dynamic_block_sparse_zone_amd import synth
from tests.helpers import compare_bf16, gpu_plan, host_bits, oracle_config, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def prism():
    import dynamic_block_sparse_zone_amd as p
    return p


def run_bwd(prism, name, **over):
    wl = synth.WORKLOADS[name]
    print(f"[bwd parity] workload={name} over={over}", flush=True)
    x = synth.make_inputs(wl, device="cpu", with_grad=True)
    dx = to_dev(x, DEV)
    pl = gpu_plan(prism, wl, dx, **over)
    o, lse = prism.attn_fwd(pl, dx["q"], dx["k"], dx["v"])
    dq, dk, dv = prism.attn_bwd(pl, dx["q"], dx["k"], dx["v"], o, lse, dx["do"])
    torch.cuda.synchronize()
    return wl, x, pl, (dq.float().cpu().numpy(), dk.float().cpu().numpy(),
                       dv.float().cpu().numpy())


def rel_err(g, r):
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))


def check_heads(orc, wl, x, grads, heads, **over):
    hb = host_bits(x)
    cfg = oracle_config(orc, wl, **over)
    opl = orc.plan(hb["q"], hb["k"], hb["v"], x["av"].numpy(), cfg)
    for h in heads:
        ref = orc.attn_bwd_head(hb["q"], hb["k"], hb["v"], hb["do"], opl, h)
        for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
            compare_bf16(g[h], r, what=f"{name} head {h} {over}")
            assert rel_err(g[h], r) < 2e-2, (name, h, rel_err(g[h], r))
    return opl


def test_bwd_full(prism, orc):
    wl, x, pl, grads = run_bwd(prism, "bwdcheck")
    check_heads(orc, wl, x, grads, range(wl.heads))


@pytest.mark.parametrize("over", [
    {"volume_mask": 1},            # all 64-token blocks: two key blocks per work-group
    {"fixed_shape": (4, 4, 8)},
    {"top_p": 0.0, "top_k": 2},
    {"top_p": 1.0},
    {"relayout": False},           # every tile gathered through the block -> token map
])
def test_bwd_variants(prism, orc, over):
    wl, x, pl, grads = run_bwd(prism, "bwdcheck", **over)
    check_heads(orc, wl, x, grads, range(wl.heads), **over)


def test_bwd_check_head(prism, orc):
    wl, x, pl, grads = run_bwd(prism, "check")
    check_heads(orc, wl, x, grads, [1])


def test_bwd_invariants(prism):
    wl, x, pl, (dq, dk, dv) = run_bwd(prism, "check", top_p=0.0, top_k=1)
    row_ptr, col = pl.export("row_ptr"), pl.export("col_idx")
    off = pl.export("blk_off")
    perm = pl.export("perm").reshape(wl.heads, -1)
    start = pl.export("blk_start")
    sid = pl.export("shape_id").reshape(wl.heads, -1)
    vol = [prism.candidate(i)[3] for i in range(16)]
    for h in range(wl.heads):
        n = int(off[h + 1] - off[h])
        chosen = np.zeros(n, bool)
        chosen[col[row_ptr[off[h]]:row_ptr[off[h + 1]]]] = True
        assert not chosen.all()
        sel_tok = np.zeros(dk.shape[1], bool)
        for j in np.nonzero(chosen)[0]:
            s0 = int(start[int(off[h]) + int(j)])
            sel_tok[perm[h, s0:s0 + vol[sid[h, s0 // 512]]]] = True
        # tokens of key blocks no query block selected: exactly zero dK and dV
        assert np.all(dk[h, ~sel_tok] == 0) and np.all(dv[h, ~sel_tok] == 0)
        assert np.any(dk[h, sel_tok] != 0)
        # softmax rows sum to one, so dK sums to zero over the keys of a head
        assert np.abs(dk[h].sum(0)).max() < 2e-2 * np.abs(dk[h]).sum(0).max() + 1e-3


def test_bwd_dense_limit_matches_autograd(prism):
    """Top-p = 1: gradients equal dense attention's (torch autograd, fp32)."""
    wl = synth.WORKLOADS["bwdcheck"]
    x = to_dev(synth.make_inputs(wl, device="cpu", with_grad=True), DEV)
    pl = gpu_plan(prism, wl, x, top_p=1.0)
    o, lse = prism.attn_fwd(pl, x["q"], x["k"], x["v"])
    dq, dk, dv = prism.attn_bwd(pl, x["q"], x["k"], x["v"], o, lse, x["do"])
    q, k, v = (x[n].float().requires_grad_(True) for n in ("q", "k", "v"))
    ref = torch.softmax(q @ k.transpose(1, 2).contiguous() / 128 ** 0.5, -1) @ v
    ref.backward(x["do"].float())
    for name, g, r in (("dQ", dq, q.grad), ("dK", dk, k.grad), ("dV", dv, v.grad)):
        compare_bf16(g.float().cpu().numpy(), r.double().cpu().numpy(), what=name)


def test_bwd_deterministic(prism):
    wl = synth.WORKLOADS["check"]
    x = to_dev(synth.make_inputs(wl, device="cpu", with_grad=True), DEV)
    pl = gpu_plan(prism, wl, x)
    o, lse = prism.attn_fwd(pl, x["q"], x["k"], x["v"])
    a = prism.attn_bwd(pl, x["q"], x["k"], x["v"], o, lse, x["do"])
    b = prism.attn_bwd(pl, x["q"], x["k"], x["v"], o, lse, x["do"])
    for u, w in zip(a, b):
        assert torch.equal(u, w)


def test_bwd_one_zone(prism, orc):
    """One 8x8x8 zone and one head: fewer dK/dV work units (4) than a
    persistent launch has work-groups per XCD."""
    wl = synth.WORKLOADS["bwdcheck"].with_(name="onezone", T=8, H=8, W=8, heads=1)
    print("[bwd parity] one zone", flush=True)
    x = synth.make_inputs(wl, device="cpu", with_grad=True)
    dx = to_dev(x, DEV)
    for over in ({"top_p": 0.0, "top_k": 1}, {"top_p": 1.0}):
        pl = gpu_plan(prism, wl, dx, **over)
        o, lse = prism.attn_fwd(pl, dx["q"], dx["k"], dx["v"])
        dq, dk, dv = prism.attn_bwd(pl, dx["q"], dx["k"], dx["v"], o, lse, dx["do"])
        torch.cuda.synchronize()
        grads = tuple(t.float().cpu().numpy() for t in (dq, dk, dv))
        check_heads(orc, wl, x, grads, [0], **over)
