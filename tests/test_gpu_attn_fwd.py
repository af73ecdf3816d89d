"""Parity of the sparse attention forward on the GPU with the fp64 oracle
(element by element on small grids, sampled query blocks on larger ones)."""
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


def run_fwd(prism, orc, name, sample=None, seed=0, **over):
    wl = synth.WORKLOADS[name] if isinstance(name, str) else name
    print(f"[fwd parity] workload={name} over={over}", flush=True)
    x = synth.make_inputs(wl, device="cpu", with_grad=False)
    dx = to_dev(x, DEV)
    pl = gpu_plan(prism, wl, dx, **over)
    o, lse = prism.attn_fwd(pl, dx["q"], dx["k"], dx["v"])
    torch.cuda.synchronize()
    hb = host_bits(x)
    cfg = oracle_config(orc, wl, **over)
    opl = orc.plan(hb["q"], hb["k"], hb["v"], x["av"].numpy(), cfg)
    rng = np.random.default_rng(seed)
    items = []
    for h in range(wl.heads):
        n = opl.nblk(h)
        rows = range(n) if sample is None else sorted(rng.choice(n, min(sample, n), False))
        items += [(h, int(i)) for i in rows]
    oo, ol = orc.attn_fwd(hb["q"], hb["k"], hb["v"], opl, items)
    og = o.float().cpu().numpy()
    lg = lse.cpu().numpy()
    got, ref, gl, rl = [], [], [], []
    for it, (h, i) in enumerate(items):
        toks = orc.tokens_of_block(opl, h, i)
        got.append(og[h, toks])
        ref.append(oo[it, :len(toks)])
        gl.append(lg[h, toks])
        rl.append(ol[it, :len(toks)])
    return wl, pl, np.concatenate(got), np.concatenate(ref), np.concatenate(gl), np.concatenate(rl)


def test_fwd_tiny_fp32_full(prism, orc):
    wl, pl, g, r, gl, rl = run_fwd(prism, orc, "tiny")
    np.testing.assert_allclose(g, r, atol=2e-5, rtol=1e-4)
    np.testing.assert_allclose(gl, rl, atol=2e-5, rtol=1e-5)


def test_fwd_fp32_mixed_volumes_d128(prism, orc):
    """The fp32 path at head_dim 128 over blocks of all three volumes (the
    structured check grid in fp32): several 64-key tiles per block and
    rows whose lists span both halves of a tile."""
    wl = synth.WORKLOADS["check"].with_(name="check_f32", dtype="f32")
    wl_, pl, g, r, gl, rl = run_fwd(prism, orc, wl)
    np.testing.assert_allclose(g, r, atol=2e-5, rtol=1e-4)
    np.testing.assert_allclose(gl, rl, atol=2e-5, rtol=1e-5)


def test_fwd_check_bf16_full(prism, orc):
    wl, pl, g, r, gl, rl = run_fwd(prism, orc, "check")
    print("check fwd err", compare_bf16(g, r, what="O"))
    np.testing.assert_allclose(gl, rl, atol=2e-3, rtol=1e-4)


def test_fwd_small_bf16_sampled(prism, orc):
    wl, pl, g, r, gl, rl = run_fwd(prism, orc, "small", sample=24)
    print("small fwd err", compare_bf16(g, r, what="O"))
    np.testing.assert_allclose(gl, rl, atol=2e-3, rtol=1e-4)


@pytest.mark.parametrize("over", [
    {"top_p": 1.0},                  # dense limit
    {"top_p": 0.0, "top_k": 1},      # one key block per query block
    {"fixed_shape": (4, 4, 8)},
    {"volume_mask": 1},              # all blocks of 64 (pairs of query blocks per unit)
    {"top_k_frac": 0.05, "top_p": 0.2},
    {"relayout": False},             # every tile gathered through the block -> token map
])
def test_fwd_variants(prism, orc, over):
    wl, pl, g, r, gl, rl = run_fwd(prism, orc, "check", **over)
    compare_bf16(g, r, what=f"O {over}")
    np.testing.assert_allclose(gl, rl, atol=2e-3, rtol=1e-4)


def test_fwd_empty_selection_gives_zero(prism, orc):
    wl, pl, g, r, gl, rl = run_fwd(prism, orc, "check", top_p=0.0, top_k=0)
    assert np.all(g == 0) and np.all(np.isneginf(gl))


def test_fwd_dense_limit_is_full_attention(prism):
    """Top-p = 1: the sparse forward equals torch's dense attention."""
    wl = synth.WORKLOADS["check"]
    x = to_dev(synth.make_inputs(wl, device="cpu", with_grad=False), DEV)
    pl = gpu_plan(prism, wl, x, top_p=1.0)
    o, _ = prism.attn_fwd(pl, x["q"], x["k"], x["v"])
    q, k, v = (x[n].float() for n in ("q", "k", "v"))
    ref = torch.softmax(q @ k.transpose(1, 2).contiguous() / 128 ** 0.5, -1) @ v
    compare_bf16(o.float().cpu().numpy(), ref.cpu().double().numpy(), what="dense")


def test_fwd_deterministic(prism):
    wl = synth.WORKLOADS["small"]
    x = to_dev(synth.make_inputs(wl, device="cpu", with_grad=False), DEV)
    pl = gpu_plan(prism, wl, x)
    a, la = prism.attn_fwd(pl, x["q"], x["k"], x["v"])
    b, lb = prism.attn_fwd(pl, x["q"], x["k"], x["v"])
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_fwd_rejects_other_kv(prism):
    wl = synth.WORKLOADS["check"]
    x = to_dev(synth.make_inputs(wl, device="cpu", with_grad=False), DEV)
    pl = gpu_plan(prism, wl, x)
    from dynamic_block_sparse_zone_amd._native import PrismError
    with pytest.raises(PrismError):
        prism.attn_fwd(pl, x["q"], x["k"].clone(), x["v"])
