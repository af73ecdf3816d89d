"""The A->V norm map on the GPU (prism_av_cross_attn) against the fp64
oracle: h_hat = CrossAttn(h, K_a, V_a) per head and a_n = ||h_hat_n||_2 over
heads and channels (paper.rainbus.top "双分支视频-音频 DiT 与跨模态交叉注意力").
h_hat is compared at the bf16 bar; the norm, an fp32 reduction of the
unrounded outputs, within 1e-2 relative.  The map then feeds the next
layer's plan (the one-layer lag of "核心方法")."""
import numpy as np
import pytest
import torch

from dynamic_block_sparse_zone_amd import synth
from tests.helpers import compare_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def prism():
    import dynamic_block_sparse_zone_amd as p
    return p


def _run(prism, orc, wl, n_audio, tokens=None, device="cpu"):
    x = synth.make_inputs(wl, device=device, with_grad=False)
    a = synth.make_audio(wl, n_audio, device=device)
    q, ka, va = x["q"].to(DEV), a["ka"].to(DEV), a["va"].to(DEV)
    print(f"[av norm] {wl.name}: {wl.heads} heads x {wl.N} tokens, {n_audio} audio tokens",
          flush=True)
    norm, o = prism.av_cross_attn(q, ka, va, want_o=True)
    torch.cuda.synchronize()
    toks = np.arange(wl.N) if tokens is None else tokens
    ref_n, ref_o = orc.av_cross(synth.to_numpy_bits(x["q"]), synth.to_numpy_bits(a["ka"]),
                                synth.to_numpy_bits(a["va"]), toks, want_o=True)
    got_o = o[:, torch.from_numpy(np.asarray(toks)).to(DEV)].float().cpu().numpy()  # [heads, n, D]
    got_n = norm.cpu().numpy()[toks]
    return got_n, got_o, ref_n, ref_o, (q, ka, va, norm, x)


@pytest.mark.parametrize("name,n_audio", [("check", 128), ("bwdcheck", 64), ("small", 320)])
def test_av_norm_matches_oracle(prism, orc, name, n_audio):
    wl = synth.WORKLOADS[name]
    toks = None if wl.N * wl.heads <= 40000 else \
        np.sort(np.random.default_rng(3).choice(wl.N, 3000, replace=False))
    got_n, got_o, ref_n, ref_o, _ = _run(prism, orc, wl, n_audio, toks)
    compare_bf16(got_o.transpose(1, 0, 2), ref_o, what=f"h_hat {name}")
    np.testing.assert_allclose(got_n, ref_n, rtol=1e-2)


def test_av_norm_full_size_sampled(prism, orc):
    """The 2K training-scale grid (1,036,800 video tokens, 40 heads) with 512
    audio tokens, on 2,000 sampled tokens."""
    wl = synth.WORKLOADS["train2k"]
    toks = np.sort(np.random.default_rng(4).choice(wl.N, 2000, replace=False))
    got_n, got_o, ref_n, ref_o, _ = _run(prism, orc, wl, 512, toks, device=DEV)
    compare_bf16(got_o.transpose(1, 0, 2), ref_o, what="h_hat train2k")
    np.testing.assert_allclose(got_n, ref_n, rtol=1e-2)


def test_av_norm_feeds_next_layer_plan(prism, orc):
    """Layer l's norm map is layer l + 1's av_norm: the plan takes it, and the
    map is deterministic, so the plan built from it is reproducible."""
    wl = synth.WORKLOADS["check"]
    x = synth.make_inputs(wl, device=DEV, with_grad=False)
    a = synth.make_audio(wl, 128, device=DEV)
    n1, _ = prism.av_cross_attn(x["q"], a["ka"], a["va"])
    n2, _ = prism.av_cross_attn(x["q"], a["ka"], a["va"])
    assert torch.equal(n1, n2)
    kw = dict(T=wl.T, H=wl.H, W=wl.W, top_k=wl.top_k, top_p=wl.top_p)
    p1 = prism.plan(x["q"], x["k"], x["v"], n1, **kw)
    p2 = prism.plan(x["q"], x["k"], x["v"], n2, **kw)
    for arr in ("audio_stats", "shape_id", "col_idx"):
        assert np.array_equal(p1.export(arr), p2.export(arr))
    assert np.any(p1.export("audio_stats") != 0)


def test_av_norm_rejects_bad_sizes(prism):
    from dynamic_block_sparse_zone_amd import _native as nat
    q = torch.zeros((1, 512, 128), dtype=torch.bfloat16, device=DEV)
    ka = torch.zeros((1, 96, 128), dtype=torch.bfloat16, device=DEV)   # not a multiple of 64
    with pytest.raises(nat.PrismError) as e:
        prism.av_cross_attn(q, ka, ka.clone())
    assert e.value.status == nat.PRISM_EINVAL
    q32 = torch.zeros((1, 512, 128), dtype=torch.float32, device=DEV)
    k32 = torch.zeros((1, 64, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(nat.PrismError) as e:
        prism.av_cross_attn(q32, k32, k32.clone())
    assert e.value.status == nat.PRISM_EUNSUPPORTED
