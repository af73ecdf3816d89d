"""Stage two's re-layout (paper.rainbus.top "方法步骤详情", stage two) is a
memory layout, not part of the method: attention over the plan's
block-contiguous copies of K and V (and the backward's copies of Q and dO)
reads exactly the tile data that gathering through the block -> token map
reads, in the same order, so O, LSE, dQ, dK and dV must agree bit for bit.
The oracle comparisons of both layouts are in test_gpu_attn_fwd.py and
test_gpu_attn_bwd.py."""
import pytest
import torch

from dynamic_block_sparse_zone_amd import synth
from tests.helpers import gpu_plan

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def prism():
    import dynamic_block_sparse_zone_amd as p
    return p


def step(prism, wl, x, relayout, bwd_workspace=None, **over):
    pl = gpu_plan(prism, wl, x, relayout=relayout, **over)
    o, lse = prism.attn_fwd(pl, x["q"], x["k"], x["v"])
    g = prism.attn_bwd(pl, x["q"], x["k"], x["v"], o, lse, x["do"], workspace=bwd_workspace)
    torch.cuda.synchronize()
    return pl, (o, lse) + tuple(g)


@pytest.mark.parametrize("name,over", [
    ("bwdcheck", {}),
    ("bwdcheck", {"volume_mask": 1}),
    ("check", {"fixed_shape": (4, 4, 8)}),
    ("check", {"top_k_frac": 0.05, "top_p": 0.2}),
    ("small", {}),
])
def test_relaid_equals_gathered(prism, name, over):
    wl = synth.WORKLOADS[name]
    print(f"[relayout] {name} {over}", flush=True)
    x = synth.make_inputs(wl, device=DEV, with_grad=True)
    _, a = step(prism, wl, x, True, **over)
    _, b = step(prism, wl, x, False, **over)
    for what, u, v in zip(("O", "LSE", "dQ", "dK", "dV"), a, b):
        assert torch.equal(u, v), f"{what} differs between the layouts ({name} {over})"


def test_backward_without_room_for_the_copies(prism):
    """A workspace that holds only the columns runs the backward without the
    copies of Q and dO, with the same result."""
    wl = synth.WORKLOADS["bwdcheck"]
    x = synth.make_inputs(wl, device=DEV, with_grad=True)
    pl = gpu_plan(prism, wl, x, relayout=True)
    full = prism.attn_bwd_workspace_bytes(pl)
    rows = wl.heads * wl.N
    assert full >= rows * 520
    small = torch.empty(rows * 8 + 256, dtype=torch.uint8, device=DEV)
    _, a = step(prism, wl, x, True)
    _, b = step(prism, wl, x, True, bwd_workspace=small)
    for what, u, v in zip(("O", "LSE", "dQ", "dK", "dV"), a, b):
        assert torch.equal(u, v), what
