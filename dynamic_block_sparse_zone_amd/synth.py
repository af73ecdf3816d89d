"""Seeded synthetic inputs shaped like the 2K video workloads on the Prism
pages (paper.rainbus.top, sections "VAE 时空压缩与超长 token 序列" and
"复现评估": ~870K video tokens per 10 s clip at inference, >1M in training,
40 heads of width 128).

This module only draws inputs.  It holds none of the method's arithmetic
and is shared by the tests, the benchmark and the CPU oracle so that all of
them see the same bytes.  No clips or benchmark items are used: the grids
below stand in for the pages' 2K-Bench workloads by shape and structure.

Layout of every tensor: [heads, T*H*W, D], token n = (t*H + h)*W + w.
The A->V norm map is [T*H*W] float32 in [0, 1].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    W: int
    heads: int
    head_dim: int
    dtype: str             # "f32" or "bf16"
    top_k: int
    top_p: float
    volume_mask: int = 7   # bit0 = 64, bit1 = 128, bit2 = 256
    fixed_shape: tuple = (0, 0, 0)
    kind: str = "structured"   # "iid" | "structured" | "background" | "smooth"
    active_frac: float = 1.0   # share of zones with content in "background"
    seed: int = 1001
    backward: bool = False
    unit_var: bool = False
    top_k_frac: float = 0.0    # > 0: k = ceil(frac * N_blk) per head instead of top_k
    cut_frames: tuple = ()     # shot cuts: from each listed frame on, new content

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def Z(self) -> int:
        return (self.T // 8) * (self.H // 8) * (self.W // 8)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # tiny forward, iid inputs, 64-token blocks only
    "tiny": Workload("tiny", 8, 16, 16, 2, 64, "f32", top_k=4, top_p=0.9, volume_mask=1,
                     kind="iid", seed=1001),
    # anisotropic per-zone sinusoids, all three volumes
    "small": Workload("small", 24, 48, 48, 8, 128, "bf16", top_k=8, top_p=0.9, seed=1002),
    # 2K inference-scale layer: mostly flat background with compact active blobs
    "infer2k": Workload("infer2k", 64, 104, 128, 40, 128, "bf16", top_k=16, top_p=0.9,
                        kind="background", active_frac=0.2, seed=1003),
    # 2K training-scale layer, forward + backward
    "train2k": Workload("train2k", 72, 120, 120, 40, 128, "bf16", top_k=16, top_p=0.9,
                        seed=1004, backward=True, unit_var=True),
    # dense limit (every block selected) at inference scale
    "dense2k": Workload("dense2k", 64, 104, 128, 40, 128, "bf16", top_k=16, top_p=1.0,
                        kind="background", active_frac=0.2, seed=1003),
    # one fixed 4x4x8 shape everywhere at inference scale
    "fixed2k": Workload("fixed2k", 64, 104, 128, 40, 128, "bf16", top_k=16, top_p=0.9,
                        kind="background", active_frac=0.2, seed=1003,
                        fixed_shape=(4, 4, 8)),
    # the pages' operating point (Top-k at 95 % sparsity, i.e. 5 % of the key
    # blocks, with Top-p 0.2) on the inference- and training-scale inputs
    "infer2k_op": Workload("infer2k_op", 64, 104, 128, 40, 128, "bf16", top_k=0, top_p=0.2,
                           kind="background", active_frac=0.2, seed=1003, top_k_frac=0.05),
    "train2k_op": Workload("train2k_op", 72, 120, 120, 40, 128, "bf16", top_k=0, top_p=0.2,
                           seed=1004, backward=True, unit_var=True, top_k_frac=0.05),
    # the same with Top-p 0.3, the contrast of the pages' Table 7
    "train2k_op3": Workload("train2k_op3", 72, 120, 120, 40, 128, "bf16", top_k=0, top_p=0.3,
                            seed=1004, backward=True, unit_var=True, top_k_frac=0.05),
    # small bf16 grid for full element-by-element checks (fwd + bwd): several
    # zones of every volume, a ragged number of blocks per head
    "check": Workload("check", 16, 24, 32, 3, 128, "bf16", top_k=3, top_p=0.9, seed=1006,
                      backward=True),
    # two shot cuts, at frame offsets 4 and 3 of their zones, for the
    # shot-cut-aware temporal zone boundaries
    "cuts": Workload("cuts", 24, 32, 32, 2, 128, "bf16", top_k=4, top_p=0.9, seed=1010,
                     kind="smooth", cut_frames=(12, 19)),
    # smallest bf16 grid with zones of every volume, for full backward checks
    "bwdcheck": Workload("bwdcheck", 8, 16, 32, 2, 128, "bf16", top_k=3, top_p=0.9, seed=1007,
                         backward=True),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _coords(wl: Workload, device):
    n = torch.arange(wl.N, device=device)
    t = n // (wl.H * wl.W)
    y = (n // wl.W) % wl.H
    x = n % wl.W
    zone = (t // 8) * ((wl.H // 8) * (wl.W // 8)) + (y // 8) * (wl.W // 8) + (x // 8)
    return t, y, x, zone


def _active_zones(wl: Workload, device, seed: int) -> torch.Tensor:
    """Boolean [Z]: 1-3 compact blobs of active zones covering ~active_frac."""
    zT, zH, zW = wl.T // 8, wl.H // 8, wl.W // 8
    if wl.kind != "background":
        return torch.ones(wl.Z, dtype=torch.bool, device=device)
    g = _gen("cpu", seed)
    nb = int(torch.randint(1, 4, (1,), generator=g))
    zt = torch.arange(zT).view(-1, 1, 1).float()
    zh = torch.arange(zH).view(1, -1, 1).float()
    zw = torch.arange(zW).view(1, 1, -1).float()
    centres = torch.rand(nb, 3, generator=g) * torch.tensor([zT, zH, zW]).float()
    # radius so that nb ellipsoids cover about active_frac of the grid
    vol = wl.active_frac * wl.Z / nb
    rad = (3 * vol / (4 * math.pi)) ** (1 / 3)
    act = torch.zeros(zT, zH, zW, dtype=torch.bool)
    for b in range(nb):
        c = centres[b]
        d2 = ((zt - c[0]) / max(1.0, rad * zT / max(zH, zW))) ** 2 + \
             ((zh - c[1]) / rad) ** 2 + ((zw - c[2]) / rad) ** 2
        act |= d2 <= 1.0
    return act.reshape(-1).to(device)


def _orthogonal(D: int, g: torch.Generator) -> torch.Tensor:
    a = torch.randn(D, D, generator=g, dtype=torch.float64)
    qm, r = torch.linalg.qr(a)
    qm = qm * torch.sign(torch.diagonal(r)).unsqueeze(0)
    return qm.float()


def _structured_head(wl: Workload, h: int, coords, act, device) -> torch.Tensor:
    """V of one head [N, D] fp32: per zone, sum over axes d of
    A_{c,d} sin(2 pi f_d x_d + phi_{c,d}) + N(0, 0.1^2); flat zones have f = 0."""
    t, y, x, zone = coords
    D, Z = wl.head_dim, wl.Z
    g = _gen(device, wl.seed * 1000 + 17 * h + 1)
    f = torch.rand(Z, 3, generator=g, device=device) * 0.5
    f = f * act.view(-1, 1).float()
    A = torch.randn(Z, D, 3, generator=g, device=device) / math.sqrt(3.0)
    phi = torch.rand(Z, D, 3, generator=g, device=device) * (2 * math.pi)
    out = torch.randn(wl.N, D, generator=g, device=device) * 0.1
    if wl.kind == "smooth":
        # one set of frequencies, amplitudes and phases for the whole grid:
        # content continuous across zone boundaries (slow, f in [0, 0.15))
        zone = torch.zeros_like(zone)
        f = f * 0.3
    xs = (t.float(), y.float(), x.float())
    for d in range(3):
        arg = (2 * math.pi) * f[zone, d].unsqueeze(1) * xs[d].unsqueeze(1) + phi[zone, :, d]
        out += A[zone, :, d] * torch.sin(arg)
        del arg
    return out


def _av_norm(wl: Workload, coords, device) -> torch.Tensor:
    """1-3 Gaussian blobs (sigma 4-12 tokens) in (h, w), modulated in time by
    1/2 + 1/2 sin(2 pi f_t t + phi), f_t in [0.25, 0.5] cycles per frame."""
    t, y, x, _ = coords
    if wl.kind == "iid":
        g = _gen(device, wl.seed * 1000 + 999)
        return torch.rand(wl.N, generator=g, device=device)
    g = _gen("cpu", wl.seed * 1000 + 998)
    nb = int(torch.randint(1, 4, (1,), generator=g))
    out = torch.zeros(wl.N, device=device)
    for _ in range(nb):
        cy, cx = float(torch.rand(1, generator=g)) * wl.H, float(torch.rand(1, generator=g)) * wl.W
        sg = 4.0 + 8.0 * float(torch.rand(1, generator=g))
        ft = 0.25 + 0.25 * float(torch.rand(1, generator=g))
        ph = 2 * math.pi * float(torch.rand(1, generator=g))
        amp = 0.5 + 0.5 * float(torch.rand(1, generator=g))
        sp = torch.exp(-(((y.float() - cy) ** 2 + (x.float() - cx) ** 2) / (2 * sg * sg)))
        tm = 0.5 + 0.5 * torch.sin(2 * math.pi * ft * t.float() + ph)
        out += amp * sp * tm
    return out.clamp_(0.0, 1.0)


def make_inputs(wl: Workload | str, device="cpu", with_grad: bool | None = None) -> dict:
    """Draw q, k, v (and d_o when the workload has a backward pass) and the
    A->V norm map.  Deterministic for a given workload and device type."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    device = torch.device(device)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    with_grad = wl.backward if with_grad is None else with_grad
    shape = (wl.heads, wl.N, wl.head_dim)
    coords = _coords(wl, device)
    q = torch.empty(shape, dtype=dt, device=device)
    k = torch.empty(shape, dtype=dt, device=device)
    v = torch.empty(shape, dtype=dt, device=device)
    do = torch.empty(shape, dtype=dt, device=device) if with_grad else None
    if wl.kind == "iid":
        g = _gen(device, wl.seed)
        for tns in (q, k, v):
            tns.copy_(torch.randn(shape, generator=g, device=device))
    else:
        act = _active_zones(wl, device, wl.seed * 1000 + 5)
        gr = _gen("cpu", wl.seed * 1000 + 7)
        for h in range(wl.heads):
            vh = _structured_head(wl, h, coords, act, device)
            R = _orthogonal(wl.head_dim, gr).to(device)
            gn = _gen(device, wl.seed * 1000 + 31 * h + 3)
            qh = vh @ R + 0.1 * torch.randn(vh.shape, generator=gn, device=device)
            kh = vh @ R + 0.1 * torch.randn(vh.shape, generator=gn, device=device)
            v[h].copy_(vh)
            q[h].copy_(qh)
            k[h].copy_(kh)
            del vh, qh, kh
        for i, tc in enumerate(wl.cut_frames):
            # a shot cut at frame tc: every later frame comes from a fresh draw
            # (other per-zone frequencies, phases and projection)
            cut = make_inputs(wl.with_(seed=wl.seed + 7919 * (i + 1), cut_frames=()),
                              device=device, with_grad=False)
            rows = slice(tc * wl.H * wl.W, wl.N)
            for name, tns in (("q", q), ("k", k), ("v", v)):
                tns[:, rows] = cut[name][:, rows]
            del cut
        if wl.unit_var:
            for tns in (q, k, v):
                sd = _global_std(tns)
                for h in range(wl.heads):
                    tns[h].copy_(tns[h].float() / sd)
    if do is not None:
        g = _gen(device, wl.seed * 1000 + 77)
        for h in range(wl.heads):
            do[h].copy_(torch.randn(shape[1:], generator=g, device=device))
    av = _av_norm(wl, coords, device).float().contiguous()
    return {"q": q, "k": k, "v": v, "do": do, "av": av, "wl": wl}


def make_audio(wl: Workload | str, n_audio: int, device="cpu") -> dict:
    """Audio keys and values [heads, n_audio, head_dim] for the A->V
    cross-attention, iid N(0, 1) from the workload's seed, in its dtype.
    (The pages give no audio token count; n_audio is a parameter.)"""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    device = torch.device(device)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    g = _gen(device, wl.seed * 1000 + 501)
    shape = (wl.heads, n_audio, wl.head_dim)
    ka = torch.randn(shape, generator=g, device=device).to(dt)
    va = torch.randn(shape, generator=g, device=device).to(dt)
    return {"ka": ka, "va": va}


def _global_std(x: torch.Tensor) -> float:
    s = 0.0
    s2 = 0.0
    for h in range(x.shape[0]):
        xf = x[h].double()
        s += float(xf.sum())
        s2 += float((xf * xf).sum())
    n = x.numel()
    var = s2 / n - (s / n) ** 2
    return math.sqrt(max(var, 1e-30))


def to_numpy_bits(x: torch.Tensor):
    """Host numpy view for the oracle: float32 as is, bf16 as raw uint16."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view("uint16")
    return x.numpy()
