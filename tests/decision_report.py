"""How far the plan's canonical arithmetic moves its discrete decisions away
from the same decisions taken in plain fp64 (test infrastructure; reported,
not a parity gate).

Two readings of the pages are compared against fp64 "math" evaluations:

* Block shapes.  The oracle takes every shape decision in fp32 in a fixed
  order (zone statistics, g_d, rho, the exact nearest-candidate test).  The
  fp64 variant recomputes the zone statistics, g_d = r_d + abar vhat_d + eps,
  rho and l*_d (xyznot.com/id "Metode" 1-2; paper.rainbus.top "方法步骤详情",
  stage one) with numpy in float64 and takes the nearest candidate by plain
  Euclidean distance.  Reported: zones whose volume or shape differs.

* Block selection.  The oracle scores block means rounded to an integer grid
  of about 9 significant bits, so that the bf16 matrix cores reproduce the
  scores exactly.  The pages define P_i = softmax(Qbar_i Kbar^T / sqrt(D))
  on the block means themselves (paper.rainbus.top "方法步骤详情", stage
  three).  The fp64 variant scores the exact fp64 block means over the same
  blocks and selects Top-k U Top-p with an fp64 cumulative sum.  Reported per
  workload: the mean and minimum Jaccard index of S_i, the share of rows whose
  S_i is identical, the selected pairs of each, and the fp64 softmax mass the
  integer-grid selection covers against the mass the fp64 selection covers.

Run as a script for the table (python tests/decision_report.py [--big]).
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

EDGES = (2, 4, 8)


def _values(x):
    """float64 values of an oracle input (float32, or bf16 as uint16 bits)."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _zones(x, T, H, W):
    """[N, C] in token order -> [Z, 8, 8, 8, C] (zone raster order)."""
    C = x.shape[-1]
    z = x.reshape(T // 8, 8, H // 8, 8, W // 8, 8, C)
    return z.transpose(0, 2, 4, 1, 3, 5, 6).reshape(-1, 8, 8, 8, C)


def _axis_var(z):
    """[Z, 3]: per zone the channel mean of the variance of the axis profiles."""
    out = []
    for ax in (1, 2, 3):
        other = tuple(a for a in (1, 2, 3) if a != ax)
        prof = z.mean(axis=other)                                  # [Z, 8, C]
        out.append(((prof - prof.mean(axis=1, keepdims=True)) ** 2).mean(axis=(1, 2)))
    return np.stack(out, axis=1)


def _ratio(s):
    tot = s.sum(axis=1, keepdims=True)
    r = np.full_like(s, 1.0 / 3.0)
    np.divide(s, tot, out=r, where=tot > 0)
    return r


def _candidates():
    out = []
    for B in (64, 128, 256):
        for a in EDGES:
            for b in EDGES:
                for c in EDGES:
                    if a * b * c == B:
                        out.append((a, b, c, B))
    return np.array(out)


def math_shapes(v, av, cfg):
    """fp64 variant of stage one: shape ids [heads, Z] and volumes."""
    cand = _candidates()
    T, H, W = cfg.T, cfg.H, cfg.W
    vals = _values(v)
    sid = np.zeros((cfg.heads, cfg.Z), np.int64)
    vol = np.zeros((cfg.heads, cfg.Z), np.int64)
    if av is not None:
        za = _zones(av.astype(np.float64).reshape(-1, 1), T, H, W)
        amean = za.mean(axis=(1, 2, 3, 4))
        abar = amean / amean.max() if amean.max() > 0 else np.zeros_like(amean)
        vhat = _ratio(_axis_var(za))
    for h in range(cfg.heads):
        z = _zones(vals[h], T, H, W)
        r = _ratio(_axis_var(z))
        sv = z.var(axis=(2, 3)).mean(axis=(1, 2))
        d = z[:, 1:] - z[:, :-1]
        tv = d.reshape(z.shape[0], -1, z.shape[-1]).var(axis=1).mean(axis=1)
        rho_raw = sv + tv
        g = r + (abar[:, None] * vhat if av is not None else 0.0) + cfg.eps
        mx = rho_raw.max()
        for m in range(cfg.Z):
            if tuple(cfg.fixed_shape) != (0, 0, 0):
                B = int(np.prod(cfg.fixed_shape))
                sid[h, m] = [tuple(c[:3]) for c in cand].index(tuple(cfg.fixed_shape))
                vol[h, m] = B
                continue
            rho = rho_raw[m] / mx if mx > 0 else 0.0
            B = 256 if mx <= 0 else 64 if rho >= cfg.tau128 else 128 if rho >= cfg.tau256 else 256
            if cfg.volume_mask == 1:
                B = 64
            S = math.log2(B)
            lg = np.log2(g[m])
            ls = -0.5 * lg + (S + 0.5 * lg.sum()) / 3.0
            ids = np.nonzero(cand[:, 3] == B)[0]
            dist = [((ls - np.log2(cand[i, :3])) ** 2).sum() for i in ids]
            sid[h, m] = ids[int(np.argmin(dist))]
            vol[h, m] = B
    return sid, vol


def exact_means(x, pl, h):
    """fp64 block means of head h over the oracle plan's blocks [n, D]."""
    vals = _values(x[h])
    n = pl.nblk(h)
    o = int(pl.blk_off[h])
    out = np.zeros((n, vals.shape[1]))
    for i in range(n):
        s, ln = int(pl.blk_start[o + i]), int(pl.blk_len[o + i])
        out[i] = vals[pl.perm[h, s:s + ln]].mean(axis=0)
    return out


def select64(s, k, p):
    """Top-k U Top-p over fp64 scores (rows of s): list of index arrays."""
    n = s.shape[1]
    k = max(0, min(k, n))
    out = []
    for row in s:
        order = np.lexsort((np.arange(n), -row))
        if p >= 1:
            L = n
        elif p > 0:
            e = np.exp(row[order] - row[order[0]])
            cum = np.cumsum(e / e.sum())
            L = int(np.searchsorted(cum, p, side="left")) + 1
            L = min(L, n)
        else:
            L = 0
        out.append(np.sort(order[:max(k, L)]))
    return out


def selection_report(orc, q, k, pl, heads):
    cfg = pl.cfg
    jac, same, pairs_i, pairs_f, mass_i, mass_f = [], 0, 0, 0, [], []
    for h in heads:
        qm, km = exact_means(q, pl, h), exact_means(k, pl, h)
        s = qm @ km.T / math.sqrt(cfg.head_dim)
        kk = cfg.k_for(pl.nblk(h))
        ref = select64(s, kk, cfg.top_p)
        P = np.exp(s - s.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        for i in range(pl.nblk(h)):
            a = orc.select_row(pl, h, i)
            b = ref[i]
            inter = len(np.intersect1d(a, b, assume_unique=True))
            uni = len(a) + len(b) - inter
            jac.append(inter / uni if uni else 1.0)
            same += int(len(a) == len(b) and inter == len(a))
            pairs_i += len(a)
            pairs_f += len(b)
            mass_i.append(P[i, a].sum())
            mass_f.append(P[i, b].sum())
    rows = len(jac)
    return {"rows": rows, "jaccard_mean": float(np.mean(jac)), "jaccard_min": float(np.min(jac)),
            "rows_identical": same / rows, "pairs_grid": pairs_i, "pairs_fp64": pairs_f,
            "mass_grid_mean": float(np.mean(mass_i)), "mass_fp64_mean": float(np.mean(mass_f))}


def shape_report(orc, v, av, pl):
    sid64, vol64 = math_shapes(v, av, pl.cfg)
    return {"zones": int(sid64.size), "volume_differs": int((vol64 != pl.volume).sum()),
            "shape_differs": int((sid64 != pl.shape_id).sum())}


def report(orc, wl, heads=None, device="cpu"):
    from dynamic_block_sparse_zone_amd import synth
    x = synth.make_inputs(wl, device=device, with_grad=False)
    bits = {n: synth.to_numpy_bits(x[n]) for n in ("q", "k", "v")}
    av = x["av"].cpu().numpy()
    cfg = orc.Config(wl.T, wl.H, wl.W, wl.heads, wl.head_dim, top_k=wl.top_k,
                     top_k_frac=wl.top_k_frac, top_p=wl.top_p, volume_mask=wl.volume_mask,
                     fixed_shape=tuple(wl.fixed_shape))
    pl = orc.plan(bits["q"], bits["k"], bits["v"], av, cfg)
    heads = range(wl.heads) if heads is None else heads
    out = {"workload": wl.name}
    out.update(shape_report(orc, bits["v"], av, pl))
    out.update(selection_report(orc, bits["q"], bits["k"], pl, heads))
    return out


def main():
    from oracle import oracle as O
    from dynamic_block_sparse_zone_amd import synth
    O.build()
    wls = [synth.WORKLOADS["tiny"], synth.WORKLOADS["check"], synth.WORKLOADS["small"],
           synth.WORKLOADS["small"].with_(name="small_op", top_k=0, top_k_frac=0.05,
                                          top_p=0.2)]
    if "--big" in sys.argv:
        # the first head of the 2K grids (a head's plan depends on its own
        # Q, K, V only; unit-variance scaling then uses this head alone)
        for name in ("infer2k", "train2k", "train2k_op"):
            wls.append(synth.WORKLOADS[name].with_(heads=1))
    for wl in wls:
        r = report(O, wl)
        print(" | ".join(f"{k}={v:.4f}" if isinstance(v, float) else f"{k}={v}"
                         for k, v in r.items()), flush=True)


if __name__ == "__main__":
    main()
