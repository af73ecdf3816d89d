"""Shared test plumbing: run the HIP path and the oracle on the same bytes."""
from __future__ import annotations

import numpy as np
import torch

from dynamic_block_sparse_zone_amd import synth


def oracle_config(O, wl, **over):
    kw = dict(top_k=wl.top_k, top_p=wl.top_p, volume_mask=wl.volume_mask,
              fixed_shape=tuple(wl.fixed_shape))
    kw.update(over)
    kw.pop("relayout", None)  # a memory layout of the kernels, not of the method
    return O.Config(wl.T, wl.H, wl.W, wl.heads, wl.head_dim, **kw)


def host_bits(x):
    return {n: (synth.to_numpy_bits(x[n]) if x.get(n) is not None else None)
            for n in ("q", "k", "v", "do")}


def gpu_plan(prism, wl, dev_x, use_audio=True, **over):
    kw = dict(top_k=wl.top_k, top_p=wl.top_p, volume_mask=wl.volume_mask,
              fixed_shape=tuple(wl.fixed_shape))
    kw.update(over)
    return prism.plan(dev_x["q"], dev_x["k"], dev_x["v"], dev_x["av"] if use_audio else None,
                      T=wl.T, H=wl.H, W=wl.W, **kw)


def to_dev(x, dev):
    return {n: (t.to(dev) if isinstance(t, torch.Tensor) else t) for n, t in x.items()}


def csr_rows(row_ptr, col, g):
    return col[row_ptr[g]:row_ptr[g + 1]]


def compare_bf16(gpu: np.ndarray, ref: np.ndarray, max_abs=2e-2, mean_abs=2e-3, what=""):
    err = np.abs(gpu.astype(np.float64) - ref)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    assert err.max() <= max_abs, f"{what}: max abs err {err.max():.3e} > {max_abs}"
    assert err.mean() <= mean_abs, f"{what}: mean abs err {err.mean():.3e} > {mean_abs}"
    return float(err.max()), float(err.mean())
