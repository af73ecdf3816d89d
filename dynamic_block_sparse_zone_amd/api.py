"""Python binding of the Prism sparse-attention library (include/prism.h).

Argument marshalling only: torch tensors supply device memory and the HIP
stream; every step of the plan and of attention runs in libprism.so.

    plan = prism.plan(q, k, v, av_norm, T=..., H=..., W=..., top_k=16, top_p=0.9)
    o, lse = prism.attn_fwd(plan, q, k, v)
    dq, dk, dv = prism.attn_bwd(plan, q, k, v, o, lse, do)

Tensors are [heads, T*H*W, head_dim] (token n = (t*H + h)*W + w), bf16 or fp32,
contiguous, on one GPU; av_norm is [T*H*W] float32 or None (first layer).
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _native as nat

_NP = {
    "zone_stats": np.float32, "audio_stats": np.float32, "shape_id": np.uint8,
    "blk_off": np.int64, "blk_start": np.int32, "qbar": np.float32, "kbar": np.float32,
    "qexp": np.int32, "kexp": np.int32, "row_ptr": np.int64, "col_idx": np.int32,
    "colt_ptr": np.int64, "colt_idx": np.int32, "perm": np.int32, "qgrid": np.uint16,
    "kgrid": np.uint16, "kv_order": np.int32, "blk_org": np.int32, "cuts": np.uint8,
    "qlo": np.uint16, "klo": np.uint16,
}


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def make_config(T, H, W, heads, head_dim, dtype, *, top_k=16, top_k_frac=0.0, top_p=0.9,
                volume_mask=7, fixed_shape=(0, 0, 0), eps=1e-4, tau128=0.5, tau256=0.25,
                need_backward=True, shape_map="power", alpha=0.5,
                cut_threshold=0.0, relayout=True) -> nat.PrismConfig:
    c = nat.PrismConfig()
    nat.lib().prism_config_default(ctypes.byref(c))
    c.T, c.H, c.W, c.heads, c.head_dim = T, H, W, heads, head_dim
    c.dtype = nat.PRISM_BF16 if dtype == torch.bfloat16 else nat.PRISM_F32
    c.top_k, c.top_k_frac, c.top_p = int(top_k), float(top_k_frac), float(top_p)
    c.volume_mask = int(volume_mask)
    for i in range(3):
        c.fixed_shape[i] = int(fixed_shape[i])
    c.eps, c.tau128, c.tau256 = float(eps), float(tau128), float(tau256)
    c.need_backward = 1 if need_backward else 0
    c.shape_map = nat.SHAPE_MAPS[shape_map] if isinstance(shape_map, str) else int(shape_map)
    c.alpha = float(alpha)
    c.cut_threshold = float(cut_threshold)
    c.relayout = 1 if relayout else 0
    return c


def workspace_bytes(cfg: nat.PrismConfig, nnz_capacity: int) -> int:
    n = ctypes.c_size_t()
    nat.check(nat.lib().prism_plan_workspace_size(ctypes.byref(cfg), int(nnz_capacity),
                                                  ctypes.byref(n)), "prism_plan_workspace_size")
    return n.value


class Plan:
    """Owns the plan handle and the device workspace it points into."""

    def __init__(self, handle, cfg, workspace, nnz, q, k, v):
        self.handle = handle
        self.cfg = cfg
        self.workspace = workspace
        self.nnz = nnz
        self.device = q.device
        self._k, self._v = k, v  # the tensors the plan was built from

    def close(self):
        if self.handle:
            nat.lib().prism_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def export(self, name: str) -> np.ndarray:
        which = nat.ARRAYS[name]
        n = ctypes.c_size_t()
        nat.check(nat.lib().prism_plan_array_bytes(self.handle, which, ctypes.byref(n)),
                  "prism_plan_array_bytes")
        out = np.empty(max(1, n.value // np.dtype(_NP[name]).itemsize), _NP[name])
        nat.check(nat.lib().prism_plan_export(self.handle, which, out.ctypes.data_as(
            ctypes.c_void_p), out.nbytes, _stream(self.device)), "prism_plan_export")
        return out[: n.value // np.dtype(_NP[name]).itemsize]

    def info(self) -> dict:
        inf = nat.PrismPlanInfo()
        nat.check(nat.lib().prism_plan_info(self.handle, ctypes.byref(inf),
                                            _stream(self.device)), "prism_plan_info")
        return {"total_blocks": inf.total_blocks, "nnz": inf.nnz,
                "max_blocks_per_head": inf.max_blocks_per_head,
                "pair_tokens": inf.pair_tokens, "shape_hist": list(inf.shape_hist),
                "kv_persistent": bool(inf.kv_persistent)}


def plan(q, k, v, av_norm=None, *, T, H, W, top_k=16, top_k_frac=0.0, top_p=0.9,
         volume_mask=7, fixed_shape=(0, 0, 0), eps=1e-4, tau128=0.5, tau256=0.25,
         need_backward=True, shape_map="power", alpha=0.5, cut_threshold=0.0,
         relayout=True, nnz_capacity=None, workspace=None) -> Plan:
    """Stages one to three (shapes, block table, pooling, selection).
    shape_map: "power" (b_d ~ g_d^-alpha; alpha = 1/2 is the pages' method),
    "isotropic", "softmax", "rank" or "entropy" (the pages' ablations).
    cut_threshold > 0: shot-cut-aware temporal zones.
    relayout: keep block-contiguous copies of K and V (and let the backward
    copy Q and dO); False gathers every tile from the caller's tensors."""
    heads, N, D = q.shape
    assert N == T * H * W and k.shape == q.shape and v.shape == q.shape
    assert q.is_contiguous() and k.is_contiguous() and v.is_contiguous()
    assert q.dtype == k.dtype == v.dtype
    if av_norm is not None:
        assert av_norm.dtype == torch.float32 and av_norm.numel() == N and av_norm.is_contiguous()
    cfg = make_config(T, H, W, heads, D, q.dtype, top_k=top_k, top_k_frac=top_k_frac,
                      top_p=top_p, volume_mask=volume_mask, fixed_shape=fixed_shape, eps=eps,
                      tau128=tau128, tau256=tau256, need_backward=need_backward,
                      shape_map=shape_map, alpha=alpha, cut_threshold=cut_threshold,
                      relayout=relayout)
    nat.check(nat.lib().prism_config_check(ctypes.byref(cfg)), "prism_config_check")
    Z = (T // 8) * (H // 8) * (W // 8)
    worst = heads * (8 * Z) ** 2
    cap = int(nnz_capacity) if nnz_capacity is not None else min(worst, max(heads * 8 * Z * 64,
                                                                            worst // 8))
    for _ in range(2):
        nbytes = workspace_bytes(cfg, cap)
        if workspace is None or workspace.numel() < nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        h = ctypes.c_void_p()
        nnz = ctypes.c_int64()
        st = nat.lib().prism_plan_create(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(av_norm), _ptr(workspace), workspace.numel(),
                                         _stream(q.device), ctypes.byref(h), ctypes.byref(nnz))
        if st == nat.PRISM_ENOMEM_WORKSPACE and nnz.value > cap:
            cap = int(nnz.value)
            workspace = None
            continue
        nat.check(st, "prism_plan_create")
        return Plan(h, cfg, workspace, int(nnz.value), q, k, v)
    raise nat.PrismError(nat.PRISM_ENOMEM_WORKSPACE, "prism_plan_create")


def attn_fwd(pl: Plan, q, k, v, o=None, lse=None):
    """Sparse attention forward; returns (o, lse) in the original token order."""
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    nat.check(nat.lib().prism_attn_fwd(pl.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       _stream(q.device)), "prism_attn_fwd")
    return o, lse


def attn_bwd_workspace_bytes(pl: Plan) -> int:
    n = ctypes.c_size_t()
    nat.check(nat.lib().prism_attn_bwd_workspace_size(ctypes.byref(pl.cfg), ctypes.byref(n)),
              "prism_attn_bwd_workspace_size")
    return n.value


def attn_bwd(pl: Plan, q, k, v, o, lse, do, dq=None, dk=None, dv=None, workspace=None):
    """Backward with the plan held constant; returns (dq, dk, dv).  Without a
    workspace one of attn_bwd_workspace_bytes(pl) is allocated; a given one
    is used as it is (one holding only the Delta / LSE columns, 8 bytes per
    token and head, runs the backward without the copies of Q and dO)."""
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(attn_bwd_workspace_bytes(pl), dtype=torch.uint8,
                                device=q.device)
    nat.check(nat.lib().prism_attn_bwd(pl.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                       workspace.numel(), _stream(q.device)), "prism_attn_bwd")
    return dq, dk, dv


def attn_bwd_noalloc(pl: Plan, q, k, v, o, lse, do, dq, dk, dv):
    """prism_attn_bwd_noalloc: the backward with its scratch in the library's
    static per-GPU array (no workspace, no allocation).  The caller passes
    the output tensors; raises PrismError (workspace too small) when the
    problem needs more scratch than the array holds."""
    nat.check(nat.lib().prism_attn_bwd_noalloc(pl.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                               _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                               _ptr(dv), _stream(q.device)),
              "prism_attn_bwd_noalloc")
    return dq, dk, dv


def av_cross_attn(q, ka, va, o=None, norm=None, want_o=False):
    """The A->V norm map: h_hat = softmax(q ka^T / sqrt(D)) va per head for
    the video queries q [heads, N, D] over the audio keys and values
    [heads, Na, D], and norm [N] = ||h_hat_n||_2 over heads and channels (the
    av_norm of the next layer's plan).  Returns (norm, o); o is None unless
    given or want_o."""
    heads, N, D = q.shape
    assert ka.shape == va.shape and ka.shape[0] == heads and ka.shape[2] == D
    assert q.is_contiguous() and ka.is_contiguous() and va.is_contiguous()
    assert q.dtype == ka.dtype == va.dtype
    if o is None and want_o:
        o = torch.empty_like(q)
    if norm is None:
        norm = torch.empty(N, dtype=torch.float32, device=q.device)
    dt = nat.PRISM_BF16 if q.dtype == torch.bfloat16 else nat.PRISM_F32
    nat.check(nat.lib().prism_av_cross_attn(_ptr(q), _ptr(ka), _ptr(va), heads, N,
                                            ka.shape[1], D, dt, _ptr(o), _ptr(norm),
                                            _stream(q.device)), "prism_av_cross_attn")
    return norm, o


def block_scores(pl: Plan, head: int) -> torch.Tensor:
    nblk = int(pl.export("blk_off")[head + 1] - pl.export("blk_off")[head])
    out = torch.empty((nblk, nblk), dtype=torch.float32, device=pl.device)
    nat.check(nat.lib().prism_block_scores(pl.handle, int(head), _ptr(out), _stream(pl.device)),
              "prism_block_scores")
    return out


def schedule_value(kind, step: int, steps: int, v0: float, v1: float) -> float:
    """A per-step sparsity schedule (prism_schedule_value): the value at step
    `step` of `steps`, from v0 at the first step to v1 at the last; kind is
    "constant", "linear" or "cosine"."""
    out = ctypes.c_float()
    k = nat.SCHEDULES[kind] if isinstance(kind, str) else int(kind)
    nat.check(nat.lib().prism_schedule_value(k, int(step), int(steps), float(v0), float(v1),
                                             ctypes.byref(out)), "prism_schedule_value")
    return out.value


def candidate(i: int) -> tuple:
    a = (ctypes.c_int32 * 4)()
    nat.check(nat.lib().prism_candidate(int(i), a), "prism_candidate")
    return tuple(a)


def timing_enable(on: bool = True) -> None:
    """Record a HIP event pair around every kernel stage (measurement)."""
    nat.check(nat.lib().prism_timing_enable(1 if on else 0), "prism_timing_enable")


def timing_read() -> dict:
    """{stage: (launches, total_ms)} since the last read; waits for the events."""
    arr = (nat.PrismStageTime * 64)()
    n = ctypes.c_int32()
    nat.check(nat.lib().prism_timing_read(arr, 64, ctypes.byref(n)), "prism_timing_read")
    return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms))
            for i in range(min(n.value, 64))}
