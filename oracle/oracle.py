"""Python face of the CPU oracle (prism_oracle.c).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's
CPU-baseline leg use this module; the product path never imports it.

Every function follows one step of Prism's Algorithm 1 (paper.rainbus.top,
section "方法步骤详情"; formulas as printed on xyznot.com/id, "Metode" 1-3):
zone statistics -> indicator / volume / shape -> zone-aware re-layout and
mean pooling -> block scores and Top-k U Top-p -> attention over the
selected blocks.  Tensors are numpy arrays laid out [heads, T*H*W, D], with
bf16 passed as its raw uint16 bit pattern.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "prism_oracle.c")

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, no fast-math, no contraction)."""
    if force or not os.path.exists(LIB_PATH) or (
        os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH)
    ):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, SRC_PATH, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(LIB_PATH)
        _lib.orc_exp2.restype = ctypes.c_float
        _lib.orc_exp2.argtypes = [ctypes.c_float]
        _lib.orc_nearest_shape.argtypes = [ctypes.c_void_p, ctypes.c_int]
        _lib.orc_lstar.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        _lib.orc_select_row.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p]
        _lib.orc_shapes.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_float, ctypes.c_float, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
            ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        _lib.orc_detect_cuts.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
        _lib.orc_nearest_shape_map.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_float]
        _lib.orc_map_target.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_float, ctypes.c_void_p]
        for name in ("orc_wlog2", "orc_wln", "orc_wexp"):
            getattr(_lib, name).restype = ctypes.c_double
            getattr(_lib, name).argtypes = [ctypes.c_double]
        _lib.orc_score_row.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        _lib.orc_quantize.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return 0
    if x.dtype == np.uint16:
        return 1
    raise TypeError(f"oracle takes float32 or bf16-as-uint16 arrays, got {x.dtype}")


# ---------------------------------------------------------------- shapes

def candidates() -> np.ndarray:
    """[16, 4] table of (bT, bH, bW, B): edges in {2,4,8}, product B."""
    out = np.zeros((16, 4), np.int32)
    n = lib().orc_candidates(_p(out))
    return out[:n]


def shape_id_of(bt: int, bh: int, bw: int) -> int:
    for i, row in enumerate(candidates()):
        if tuple(row[:3]) == (bt, bh, bw):
            return i
    raise ValueError(f"({bt},{bh},{bw}) is not a candidate shape")


def lstar(g, B: int) -> np.ndarray:
    g = np.ascontiguousarray(g, np.float32)
    out = np.zeros(3, np.float64)
    lib().orc_lstar(_p(g), B, _p(out))
    return out


def nearest_shape(g, B: int) -> int:
    g = np.ascontiguousarray(g, np.float32)
    return lib().orc_nearest_shape(_p(g), B)


def exp2(x: float) -> float:
    return lib().orc_exp2(float(x))


# shape mappings (ids as in include/prism.h's prism_shape_map)
MAP_POWER, MAP_ISOTROPIC, MAP_SOFTMAX, MAP_RANK, MAP_ENTROPY = range(5)


def map_target(g, B: int, shape_map: int, alpha: float = 0.5) -> np.ndarray:
    g = np.ascontiguousarray(g, np.float32)
    out = np.zeros(3, np.float64)
    assert lib().orc_map_target(_p(g), B, shape_map, np.float32(alpha), _p(out)) == 0
    return out


def nearest_shape_map(g, B: int, shape_map: int, alpha: float = 0.5) -> int:
    g = np.ascontiguousarray(g, np.float32)
    return lib().orc_nearest_shape_map(_p(g), B, shape_map, np.float32(alpha))


def wlog2(x: float) -> float:
    return lib().orc_wlog2(float(x))


def wln(x: float) -> float:
    return lib().orc_wln(float(x))


def wexp(x: float) -> float:
    return lib().orc_wexp(float(x))


# ---------------------------------------------------------------- config

@dataclass
class Config:
    T: int
    H: int
    W: int
    heads: int
    head_dim: int
    top_k: int = 16
    top_k_frac: float = 0.0
    top_p: float = 0.9
    volume_mask: int = 7
    fixed_shape: tuple = (0, 0, 0)
    eps: float = 1e-4
    tau128: float = 0.5
    tau256: float = 0.25
    shape_map: int = 0       # MAP_POWER
    alpha: float = 0.5
    cut_threshold: float = 0.0   # > 0: shot-cut-aware temporal zones

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def Z(self) -> int:
        return (self.T // 8) * (self.H // 8) * (self.W // 8)

    def k_for(self, nblk: int) -> int:
        """Top-k size: a block count, or ceil(frac * N_blk) when frac > 0."""
        if self.top_k_frac > 0:
            k = int(math.ceil(np.float64(np.float32(self.top_k_frac)) * nblk))
        else:
            k = self.top_k
        return max(0, min(k, nblk))


@dataclass
class Plan:
    cfg: Config
    vstats: np.ndarray            # [heads, Z, 5]
    astats: np.ndarray | None     # [Z, 4]
    g: np.ndarray                 # [heads, Z, 3]
    volume: np.ndarray            # [heads, Z]
    shape_id: np.ndarray          # [heads, Z] uint8
    blk_off: np.ndarray           # [heads + 1] int64
    blk_start: np.ndarray         # [G] int32 (permuted row of the block's first token)
    blk_len: np.ndarray           # [G] int32
    perm: np.ndarray              # [heads, N] int32 permuted position -> token
    qbar: np.ndarray              # [G, D] fp32
    kbar: np.ndarray              # [G, D] fp32
    qgrid: np.ndarray             # [G, D] fp32 (integers): the grid's high part
    qexp: np.ndarray              # [G] int32
    kgrid: np.ndarray
    kexp: np.ndarray
    qlo: np.ndarray               # [G, D] fp32 (integers): the grid's low part
    klo: np.ndarray
    rows: dict = field(default_factory=dict)   # (head, local block) -> selected local key ids
    cuts: np.ndarray | None = None             # [T] uint8 shot cuts (cut_threshold > 0)

    def nblk(self, h: int) -> int:
        return int(self.blk_off[h + 1] - self.blk_off[h])


def zone_stats(v: np.ndarray, cfg: Config) -> np.ndarray:
    out = np.zeros((cfg.heads, cfg.Z, 5), np.float32)
    rc = lib().orc_zone_stats(_p(v), _dtype_code(v), cfg.T, cfg.H, cfg.W, cfg.heads,
                              cfg.head_dim, _p(out))
    assert rc == 0
    return out


def audio_stats(a: np.ndarray, cfg: Config) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float32)
    out = np.zeros((cfg.Z, 4), np.float32)
    rc = lib().orc_audio_stats(_p(a), cfg.T, cfg.H, cfg.W, _p(out))
    assert rc == 0
    return out


def detect_cuts(v: np.ndarray, cfg: Config):
    """Shot cuts from the frame-difference energy of V: (cuts [T] uint8,
    energy [T] fp64)."""
    cuts = np.zeros(cfg.T, np.uint8)
    energy = np.zeros(cfg.T, np.float64)
    rc = lib().orc_detect_cuts(_p(v), _dtype_code(v), cfg.T, cfg.H, cfg.W, cfg.heads,
                               cfg.head_dim, np.float32(cfg.cut_threshold), _p(cuts),
                               _p(energy))
    assert rc == 0
    return cuts, energy


def cut_caps(cuts: np.ndarray, T: int) -> np.ndarray:
    cap = np.zeros(T // 8, np.int32)
    lib().orc_cut_caps(_p(np.ascontiguousarray(cuts, np.uint8)), T, _p(cap))
    return cap


def shapes(vstats, astats, cfg: Config, zt_cap=None):
    fixed = -1 if tuple(cfg.fixed_shape) == (0, 0, 0) else shape_id_of(*cfg.fixed_shape)
    sid = np.zeros((cfg.heads, cfg.Z), np.uint8)
    g = np.zeros((cfg.heads, cfg.Z, 3), np.float32)
    vol = np.zeros((cfg.heads, cfg.Z), np.int32)
    cap = None if zt_cap is None else np.ascontiguousarray(zt_cap, np.int32)
    zpt = (cfg.H // 8) * (cfg.W // 8)
    rc = lib().orc_shapes(_p(vstats), _p(astats), cfg.heads, cfg.Z, np.float32(cfg.eps),
                          np.float32(cfg.tau128), np.float32(cfg.tau256), cfg.volume_mask,
                          fixed, cfg.shape_map, np.float32(cfg.alpha), _p(cap), zpt, _p(sid),
                          _p(g), _p(vol))
    assert rc == 0
    return sid, g, vol


def block_table(shape_id: np.ndarray, cfg: Config):
    cand = candidates()
    G = int(sum(512 // cand[s, 3] for s in shape_id.reshape(-1)))
    off = np.zeros(cfg.heads + 1, np.int64)
    start = np.zeros(G, np.int32)
    ln = np.zeros(G, np.int32)
    lib().orc_block_table(_p(shape_id), cfg.heads, cfg.Z, _p(off), _p(start), _p(ln))
    return off, start, ln


def perm_map(shape_id: np.ndarray, cfg: Config) -> np.ndarray:
    perm = np.zeros((cfg.heads, cfg.N), np.int32)
    lib().orc_perm_map(_p(shape_id), cfg.T, cfg.H, cfg.W, cfg.heads, _p(perm))
    return perm


def pool(x: np.ndarray, shape_id, blk_off, cfg: Config) -> np.ndarray:
    G = int(blk_off[-1])
    out = np.zeros((G, cfg.head_dim), np.float32)
    lib().orc_pool(_p(x), _dtype_code(x), cfg.T, cfg.H, cfg.W, cfg.heads, cfg.head_dim,
                   _p(shape_id), _p(blk_off), _p(out))
    return out


def quantize(xbar: np.ndarray):
    """Two-level integer grid of pooled rows: (hi [rows, D], E [rows],
    lo [rows, D]) with x ~ 2^E (hi + 2^-8 lo)."""
    xbar = np.ascontiguousarray(xbar, np.float32)
    q = np.zeros_like(xbar)
    lo = np.zeros_like(xbar)
    e = np.zeros(xbar.shape[0], np.int32)
    lib().orc_quantize(_p(xbar), xbar.shape[0], xbar.shape[1], _p(q), _p(lo), _p(e))
    return q, e, lo


def plan(q, k, v, av_norm, cfg: Config) -> Plan:
    """Stages one to three up to the pooled, integer-grid block means."""
    vs = zone_stats(v, cfg)
    ast = None if av_norm is None else audio_stats(av_norm, cfg)
    cuts = None
    if cfg.cut_threshold > 0:
        cuts, _ = detect_cuts(v, cfg)
    sid, g, vol = shapes(vs, ast, cfg, None if cuts is None else cut_caps(cuts, cfg.T))
    off, start, ln = block_table(sid, cfg)
    perm = perm_map(sid, cfg)
    qbar = pool(q, sid, off, cfg)
    kbar = pool(k, sid, off, cfg)
    qg, qe, ql = quantize(qbar)
    kg, ke, kl = quantize(kbar)
    pl = Plan(cfg, vs, ast, g, vol, sid, off, start, ln, perm, qbar, kbar, qg, qe, kg, ke, ql,
              kl)
    pl.cuts = cuts
    return pl


def score_row(pl: Plan, h: int, i: int) -> np.ndarray:
    """Block scores s_ij (fp32) of local query block i of head h."""
    o, n = int(pl.blk_off[h]), pl.nblk(h)
    s = np.zeros(n, np.float32)
    qrow = np.ascontiguousarray(pl.qgrid[o + i])
    qlo = np.ascontiguousarray(pl.qlo[o + i])
    kg = np.ascontiguousarray(pl.kgrid[o:o + n])
    kl = np.ascontiguousarray(pl.klo[o:o + n])
    ke = np.ascontiguousarray(pl.kexp[o:o + n])
    lib().orc_score_row(_p(qrow), _p(qlo), int(pl.qexp[o + i]), _p(kg), _p(kl), _p(ke), n,
                        pl.cfg.head_dim, _p(s))
    return s


def select_from_scores(s: np.ndarray, k: int, p: float) -> np.ndarray:
    s = np.ascontiguousarray(s, np.float32)
    out = np.zeros(max(1, s.shape[0]), np.int32)
    cnt = lib().orc_select_row(_p(s), s.shape[0], k, np.float32(p), _p(out))
    return out[:cnt].copy()


def select_row(pl: Plan, h: int, i: int) -> np.ndarray:
    key = (h, i)
    if key not in pl.rows:
        s = score_row(pl, h, i)
        pl.rows[key] = select_from_scores(s, pl.cfg.k_for(pl.nblk(h)), pl.cfg.top_p)
    return pl.rows[key]


def select_all(pl: Plan, heads=None, threads: int = 1):
    """Full CSR over the listed heads: (row_ptr [G+1] int64 over all blocks,
    col_idx int32).  Rows of heads not listed are empty.  Rows are
    independent; with threads > 1 they are computed by that many host
    threads (the C calls release the interpreter lock), which changes no
    result."""
    heads = range(pl.cfg.heads) if heads is None else heads
    G = int(pl.blk_off[-1])
    counts = np.zeros(G, np.int64)
    lists = {}
    todo = [(h, i) for h in heads for i in range(pl.nblk(h))]
    if threads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda hi: select_row(pl, *hi), todo, chunksize=64))
    for h, i in todo:
        r = select_row(pl, h, i)
        lists[int(pl.blk_off[h]) + i] = r
        counts[int(pl.blk_off[h]) + i] = len(r)
    row_ptr = np.zeros(G + 1, np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col = np.zeros(int(row_ptr[-1]), np.int32)
    for g, r in lists.items():
        col[row_ptr[g]:row_ptr[g + 1]] = r
    return row_ptr, col


# ---------------------------------------------------------------- attention

def _items(pl: Plan, items):
    ih = np.array([h for h, _ in items], np.int32)
    ib = np.array([b for _, b in items], np.int32)
    sels = [select_row(pl, h, b) for h, b in items]
    ptr = np.zeros(len(items) + 1, np.int64)
    np.cumsum([len(s) for s in sels], out=ptr[1:])
    idx = np.concatenate(sels).astype(np.int32) if sels else np.zeros(0, np.int32)
    return ih, ib, ptr, np.ascontiguousarray(idx)


def attn_fwd(q, k, v, pl: Plan, items):
    """O and LSE for (head, local query block) items.
    Returns o [n, 256, D] fp64 and lse [n, 256] (rows in permuted order)."""
    cfg = pl.cfg
    ih, ib, ptr, idx = _items(pl, items)
    o = np.zeros((len(items), 256, cfg.head_dim), np.float64)
    lse = np.zeros((len(items), 256), np.float64)
    lib().orc_attn_fwd(_p(q), _p(k), _p(v), _dtype_code(q), ctypes.c_int64(cfg.N),
                       cfg.head_dim, _p(pl.perm), _p(pl.blk_off), _p(pl.blk_start),
                       _p(pl.blk_len), len(items), _p(ih), _p(ib), _p(ptr), _p(idx),
                       _p(o), _p(lse))
    return o, lse


def attn_bwd_q(q, k, v, do, pl: Plan, items):
    cfg = pl.cfg
    ih, ib, ptr, idx = _items(pl, items)
    dq = np.zeros((len(items), 256, cfg.head_dim), np.float64)
    lib().orc_attn_bwd_q(_p(q), _p(k), _p(v), _p(do), _dtype_code(q), ctypes.c_int64(cfg.N),
                         cfg.head_dim, _p(pl.perm), _p(pl.blk_off), _p(pl.blk_start),
                         _p(pl.blk_len), len(items), _p(ih), _p(ib), _p(ptr), _p(idx),
                         _p(dq))
    return dq


def attn_bwd_kv(q, k, v, do, pl: Plan, items, threads: int = 1, split: int = 1):
    """dK, dV for (head, local key block) items; needs every row of the
    items' heads, so it selects those heads in full.  A key block's gradient
    is a sum over the query blocks that selected it; with split > 1 that list
    is cut into up to `split` parts computed as separate items (in parallel)
    whose fp64 results are then added, which changes only the order of the
    fp64 additions."""
    cfg = pl.cfg
    heads = sorted({h for h, _ in items})
    row_ptr, col = select_all(pl, heads, threads=threads)
    subs = []     # (item index, head, key block, query blocks)
    for it, (h, j) in enumerate(items):
        o = int(pl.blk_off[h])
        lst = [i for i in range(pl.nblk(h))
               if np.any(col[row_ptr[o + i]:row_ptr[o + i + 1]] == j)]
        parts = max(1, min(split, len(lst)))
        for part in np.array_split(np.array(lst, np.int32), parts):
            subs.append((it, h, j, part))
    tptr = np.zeros(len(subs) + 1, np.int64)
    np.cumsum([len(s[3]) for s in subs], out=tptr[1:])
    tidx = (np.ascontiguousarray(np.concatenate([s[3] for s in subs]).astype(np.int32))
            if subs else np.zeros(0, np.int32))
    ih = np.array([s[1] for s in subs], np.int32)
    ib = np.array([s[2] for s in subs], np.int32)
    sdk = np.zeros((len(subs), 256, cfg.head_dim), np.float64)
    sdv = np.zeros((len(subs), 256, cfg.head_dim), np.float64)
    lib().orc_attn_bwd_kv(_p(q), _p(k), _p(v), _p(do), _dtype_code(q), ctypes.c_int64(cfg.N),
                          cfg.head_dim, _p(pl.perm), _p(pl.blk_off), _p(pl.blk_start),
                          _p(pl.blk_len), _p(row_ptr), _p(col), len(subs), _p(ih), _p(ib),
                          _p(tptr), _p(tidx), _p(sdk), _p(sdv))
    dk = np.zeros((len(items), 256, cfg.head_dim), np.float64)
    dv = np.zeros((len(items), 256, cfg.head_dim), np.float64)
    for s, (it, _, _, _) in enumerate(subs):
        dk[it] += sdk[s]
        dv[it] += sdv[s]
    return dk, dv


def tokens_of_block(pl: Plan, h: int, i: int) -> np.ndarray:
    """Original token indices of local block i of head h, in permuted order."""
    g = int(pl.blk_off[h]) + i
    s, n = int(pl.blk_start[g]), int(pl.blk_len[g])
    return pl.perm[h, s:s + n]


def attn_bwd_head(q, k, v, do, pl: Plan, h: int):
    """dQ, dK, dV of head h ([N, D] fp64 each, original token order), walking
    every query row once over the head's full selection."""
    cfg = pl.cfg
    row_ptr, col = select_all(pl, [h])
    dq = np.zeros((cfg.N, cfg.head_dim), np.float64)
    dk = np.zeros_like(dq)
    dv = np.zeros_like(dq)
    lib().orc_attn_bwd_head(_p(q), _p(k), _p(v), _p(do), _dtype_code(q), ctypes.c_int64(cfg.N),
                            cfg.head_dim, _p(pl.perm), _p(pl.blk_off), _p(pl.blk_start),
                            _p(pl.blk_len), _p(row_ptr), _p(col), h, _p(dq), _p(dk), _p(dv))
    return dq, dk, dv


# ---------------------------------------------------------------- A->V norm map

def av_cross(q, ka, va, tokens, want_o: bool = False):
    """A->V cross-attention of video queries q [heads, N, D] over audio keys
    and values ka, va [heads, Na, D] at the listed tokens: the norm
    ||h_hat_n||_2 over all heads and channels (fp64), and optionally h_hat
    [len(tokens), heads, D]."""
    heads, N, D = q.shape
    Na = ka.shape[1]
    tokens = np.ascontiguousarray(tokens, np.int64)
    norm = np.zeros(len(tokens), np.float64)
    o = np.zeros((len(tokens), heads, D), np.float64) if want_o else None
    rc = lib().orc_av_cross(_p(q), _p(ka), _p(va), _dtype_code(q), heads, ctypes.c_int64(N),
                            ctypes.c_int64(Na), D, len(tokens), _p(tokens), _p(norm), _p(o))
    assert rc == 0
    return (norm, o) if want_o else norm
