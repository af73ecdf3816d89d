"""ctypes declarations of the C ABI in include/prism.h (libprism.so).

Loading fails loudly when the HIP library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libprism.so")

PRISM_OK = 0
PRISM_EINVAL = 1
PRISM_EUNSUPPORTED = 2
PRISM_ENOMEM_WORKSPACE = 3
PRISM_EDEVICE = 4
PRISM_ESTATE = 5

PRISM_F32 = 0
PRISM_BF16 = 1

SHAPE_MAPS = {"power": 0, "isotropic": 1, "softmax": 2, "rank": 3, "entropy": 4}
SCHEDULES = {"constant": 0, "linear": 1, "cosine": 2}

NOALLOC_SCRATCH_BYTES = 128 << 20   # PRISM_NOALLOC_SCRATCH_BYTES

ARRAYS = {
    "zone_stats": 0, "audio_stats": 1, "shape_id": 2, "blk_off": 3, "blk_start": 4,
    "qbar": 5, "kbar": 6, "qexp": 7, "kexp": 8, "row_ptr": 9, "col_idx": 10,
    "colt_ptr": 11, "colt_idx": 12, "perm": 13, "qgrid": 14, "kgrid": 15, "kv_order": 16,
    "blk_org": 17, "cuts": 18, "qlo": 19, "klo": 20,
}

EXPORTED = [
    "prism_config_default", "prism_config_check", "prism_plan_workspace_size",
    "prism_plan_create", "prism_plan_destroy", "prism_attn_fwd",
    "prism_attn_bwd_workspace_size", "prism_attn_bwd", "prism_attn_bwd_noalloc",
    "prism_av_cross_attn", "prism_block_scores",
    "prism_plan_array_bytes", "prism_plan_export", "prism_plan_info", "prism_candidate",
    "prism_schedule_value",
    "prism_status_str", "prism_timing_enable", "prism_timing_read",
]


class PrismConfig(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("top_k_frac", ctypes.c_float), ("top_p", ctypes.c_float),
        ("volume_mask", ctypes.c_uint32), ("fixed_shape", ctypes.c_int32 * 3),
        ("eps", ctypes.c_float), ("tau128", ctypes.c_float), ("tau256", ctypes.c_float),
        ("need_backward", ctypes.c_int32), ("shape_map", ctypes.c_int32),
        ("alpha", ctypes.c_float), ("cut_threshold", ctypes.c_float),
        ("relayout", ctypes.c_int32),
    ]


class PrismPlanInfo(ctypes.Structure):
    _fields_ = [
        ("total_blocks", ctypes.c_int64), ("nnz", ctypes.c_int64),
        ("max_blocks_per_head", ctypes.c_int64), ("pair_tokens", ctypes.c_double),
        ("shape_hist", ctypes.c_int64 * 16), ("kv_persistent", ctypes.c_int32),
    ]


class PrismStageTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


class PrismError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cfgp = ctypes.POINTER(PrismConfig)
        L.prism_config_default.argtypes = [cfgp]
        L.prism_config_default.restype = None
        L.prism_config_check.argtypes = [cfgp]
        L.prism_plan_workspace_size.argtypes = [cfgp, i64, ctypes.POINTER(sz)]
        L.prism_plan_create.argtypes = [cfgp, vp, vp, vp, vp, vp, sz, vp,
                                        ctypes.POINTER(vp), ctypes.POINTER(i64)]
        L.prism_plan_destroy.argtypes = [vp]
        L.prism_plan_destroy.restype = None
        L.prism_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.prism_attn_bwd_workspace_size.argtypes = [cfgp, ctypes.POINTER(sz)]
        L.prism_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.prism_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.prism_av_cross_attn.argtypes = [vp, vp, vp, i32, i64, i32, i32, i32, vp, vp, vp]
        L.prism_block_scores.argtypes = [vp, i32, vp, vp]
        L.prism_plan_array_bytes.argtypes = [vp, i32, ctypes.POINTER(sz)]
        L.prism_plan_export.argtypes = [vp, i32, vp, sz, vp]
        L.prism_plan_info.argtypes = [vp, ctypes.POINTER(PrismPlanInfo), vp]
        L.prism_candidate.argtypes = [i32, ctypes.POINTER(ctypes.c_int32)]
        L.prism_schedule_value.argtypes = [i32, i64, i64, ctypes.c_float, ctypes.c_float,
                                           ctypes.POINTER(ctypes.c_float)]
        L.prism_timing_enable.argtypes = [i32]
        L.prism_timing_read.argtypes = [ctypes.POINTER(PrismStageTime), i32,
                                        ctypes.POINTER(ctypes.c_int32)]
        L.prism_status_str.argtypes = [ctypes.c_int]
        L.prism_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(s: int) -> str:
    return lib().prism_status_str(int(s)).decode()


def check(status: int, where: str) -> None:
    if status != PRISM_OK:
        raise PrismError(status, where)
