"""MI355X (gfx950) implementation of Prism's dynamic block-sparse video
self-attention: zone statistics, content-adaptive block shapes, zone-aware
re-layout, Top-k U Top-p block selection and sparse attention forward and
backward, behind the C ABI of include/prism.h."""
from .api import (Plan, attn_bwd, attn_bwd_noalloc, attn_bwd_workspace_bytes, attn_fwd,
                  av_cross_attn, block_scores, candidate, make_config, plan, schedule_value,
                  timing_enable, timing_read, workspace_bytes)

__all__ = ["Plan", "plan", "attn_fwd", "attn_bwd", "attn_bwd_noalloc",
           "attn_bwd_workspace_bytes", "av_cross_attn", "block_scores",
           "candidate", "make_config", "schedule_value", "workspace_bytes", "timing_enable",
           "timing_read"]
