// Host-side launchers of the gfx950 kernels (one translation unit each).
#pragma once
#include "prism_common.h"
#include <vector>

namespace prism {

bool launch_zone_stats(const void* v, int dtype, int D, int H, int W, int Z, int heads,
                       int64_t N, float* out, hipStream_t st);
bool launch_audio_stats(const float* a, int H, int W, int Z, float* out, hipStream_t st);
bool launch_cuts(const PlanDev& P, const void* v, float kappa, hipStream_t st);
bool launch_shapes(const PlanDev& P, int have_audio, const prism_config& c, int fixed_id,
                   hipStream_t st);
bool launch_blk_off(const PlanDev& P, hipStream_t st);
bool launch_pool(const PlanDev& P, const void* q, const void* k, hipStream_t st);
bool launch_block_scores(const PlanDev& P, int64_t g0, int n, float* out, hipStream_t st);
bool launch_select(const PlanDev& P, int64_t g0, int n, const prism_config& c, int last,
                   hipStream_t st);
bool launch_transpose(const PlanDev& P, int64_t g0, int n, int last, hipStream_t st);
bool launch_perm_map(const PlanDev& P, int32_t* out, hipStream_t st);
bool launch_sum_i64(const int64_t* in, int64_t n, int64_t* out, hipStream_t st);
// the dK/dV work-unit order (after the transpose)
bool launch_unit_order_k(const PlanDev& P, hipStream_t st);

bool launch_attn_fwd(const PlanDev& P, const void* q, const void* k, const void* v, void* o,
                     float* lse, hipStream_t st);

// the backward's inputs and its scratch (per-token columns in the original
// token order)
struct BwdDev {
  const void* q;
  const void* k;
  const void* v;
  const void* d_o;
  float* delta;    // [heads][N] rowsum(dO * O)
  float* lse2;     // [heads][N] log2(e) * LSE
  // with the re-layout: Q, dO, Delta and log2(e) * LSE in block-contiguous
  // order (rows swizzled as the plan's K and V copies), else null
  uint16_t* qp;
  uint16_t* dop;
  float* delta_p;
  float* lse2_p;
};
// Rows of two [heads][N][128] bf16 tensors (and, when fa is given, of two
// [heads][N] float columns) into block-contiguous order with swizzled chunks.
bool launch_relayout(const PlanDev& P, const void* a, const void* b, const float* fa,
                     const float* fb, uint16_t* ap, uint16_t* bp, float* fap, float* fbp,
                     hipStream_t st);
bool launch_bwd_prep(const PlanDev& P, const BwdDev& B, const void* o, const float* lse,
                     hipStream_t st);
bool launch_bwd_dkdv(const PlanDev& P, const BwdDev& B, void* dk, void* dv, hipStream_t st);
bool launch_bwd_dq(const PlanDev& P, const BwdDev& B, void* dq, hipStream_t st);

// the A->V cross-attention and its per-token output norm (the next layer's
// av_norm map)
bool launch_av_cross(const void* q, const void* ka, const void* va, int heads, int64_t N,
                     int Na, void* o, float* norm, hipStream_t st);

// stage timing (measurement support)
void stage_begin(const char* name, hipStream_t st);
void stage_end(hipStream_t st);

}  // namespace prism
