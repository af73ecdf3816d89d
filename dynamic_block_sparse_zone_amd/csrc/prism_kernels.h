// Host-side launchers of the gfx950 kernels (one translation unit each).
#pragma once
#include "prism_common.h"
#include <vector>

namespace prism {

bool launch_zone_stats(const void* v, int dtype, int D, int H, int W, int Z, int heads,
                       int64_t N, float* out, hipStream_t st);
bool launch_audio_stats(const float* a, int H, int W, int Z, float* out, hipStream_t st);
bool launch_shapes(const PlanDev& P, int have_audio, const prism_config& c, int fixed_id,
                   hipStream_t st);
bool launch_blk_off(const PlanDev& P, hipStream_t st);
bool launch_permute_pool(const PlanDev& P, const void* q, const void* k, const void* v,
                         hipStream_t st);
bool launch_block_scores(const PlanDev& P, int64_t g0, int n, float* out, hipStream_t st);
bool launch_select(const PlanDev& P, int64_t g0, int n, const prism_config& c, int last,
                   hipStream_t st);
bool launch_transpose(const PlanDev& P, int64_t g0, int n, int last, hipStream_t st);
bool launch_perm_map(const PlanDev& P, int32_t* out, hipStream_t st);
bool launch_sum_i64(const int64_t* in, int64_t n, int64_t* out, hipStream_t st);
// the dK/dV work-unit order (after the transpose)
bool launch_unit_order_k(const PlanDev& P, const std::vector<int64_t>& off, hipStream_t st);

bool launch_attn_fwd(const PlanDev& P, const void* q, void* o, float* lse, hipStream_t st);

struct BwdDev {
  float* delta;    // [heads][N] rowsum(dO * O), permuted order
  float* lse_p;    // [heads][N] lse, permuted order
  void* qp;        // [heads][N][D] permuted Q (swizzled like K/V)
  void* dop;       // [heads][N][D] permuted dO
};
bool launch_bwd_prep(const PlanDev& P, const BwdDev& B, const void* q, const void* o,
                     const float* lse, const void* d_o, hipStream_t st);
bool launch_bwd_dkdv(const PlanDev& P, const BwdDev& B, void* dk, void* dv, hipStream_t st);
bool launch_bwd_dq(const PlanDev& P, const BwdDev& B, void* dq, hipStream_t st);

// stage timing (measurement support)
void stage_begin(const char* name, hipStream_t st);
void stage_end(hipStream_t st);

}  // namespace prism
