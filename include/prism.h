/*
 * prism.h -- C ABI of an MI355X (gfx950) implementation of Prism's dynamic
 * block-sparse video self-attention ("Prism: Dynamic Sparse Attention for
 * Native 2K Joint Video-Audio Generation Model Training", arXiv 2610.05416).
 *
 * The method (paper.rainbus.top, section "方法步骤详情", five stages; formulas
 * on xyznot.com/id, "Metode" 1-3):
 *   1. per 8x8x8 macro-zone and head: directional variance ratio r_{v,d} of
 *      the axis-mean-pooled V, audio coupling abar and directional variance
 *      vhat_{a,d} of the cached A->V cross-attention norm map, indicator
 *      g_d = r_{v,d} + abar vhat_{a,d} + eps, density rho -> block volume
 *      B in {64,128,256}, block shape nearest (in log2 space) to the
 *      continuous optimum b_d ~ g_d^(-1/2) among 16 candidates;
 *   2. zone-aware re-layout of the tokens into block-contiguous order;
 *   3. mean-pooled block representatives, block scores
 *      P_i = softmax(Qbar_i Kbar^T / sqrt(D)), S_i = TopK(P_i,k) U TopP(P_i,p);
 *   4. attention of every query block over the tokens of S_i only;
 *   5. results back in the original token order.
 * The plan (stages 1-3) is a constant for the backward pass: gradients flow
 * only through attention on the selected blocks (same page, "技术新颖性").
 *
 * Conventions for every entry point:
 *   - tensors are contiguous [heads][T*H*W][head_dim], token n =
 *     (t*H + h)*W + w (row-major t, h, w), element type cfg->dtype;
 *   - every tensor pointer is DEVICE memory unless stated otherwise;
 *   - `stream` is a hipStream_t (NULL = the default stream); all device work
 *     is enqueued on it, and a call returns once its work is enqueued except
 *     where a host read-back is stated;
 *   - the library allocates no device memory: the caller provides every
 *     buffer and the plan workspace, and keeps them alive while a plan that
 *     points into them is in use;
 *   - no call aborts or prints; failures are returned as prism_status.
 *     Asynchronous device faults surface as PRISM_EDEVICE from a later call.
 *   - plans may be used from any host thread, but two calls that use one
 *     plan must not run concurrently on different streams (prism_attn_bwd
 *     keeps the start counters of its dK/dV launch in the plan workspace;
 *     two overlapping backward calls on one plan would share them, which
 *     slows both and changes no result).
 */
#ifndef PRISM_H
#define PRISM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PRISM_OK = 0,
  PRISM_EINVAL = 1,             /* bad argument: NULL pointer, size, hyper-parameter */
  PRISM_EUNSUPPORTED = 2,       /* valid, but not provided (dtype / head_dim combination) */
  PRISM_ENOMEM_WORKSPACE = 3,   /* caller's workspace too small; see *_needed outputs */
  PRISM_EDEVICE = 4,            /* HIP runtime reported an error */
  PRISM_ESTATE = 5              /* arguments do not match the plan they are used with */
} prism_status;

typedef enum { PRISM_F32 = 0, PRISM_BF16 = 1 } prism_dtype;

/* Block-shape mapping from the indicator g_d to the target point l in log2
 * space (sum_d l_d = S = log2 B); the shape is the candidate of volume B
 * nearest to l.  PRISM_MAP_POWER with alpha = 1/2 is the pages' method,
 * b_d ~ g_d^(-1/2) (xyznot.com/id "Metode" 2).  The others are the
 * ablations that paper.rainbus.top "技术新颖性" (Table 10) names without
 * formulas, in these readings:
 *   PRISM_MAP_POWER      l_d = -alpha log2 g_d + (S + alpha sum log2 g) / 3
 *                        (b_d ~ g_d^(-alpha); the pages try 1/3, 1/2, 2)
 *   PRISM_MAP_ISOTROPIC  l_d = S / 3 (the most cubic candidate)
 *   PRISM_MAP_SOFTMAX    l_d = S softmax(-g)_d
 *   PRISM_MAP_RANK       l_d = S / 3 + rank_d - 1, rank 0 = largest g_d
 *   PRISM_MAP_ENTROPY    l_d = S i_d / sum i, i_d = -ln(g_d / sum g)
 * Every mapping other than alpha = 1/2 is evaluated in fp64 in a fixed
 * order with a written logarithm and exponential. */
typedef enum {
  PRISM_MAP_POWER = 0,
  PRISM_MAP_ISOTROPIC = 1,
  PRISM_MAP_SOFTMAX = 2,
  PRISM_MAP_RANK = 3,
  PRISM_MAP_ENTROPY = 4
} prism_shape_map;

/* Hyper-parameters and problem size.  Defaults (prism_config_default) are
 * the pages' constants: eps = 1e-4, tau_128 = 0.5, tau_256 = 0.25
 * (paper.rainbus.top "方法步骤详情" and "复现评估"). */
typedef struct {
  int32_t T, H, W;        /* token grid; each a positive multiple of 8 (zones are 8x8x8) */
  int32_t heads;          /* >= 1 */
  int32_t head_dim;       /* 64 or 128; the bf16 attention kernels take 128 */
  int32_t dtype;          /* prism_dtype of Q, K, V, O, dO, dQ, dK, dV */
  int32_t top_k;          /* Top-k size in key blocks (>= 0, clamped to the head's block count) */
  float top_k_frac;       /* > 0: Top-k size = ceil(top_k_frac * N_blk) instead of top_k */
  float top_p;            /* Top-p mass in [0, inf); >= 1 selects every block, 0 = Top-k only */
  uint32_t volume_mask;   /* allowed volumes: bit0 = 64, bit1 = 128, bit2 = 256 (nonzero) */
  int32_t fixed_shape[3]; /* {0,0,0}: dynamic shapes; else one (bT,bH,bW) candidate for all zones */
  float eps;              /* indicator floor, added to every g_d */
  float tau128;           /* rho < tau128 -> volume >= 128 */
  float tau256;           /* rho < tau256 -> volume 256 */
  int32_t need_backward;  /* nonzero: also build the key-major lists prism_attn_bwd needs */
  int32_t shape_map;      /* prism_shape_map (default PRISM_MAP_POWER) */
  float alpha;            /* exponent of PRISM_MAP_POWER, >= 0 (default 1/2) */
  float cut_threshold;    /* > 0: shot-cut-aware temporal zones (paper.rainbus.top
                             "独立分析的弱点" (1)): frame t starts a shot cut when its
                             frame-difference energy of V, e_t = mean over heads, tokens
                             and channels of (V_t - V_{t-1})^2 (fp64), exceeds
                             cut_threshold * mean_t e_t; a zone with a cut at offset c
                             of its 8 frames takes only blocks with b_T <= the largest
                             power of two dividing c (at least 2), and at most 128 tokens
                             when that is 2.  0 (default): fixed 8-frame zones. */
  int32_t relayout;       /* stage two's re-layout (paper.rainbus.top "方法步骤详情", stage
                             two), bf16 with head_dim 128: nonzero (default) = the plan
                             keeps copies of K and V in block-contiguous order, and
                             prism_attn_bwd copies Q and dO the same way when its
                             workspace holds them, so that every attention tile is one
                             contiguous run; 0 = no copies: every tile is gathered from
                             the caller's tensors through the block -> token map.  The
                             results are identical; the copies take 2 x heads x N x 256
                             bytes in the plan's workspace (and the same again, plus 8
                             bytes per token and head, in the backward's) and make the
                             attention kernels 2-7 % faster.  With copies the plan holds
                             K and V as they were at its creation. */
} prism_config;

/* Opaque plan: block shapes, block table and selected key-block lists of
 * one layer call.  Host object; its device arrays live in the caller's
 * workspace. */
typedef struct prism_plan_s prism_plan_t;

/* Fill *cfg with the defaults above (T=H=W=8, heads=1, head_dim=128, bf16,
 * top_k=16, top_p=0.9, all volumes, dynamic shapes, need_backward=1,
 * PRISM_MAP_POWER with alpha = 1/2). */
void prism_config_default(prism_config* cfg);

/* Host-only validation of a configuration; no device work.  PRISM_EINVAL for
 * a malformed configuration; PRISM_EUNSUPPORTED for T*H*W >= 2^24 tokens per
 * head (the kernels address one head's rows with 32-bit byte offsets) or a
 * head_dim other than 64 and 128. */
prism_status prism_config_check(const prism_config* cfg);

/* Bytes of device workspace prism_plan needs for `cfg` when up to
 * nnz_capacity (query block, key block) pairs may be selected over all
 * heads.  nnz_capacity < 0 asks for the worst case (every block selected).
 * Host-only. */
prism_status prism_plan_workspace_size(const prism_config* cfg, int64_t nnz_capacity,
                                       size_t* bytes);

/* Stages 1-3: builds a plan (zone statistics, shapes, the block table of the
 * block-contiguous re-layout of stage 2, pooled means, block scores and the
 * selected key-block lists).  The re-layout itself is never materialised:
 * the attention kernels gather each block's rows from q, k, v (and dO)
 * through the block -> token map, so the plan holds no copy of any tensor.
 *   q, k, v       device [heads][N][head_dim] of cfg->dtype
 *   av_norm       device [N] float32 A->V norm map cached from the previous
 *                 layer, or NULL for the first layer (g = r + eps)
 *   workspace     device buffer of workspace_bytes; at least
 *                 prism_plan_workspace_size(cfg, nnz_capacity) where
 *                 nnz_capacity is derived from workspace_bytes
 *   plan_out      receives a new plan (free with prism_plan_destroy)
 *   nnz_out       receives the number of selected (query block, key block)
 *                 pairs over all heads (may be NULL)
 * Reads back two small arrays to the host (per-head block counts and the
 * pair count), so it synchronises `stream` twice.  If the selection does not
 * fit the workspace it returns PRISM_ENOMEM_WORKSPACE with *nnz_out set to
 * the pair count needed and no plan.  prism_attn_fwd/bwd read q, k and v
 * themselves: they must be the tensors the plan was built from, unchanged. */
prism_status prism_plan_create(const prism_config* cfg, const void* q, const void* k,
                               const void* v, const float* av_norm, void* workspace,
                               size_t workspace_bytes, void* stream, prism_plan_t** plan_out,
                               int64_t* nnz_out);

void prism_plan_destroy(prism_plan_t* plan);

/* Stage 4-5 forward: O = softmax over the selected key tokens of
 * (q k^T / sqrt(head_dim)) times v, for every query token, written in the
 * original token order; lse [heads][N] float32 (natural log of the softmax
 * normaliser), needed by the backward pass.
 * q, k, v must be the tensors the plan was built from (k and v are checked
 * by address: PRISM_ESTATE otherwise).  o: device [heads][N][head_dim]. */
prism_status prism_attn_fwd(const prism_plan_t* plan, const void* q, const void* k,
                            const void* v, void* o, float* lse, void* stream);

/* Bytes of device workspace prism_attn_bwd needs: 8 per token and head
 * (Delta = rowsum(dO * O) and log2(e) * LSE), and with cfg->relayout (bf16,
 * head_dim 128) 520 per token and head (also Q, dO and those two columns in
 * block-contiguous order).  prism_attn_bwd given only the first amount runs
 * without the copies.  Host-only. */
prism_status prism_attn_bwd_workspace_size(const prism_config* cfg, size_t* bytes);

/* Backward with the plan held constant: given dO = dL/dO, writes
 * dq, dk, dv (device [heads][N][head_dim], original token order).
 * o and lse are those prism_attn_fwd produced for the same plan and inputs.
 * Needs a plan built with need_backward; key blocks that no query block
 * selected receive zero gradient.  Deterministic (no floating-point
 * atomics; the dK/dV launch orders its work by the plan's unit order and, for
 * plans selecting at least half of all block pairs, starts the work-groups of
 * each XCD together, which affects timing only). */
prism_status prism_attn_bwd(const prism_plan_t* plan, const void* q, const void* k,
                            const void* v, const void* o, const float* lse, const void* d_o,
                            void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Size of the per-GPU scratch array of prism_attn_bwd_noalloc (128 MiB). */
#define PRISM_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* prism_attn_bwd for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments and results as prism_attn_bwd
 * without the workspace: the backward's scratch lives in a static device
 * array of PRISM_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends.  The call allocates nothing (no hipMalloc,
 * no hipFree, no event creation; the stage timing of prism_timing_enable
 * skips it).  It makes no copies of Q and dO (the 8 bytes per token and head
 * of the columns are all it keeps) and returns PRISM_ENOMEM_WORKSPACE, before
 * any device work, when those exceed the array.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two host threads) race and must not be issued; calls ordered on
 * one stream are safe, since each fully rewrites the scratch it reads. */
prism_status prism_attn_bwd_noalloc(const prism_plan_t* plan, const void* q, const void* k,
                                    const void* v, const void* o, const float* lse,
                                    const void* d_o, void* dq, void* dk, void* dv,
                                    void* stream);

/* The A->V norm map of the next layer: the audio-to-video cross-attention
 * h_hat = CrossAttn(h, K_a, V_a) of the video tokens over the audio tokens
 * and, in its epilogue, the L2 norm of each video position's output
 * (paper.rainbus.top "双分支视频-音频 DiT 与跨模态交叉注意力" and
 * "核心方法": the norm says how much audio a position absorbed; the norms of
 * one layer are cached and guide the block shapes of the next).
 *   q         device [heads][n_video][head_dim]: the video queries
 *             (n_video = T*H*W tokens, row-major t, h, w)
 *   ka, va    device [heads][n_audio][head_dim]: audio keys and values
 *   o         device [heads][n_video][head_dim] output h_hat per head
 *             (softmax(q ka^T / sqrt(head_dim)) va), or NULL to skip it
 *   norm_out  device [n_video] float32: a_n = sqrt(sum over heads and
 *             channels of h_hat^2), the concatenated head outputs before any
 *             output projection; it is the av_norm argument of the next
 *             layer's prism_plan_create
 * bf16 with head_dim 128 only (PRISM_EUNSUPPORTED otherwise); n_video a
 * multiple of 256 (any T, H, W that are multiples of 8), n_audio a multiple
 * of 64, both below 2^24 (PRISM_EINVAL / PRISM_EUNSUPPORTED).  Dense
 * attention over every audio token, deterministic, no scratch. */
prism_status prism_av_cross_attn(const void* q, const void* ka, const void* va, int32_t heads,
                                 int64_t n_video, int32_t n_audio, int32_t head_dim,
                                 int32_t dtype, void* o, float* norm_out, void* stream);

/* Per-step sparsity schedules (paper.rainbus.top "独立分析的弱点" (4): a loose
 * Top-p early and a tighter one later, or a value that follows the denoising
 * step).  The value of a hyper-parameter (top_p, top_k_frac, ...) at step
 * `step` of `steps` (progress s = step / (steps - 1), clamped to [0, 1]; a
 * single step is s = 0), going from v0 at the first step to v1 at the last:
 *   PRISM_SCHED_CONSTANT  v0
 *   PRISM_SCHED_LINEAR    v0 + (v1 - v0) s
 *   PRISM_SCHED_COSINE    v1 + (v0 - v1) (1 + cos(pi s)) / 2
 * evaluated in double and rounded to float.  The caller sets the value into
 * the prism_config of that step's plan.  Host-only; PRISM_EINVAL for an
 * unknown kind, steps < 1 or non-finite ends. */
typedef enum {
  PRISM_SCHED_CONSTANT = 0,
  PRISM_SCHED_LINEAR = 1,
  PRISM_SCHED_COSINE = 2
} prism_schedule_kind;
prism_status prism_schedule_value(int32_t kind, int64_t step, int64_t steps, float v0, float v1,
                                  float* out);

/* Block scores of one head (stage 3): out_scores device float32
 * [N_blk(head)][N_blk(head)], s_ij = Qbar_i . Kbar_j / sqrt(head_dim) with
 * both means on the two-level integer grid x ~ 2^E (hi + 2^-8 lo) of
 * prism_plan_export's QGRID/QLO/QEXP and KGRID/KLO/KEXP (about 17
 * significant bits): the dot product of the grid values is formed exactly
 * and rounded once to float32 before the 1/sqrt(head_dim) scaling. */
prism_status prism_block_scores(const prism_plan_t* plan, int32_t head, float* out_scores,
                                void* stream);

/* Plan arrays that can be copied out for inspection. */
typedef enum {
  PRISM_ARR_ZONE_STATS = 0,   /* float32 [heads][Z][5]: sigma2_T, sigma2_H, sigma2_W, SV, TV */
  PRISM_ARR_AUDIO_STATS = 1,  /* float32 [Z][4]: audio sigma2_T, _H, _W, zone mean (zeros if no map) */
  PRISM_ARR_SHAPE_ID = 2,     /* uint8 [heads][Z]: candidate id (see prism_candidate) */
  PRISM_ARR_BLK_OFF = 3,      /* int64 [heads+1]: first global block id of each head */
  PRISM_ARR_BLK_START = 4,    /* int32 [G]: first permuted row of each block within its head */
  PRISM_ARR_QBAR = 5,         /* float32 [G][head_dim]: block-mean of Q */
  PRISM_ARR_KBAR = 6,         /* float32 [G][head_dim]: block-mean of K */
  PRISM_ARR_QEXP = 7,         /* int32 [G]: E with Qbar ~ 2^E * QGRID */
  PRISM_ARR_KEXP = 8,         /* int32 [G] */
  PRISM_ARR_ROW_PTR = 9,      /* int64 [G+1]: CSR row pointer over global query blocks */
  PRISM_ARR_COL_IDX = 10,     /* int32 [nnz]: selected key blocks (local ids, ascending) */
  PRISM_ARR_COLT_PTR = 11,    /* int64 [G+1]: key-major pointer (need_backward) */
  PRISM_ARR_COLT_IDX = 12,    /* int32 [nnz]: query blocks selecting each key block, ascending */
  PRISM_ARR_PERM = 13,        /* int32 [heads][N]: original token of each permuted row */
  PRISM_ARR_QGRID = 14,       /* uint16 (bf16 bits) [G][head_dim]: high part of the grid of Qbar */
  PRISM_ARR_KGRID = 15,       /* uint16 (bf16 bits) [G][head_dim] */
  PRISM_ARR_KV_ORDER = 16,    /* int32 [heads][N/128] (need_backward): the dK/dV kernel's work
                                 units (128 permuted key rows) of each head, in the order it
                                 takes them: longest walk first (the longest key-major list
                                 among the unit's blocks, in 64-row tiles, capped at 16383),
                                 ties by unit index.  A scheduling order only: dK and dV do
                                 not depend on it. */
  PRISM_ARR_BLK_ORG = 17,     /* int32 [G]: original token (within its head) of each block's
                                 first row: with the block's shape this gives every row's
                                 token in closed form */
  PRISM_ARR_CUTS = 18,        /* uint8 [T] (cut_threshold > 0): 1 where a shot cut starts */
  PRISM_ARR_QLO = 19,         /* uint16 (bf16 bits) [G][head_dim]: low part of the grid of
                                 Qbar, Qbar ~ 2^QEXP (QGRID + 2^-8 QLO) */
  PRISM_ARR_KLO = 20          /* uint16 (bf16 bits) [G][head_dim] */
} prism_array;

/* Size in bytes of a plan array. Host-only. */
prism_status prism_plan_array_bytes(const prism_plan_t* plan, int32_t which, size_t* bytes);

/* Copy a plan array into HOST memory dst (dst_bytes >= its size);
 * synchronises `stream`. */
prism_status prism_plan_export(const prism_plan_t* plan, int32_t which, void* dst,
                               size_t dst_bytes, void* stream);

/* Host-side plan summary. */
typedef struct {
  int64_t total_blocks;       /* G = sum over heads of N_blk */
  int64_t nnz;                /* selected (query block, key block) pairs */
  int64_t max_blocks_per_head;
  double pair_tokens;         /* sum over selected pairs of B_i * B_j */
  int64_t shape_hist[16];     /* zones per candidate shape, over all heads */
  int32_t kv_persistent;      /* 1: prism_attn_bwd runs dK/dV as the ordered persistent
                                 launch (plans selecting at least half of all block pairs);
                                 0: one work-group per unit */
} prism_plan_info_t;

/* Fills *info; pair_tokens needs one device read-back (synchronises). */
prism_status prism_plan_info(const prism_plan_t* plan, prism_plan_info_t* info, void* stream);

/* Candidate shape table, id order: by volume, then lexicographic (bT,bH,bW).
 * Writes bT, bH, bW, B of candidate `id` (0..15). Host-only. */
prism_status prism_candidate(int32_t id, int32_t* out4);

/* Measurement support.  While enabled, every kernel stage the library
 * enqueues is bracketed by a pair of HIP events recorded on the stage's own
 * stream (stage names: plan.stats, plan.shapes, plan.pool, plan.scores,
 * plan.select, plan.transpose, plan.order, attn.fwd, bwd.prep, bwd.dkdv,
 * bwd.dq, av.cross).
 * Host-only; off by default. */
prism_status prism_timing_enable(int32_t enable);

typedef struct {
  char name[32];
  int64_t launches;   /* recorded launches of this stage */
  double total_ms;    /* sum of their event-to-event durations */
} prism_stage_time;

/* Aggregates and clears the recorded stages: writes up to max entries to
 * out (host memory) and the number of distinct stages to *count.  Waits for
 * the recorded events to complete. */
prism_status prism_timing_read(prism_stage_time* out, int32_t max, int32_t* count);

const char* prism_status_str(prism_status s);

#ifdef __cplusplus
}
#endif
#endif /* PRISM_H */
