// Host side of the C ABI declared in include/prism.h: validation, workspace
// carving and the order of the kernel launches.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "prism_common.h"
#include "prism_kernels.h"

using namespace prism;

struct prism_plan_s {
  prism_config cfg;
  PlanDev P;
  std::vector<int64_t> blk_off;  // host copy, heads + 1
  int64_t nnz;
  int64_t max_blocks;
  const void* k;
  const void* v;
  int32_t* perm;  // device [heads][N], written on export
};

// ---------------------------------------------------------------- stage timing
namespace prism {
namespace {
struct StageRec {
  std::string name;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<StageRec> g_recs;
std::vector<hipEvent_t> g_pool;
hipEvent_t pool_get() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

void stage_begin(const char* name, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing) return;
  StageRec r{name, pool_get(), pool_get()};
  if (!r.a || !r.b) return;
  (void)hipEventRecord(r.a, st);
  g_recs.push_back(r);
}

void stage_end(hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing || g_recs.empty()) return;
  (void)hipEventRecord(g_recs.back().b, st);
}
}  // namespace prism

namespace {

int64_t zones_of(const prism_config& c) {
  return (int64_t)(c.T / 8) * (c.H / 8) * (c.W / 8);
}

int fixed_id_of(const prism_config& c) {
  if (c.fixed_shape[0] == 0 && c.fixed_shape[1] == 0 && c.fixed_shape[2] == 0) return -1;
  for (int i = 0; i < kNumShapes; i++)
    if (h_shapes[i].bt == c.fixed_shape[0] && h_shapes[i].bh == c.fixed_shape[1] &&
        h_shapes[i].bw == c.fixed_shape[2])
      return i;
  return -2;
}

// selection density from which the dK/dV kernel runs persistent over the
// planned unit order (measured: 0.86 gains 3-4 %, 0.15 loses 6 %)
constexpr double kPersistDensity = 0.5;

// Sequential sub-allocator over the caller's workspace (256-byte aligned);
// with a null base it only measures.
struct Arena {
  char* base;
  size_t off = 0;
  template <class T>
  T* take(int64_t count) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? (T*)(base + off) : nullptr;
    off += (size_t)count * sizeof(T);
    return p;
  }
};

// Carves the plan arrays; returns bytes used for a given pair capacity.
size_t carve(const prism_config& c, int64_t cap, char* base, PlanDev* P, int32_t** perm) {
  Arena A{base};
  const int64_t Z = zones_of(c);
  const int64_t N = (int64_t)c.T * c.H * c.W;
  const int64_t maxblk = 8 * Z;
  const int64_t G = (int64_t)c.heads * maxblk;
  const int D = c.head_dim;
  P->T = c.T;
  P->H = c.H;
  P->W = c.W;
  P->heads = c.heads;
  P->D = D;
  P->dtype = c.dtype;
  P->Z = (int)Z;
  P->N = N;
  P->vstats = A.take<float>((int64_t)c.heads * Z * 5);
  P->astats = A.take<float>(Z * 4);
  P->shape_id = A.take<uint8_t>((int64_t)c.heads * Z);
  P->zone_base = A.take<int32_t>((int64_t)c.heads * Z);
  P->nblk = A.take<int32_t>(c.heads);
  P->blk_off = A.take<int64_t>(c.heads + 1);
  P->blk_start = A.take<int32_t>(G);
  P->blk_org = A.take<int32_t>(G);
  P->blk_shape = A.take<uint8_t>(G);
  P->blk_head = A.take<int32_t>(G);
  P->qbar = A.take<float>(G * D);
  P->kbar = A.take<float>(G * D);
  P->qgrid = A.take<uint16_t>(G * D);
  P->kgrid = A.take<uint16_t>(G * D);
  P->qlo = A.take<uint16_t>(G * D);
  P->klo = A.take<uint16_t>(G * D);
  P->qexp = A.take<int32_t>(G);
  P->kexp = A.take<int32_t>(G);
  // stage two's copies of K and V (bf16, head_dim 128)
  P->relayout = c.relayout && c.dtype == PRISM_BF16 && c.head_dim == 128;
  P->kp = P->relayout ? A.take<uint16_t>((int64_t)c.heads * N * 128) : nullptr;
  P->vp = P->relayout ? A.take<uint16_t>((int64_t)c.heads * N * 128) : nullptr;
  P->scores = A.take<float>(maxblk * maxblk);
  P->selmask = A.take<unsigned long long>(maxblk * ((maxblk + 63) / 64));
  P->volm = A.take<unsigned long long>(3 * ((maxblk + 63) / 64));
  P->row_cnt = A.take<int32_t>(G);
  P->row_key = A.take<uint32_t>(G);
  P->row_tie = A.take<int32_t>(G);
  P->row_ptr = A.take<int64_t>(G + 1);
  P->row_cost = A.take<int64_t>(G);
  P->counters = A.take<int64_t>(8);
  int32_t* pm = A.take<int32_t>((int64_t)c.heads * N);
  if (perm) *perm = pm;
  if (c.need_backward) {
    P->colt_ptr = A.take<int64_t>(G + 1);
    P->colt_cnt = A.take<int32_t>(G);
    P->chunk_cnt = A.take<int32_t>((maxblk / 64 + 1) * maxblk);
    P->chunk_cost = A.take<int32_t>((maxblk / 64 + 1) * maxblk);
    P->korder = A.take<int32_t>((int64_t)c.heads * (N / 128));
    P->colt_cost = A.take<int64_t>(G);
    P->sync = A.take<int32_t>(128);
  } else {
    P->colt_ptr = nullptr;
    P->colt_cnt = nullptr;
    P->chunk_cnt = nullptr;
    P->chunk_cost = nullptr;
    P->korder = nullptr;
    P->colt_cost = nullptr;
    P->sync = nullptr;
  }
  P->kv_persist = 0;
  P->cut_part = A.take<double>((int64_t)c.T * c.heads);
  P->cut_energy = A.take<double>(c.T);
  P->cuts = A.take<uint8_t>(c.T);
  P->zt_cap = A.take<int32_t>(c.T / 8);
  P->col_idx = A.take<int32_t>(cap);
  P->colt_idx = c.need_backward ? A.take<int32_t>(cap) : nullptr;
  P->cap = cap;
  return A.off + 256;
}

size_t per_pair_bytes(const prism_config& c) { return c.need_backward ? 8 : 4; }

// the configuration asks for stage two's copies and the kernels take them
bool relaid_config(const prism_config& c) {
  return c.relayout && c.dtype == PRISM_BF16 && c.head_dim == 128;
}

// The backward's workspace: Delta and log2(e) * LSE per token (token
// order), and with the copies Q, dO and both columns in block-contiguous
// order.  The same carving serves sizing (base null) and use.
struct BwdCarve {
  float *delta, *lse2, *delta_p, *lse2_p;
  uint16_t *qp, *dop;
};
size_t bwd_carve(const prism_config& c, bool relaid, char* base, BwdCarve* out) {
  const int64_t rows = (int64_t)c.heads * c.T * c.H * c.W;
  Arena A{base};
  BwdCarve b{};
  b.delta = A.take<float>(rows);
  b.lse2 = A.take<float>(rows);
  if (relaid) {
    b.qp = A.take<uint16_t>(rows * 128);
    b.dop = A.take<uint16_t>(rows * 128);
    b.delta_p = A.take<float>(rows);
    b.lse2_p = A.take<float>(rows);
  }
  if (out) *out = b;
  return A.off + 256;
}
size_t bwd_workspace_bytes(const prism_config& c, bool relaid) {
  return bwd_carve(c, relaid, nullptr, nullptr);
}

}  // namespace

extern "C" {

void prism_config_default(prism_config* c) {
  if (!c) return;
  memset(c, 0, sizeof(*c));
  c->T = c->H = c->W = 8;
  c->heads = 1;
  c->head_dim = 128;
  c->dtype = PRISM_BF16;
  c->top_k = 16;
  c->top_k_frac = 0.0f;
  c->top_p = 0.9f;
  c->volume_mask = 7u;
  c->eps = 1e-4f;
  c->tau128 = 0.5f;
  c->tau256 = 0.25f;
  c->need_backward = 1;
  c->shape_map = PRISM_MAP_POWER;
  c->alpha = 0.5f;
  c->cut_threshold = 0.0f;
  c->relayout = 1;
}

prism_status prism_config_check(const prism_config* c) {
  if (!c) return PRISM_EINVAL;
  if (c->T <= 0 || c->H <= 0 || c->W <= 0 || c->T % 8 || c->H % 8 || c->W % 8)
    return PRISM_EINVAL;
  if (c->heads <= 0) return PRISM_EINVAL;
  // one head's rows of 128 bf16 channels are addressed with 32-bit byte
  // offsets by the attention kernels: T*H*W < 2^24
  if ((int64_t)c->T * c->H * c->W >= ((int64_t)1 << 24)) return PRISM_EUNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return PRISM_EUNSUPPORTED;
  if (c->dtype != PRISM_F32 && c->dtype != PRISM_BF16) return PRISM_EINVAL;
  if (c->top_k < 0) return PRISM_EINVAL;
  if (!(c->top_k_frac >= 0.0f) || !isfinite(c->top_k_frac)) return PRISM_EINVAL;
  if (!(c->top_p >= 0.0f)) return PRISM_EINVAL;  // also rejects NaN
  if ((c->volume_mask & 7u) == 0 || (c->volume_mask & ~7u)) return PRISM_EINVAL;
  if (fixed_id_of(*c) == -2) return PRISM_EINVAL;
  if (!(c->eps > 0.0f) || !isfinite(c->eps)) return PRISM_EINVAL;
  if (!(c->tau256 >= 0.0f) || !(c->tau128 >= c->tau256) || !isfinite(c->tau128))
    return PRISM_EINVAL;
  if (c->shape_map < PRISM_MAP_POWER || c->shape_map > PRISM_MAP_ENTROPY) return PRISM_EINVAL;
  if (!(c->alpha >= 0.0f) || !isfinite(c->alpha)) return PRISM_EINVAL;
  if (!(c->cut_threshold >= 0.0f) || !isfinite(c->cut_threshold)) return PRISM_EINVAL;
  return PRISM_OK;
}

prism_status prism_plan_workspace_size(const prism_config* c, int64_t nnz_capacity,
                                       size_t* bytes) {
  prism_status s = prism_config_check(c);
  if (s != PRISM_OK) return s;
  if (!bytes) return PRISM_EINVAL;
  if (nnz_capacity < 0) {
    int64_t mb = 8 * zones_of(*c);
    nnz_capacity = (int64_t)c->heads * mb * mb;
  }
  PlanDev P;
  *bytes = carve(*c, nnz_capacity, nullptr, &P, nullptr);
  return PRISM_OK;
}

prism_status prism_plan_create(const prism_config* c, const void* q, const void* k,
                               const void* v, const float* av_norm, void* workspace,
                               size_t workspace_bytes, void* stream, prism_plan_t** plan_out,
                               int64_t* nnz_out) {
  prism_status s = prism_config_check(c);
  if (s != PRISM_OK) return s;
  if (!q || !k || !v || !workspace || !plan_out) return PRISM_EINVAL;
  *plan_out = nullptr;
  hipStream_t st = (hipStream_t)stream;
  PlanDev P;
  size_t fixed = carve(*c, 0, nullptr, &P, nullptr);
  if (workspace_bytes < fixed) {
    if (nnz_out) *nnz_out = -1;
    return PRISM_ENOMEM_WORKSPACE;
  }
  int64_t cap = (int64_t)((workspace_bytes - fixed) / per_pair_bytes(*c));
  int32_t* perm = nullptr;
  carve(*c, cap, (char*)workspace, &P, &perm);
  const int fixed_id = fixed_id_of(*c);

  PRISM_HIP(hipGetLastError());
  stage_begin("plan.stats", st);
  bool ok = launch_zone_stats(v, c->dtype, c->head_dim, c->H, c->W, P.Z, c->heads, P.N,
                              P.vstats, st);
  if (av_norm)
    ok = ok && launch_audio_stats(av_norm, c->H, c->W, P.Z, P.astats, st);
  else
    PRISM_HIP(hipMemsetAsync(P.astats, 0, sizeof(float) * 4 * P.Z, st));
  if (c->cut_threshold > 0.0f) ok = ok && launch_cuts(P, v, c->cut_threshold, st);
  stage_end(st);
  stage_begin("plan.shapes", st);
  ok = ok && launch_shapes(P, av_norm != nullptr, *c, fixed_id, st);
  ok = ok && launch_blk_off(P, st);
  stage_end(st);
  if (!ok) return PRISM_EDEVICE;
  std::vector<int64_t> off(c->heads + 1);
  PRISM_HIP(hipMemcpyAsync(off.data(), P.blk_off, sizeof(int64_t) * (c->heads + 1),
                           hipMemcpyDeviceToHost, st));
  PRISM_HIP(hipStreamSynchronize(st));
  int64_t maxb = 0;
  for (int h = 0; h < c->heads; h++) maxb = std::max(maxb, off[h + 1] - off[h]);

  stage_begin("plan.pool", st);
  ok = launch_pool(P, q, k, st);
  stage_end(st);
  if (ok && P.relayout) {
    stage_begin("plan.relayout", st);
    ok = launch_relayout(P, k, v, nullptr, nullptr, P.kp, P.vp, nullptr, nullptr, st);
    stage_end(st);
  }
  PRISM_HIP(hipMemsetAsync(P.counters, 0, sizeof(int64_t) * 8, st));
  for (int h = 0; h < c->heads && ok; h++) {
    int n = (int)(off[h + 1] - off[h]);
    stage_begin("plan.scores", st);
    ok = launch_block_scores(P, off[h], n, P.scores, st);
    stage_end(st);
    stage_begin("plan.select", st);
    ok = ok && launch_select(P, off[h], n, *c, h == c->heads - 1, st);
    stage_end(st);
    // the key-major lists of the head, from its selection mask (writes past
    // the capacity are dropped; the plan then fails below)
    if (c->need_backward) {
      stage_begin("plan.transpose", st);
      ok = ok && launch_transpose(P, off[h], n, h == c->heads - 1, st);
      stage_end(st);
    }
  }
  if (!ok) return PRISM_EDEVICE;
  int64_t nnz = 0;
  PRISM_HIP(hipMemcpyAsync(&nnz, P.counters, sizeof(int64_t), hipMemcpyDeviceToHost, st));
  PRISM_HIP(hipStreamSynchronize(st));
  if (nnz_out) *nnz_out = nnz;
  if (nnz > cap) return PRISM_ENOMEM_WORKSPACE;
  if (c->need_backward) {
    stage_begin("plan.order", st);
    ok = launch_unit_order_k(P, st);
    stage_end(st);
    if (!ok) return PRISM_EDEVICE;
  }
  // the dK/dV kernel takes the ordered persistent launch when at least half
  // of all (query block, key block) pairs are selected
  double pairs_all = 0.0;
  for (int h = 0; h < c->heads; h++) pairs_all += (double)(off[h + 1] - off[h]) * (off[h + 1] - off[h]);
  P.kv_persist = c->need_backward && (double)nnz >= kPersistDensity * pairs_all;
  PRISM_HIP(hipGetLastError());
  prism_plan_s* pl = new prism_plan_s;
  pl->cfg = *c;
  pl->P = P;
  pl->blk_off = off;
  pl->nnz = nnz;
  pl->max_blocks = maxb;
  pl->k = k;
  pl->v = v;
  pl->perm = perm;
  *plan_out = pl;
  return PRISM_OK;
}

void prism_plan_destroy(prism_plan_t* plan) { delete plan; }

prism_status prism_attn_fwd(const prism_plan_t* plan, const void* q, const void* k,
                            const void* v, void* o, float* lse, void* stream) {
  if (!plan || !q || !k || !v || !o || !lse) return PRISM_EINVAL;
  if (k != plan->k || v != plan->v) return PRISM_ESTATE;
  const prism_config& c = plan->cfg;
  if (!((c.dtype == PRISM_BF16 && c.head_dim == 128) || c.dtype == PRISM_F32))
    return PRISM_EUNSUPPORTED;
  PRISM_HIP(hipGetLastError());
  stage_begin("attn.fwd", (hipStream_t)stream);
  bool ok = launch_attn_fwd(plan->P, q, k, v, o, lse, (hipStream_t)stream);
  stage_end((hipStream_t)stream);
  return ok ? PRISM_OK : PRISM_EDEVICE;
}

prism_status prism_attn_bwd_workspace_size(const prism_config* c, size_t* bytes) {
  prism_status s = prism_config_check(c);
  if (s != PRISM_OK) return s;
  if (!bytes) return PRISM_EINVAL;
  *bytes = bwd_workspace_bytes(*c, relaid_config(*c));
  return PRISM_OK;
}

}  // extern "C"

namespace {

// The backward with its scratch (Delta and log2(e) * LSE per token, and
// with `copies` and room for them the block-contiguous copies of Q and dO)
// carved from `workspace`.  `timed`: record the stage events of the
// measurement support (which may create HIP events).
prism_status bwd_run(const prism_plan_t* plan, const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* d_o, void* dq, void* dk,
                     void* dv, void* workspace, size_t workspace_bytes, hipStream_t st,
                     bool timed, bool copies) {
  if (!plan || !q || !k || !v || !o || !lse || !d_o || !dq || !dk || !dv || !workspace)
    return PRISM_EINVAL;
  if (k != plan->k || v != plan->v) return PRISM_ESTATE;
  const prism_config& c = plan->cfg;
  if (!c.need_backward) return PRISM_ESTATE;
  if (!(c.dtype == PRISM_BF16 && c.head_dim == 128)) return PRISM_EUNSUPPORTED;
  // the copies of Q and dO when the configuration asks for them and the
  // workspace holds them; else the query tiles are gathered
  const bool relaid =
      copies && relaid_config(c) && workspace_bytes >= bwd_workspace_bytes(c, true);
  if (workspace_bytes < bwd_workspace_bytes(c, relaid)) return PRISM_ENOMEM_WORKSPACE;
  BwdCarve W;
  bwd_carve(c, relaid, (char*)workspace, &W);
  BwdDev B;
  B.q = q;
  B.k = k;
  B.v = v;
  B.d_o = d_o;
  B.delta = W.delta;
  B.lse2 = W.lse2;
  B.qp = W.qp;
  B.dop = W.dop;
  B.delta_p = W.delta_p;
  B.lse2_p = W.lse2_p;
  PRISM_HIP(hipGetLastError());
  if (timed) stage_begin("bwd.prep", st);
  bool ok = launch_bwd_prep(plan->P, B, o, lse, st);
  if (timed) stage_end(st);
  if (timed) stage_begin("bwd.dkdv", st);
  ok = ok && launch_bwd_dkdv(plan->P, B, dk, dv, st);
  if (timed) stage_end(st);
  if (timed) stage_begin("bwd.dq", st);
  ok = ok && launch_bwd_dq(plan->P, B, dq, st);
  if (timed) stage_end(st);
  return ok ? PRISM_OK : PRISM_EDEVICE;
}

// Scratch of the allocation-free backward: one copy per GPU, held from the
// library's load until the process ends.  In host code `scratch` names a
// host-side stand-in; the device address of each GPU's copy comes from
// hipGetSymbolAddress with that GPU current, and only that address is used.
static __device__ __align__(256) char scratch[PRISM_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

prism_status scratch_address(void** out) {
  int dev = -1;
  PRISM_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return PRISM_EDEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PRISM_EDEVICE;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return PRISM_OK;
}

}  // namespace

extern "C" {

prism_status prism_attn_bwd(const prism_plan_t* plan, const void* q, const void* k,
                            const void* v, const void* o, const float* lse, const void* d_o,
                            void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return bwd_run(plan, q, k, v, o, lse, d_o, dq, dk, dv, workspace, workspace_bytes,
                 (hipStream_t)stream, true, true);
}

prism_status prism_attn_bwd_noalloc(const prism_plan_t* plan, const void* q, const void* k,
                                    const void* v, const void* o, const float* lse,
                                    const void* d_o, void* dq, void* dk, void* dv,
                                    void* stream) {
  if (!plan) return PRISM_EINVAL;
  prism_status s = prism_config_check(&plan->cfg);
  if (s != PRISM_OK) return s;
  // (no copies of Q and dO: the columns alone must fit the array)
  if (bwd_workspace_bytes(plan->cfg, false) > (size_t)PRISM_NOALLOC_SCRATCH_BYTES)
    return PRISM_ENOMEM_WORKSPACE;
  void* ws = nullptr;
  s = scratch_address(&ws);
  if (s != PRISM_OK) return s;
  return bwd_run(plan, q, k, v, o, lse, d_o, dq, dk, dv, ws, PRISM_NOALLOC_SCRATCH_BYTES,
                 (hipStream_t)stream, false, false);
}

prism_status prism_av_cross_attn(const void* q, const void* ka, const void* va, int32_t heads,
                                 int64_t n_video, int32_t n_audio, int32_t head_dim,
                                 int32_t dtype, void* o, float* norm_out, void* stream) {
  if (!q || !ka || !va || !norm_out || heads <= 0 || n_video <= 0 || n_audio <= 0)
    return PRISM_EINVAL;
  if (dtype != PRISM_BF16 || head_dim != 128) return PRISM_EUNSUPPORTED;
  // rows come in work-groups of 256 and audio keys in tiles of 64; one
  // head's rows are addressed with 32-bit byte offsets
  if (n_video % 256 || n_audio % 64) return PRISM_EINVAL;
  if (n_video >= ((int64_t)1 << 24) || n_audio >= (1 << 24)) return PRISM_EUNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  PRISM_HIP(hipGetLastError());
  stage_begin("av.cross", st);
  const bool ok = launch_av_cross(q, ka, va, heads, n_video, n_audio, o, norm_out, st);
  stage_end(st);
  return ok ? PRISM_OK : PRISM_EDEVICE;
}

prism_status prism_block_scores(const prism_plan_t* plan, int32_t head, float* out,
                                void* stream) {
  if (!plan || !out || head < 0 || head >= plan->cfg.heads) return PRISM_EINVAL;
  int n = (int)(plan->blk_off[head + 1] - plan->blk_off[head]);
  PRISM_HIP(hipGetLastError());
  if (!launch_block_scores(plan->P, plan->blk_off[head], n, out, (hipStream_t)stream))
    return PRISM_EDEVICE;
  return PRISM_OK;
}

static const void* array_ptr(const prism_plan_t* pl, int which, size_t* bytes) {
  const PlanDev& P = pl->P;
  const prism_config& c = pl->cfg;
  const int64_t G = pl->blk_off[c.heads];
  const int64_t Z = P.Z;
  switch (which) {
    case PRISM_ARR_ZONE_STATS: *bytes = sizeof(float) * c.heads * Z * 5; return P.vstats;
    case PRISM_ARR_AUDIO_STATS: *bytes = sizeof(float) * Z * 4; return P.astats;
    case PRISM_ARR_SHAPE_ID: *bytes = (size_t)c.heads * Z; return P.shape_id;
    case PRISM_ARR_BLK_OFF: *bytes = sizeof(int64_t) * (c.heads + 1); return P.blk_off;
    case PRISM_ARR_BLK_START: *bytes = sizeof(int32_t) * G; return P.blk_start;
    case PRISM_ARR_QBAR: *bytes = sizeof(float) * G * c.head_dim; return P.qbar;
    case PRISM_ARR_KBAR: *bytes = sizeof(float) * G * c.head_dim; return P.kbar;
    case PRISM_ARR_QEXP: *bytes = sizeof(int32_t) * G; return P.qexp;
    case PRISM_ARR_KEXP: *bytes = sizeof(int32_t) * G; return P.kexp;
    case PRISM_ARR_ROW_PTR: *bytes = sizeof(int64_t) * (G + 1); return P.row_ptr;
    case PRISM_ARR_COL_IDX: *bytes = sizeof(int32_t) * pl->nnz; return P.col_idx;
    case PRISM_ARR_COLT_PTR:
      *bytes = c.need_backward ? sizeof(int64_t) * (G + 1) : 0;
      return P.colt_ptr;
    case PRISM_ARR_COLT_IDX:
      *bytes = c.need_backward ? sizeof(int32_t) * pl->nnz : 0;
      return P.colt_idx;
    case PRISM_ARR_PERM: *bytes = sizeof(int32_t) * c.heads * P.N; return pl->perm;
    case PRISM_ARR_QGRID: *bytes = sizeof(uint16_t) * G * c.head_dim; return P.qgrid;
    case PRISM_ARR_KGRID: *bytes = sizeof(uint16_t) * G * c.head_dim; return P.kgrid;
    case PRISM_ARR_KV_ORDER:
      *bytes = c.need_backward ? sizeof(int32_t) * c.heads * (P.N / 128) : 0;
      return P.korder;
    case PRISM_ARR_BLK_ORG: *bytes = sizeof(int32_t) * G; return P.blk_org;
    case PRISM_ARR_CUTS: *bytes = c.cut_threshold > 0.0f ? (size_t)c.T : 0; return P.cuts;
    case PRISM_ARR_QLO: *bytes = sizeof(uint16_t) * G * c.head_dim; return P.qlo;
    case PRISM_ARR_KLO: *bytes = sizeof(uint16_t) * G * c.head_dim; return P.klo;
    default: *bytes = 0; return nullptr;
  }
}

prism_status prism_plan_array_bytes(const prism_plan_t* plan, int32_t which, size_t* bytes) {
  if (!plan || !bytes) return PRISM_EINVAL;
  const void* p = array_ptr(plan, which, bytes);
  if (!p && *bytes) return PRISM_EINVAL;
  if (which < 0 || which > PRISM_ARR_KLO) return PRISM_EINVAL;
  return PRISM_OK;
}

prism_status prism_plan_export(const prism_plan_t* plan, int32_t which, void* dst,
                               size_t dst_bytes, void* stream) {
  if (!plan || !dst || which < 0 || which > PRISM_ARR_KLO) return PRISM_EINVAL;
  size_t bytes = 0;
  const void* p = array_ptr(plan, which, &bytes);
  if (dst_bytes < bytes) return PRISM_EINVAL;
  if (bytes == 0) return PRISM_OK;
  hipStream_t st = (hipStream_t)stream;
  PRISM_HIP(hipGetLastError());
  if (which == PRISM_ARR_PERM && !launch_perm_map(plan->P, plan->perm, st)) return PRISM_EDEVICE;
  PRISM_HIP(hipMemcpyAsync(dst, p, bytes, hipMemcpyDeviceToHost, st));
  PRISM_HIP(hipStreamSynchronize(st));
  return PRISM_OK;
}

prism_status prism_plan_info(const prism_plan_t* plan, prism_plan_info_t* info, void* stream) {
  if (!plan || !info) return PRISM_EINVAL;
  const prism_config& c = plan->cfg;
  const int64_t G = plan->blk_off[c.heads];
  hipStream_t st = (hipStream_t)stream;
  memset(info, 0, sizeof(*info));
  info->total_blocks = G;
  info->nnz = plan->nnz;
  info->max_blocks_per_head = plan->max_blocks;
  info->kv_persistent = plan->P.kv_persist;
  PRISM_HIP(hipGetLastError());
  if (!launch_sum_i64(plan->P.row_cost, G, plan->P.counters + 4, st)) return PRISM_EDEVICE;
  int64_t pt = 0;
  PRISM_HIP(hipMemcpyAsync(&pt, plan->P.counters + 4, sizeof(int64_t), hipMemcpyDeviceToHost,
                           st));
  std::vector<uint8_t> sid((size_t)c.heads * plan->P.Z);
  PRISM_HIP(hipMemcpyAsync(sid.data(), plan->P.shape_id, sid.size(), hipMemcpyDeviceToHost, st));
  PRISM_HIP(hipStreamSynchronize(st));
  info->pair_tokens = (double)pt;
  for (uint8_t s : sid) info->shape_hist[s < 16 ? s : 0]++;
  return PRISM_OK;
}

prism_status prism_schedule_value(int32_t kind, int64_t step, int64_t steps, float v0, float v1,
                                  float* out) {
  if (!out || steps < 1 || !isfinite(v0) || !isfinite(v1)) return PRISM_EINVAL;
  double s = steps > 1 ? (double)step / (double)(steps - 1) : 0.0;
  s = s < 0.0 ? 0.0 : s > 1.0 ? 1.0 : s;
  const double a = v0, b = v1;
  double v;
  switch (kind) {
    case PRISM_SCHED_CONSTANT: v = a; break;
    case PRISM_SCHED_LINEAR: v = a + (b - a) * s; break;
    case PRISM_SCHED_COSINE: v = b + (a - b) * (1.0 + cos(M_PI * s)) * 0.5; break;
    default: return PRISM_EINVAL;
  }
  *out = (float)v;
  return PRISM_OK;
}

prism_status prism_candidate(int32_t id, int32_t* out4) {
  if (id < 0 || id >= kNumShapes || !out4) return PRISM_EINVAL;
  out4[0] = h_shapes[id].bt;
  out4[1] = h_shapes[id].bh;
  out4[2] = h_shapes[id].bw;
  out4[3] = h_shapes[id].volume;
  return PRISM_OK;
}

prism_status prism_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(prism::g_tmu);
  prism::g_timing = enable != 0;
  return PRISM_OK;
}

prism_status prism_timing_read(prism_stage_time* out, int32_t max, int32_t* count) {
  if (!count || max < 0 || (max > 0 && !out)) return PRISM_EINVAL;
  std::lock_guard<std::mutex> lk(prism::g_tmu);
  std::vector<prism_stage_time> agg;
  prism_status status = PRISM_OK;
  for (auto& r : prism::g_recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      status = PRISM_EDEVICE;
    size_t i = 0;
    for (; i < agg.size(); i++)
      if (r.name == agg[i].name) break;
    if (i == agg.size()) {
      prism_stage_time t;
      memset(&t, 0, sizeof(t));
      strncpy(t.name, r.name.c_str(), sizeof(t.name) - 1);
      agg.push_back(t);
    }
    agg[i].launches++;
    agg[i].total_ms += ms;
    prism::g_pool.push_back(r.a);
    prism::g_pool.push_back(r.b);
  }
  prism::g_recs.clear();
  *count = (int32_t)agg.size();
  for (int32_t i = 0; i < (int32_t)agg.size() && i < max; i++) out[i] = agg[i];
  return status;
}

const char* prism_status_str(prism_status s) {
  switch (s) {
    case PRISM_OK: return "ok";
    case PRISM_EINVAL: return "invalid argument";
    case PRISM_EUNSUPPORTED: return "unsupported configuration";
    case PRISM_ENOMEM_WORKSPACE: return "workspace too small";
    case PRISM_EDEVICE: return "HIP runtime error";
    case PRISM_ESTATE: return "arguments do not match the plan";
    default: return "unknown status";
  }
}

}  // extern "C"
