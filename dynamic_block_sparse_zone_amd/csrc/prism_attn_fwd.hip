// Sparse attention forward over the selected, variable-shape blocks
// (paper.rainbus.top "方法步骤详情", stages four and five): each query tile
// iterates only over the key blocks of its S_i with an online softmax
// (running maximum and running sum), and its output rows are written straight
// back to their original token positions.
//
// gfx950 design (bf16, head_dim 128):
//  * a work-group of 4 waves owns 128 consecutive permuted query rows (one
//    block of 128, half a block of 256, or two blocks of 64 whose key lists
//    are walked as one merged list, each half computing only its own blocks);
//  * every wave owns 32 query rows and computes S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16 (K from LDS, Q in registers), so that each lane
//    holds one query row's scores and the softmax needs one cross-lane step;
//  * O^T += V^T P^T reuses the score registers as the B operand directly; the
//    V^T fragments come from the row-major V tile by ds_read_b64_tr_b16;
//  * K/V tiles of 64 keys are double-buffered in LDS; the next tile's global
//    loads are in flight while the current one is computed;
//  * the softmax maximum is only moved when it grows by more than 2^8, so the
//    accumulator rescale is rare.
#include "prism_common.h"
#include "prism_kernels.h"

namespace prism {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Merged walk over the ascending key-block lists of the query blocks of one
// work unit (1, 2 or 4 lists): yields each key block once, with a bit mask of
// the lists that hold it.
struct UnionIter {
  const int32_t* col;
  int64_t a[4], e[4];
  int head[4];
  int n;
  __device__ void init(const int32_t* c, int nl) {
    col = c;
    n = nl;
#pragma unroll
    for (int i = 0; i < 4; i++) head[i] = (i < n && a[i] < e[i]) ? col[a[i]] : 0x7fffffff;
  }
  __device__ bool next(int& j, int& mask) {
    int best = head[0];
#pragma unroll
    for (int i = 1; i < 4; i++) best = head[i] < best ? head[i] : best;
    if (best == 0x7fffffff) return false;
    mask = 0;
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (head[i] == best) {
        mask |= 1 << i;
        a[i]++;
        head[i] = a[i] < e[i] ? col[a[i]] : 0x7fffffff;
      }
    j = best;
    return true;
  }
};

struct TileDesc {
  int64_t row;  // first permuted row of the 64-key tile
  int mask;     // lists (query blocks of the unit) that selected it
};

// 64-key tiles of the merged walk
struct TileIter {
  UnionIter U;
  const int32_t* blk_start;
  const uint8_t* blk_shape;
  int64_t hoff;
  int64_t row;
  int t, nt, mask;
  bool valid;
  __device__ void start() {
    valid = true;
    t = 0;
    nt = 0;
    advance();
  }
  __device__ void advance() {
    if (valid && t + 1 < nt) {
      t++;
      row += 64;
      return;
    }
    int j;
    valid = U.next(j, mask);
    if (valid) {
      row = blk_start[hoff + j];
      nt = d_shapes[block_shape_at(blk_shape, hoff + j)].volume >> 6;
      t = 0;
    }
  }
  __device__ TileDesc take() {
    TileDesc d{row, mask};
    advance();
    return d;
  }
};

__device__ inline bf16x8 lds_row_chunk(const uint16_t* tile, int row, int chunk) {
  const uint4* p = (const uint4*)(tile + row * 128 + ((chunk ^ chunk_swizzle(row)) << 3));
  return __builtin_bit_cast(bf16x8, *p);
}

// A-operand fragment of X^T (rows = channel d, k = 16 keys of chunk c) from
// a row-major, swizzled 64 x 128 tile X, keys in the order
// {16c+4hl+0..3, 16c+8+4hl+0..3} for lane half hl.
__device__ inline bf16x8 lds_trans_frag(const uint16_t* tile, int c, int db, int lane) {
  const int hl = lane >> 5;
  const int rowA = 16 * c + 4 * hl + ((lane & 15) >> 2);
  const int rowB = rowA + 8;
  const int chunk = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int off = 4 * (lane & 1);
  const uint16_t* pa = tile + rowA * 128 + ((chunk ^ chunk_swizzle(rowA)) << 3) + off;
  const uint16_t* pb = tile + rowB * 128 + ((chunk ^ chunk_swizzle(rowB)) << 3) + off;
  s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pa);
  s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pb);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  // one v_cvt_pk_bf16_f32 (round to nearest even)
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Query rows per work-group and pipeline depth of the K/V tile ring.
constexpr int kFwdRows = 256;
constexpr int kFwdWaves = kFwdRows / 32;
constexpr int kRing = 4;
// s_waitcnt immediates (vmcnt in bits 3:0, expcnt and lgkmcnt left at their
// maxima) for 8, 4 and 0 outstanding vector-memory operations: one K/V tile
// pair is four operations per wave
constexpr int kWaitVm8 = 0x0F78, kWaitVm4 = 0x0F74, kWaitVm0 = 0x0F70;

__global__ __launch_bounds__(kFwdWaves * 64, 1) void k_attn_fwd_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vp, const uint8_t* __restrict__ shape_id,
    const int32_t* __restrict__ zone_base, const int64_t* __restrict__ blk_off,
    const int32_t* __restrict__ blk_start, const uint8_t* __restrict__ blk_shape,
    const int64_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int H, int W,
    int Z, int64_t N, float c_log2, uint16_t* __restrict__ o, float* __restrict__ lse) {
  // ring of kRing K/V tile pairs: three tiles in flight while one is used.
  // One variable per slot, addressed with compile-time slot numbers, so the
  // compiler can tell an in-flight tile load from the slot being read.
  __shared__ __attribute__((aligned(16))) uint16_t sK0[64 * 128], sK1[64 * 128], sK2[64 * 128],
      sK3[64 * 128];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[64 * 128], sV1[64 * 128], sV2[64 * 128],
      sV3[64 * 128];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int64_t upH = N / kFwdRows;
  const int64_t unit = xcd_unit(blockIdx.x, gridDim.x);
  const int h = (int)(unit / upH);
  const int64_t r0 = (unit - (int64_t)h * upH) * kFwdRows;
  const int m = (int)(r0 >> 9);
  const int sid = shape_id[(int64_t)h * Z + m];
  const Shape sh = d_shapes[sid];
  const int B = sh.volume;
  const int rz = (int)(r0 & 511);
  const int64_t hoff = blk_off[h];
  const int64_t gfirst = hoff + zone_base[(int64_t)h * Z + m] + rz / B;
  const int nlists = B >= kFwdRows ? 1 : kFwdRows / B;  // query blocks in the unit
  const int slot = __builtin_amdgcn_readfirstlane((32 * wv) / B < nlists ? (32 * wv) / B : 0);

  TileIter it;
  for (int i = 0; i < 4; i++) {
    const int64_t g = gfirst + (i < nlists ? i : 0);
    it.U.a[i] = row_ptr[g];
    it.U.e[i] = row_ptr[g + 1];
  }
  it.U.init(col_idx, nlists);
  it.blk_start = blk_start;
  it.blk_shape = blk_shape;
  it.hoff = hoff;
  it.start();

  // query fragments: row p of this wave, 8 chunks of 16 channels
  const int64_t p = r0 + wv * 32 + l32;
  const int64_t tok = token_of(sh, m, (int)(p & 511), H, W);
  const uint16_t* qrow = q + ((int64_t)h * N + tok) * 128;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; kk++)
    qf[kk] = __builtin_bit_cast(bf16x8, *(const uint4*)(qrow + kk * 16 + hl * 8));
  // the query fragments land before any tile load is issued, so waits in the
  // ring only ever concern tiles
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[db][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  const uint4* kbase = (const uint4*)(kp + (int64_t)h * N * 128);
  const uint4* vbase = (const uint4*)(vp + (int64_t)h * N * 128);
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  // one 64-row K tile and V tile (16 KB each, already in LDS layout) straight
  // into a ring slot: wave w moves the 1 KB pieces w and w + 8 of each
  // The slot address goes through an opaque LDS offset: the loads then carry
  // no object identity, and the compiler adds no conservative wait of its own
  // before the reads of other slots (the ring's explicit waits order them).
  auto stage = [&](uint16_t* dK, uint16_t* dV, int64_t row) {
    const uint4* ks = kbase + row * 16;
    const uint4* vs = vbase + row * 16;
    const uint32_t oK = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)dK);
    const uint32_t oV = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)dV);
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const uint32_t piece = i * 512 + wvu * 64;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(ks + piece + lane),
          (__attribute__((address_space(3))) void*)(uintptr_t)(oK + piece * 16), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(vs + piece + lane),
          (__attribute__((address_space(3))) void*)(uintptr_t)(oV + piece * 16), 16, 0, 0);
    }
  };
  auto compute = [&](const uint16_t* Ks, const uint16_t* Vs) {
    f32x16 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int r = 0; r < 16; r++) st[kb][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; kk++)
#pragma unroll
      for (int kb = 0; kb < 2; kb++) {
        bf16x8 a = lds_row_chunk(Ks, 32 * kb + l32, 2 * kk + hl);
        st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], st[kb], 0, 0, 0);
      }
    float mx = st[0][0];
#pragma unroll
    for (int r = 1; r < 16; r++) mx = fmaxf(mx, st[0][r]);
#pragma unroll
    for (int r = 0; r < 16; r++) mx = fmaxf(mx, st[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mt = mx * c_log2;
    const bool need = mt > m_run + 8.0f;
    if (__any(need)) {
      const float mnew = need ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[db][r] *= alpha;
      m_run = mnew;
    }
    const float negm = -m_run;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int r = 8 * (c & 1) + 2 * e;
        float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[c >> 1][r], c_log2, negm));
        float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[c >> 1][r + 1], c_log2, negm));
        l_run += p0 + p1;
        pk[e] = pack_bf16x2(p0, p1);
      }
      bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
#pragma unroll
      for (int db = 0; db < 4; db++) {
        bf16x8 va = lds_trans_frag(Vs, c, db, lane);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, acc[db], 0, 0, 0);
      }
    }
  };

  // Every step issues exactly one tile pair (four loads per wave): past the
  // end of the lists it re-reads the last real tile into a slot that is never
  // computed on.  With a fixed count of loads per step, "at most eight loads
  // outstanding" provably means the slot about to be read has landed, and the
  // compiler needs no wait of its own between the ring and the reads.
  uint32_t ring_mask = 0;  // query-block masks of the tiles in the ring, a byte per slot
  int nreal = 0;           // real tiles issued
  int64_t last_row = 0;
  auto issue = [&](int b, uint16_t* dK, uint16_t* dV) {
    int64_t row = last_row;
    uint32_t mask = 0;
    if (it.valid) {
      const TileDesc d = it.take();
      row = d.row;
      mask = (uint32_t)d.mask;
      last_row = row;
      nreal++;
    }
    ring_mask = (ring_mask & ~(0xffu << (8 * b))) | (mask << (8 * b));
    stage(dK, dV, row);
  };
  issue(0, sK0, sV0);
  issue(1, sK1, sV1);
  issue(2, sK2, sV2);
  // step for tile j in slot S: its loads and every older one are done once at
  // most the eight of tiles j+1 and j+2 are pending; the barrier then also
  // says every wave has finished with tile j-1, whose slot is refilled
#define PRISM_FWD_STEP(S, KS, VS, KN, VN)                        \
  if (j + (S) >= nreal) break;                                   \
  __builtin_amdgcn_s_waitcnt(kWaitVm8);                          \
  __builtin_amdgcn_s_barrier();                                  \
  asm volatile("" ::: "memory"); /* no LDS access moves above */ \
  {                                                              \
    const uint32_t tile_mask = (ring_mask >> (8 * (S))) & 0xffu; \
    issue(((S) + 3) & 3, KN, VN);                                \
    if ((tile_mask >> slot) & 1u) compute(KS, VS);               \
  }
  for (int j = 0;; j += 4) {
    PRISM_FWD_STEP(0, sK0, sV0, sK3, sV3)
    PRISM_FWD_STEP(1, sK1, sV1, sK0, sV0)
    PRISM_FWD_STEP(2, sK2, sV2, sK1, sV1)
    PRISM_FWD_STEP(3, sK3, sV3, sK2, sV2)
  }
#undef PRISM_FWD_STEP
  // no tile load may still be writing LDS when the work-group ends
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  uint16_t* orow = o + ((int64_t)h * N + tok) * 128;
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      uint2 u;
      u.x = pack_bf16x2(acc[db][4 * jj + 0] * inv, acc[db][4 * jj + 1] * inv);
      u.y = pack_bf16x2(acc[db][4 * jj + 2] * inv, acc[db][4 * jj + 3] * inv);
      *(uint2*)(orow + 32 * db + 8 * jj + 4 * hl) = u;
    }
  if (hl == 0)
    lse[(int64_t)h * N + tok] =
        l_tot > 0.0f ? m_run * 0.69314718055994530942f + logf(l_tot) : -INFINITY;
}

// ---------------------------------------------------------------- fp32 path
// Plain fp32 kernel (small problems, fp32 inputs): one thread per query row,
// K/V tiles of 64 rows staged in LDS, exact expf online softmax.
template <int D>
__global__ __launch_bounds__(64) void k_attn_fwd_f32(
    const float* __restrict__ q, const float* __restrict__ kp, const float* __restrict__ vp,
    const uint8_t* __restrict__ shape_id, const int32_t* __restrict__ zone_base,
    const int64_t* __restrict__ blk_off, const int32_t* __restrict__ blk_start,
    const uint8_t* __restrict__ blk_shape, const int64_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int H, int W, int Z, int64_t N, float scale,
    float* __restrict__ o, float* __restrict__ lse) {
  __shared__ float Ks[64][D], Vs[64][D];
  const int64_t tpH = N >> 6;
  const int h = (int)(blockIdx.x / tpH);
  const int64_t r0 = (blockIdx.x - (int64_t)h * tpH) << 6;
  const int m = (int)(r0 >> 9);
  const Shape sh = d_shapes[shape_id[(int64_t)h * Z + m]];
  const int64_t hoff = blk_off[h];
  const int64_t g = hoff + zone_base[(int64_t)h * Z + m] + (int)(r0 & 511) / sh.volume;
  const int64_t p = r0 + threadIdx.x;
  const int64_t tok = token_of(sh, m, (int)(p & 511), H, W);
  float qv[D], ov[D];
  for (int c = 0; c < D; c++) {
    qv[c] = q[((int64_t)h * N + tok) * D + c];
    ov[c] = 0.0f;
  }
  float mrun = -INFINITY, lrun = 0.0f;
  for (int64_t e = row_ptr[g]; e < row_ptr[g + 1]; e++) {
    int j = col_idx[e];
    int64_t start = blk_start[hoff + j];
    int nt = d_shapes[block_shape_at(blk_shape, hoff + j)].volume >> 6;
    for (int t = 0; t < nt; t++) {
      __syncthreads();
      for (int i = threadIdx.x; i < 64 * D; i += 64) {
        Ks[i / D][i % D] = kp[((int64_t)h * N + start + 64 * t) * D + i];
        Vs[i / D][i % D] = vp[((int64_t)h * N + start + 64 * t) * D + i];
      }
      __syncthreads();
      for (int r = 0; r < 64; r++) {
        float s = 0.0f;
        for (int c = 0; c < D; c++) s = __builtin_fmaf(qv[c], Ks[r][c], s);
        s *= scale;
        if (s > mrun) {
          float a = expf(mrun - s);
          lrun *= a;
          for (int c = 0; c < D; c++) ov[c] *= a;
          mrun = s;
        }
        float pr = expf(s - mrun);
        lrun += pr;
        for (int c = 0; c < D; c++) ov[c] = __builtin_fmaf(pr, Vs[r][c], ov[c]);
      }
    }
  }
  float inv = lrun > 0.0f ? 1.0f / lrun : 0.0f;
  for (int c = 0; c < D; c++) o[((int64_t)h * N + tok) * D + c] = ov[c] * inv;
  lse[(int64_t)h * N + tok] = lrun > 0.0f ? mrun + logf(lrun) : -INFINITY;
}

bool launch_attn_fwd(const PlanDev& P, const void* q, void* o, float* lse, hipStream_t st) {
  if (P.dtype == PRISM_BF16 && P.D == 128) {
    dim3 grid((unsigned)(P.heads * (P.N / kFwdRows))), block(kFwdWaves * 64);
    float c_log2 = (float)(1.4426950408889634 / sqrt(128.0));
    hipLaunchKernelGGL(k_attn_fwd_bf16, grid, block, 0, st, (const uint16_t*)q,
                       (const uint16_t*)P.kp, (const uint16_t*)P.vp, P.shape_id, P.zone_base,
                       P.blk_off, P.blk_start, P.blk_shape, P.row_ptr, P.col_idx, P.H, P.W, P.Z,
                       P.N, c_log2, (uint16_t*)o, lse);
  } else if (P.dtype == PRISM_F32 && (P.D == 64 || P.D == 128)) {
    dim3 grid((unsigned)(P.heads * (P.N >> 6))), block(64);
    float scale = (float)(1.0 / sqrt((double)P.D));
    if (P.D == 64)
      hipLaunchKernelGGL((k_attn_fwd_f32<64>), grid, block, 0, st, (const float*)q,
                         (const float*)P.kp, (const float*)P.vp, P.shape_id, P.zone_base,
                         P.blk_off, P.blk_start, P.blk_shape, P.row_ptr, P.col_idx, P.H, P.W,
                         P.Z, P.N, scale, (float*)o, lse);
    else
      hipLaunchKernelGGL((k_attn_fwd_f32<128>), grid, block, 0, st, (const float*)q,
                         (const float*)P.kp, (const float*)P.vp, P.shape_id, P.zone_base,
                         P.blk_off, P.blk_start, P.blk_shape, P.row_ptr, P.col_idx, P.H, P.W,
                         P.Z, P.N, scale, (float*)o, lse);
  } else {
    return false;
  }
  return hipGetLastError() == hipSuccess;
}

}  // namespace prism
