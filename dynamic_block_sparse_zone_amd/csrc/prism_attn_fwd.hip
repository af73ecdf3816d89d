// Sparse attention forward over the selected, variable-shape blocks
// (paper.rainbus.top "方法步骤详情", stages four and five): each query tile
// iterates only over the key blocks of its S_i with an online softmax
// (running maximum and running sum), and its output rows are written straight
// back to their original token positions.
//
// gfx950 design (bf16, head_dim 128):
//  * a work-group of 8 waves owns 256 consecutive permuted query rows (one
//    block of 256, two of 128 or four of 64, whose key lists are walked as
//    one merged list, each wave computing only the blocks of its own list);
//  * every wave owns 32 query rows and computes S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16 (K from LDS, Q in registers), so that each lane
//    holds one query row's scores and the softmax needs one cross-lane step;
//  * O^T += V^T P^T takes the bf16 probabilities as the B operand directly;
//    the V^T fragments come from the row-major V tile by ds_read_b64_tr_b16;
//  * K/V tiles of 64 keys come from the plan's re-laid copies (or are
//    gathered from the caller's K and V through the block -> token map) and
//    stream through a 4-slot LDS ring: the barrier of
//    step j publishes tile j + 1 and frees the slot of tile j - 1 for tile
//    j + 3, so while tile j is computed the next one is already readable;
//  * the fragment reads that open each matrix stretch are issued one stretch
//    early (the first K fragments of tile j + 1 during the P V of tile j,
//    the first V fragments during the softmax), so the two waves of a SIMD,
//    which run in step, do not both wait for LDS at the start of a stretch;
//  * the row maximum crosses the two 32-lane halves with v_permlane32_swap
//    (an LDS-free exchange: a ds_bpermute would make every later LDS wait of
//    the tile a full drain of the prefetched reads);
//  * the softmax maximum is only moved when it grows by more than 2^8, so the
//    accumulator rescale is rare.
#include "prism_attn_common.h"
#include "prism_kernels.h"

namespace prism {

constexpr int kFwdRows = 256;             // query rows per work-group
constexpr int kFwdWaves = kFwdRows / 32;  // one wave per 32 rows
// loads per wave per K/V tile pair: 2 x 16 KB over 8 waves in 1 KB pieces
constexpr int kFwdLoads = 2 * kTile / (kFwdWaves * 1024);

// kRelaid: k and v are the plan's block-contiguous copies and blk_base holds
// each block's first permuted row; else k and v are the caller's tensors and
// blk_base each block's first token
template <bool kRelaid>
__global__ __launch_bounds__(kFwdWaves * 64, 1) void k_attn_fwd_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint8_t* __restrict__ shape_id,
    const int32_t* __restrict__ zone_base, const int64_t* __restrict__ blk_off,
    const int32_t* __restrict__ blk_base, const uint8_t* __restrict__ blk_shape,
    const int64_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int H, int W,
    int Z, int64_t N, float c_log2, uint16_t* __restrict__ o, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) char ringK[kRing * kTile];
  __shared__ __attribute__((aligned(16))) char ringV[kRing * kTile];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int64_t upH = N / kFwdRows;
  const int64_t unit = xcd_unit(blockIdx.x, gridDim.x);
  const int h = (int)(unit / upH);
  const int64_t r0 = (unit - (int64_t)h * upH) * kFwdRows;
  const int m = (int)(r0 >> 9);
  const Shape sh = d_shapes[shape_id[(int64_t)h * Z + m]];
  const int B = sh.volume;
  const int rz = (int)(r0 & 511);
  const int64_t hoff = blk_off[h];
  const int nlists = B >= kFwdRows ? 1 : kFwdRows / B;  // query blocks in the unit
  const int mylist = (32 * wvu) / B < nlists ? (32 * wvu) / B : 0;

  TileIter it;
  it.init(row_ptr, col_idx, hoff + zone_base[(int64_t)h * Z + m] + rz / B, nlists, blk_base,
          blk_shape, hoff);

  // query fragments: row p of this wave, 8 chunks of 16 channels
  const int64_t p = r0 + wv * 32 + l32;
  const int64_t tok = token_of(sh, m, (int)(p & 511), H, W);
  const uint16_t* qrow = q + ((int64_t)h * N + tok) * 128;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; kk++)
    qf[kk] = __builtin_bit_cast(bf16x8, *(const uint4*)(qrow + kk * 16 + hl * 8));
  // the fragments land before any tile load is issued (the empty asm
  // consumes them), so the ring's waits only ever concern tiles
#pragma unroll
  for (int kk = 0; kk < 8; kk++) asm volatile("" : "+v"(qf[kk]));
  uint32_t ro[8], to[4][2];
  row_offsets(lane, ro);
  tr_offsets(lane, to);

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[db][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // this head's K and V (N rows of 256 B) as buffers
  const __amdgpu_buffer_rsrc_t rsK = buffer_of(k + (int64_t)h * N * 128, (uint32_t)(N * 256));
  const __amdgpu_buffer_rsrc_t rsV = buffer_of(v + (int64_t)h * N * 128, (uint32_t)(N * 256));
  const uint32_t lK = lds_offset(ringK), lV = lds_offset(ringV);
  // tile t of the block (base org, shape sid) from K and from V into slot
  // b: wave w fills the 1 KB pieces w, w + 8 of each (the same chunks of the
  // same rows of both)
  auto stage = [&](int b, uint32_t org, int sid, int t) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const uint32_t piece = i * 512 + wvu * 64;
      const uint32_t src = tile_src<kRelaid>(org, sid, t, piece + lane, H, W);
      dma16(rsK, src, lK + b * kTile + piece * 16);
      dma16(rsV, src, lV + b * kTile + piece * 16);
    }
  };
  uint32_t ring_mask = 0;  // list masks of the tiles in the ring, a byte per slot
  int nreal = 0;           // real tiles issued
  uint32_t last_org = 0;   // the last real tile (re-read past the end)
  int last_sid = 0, last_t = 0;
  auto issue = [&](int b) {
    uint32_t mask = 0;
    if (it.valid) {
      last_org = it.org();
      last_sid = it.sid();
      last_t = it.t;
      mask = (uint32_t)it.mask;
      nreal++;
      it.advance();
    }
    ring_mask = (ring_mask & ~(0xffu << (8 * b))) | (mask << (8 * b));
    stage(b, last_org, last_sid, last_t);
  };
  // step j: tiles j and j + 1 have landed (each wave waits for its own
  // pieces, the barrier for everybody's), every wave is done with tile
  // j - 1, and its slot takes tile j + 3
  auto ring_step = [&](int j) {
    __builtin_amdgcn_s_waitcnt(wait_vm(kFwdLoads));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue((j + kRing - 1) & (kRing - 1));
  };
  auto listed = [&](int j) {
    return ((ring_mask >> (8 * (j & (kRing - 1)) + mylist)) & 1u) != 0;
  };
  // fragment i (0..15) of S^T = K Q^T: channels 16 (i / 2).., keys 32 (i % 2)..
  auto kfrag = [&](const char* sk, int i) { return ld_frag(sk + (i & 1) * 8192 + ro[i >> 1]); };
  // fragment t (0..15) of O^T += V^T P^T: keys 16 (t / 4).., channels 32 (t % 4)..
  auto vfrag = [&](const char* sv, int t) {
    return ld_tfrag(sv + (t >> 2) * 4096 + to[t & 3][0], sv + (t >> 2) * 4096 + to[t & 3][1]);
  };
  constexpr int kPre = 4;  // fragments read one stretch early
  bf16x8 kpre[kPre];
  int kpre_tile = -1;  // the tile whose first K fragments kpre holds
  // one tile: S^T = K Q^T, online softmax, O^T += V^T P^T
  auto compute = [&](int j) {
    const char* sk = ringK + (j & (kRing - 1)) * kTile;
    const char* sv = ringV + (j & (kRing - 1)) * kTile;
    if (kpre_tile != j) {
#pragma unroll
      for (int i = 0; i < kPre; i++) kpre[i] = kfrag(sk, i);
    }
    f32x16 st[2];
#pragma unroll
    for (int i = 0; i < 16; i++)
      st[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(i < kPre ? kpre[i] : kfrag(sk, i),
                                                          qf[i >> 1], i < 2 ? f32x16{} : st[i & 1],
                                                          0, 0, 0);
    // the first V fragments of P V are read while the softmax runs
    bf16x8 vpre[kPre];
#pragma unroll
    for (int t = 0; t < kPre; t++) vpre[t] = vfrag(sv, t);
    // (the fences keep such early reads where they are written)
    __builtin_amdgcn_sched_barrier(0);
    float mx = st[0][0];
#pragma unroll
    for (int r = 1; r < 16; r++) mx = fmaxf(mx, st[0][r]);
#pragma unroll
    for (int r = 0; r < 16; r++) mx = fmaxf(mx, st[1][r]);
    {
      const uint32_t mb = __builtin_bit_cast(uint32_t, mx);
      const auto sw = __builtin_amdgcn_permlane32_swap(mb, mb, false, false);
      mx = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]),
                 __builtin_bit_cast(float, (uint32_t)sw[1]));
    }
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
    bf16x8 pb[4];
#pragma unroll
    for (int c = 0; c < 4; c++) {
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int r = 8 * (c & 1) + 2 * e;
        float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[c >> 1][r], c_log2, negm));
        float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[c >> 1][r + 1], c_log2, negm));
        pk[e] = pk2(p0, p1);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e]), kOnes2,
                                                l_run, false);
      }
      pb[c] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
    // the first K fragments of the next tile (published by this step's
    // barrier) are read while P V runs
    const char* skn = ringK + ((j + 1) & (kRing - 1)) * kTile;
#pragma unroll
    for (int i = 0; i < kPre; i++) kpre[i] = kfrag(skn, i);
    kpre_tile = j + 1;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 16; t++)
      acc[t & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t < kPre ? vpre[t] : vfrag(sv, t),
                                                           pb[t >> 2], acc[t & 3], 0, 0, 0);
  };
  issue(0);
  issue(1);
  issue(2);
  int j = 0;
  while (true) {
    // tiles outside this wave's list only move the ring along
    while (j < nreal && !listed(j)) ring_step(j++);
    if (j >= nreal) break;
    ring_step(j);
    compute(j);
    j++;
  }
  // no tile load may still be writing LDS when the work-group ends
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  uint16_t* orow = o + ((int64_t)h * N + tok) * 128;
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      uint2 u;
      u.x = pk2(acc[db][4 * jj + 0] * inv, acc[db][4 * jj + 1] * inv);
      u.y = pk2(acc[db][4 * jj + 2] * inv, acc[db][4 * jj + 3] * inv);
      *(uint2*)(orow + 32 * db + 8 * jj + 4 * hl) = u;
    }
  if (hl == 0)
    lse[(int64_t)h * N + tok] =
        l_tot > 0.0f ? m_run * 0.69314718055994530942f + logf(l_tot) : -INFINITY;
}

// ---------------------------------------------------------------- fp32 path
// fp32 inputs (small problems): the same online softmax on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32).  A work-group of two waves owns the 64
// rows of one permuted query tile (32 rows per wave, its Q fragments in
// registers); each 64-key tile of the row's blocks is gathered into LDS
// through the block -> token map (rows padded by one word, so that the 32
// lanes reading one channel of 32 keys touch distinct banks); per 32-key
// half, S = Q K^T, then the row maxima and sums by lane shuffles within
// each 32-lane half, and O += P V with P passed through LDS into the A
// operand's layout.  Output layout of a 32 x 32 product: lane l holds column
// l % 32 of rows 8 (r / 4) + 4 (l / 32) + r % 4, r = 0..15.
template <int D>
__global__ __launch_bounds__(128) void k_attn_fwd_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const uint8_t* __restrict__ shape_id, const int32_t* __restrict__ zone_base,
    const int64_t* __restrict__ blk_off, const int32_t* __restrict__ blk_org,
    const uint8_t* __restrict__ blk_shape, const int64_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int H, int W, int Z, int64_t N, float scale,
    float* __restrict__ o, float* __restrict__ lse) {
  constexpr int DP = D + 1;  // padded LDS row
  constexpr int NB = D / 32;  // 32-channel output blocks
  __shared__ float Ks[64 * DP], Vs[64 * DP];
  __shared__ float Ps[2][32 * 33];
  __shared__ int64_t rowtok[64];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int64_t tpH = N >> 6;
  const int h = (int)(blockIdx.x / tpH);
  const int64_t r0 = (blockIdx.x - (int64_t)h * tpH) << 6;
  const int m = (int)(r0 >> 9);
  const Shape sh = d_shapes[shape_id[(int64_t)h * Z + m]];
  const int64_t hoff = blk_off[h];
  const int64_t g = hoff + zone_base[(int64_t)h * Z + m] + (int)(r0 & 511) / sh.volume;
  // this wave's query rows as A operands: lane l holds row l % 32, channel
  // 2 kk + l / 32 of step kk
  const int64_t qtok = token_of(sh, m, (int)((r0 + 32 * wv + l32) & 511), H, W);
  float qa[D / 2];
#pragma unroll
  for (int kk = 0; kk < D / 2; kk++) qa[kk] = q[((int64_t)h * N + qtok) * D + 2 * kk + hl];
  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[nb][r] = 0.0f;
  // running maximum and sum of the rows this lane's registers hold
  float mrun[16], lrun[16];
#pragma unroll
  for (int r = 0; r < 16; r++) {
    mrun[r] = -INFINITY;
    lrun[r] = 0.0f;
  }
  float* ps = Ps[wv];
  for (int64_t e = row_ptr[g]; e < row_ptr[g + 1]; e++) {
    const int j = col_idx[e];
    const uint32_t org = (uint32_t)blk_org[hoff + j];
    const int sid = block_shape_at(blk_shape, hoff + j);
    const int nt = d_shapes[sid].volume >> 6;
    for (int t = 0; t < nt; t++) {
      __syncthreads();  // the previous tile's readers are done
      if (tid < 64) rowtok[tid] = (int64_t)h * N + org + block_row_offset(sid, 64u * t + tid, H, W);
      __syncthreads();
      for (int i = tid; i < 64 * D; i += 128) {
        const int r = i / D, c = i % D;
        Ks[r * DP + c] = k[rowtok[r] * D + c];
        Vs[r * DP + c] = v[rowtok[r] * D + c];
      }
      __syncthreads();
#pragma unroll
      for (int kb = 0; kb < 2; kb++) {
        // S = Q K^T over keys 32 kb .. 32 kb + 31: B operand lane l holds
        // key 32 kb + l % 32, channel 2 kk + l / 32
        f32x16 sc;
#pragma unroll
        for (int r = 0; r < 16; r++) sc[r] = 0.0f;
        const float* kr = Ks + (32 * kb + l32) * DP + hl;
#pragma unroll
        for (int kk = 0; kk < D / 2; kk++)
          sc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[kk], kr[2 * kk], sc, 0, 0, 0);
        // online softmax per row: maxima and sums over the 32 lanes of a half
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const float sv = sc[r] * scale;
          float mx = sv;
#pragma unroll
          for (int off = 16; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
          const float mnew = fmaxf(mrun[r], mx);
          const float alpha = mrun[r] == -INFINITY ? 0.0f : expf(mrun[r] - mnew);
          const float pv = expf(sv - mnew);
          float sum = pv;
#pragma unroll
          for (int off = 16; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
          lrun[r] = lrun[r] * alpha + sum;
          mrun[r] = mnew;
#pragma unroll
          for (int nb = 0; nb < NB; nb++) acc[nb][r] *= alpha;
          ps[(8 * (r >> 2) + 4 * hl + (r & 3)) * 33 + l32] = pv;
        }
        __syncthreads();
        // O += P V: A lane l holds row l % 32, key 2 kk + l / 32 of the half;
        // B lane l holds key 32 kb + 2 kk + l / 32, channel 32 nb + l % 32
#pragma unroll
        for (int kk = 0; kk < 16; kk++) {
          const float pa = ps[l32 * 33 + 2 * kk + hl];
          const float* vr = Vs + (32 * kb + 2 * kk + hl) * DP + l32;
#pragma unroll
          for (int nb = 0; nb < NB; nb++)
            acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(pa, vr[32 * nb], acc[nb], 0, 0, 0);
        }
        __syncthreads();  // P is rewritten by the next half
      }
    }
  }
  // rows 8 (r / 4) + 4 hl + r % 4 of this wave's 32; lane l holds channel
  // 32 nb + l % 32
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int i = 8 * (r >> 2) + 4 * hl + (r & 3);
    const int64_t tok = token_of(sh, m, (int)((r0 + 32 * wv + i) & 511), H, W);
    const float inv = lrun[r] > 0.0f ? 1.0f / lrun[r] : 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; nb++) o[((int64_t)h * N + tok) * D + 32 * nb + l32] = acc[nb][r] * inv;
    if (l32 == 0) lse[(int64_t)h * N + tok] = lrun[r] > 0.0f ? mrun[r] + logf(lrun[r]) : -INFINITY;
  }
}

bool launch_attn_fwd(const PlanDev& P, const void* q, const void* k, const void* v, void* o,
                     float* lse, hipStream_t st) {
  if (P.dtype == PRISM_BF16 && P.D == 128) {
    dim3 grid((unsigned)(P.heads * (P.N / kFwdRows))), block(kFwdWaves * 64);
    float c_log2 = (float)(1.4426950408889634 / sqrt(128.0));
    if (P.relayout)
      hipLaunchKernelGGL(k_attn_fwd_bf16<true>, grid, block, 0, st, (const uint16_t*)q, P.kp,
                         P.vp, P.shape_id, P.zone_base, P.blk_off, P.blk_start, P.blk_shape,
                         P.row_ptr, P.col_idx, P.H, P.W, P.Z, P.N, c_log2, (uint16_t*)o, lse);
    else
      hipLaunchKernelGGL(k_attn_fwd_bf16<false>, grid, block, 0, st, (const uint16_t*)q,
                         (const uint16_t*)k, (const uint16_t*)v, P.shape_id, P.zone_base,
                         P.blk_off, P.blk_org, P.blk_shape, P.row_ptr, P.col_idx, P.H, P.W,
                         P.Z, P.N, c_log2, (uint16_t*)o, lse);
  } else if (P.dtype == PRISM_F32 && (P.D == 64 || P.D == 128)) {
    dim3 grid((unsigned)(P.heads * (P.N >> 6))), block(128);
    float scale = (float)(1.0 / sqrt((double)P.D));
    if (P.D == 64)
      hipLaunchKernelGGL((k_attn_fwd_f32<64>), grid, block, 0, st, (const float*)q,
                         (const float*)k, (const float*)v, P.shape_id, P.zone_base,
                         P.blk_off, P.blk_org, P.blk_shape, P.row_ptr, P.col_idx, P.H, P.W,
                         P.Z, P.N, scale, (float*)o, lse);
    else
      hipLaunchKernelGGL((k_attn_fwd_f32<128>), grid, block, 0, st, (const float*)q,
                         (const float*)k, (const float*)v, P.shape_id, P.zone_base,
                         P.blk_off, P.blk_org, P.blk_shape, P.row_ptr, P.col_idx, P.H, P.W,
                         P.Z, P.N, scale, (float*)o, lse);
  } else {
    return false;
  }
  return hipGetLastError() == hipSuccess;
}

}  // namespace prism
