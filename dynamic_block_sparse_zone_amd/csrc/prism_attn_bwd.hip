// Sparse attention backward with the plan held constant (paper.rainbus.top,
// "技术新颖性": shapes and selections are detached, gradients flow only
// through attention on the selected blocks).  With P = softmax over the
// selected keys, dP = dO V^T, Delta = rowsum(dO * O), dS = P (dP - Delta):
//   dV = P^T dO,  dK = dS^T Q / sqrt(D),  dQ = dS K / sqrt(D).
//
// gfx950 design (bf16, head_dim 128), deterministic (no atomics):
//  * prep: Delta and log2(e) * LSE per token (original order) and, with the
//    re-layout, copies of Q, dO and both columns in block-contiguous order;
//    every tile of Q, dO (and the LSE / Delta columns) comes from those
//    copies and every K, V tile from the plan's (or, without copies, each is
//    gathered from the caller's tensors through the block -> token map);
//  * dK/dV: a work-group owns 128 permuted key rows (4 waves x 32 keys, K and
//    V of its keys in registers, dK/dV accumulators pinned to AGPRs) and
//    walks the query blocks whose S_i holds its key blocks (key-major lists);
//    Q and dO tiles with their LSE and Delta columns stream through a 4-slot
//    LDS ring; per 32-query slice it forms S = Q K^T and dP = dO V^T, then
//    dV^T += dO^T P and dK^T += Q^T dS with the transposed operands read by
//    ds_read_b64_tr_b16.  One wave per SIMD: a tile's 64 MFMAs run in a
//    fixed, fenced order with each fragment read eight MFMAs ahead (the
//    next tile's first ones during this tile's last products) and the dS
//    arithmetic of one slice under the products of the other.  For dense
//    selections the launch is persistent: each XCD's work-groups take its
//    units in the plan's order (longest walk first) a generation at a time,
//    so that walks of equal length share the XCD's L2 (it fetches 2x the
//    bytes per flop of the query-major kernels, which gained nothing from
//    this; sparse selections share too little and keep one unit per
//    work-group);
//  * dQ: a work-group owns 256 permuted query rows (8 waves) and walks its
//    key blocks as the forward does: S^T = K Q^T, dP^T = V dO^T,
//    dQ^T += K^T dS^T, the tile's 48 MFMAs again in a fenced order.
#include "prism_attn_common.h"
#include "prism_kernels.h"

namespace prism {

// dK/dV work units: 128 key rows, 4 waves x 32 keys; each query tile of the
// ring carries its Q and dO tiles and its LSE and Delta columns.
constexpr int kKvRows = 128;
constexpr int kKvWaves = kKvRows / 32;
// loads per wave per query tile: 2 x 16 KB in 1 KB pieces over 4 waves, plus
// one 256-byte column load
constexpr int kKvLoads = 2 * kTile / (kKvWaves * 1024) + 1;
// dQ work units: 256 query rows, 8 waves x 32 rows; K/V tile pairs as in the
// forward
constexpr int kDqRows = 256;
constexpr int kDqWaves = kDqRows / 32;
constexpr int kDqLoads = 2 * kTile / (kDqWaves * 1024);

// ---------------------------------------------------------------- prep
// Per token row (all heads, original order): Delta = rowsum(dO * O) and
// log2(e) * LSE.  One wave per row, 8 rows per block of 512 threads; lane l
// holds channels 2l, 2l + 1.
__global__ __launch_bounds__(512) void k_bwd_prep(const uint16_t* __restrict__ o,
                                                  const uint16_t* __restrict__ d_o,
                                                  const float* __restrict__ lse, int64_t rows,
                                                  float* __restrict__ delta,
                                                  float* __restrict__ lse2) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint32_t dv = *(const uint32_t*)(d_o + row * 128 + lane * 2);
  const uint32_t ov = *(const uint32_t*)(o + row * 128 + lane * 2);
  float s = __uint_as_float(dv << 16) * __uint_as_float(ov << 16);
  s = __builtin_fmaf(__uint_as_float(dv & 0xffff0000u), __uint_as_float(ov & 0xffff0000u), s);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) {
    delta[row] = s;
    lse2[row] = lse[row] * 1.44269504088896340736f;
  }
}

// ---------------------------------------------------------------- dK, dV
// kRelaid: q, d_o, lse2 and delta are the block-contiguous copies and
// blk_base holds each block's first permuted row; else they are in token
// order and blk_base holds each block's first token
template <bool kRelaid>
__global__ __launch_bounds__(kKvWaves * 64, 1) void k_bwd_dkdv(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse2, const float* __restrict__ delta,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint8_t* __restrict__ shape_id, const int32_t* __restrict__ zone_base,
    const int64_t* __restrict__ blk_off, const int32_t* __restrict__ blk_base,
    const uint8_t* __restrict__ blk_shape, const int64_t* __restrict__ colt_ptr,
    const int32_t* __restrict__ colt_idx, int H, int W, int Z, int64_t N, float c_log2,
    float scale, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int64_t nunits,
    const int32_t* __restrict__ order, int32_t* sync) {
  // ring of query-tile slots: Q and dO tiles, and the LSE and Delta columns
  // (two objects, so that the reads of each carry their own alias scope)
  __shared__ __attribute__((aligned(16))) char ring[kRing * 2 * kTile];
  __shared__ __attribute__((aligned(16))) float ringc[kRing * 128];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int64_t upH = N / kKvRows;
  // persistent (sync given) or one unit per work-group
  const UnitLoop L(nunits);
  const int ngen = sync ? L.ngen : 1;
  for (int gen = 0; gen < ngen; gen++) {
  int64_t unit = xcd_unit(blockIdx.x, gridDim.x);
  if (sync) {
    L.start(sync, gen);
    unit = L.unit(order, upH, gen);
    if (unit < 0) continue;
  }
  {
  const int h = (int)(unit / upH);
  const int64_t r0 = (unit - (int64_t)h * upH) * kKvRows;
  const int m = (int)(r0 >> 9);
  const Shape sh = d_shapes[shape_id[(int64_t)h * Z + m]];
  const int B = sh.volume;
  const int rz = (int)(r0 & 511);
  const int64_t hoff = blk_off[h];
  const int nlists = B >= kKvRows ? 1 : kKvRows / B;  // key blocks in the unit
  const int mylist = (32 * wvu) / B < nlists ? (32 * wvu) / B : 0;

  // this wave's 32 keys: K and V rows as MFMA B operands (k = channel)
  const int64_t hrow = (int64_t)h * N;
  const int64_t ktok = token_of(sh, m, (int)((r0 + wv * 32 + l32) & 511), H, W);
  bf16x8 kr[8], vr[8];
#pragma unroll
  for (int kk = 0; kk < 8; kk++) {
    kr[kk] = row_chunk(k, hrow + ktok, 2 * kk + hl);
    vr[kk] = row_chunk(v, hrow + ktok, 2 * kk + hl);
  }
  // the key fragments land before any tile load is issued, so the ring's
  // waits only ever concern tiles (the empty asm consumes them here)
#pragma unroll
  for (int kk = 0; kk < 8; kk++) asm volatile("" : "+v"(kr[kk]), "+v"(vr[kk]));
  f32x16 dkt[4], dvt[4];
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int r = 0; r < 16; r++) {
      dkt[db][r] = 0.0f;
      dvt[db][r] = 0.0f;
    }
#pragma unroll
  for (int db = 0; db < 4; db++) asm volatile("" : "+a"(dkt[db]), "+a"(dvt[db]));
  uint32_t ro[8], to[4][2];
  row_offsets(lane, ro);
  tr_offsets(lane, to);

  TileIter it;
  it.init(colt_ptr, colt_idx, hoff + zone_base[(int64_t)h * Z + m] + rz / B, nlists, blk_base,
          blk_shape, hoff);
  const __amdgpu_buffer_rsrc_t rsQ = buffer_of(q + hrow * 128, (uint32_t)(N * 256));
  const __amdgpu_buffer_rsrc_t rsD = buffer_of(d_o + hrow * 128, (uint32_t)(N * 256));
  // waves 0 and 2 bring the LSE column, waves 1 and 3 Delta (both pairs write
  // the same values), so that every wave issues the same nine loads per tile
  const __amdgpu_buffer_rsrc_t rsC =
      buffer_of((wvu & 1) ? delta + hrow : lse2 + hrow, (uint32_t)(N * 4));
  const uint32_t lring = lds_offset(ring);
  const uint32_t lcol = lds_offset(ringc) + (wvu & 1) * 256;
  // tile t of the query block (base org, shape sid) from Q and dO, with its
  // LSE or Delta column, into slot b
  auto stage = [&](int b, uint32_t org, int sid, int t) {
    const uint32_t o = lring + b * 2 * kTile;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t piece = i * 256 + wvu * 64;
      const uint32_t src = tile_src<kRelaid>(org, sid, t, piece + lane, H, W);
      dma16(rsQ, src, o + piece * 16);
      dma16(rsD, src, o + kTile + piece * 16);
    }
    dma4(rsC, col_src<kRelaid>(org, sid, t, lane, H, W), lcol + b * 512);
  };

  uint32_t ring_f = 0;  // list masks of the tiles in the ring, a byte per slot
  int nreal = 0;        // real tiles issued; later slots re-read the last one
  uint32_t last_org = 0;
  int last_sid = 0, last_t = 0;
  auto issue = [&](int b) {
    uint32_t f = 0;
    if (it.valid) {
      last_org = it.org();
      last_sid = it.sid();
      last_t = it.t;
      f = (uint32_t)it.mask;
      nreal++;
      it.advance();
    }
    ring_f = (ring_f & ~(0xffu << (8 * b))) | (f << (8 * b));
    stage(b, last_org, last_sid, last_t);
  };
  issue(0);
  issue(1);
  issue(2);
  // one ring step per tile, in every wave
  // step j: tiles j and j + 1 have landed, so the first fragments of tile
  // j + 1 can be read during the last slots of tile j
  auto ring_step = [&](int j) {
    __builtin_amdgcn_s_waitcnt(wait_vm(kKvLoads));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue((j + kRing - 1) & (kRing - 1));
  };
  auto listed = [&](int j) { return ((ring_f >> (8 * (j & (kRing - 1)) + mylist)) & 1u) != 0; };
  // fragments read ahead of their MFMA; a divisor of the tile's 64 slots,
  // so that slot t and the next tile's slot t + kWin - 64 share win[t % kWin]
  constexpr int kWin = 8;
  static_assert(64 % kWin == 0, "window must divide the slots of a tile");
  bf16x8 win[kWin];
  int pre_tile = -1;  // the tile whose first kWin fragments win holds
  int j = 0;
  while (true) {
    // tiles whose query block does not list this wave's key block only move
    // the ring along (a loop of its own, so the accumulators stay in place)
    while (j < nreal && !listed(j)) ring_step(j++);
    if (j >= nreal) break;
    ring_step(j);
    const char* sq = ring + (j & (kRing - 1)) * 2 * kTile;  // Q tile
    const char* sd = sq + kTile;                            // dO tile
    const char* sqn = ring + ((j + 1) & (kRing - 1)) * 2 * kTile;  // next tile
    const char* sdn = sqn + kTile;
    const float* sl = ringc + (j & (kRing - 1)) * 128;      // log2(e) LSE
    const float* sdl = sl + 64;                             // Delta
    // The tile's 64 MFMAs in a fixed order, one per slot:
    //   ops  0..15  S = Q K^T and dP = dO V^T of query half 0 (alternating)
    //   ops 16..31  the same for half 1, while half 0's dS is formed
    //   ops 32..47  dV^T += dO^T P, dK^T += Q^T dS of half 0, while half 1's
    //               dS is formed
    //   ops 48..63  the same for half 1.
    // Each op's fragment is read kWin slots ahead (the last slots read the
    // first fragments of the next tile), and a scheduling fence closes every
    // slot, so LDS latency and the VALU work hide under the MFMAs already
    // issued.
    auto frag = [&](int t) -> bf16x8 {
      if (t < 32) {
        const char* base = (t & 1) ? sd : sq;
        return ld_frag(base + (t >> 4) * 8192 + ro[(t & 15) >> 1]);
      }
      const int u = t - 32, cc = ((u >> 4) * 2 + ((u & 15) >> 3)) * 4096, db = (u & 7) >> 1;
      const char* base = (t & 1) ? sq : sd;
      return ld_tfrag(base + cc + to[db][0], base + cc + to[db][1]);
    };
    f32x16 s[2], dp[2];
    uint32_t pp[2][8], ps[2][8];
    f32x4 Lc[2][4], Dc[2][4];
    float pv_prev = 0.0f, sv_prev = 0.0f;
    if (pre_tile != j) {
#pragma unroll
      for (int t = 0; t < kWin; t++) win[t] = frag(t);
    }
    auto slot = [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      const bf16x8 f = win[t % kWin];
      if constexpr (t + kWin < 64) {
        win[t % kWin] = frag(t + kWin);
      } else {
        constexpr int n = t + kWin - 64;  // an S/dP fragment of the next tile
        win[t % kWin] = ld_frag(((n & 1) ? sdn : sqn) + (n >> 4) * 8192 + ro[(n & 15) >> 1]);
      }
      if constexpr (t >= 12 && t < 44 && (t & 3) == 0) {
        // the LSE and Delta values of the dS rows formed four slots on
        constexpr int qb = (t - 12) >> 4, jj = ((t - 12) & 15) >> 2;
        Lc[qb][jj] = *(const f32x4*)(sl + 32 * qb + 8 * jj + 4 * hl);
        Dc[qb][jj] = *(const f32x4*)(sdl + 32 * qb + 8 * jj + 4 * hl);
      }
      if constexpr (t < 32) {
        constexpr int qb = t >> 4, kk = (t & 15) >> 1;
        if constexpr (t & 1)
          dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, vr[kk], kk ? dp[qb] : f32x16{}, 0,
                                                           0, 0);
        else
          s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, kr[kk], kk ? s[qb] : f32x16{}, 0, 0,
                                                          0);
      } else {
        constexpr int u = t - 32, qb = u >> 4, c = (u & 15) >> 3, db = (u & 7) >> 1;
        if constexpr (t & 1) {
          const bf16x8 bs = __builtin_bit_cast(
              bf16x8, make_uint4(ps[qb][4 * c], ps[qb][4 * c + 1], ps[qb][4 * c + 2],
                                 ps[qb][4 * c + 3]));
          dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, bs, dkt[db], 0, 0, 0);
        } else {
          const bf16x8 bp = __builtin_bit_cast(
              bf16x8, make_uint4(pp[qb][4 * c], pp[qb][4 * c + 1], pp[qb][4 * c + 2],
                                 pp[qb][4 * c + 3]));
          dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, bp, dvt[db], 0, 0, 0);
        }
      }
      if constexpr (t >= 16 && t < 48) {
        // one element of the dS of the half whose S and dP are complete:
        // row q = 32qb + 8jj + 4hl + i of this lane, r = 4jj + i
        constexpr int qb = (t - 16) >> 4, r = (t - 16) & 15, jj = r >> 2, i = r & 3;
        const float pv =
            __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], c_log2, -Lc[qb][jj][i]));
        const float sv = pv * (dp[qb][r] - Dc[qb][jj][i]);
        if constexpr (r & 1) {
          pp[qb][r >> 1] = pk2(pv_prev, pv);
          ps[qb][r >> 1] = pk2(sv_prev, sv);
        }
        pv_prev = pv;
        sv_prev = sv;
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    unrolled<64>(slot);
    pre_tile = j + 1;
    // pin the accumulators to the accumulation registers across the loop
    // (otherwise they are parked in ordinary registers and copied both ways
    // on every tile)
#pragma unroll
    for (int db = 0; db < 4; db++) asm volatile("" : "+a"(dkt[db]), "+a"(dvt[db]));
    j++;
  }
  // no tile load may still be writing LDS when the work-group ends
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  // lane holds key r0 + 32wv + l32, channels 32db + 8j + 4hl + 0..3
  const int64_t p = r0 + wv * 32 + l32;
  const int64_t tok = token_of(sh, m, (int)(p & 511), H, W);
  uint16_t* dkr = dk + (hrow + tok) * 128;
  uint16_t* dvr = dv + (hrow + tok) * 128;
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint2 a, b;
      a.x = pk2(dkt[db][4 * j] * scale, dkt[db][4 * j + 1] * scale);
      a.y = pk2(dkt[db][4 * j + 2] * scale, dkt[db][4 * j + 3] * scale);
      b.x = pk2(dvt[db][4 * j], dvt[db][4 * j + 1]);
      b.y = pk2(dvt[db][4 * j + 2], dvt[db][4 * j + 3]);
      *(uint2*)(dkr + 32 * db + 8 * j + 4 * hl) = a;
      *(uint2*)(dvr + 32 * db + 8 * j + 4 * hl) = b;
    }
  }
  }
}

// ---------------------------------------------------------------- dQ
// kRelaid: k and v are the plan's block-contiguous copies and blk_base holds
// each block's first permuted row; else the caller's tensors and first tokens
// (this work-group's own Q, dO, LSE and Delta rows are read in token order)
template <bool kRelaid>
__global__ __launch_bounds__(kDqWaves * 64, 1) void k_bwd_dq(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse2, const float* __restrict__ delta,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint8_t* __restrict__ shape_id, const int32_t* __restrict__ zone_base,
    const int64_t* __restrict__ blk_off, const int32_t* __restrict__ blk_base,
    const uint8_t* __restrict__ blk_shape, const int64_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int H, int W, int Z, int64_t N, float c_log2,
    float scale, uint16_t* __restrict__ dq) {
  __shared__ __attribute__((aligned(16))) char ringK[kRing * kTile];
  __shared__ __attribute__((aligned(16))) char ringV[kRing * kTile];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int64_t upH = N / kDqRows;
  const int64_t unit = xcd_unit(blockIdx.x, gridDim.x);
  const int h = (int)(unit / upH);
  const int64_t r0 = (unit - (int64_t)h * upH) * kDqRows;
  const int m = (int)(r0 >> 9);
  const Shape sh = d_shapes[shape_id[(int64_t)h * Z + m]];
  const int B = sh.volume;
  const int rz = (int)(r0 & 511);
  const int64_t hoff = blk_off[h];
  const int nlists = B >= kDqRows ? 1 : kDqRows / B;  // query blocks in the unit
  const int mylist = (32 * wvu) / B < nlists ? (32 * wvu) / B : 0;

  TileIterS it;
  it.init(row_ptr, col_idx, hoff + zone_base[(int64_t)h * Z + m] + rz / B, nlists, blk_base,
          blk_shape, hoff);

  // this wave's 32 query rows: Q and dO as MFMA B operands, LSE and Delta of
  // the lane's row
  const int64_t hrow = (int64_t)h * N;
  const int64_t qtok = token_of(sh, m, (int)((r0 + wv * 32 + l32) & 511), H, W);
  const int64_t qrow = hrow + qtok;
  bf16x8 qf[8], df[8];
#pragma unroll
  for (int kk = 0; kk < 8; kk++) {
    qf[kk] = row_chunk(q, qrow, 2 * kk + hl);
    df[kk] = row_chunk(d_o, qrow, 2 * kk + hl);
  }
  float L = lse2[qrow];
  float Dl = delta[qrow];
  // all of it lands before any tile load is issued (the empty asm consumes
  // it), so the ring's waits only ever concern tiles
#pragma unroll
  for (int kk = 0; kk < 8; kk++) asm volatile("" : "+v"(qf[kk]), "+v"(df[kk]));
  asm volatile("" : "+v"(L), "+v"(Dl));
  uint32_t ro[8], to[4][2];
  row_offsets(lane, ro);
  tr_offsets(lane, to);
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[db][r] = 0.0f;

  const __amdgpu_buffer_rsrc_t rsK = buffer_of(k + hrow * 128, (uint32_t)(N * 256));
  const __amdgpu_buffer_rsrc_t rsV = buffer_of(v + hrow * 128, (uint32_t)(N * 256));
  const uint32_t lK = lds_offset(ringK), lV = lds_offset(ringV);
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
  uint32_t last_org = 0;
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
  auto ring_step = [&](int j) {
    __builtin_amdgcn_s_waitcnt(wait_vm(2 * kDqLoads));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue((j + kRing - 1) & (kRing - 1));
  };
  auto listed = [&](int j) {
    return ((ring_mask >> (8 * (j & (kRing - 1)) + mylist)) & 1u) != 0;
  };
  issue(0);
  issue(1);
  issue(2);
  int j = 0;
  while (true) {
    while (j < nreal && !listed(j)) ring_step(j++);
    if (j >= nreal) break;
    ring_step(j);
    const char* sk = ringK + (j & (kRing - 1)) * kTile;
    const char* sv = ringV + (j & (kRing - 1)) * kTile;
    // The tile's 48 MFMAs in a fixed order, one per slot:
    //   ops  0..15  S^T = K Q^T and dP^T = V dO^T of keys 0..31 (alternating)
    //   ops 16..31  the same for keys 32..63, while the dS of keys 0..31 is
    //               formed (lane: query l32, keys 8r' + 4hl + i)
    //   ops 32..47  dQ^T += K^T dS^T, 16 keys per group of four, while the
    //               dS of keys 32..63 is formed.
    // Each op's fragment is read kWin slots ahead and a scheduling fence
    // closes every slot.
    constexpr int kWin = 3;
    auto frag = [&](auto tc) -> bf16x8 {
      constexpr int t = decltype(tc)::value;
      if constexpr (t < 32) {
        return ld_frag(((t & 1) ? sv : sk) + (t >> 4) * 8192 + ro[(t & 15) >> 1]);
      } else {
        constexpr int c = (t - 32) >> 2, db = (t - 32) & 3;
        return ld_tfrag(sk + c * 4096 + to[db][0], sk + c * 4096 + to[db][1]);
      }
    };
    f32x16 st[2], dpt[2];
    uint32_t pk[4][4];
    float prev = 0.0f;
    bf16x8 win[kWin];
    unrolled<kWin>([&](auto tc) { win[decltype(tc)::value] = frag(tc); });
    // dS element e (0..31): the B operand bs[e / 8], row r of key half e / 16
    auto ds_elem = [&](auto ec) {
      constexpr int e = decltype(ec)::value, c = e >> 3, i = e & 7;
      constexpr int r = 8 * (c & 1) + i, kb = c >> 1;
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][r], c_log2, -L));
      const float sv = pv * (dpt[kb][r] - Dl);
      if constexpr (i & 1) pk[c][i >> 1] = pk2(prev, sv);
      prev = sv;
    };
    auto slot = [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      const bf16x8 f = win[t % kWin];
      if constexpr (t + kWin < 48)
        win[t % kWin] = frag(std::integral_constant<int, t + kWin>{});
      if constexpr (t < 32) {
        constexpr int kb = t >> 4, kk = (t & 15) >> 1;
        if constexpr (t & 1)
          dpt[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, df[kk], kk ? dpt[kb] : f32x16{},
                                                            0, 0, 0);
        else
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[kk], kk ? st[kb] : f32x16{},
                                                           0, 0, 0);
      } else {
        constexpr int c = (t - 32) >> 2, db = (t - 32) & 3;
        const bf16x8 bs =
            __builtin_bit_cast(bf16x8, make_uint4(pk[c][0], pk[c][1], pk[c][2], pk[c][3]));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, bs, acc[db], 0, 0, 0);
      }
      // keys 0..31 one element a slot from slot 17, keys 32..63 two a slot
      // from slot 33 (a slot after the last product they read)
      if constexpr (t >= 17 && t < 33) ds_elem(std::integral_constant<int, t - 17>{});
      if constexpr (t >= 33 && t < 41) {
        ds_elem(std::integral_constant<int, 16 + 2 * (t - 33)>{});
        ds_elem(std::integral_constant<int, 17 + 2 * (t - 33)>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    unrolled<48>(slot);
    j++;
  }
  // no tile load may still be writing LDS when the work-group ends
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  uint16_t* row = dq + qrow * 128;
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      uint2 u;
      u.x = pk2(acc[db][4 * jj] * scale, acc[db][4 * jj + 1] * scale);
      u.y = pk2(acc[db][4 * jj + 2] * scale, acc[db][4 * jj + 3] * scale);
      *(uint2*)(row + 32 * db + 8 * jj + 4 * hl) = u;
    }
}

// ---------------------------------------------------------------- launch
// dK/dV runs persistent: one work-group per compute unit (a multiple of 8:
// one share per XCD).
static int persistent_grid() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n = 256;
  n &= ~7;
  return n < 8 ? 8 : n;
}

// the start counters to zero (a fill kernel, not a memset, so that the
// launch sequence can be captured into a graph)
__global__ void k_clear_sync(int32_t* p) { p[threadIdx.x] = 0; }

static const float kCLog2 = (float)(1.4426950408889634 / 11.313708498984761);
static const float kScale = (float)(1.0 / 11.313708498984761);

bool launch_bwd_prep(const PlanDev& P, const BwdDev& Bd, const void* o, const float* lse,
                     hipStream_t st) {
  if (!(P.dtype == PRISM_BF16 && P.D == 128)) return false;
  const int64_t rows = P.heads * P.N;
  hipLaunchKernelGGL(k_bwd_prep, dim3((unsigned)((rows + 7) / 8)), dim3(512), 0, st,
                     (const uint16_t*)o, (const uint16_t*)Bd.d_o, lse, rows, Bd.delta, Bd.lse2);
  if (hipGetLastError() != hipSuccess) return false;
  // the copies dK/dV streams its query tiles from
  return !Bd.qp || launch_relayout(P, Bd.q, Bd.d_o, Bd.lse2, Bd.delta, Bd.qp, Bd.dop, Bd.lse2_p,
                                   Bd.delta_p, st);
}

bool launch_bwd_dkdv(const PlanDev& P, const BwdDev& Bd, void* dk, void* dv, hipStream_t st) {
  if (!(P.dtype == PRISM_BF16 && P.D == 128)) return false;
  // the ordered persistent launch pays where units share most of their
  // tiles (dense selections); sparse plans take one unit per work-group
  const int64_t nunits = P.heads * (P.N / kKvRows);
  if (P.kv_persist) hipLaunchKernelGGL(k_clear_sync, dim3(1), dim3(128), 0, st, P.sync);
  dim3 grid((unsigned)(P.kv_persist ? persistent_grid() : nunits)), block(kKvWaves * 64);
  if (Bd.qp)
    hipLaunchKernelGGL(k_bwd_dkdv<true>, grid, block, 0, st, Bd.qp, Bd.dop, Bd.lse2_p,
                       Bd.delta_p, (const uint16_t*)Bd.k, (const uint16_t*)Bd.v, P.shape_id,
                       P.zone_base, P.blk_off, P.blk_start, P.blk_shape, P.colt_ptr,
                       P.colt_idx, P.H, P.W, P.Z, P.N, kCLog2, kScale, (uint16_t*)dk,
                       (uint16_t*)dv, nunits, P.korder, P.kv_persist ? P.sync : nullptr);
  else
    hipLaunchKernelGGL(k_bwd_dkdv<false>, grid, block, 0, st, (const uint16_t*)Bd.q,
                       (const uint16_t*)Bd.d_o, Bd.lse2, Bd.delta, (const uint16_t*)Bd.k,
                       (const uint16_t*)Bd.v, P.shape_id, P.zone_base, P.blk_off, P.blk_org,
                       P.blk_shape, P.colt_ptr, P.colt_idx, P.H, P.W, P.Z, P.N, kCLog2,
                       kScale, (uint16_t*)dk, (uint16_t*)dv, nunits, P.korder,
                       P.kv_persist ? P.sync : nullptr);
  return hipGetLastError() == hipSuccess;
}

bool launch_bwd_dq(const PlanDev& P, const BwdDev& Bd, void* dq, hipStream_t st) {
  if (!(P.dtype == PRISM_BF16 && P.D == 128)) return false;
  dim3 grid((unsigned)(P.heads * (P.N / kDqRows))), block(kDqWaves * 64);
  if (P.relayout)
    hipLaunchKernelGGL(k_bwd_dq<true>, grid, block, 0, st, (const uint16_t*)Bd.q,
                       (const uint16_t*)Bd.d_o, Bd.lse2, Bd.delta, P.kp, P.vp, P.shape_id,
                       P.zone_base, P.blk_off, P.blk_start, P.blk_shape, P.row_ptr, P.col_idx,
                       P.H, P.W, P.Z, P.N, kCLog2, kScale, (uint16_t*)dq);
  else
    hipLaunchKernelGGL(k_bwd_dq<false>, grid, block, 0, st, (const uint16_t*)Bd.q,
                       (const uint16_t*)Bd.d_o, Bd.lse2, Bd.delta, (const uint16_t*)Bd.k,
                       (const uint16_t*)Bd.v, P.shape_id, P.zone_base, P.blk_off, P.blk_org,
                       P.blk_shape, P.row_ptr, P.col_idx, P.H, P.W, P.Z, P.N, kCLog2, kScale,
                       (uint16_t*)dq);
  return hipGetLastError() == hipSuccess;
}

}  // namespace prism
