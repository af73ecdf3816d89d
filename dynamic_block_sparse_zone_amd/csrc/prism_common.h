// Internal definitions shared by the gfx950 kernels and the host side of the
// library.  Not part of the public ABI (include/prism.h is).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/prism.h"

namespace prism {

// ---------------------------------------------------------------- shapes
// The 16 candidate block shapes (bT, bH, bW): every edge in {2,4,8}, edge
// product B in {64,128,256} (paper.rainbus.top "核心方法").  Order: by B,
// then lexicographic; the index is the shape id used everywhere.
struct Shape {
  int8_t bt, bh, bw;
  int8_t log2_bt, log2_bh, log2_bw;
  int16_t volume;
};

#define PRISM_SHAPES                                                                   \
  {{2, 4, 8, 1, 2, 3, 64},   {2, 8, 4, 1, 3, 2, 64},   {4, 2, 8, 2, 1, 3, 64},          \
   {4, 4, 4, 2, 2, 2, 64},   {4, 8, 2, 2, 3, 1, 64},   {8, 2, 4, 3, 1, 2, 64},          \
   {8, 4, 2, 3, 2, 1, 64},   {2, 8, 8, 1, 3, 3, 128},  {4, 4, 8, 2, 2, 3, 128},         \
   {4, 8, 4, 2, 3, 2, 128},  {8, 2, 8, 3, 1, 3, 128},  {8, 4, 4, 3, 2, 2, 128},         \
   {8, 8, 2, 3, 3, 1, 128},  {4, 8, 8, 2, 3, 3, 256},  {8, 4, 8, 3, 2, 3, 256},         \
   {8, 8, 4, 3, 3, 2, 256}}

static constexpr int kNumShapes = 16;
// first id and count of each volume class: 64 -> [0,7), 128 -> [7,13), 256 -> [13,16)
__host__ __device__ inline int shape_first(int volume) {
  return volume == 64 ? 0 : volume == 128 ? 7 : 13;
}
__host__ __device__ inline int shape_count(int volume) {
  return volume == 64 ? 7 : volume == 128 ? 6 : 3;
}

static __constant__ Shape d_shapes[kNumShapes] = PRISM_SHAPES;
static const Shape h_shapes[kNumShapes] = PRISM_SHAPES;
static constexpr Shape kShapeTable[kNumShapes] = PRISM_SHAPES;

// log2 of one edge of every candidate, two bits per shape id, so that a
// kernel can look an edge up by arithmetic alone (no memory access):
// log2(edge) = (kLog2X >> 2 * id) & 3.
constexpr uint32_t pack_edge_log2(int axis) {
  uint32_t r = 0;
  for (int i = 0; i < kNumShapes; i++) {
    const Shape& s = kShapeTable[i];
    r |= (uint32_t)(axis == 0 ? s.log2_bt : axis == 1 ? s.log2_bh : s.log2_bw) << (2 * i);
  }
  return r;
}
constexpr uint32_t kLog2H = pack_edge_log2(1);
constexpr uint32_t kLog2W = pack_edge_log2(2);

// Token offset of row u (0..B-1, raster order t, h, w inside the block) of a
// block of shape `sid` from the block's first token, on a grid of H x W
// tokens per frame.  With the block's first token this is the closed-form
// map from a block-contiguous row to its original token, so kernels can read
// a block's rows straight from the original [N][D] layout.
__host__ __device__ inline uint32_t block_row_offset(int sid, uint32_t u, int H, int W) {
  const uint32_t lw = (kLog2W >> (2 * sid)) & 3u, lh = (kLog2H >> (2 * sid)) & 3u;
  return (u >> (lh + lw)) * (uint32_t)(H * W) + ((u >> lw) & ((1u << lh) - 1u)) * (uint32_t)W +
         (u & ((1u << lw) - 1u));
}

// Original token of permuted row r (0..511) of zone m for a zone shape:
// blocks in raster order over the zone's block grid, tokens in raster order
// inside each block.
__host__ __device__ inline int64_t token_of(const Shape& s, int m, int r, int H, int W) {
  int zH = H >> 3, zW = W >> 3;
  int mt = m / (zH * zW), rem = m - mt * (zH * zW);
  int mh = rem / zW, mw = rem - mh * zW;
  int lgB = s.log2_bt + s.log2_bh + s.log2_bw;
  int jl = r >> lgB, u = r & ((1 << lgB) - 1);
  int lnbH = 3 - s.log2_bh, lnbW = 3 - s.log2_bw;
  int jt = jl >> (lnbH + lnbW);
  int jh = (jl >> lnbW) & ((1 << lnbH) - 1);
  int jw = jl & ((1 << lnbW) - 1);
  int ut = u >> (s.log2_bh + s.log2_bw);
  int uh = (u >> s.log2_bw) & ((1 << s.log2_bh) - 1);
  int uw = u & ((1 << s.log2_bw) - 1);
  int t = (mt << 3) + (jt << s.log2_bt) + ut;
  int y = (mh << 3) + (jh << s.log2_bh) + uh;
  int w = (mw << 3) + (jw << s.log2_bw) + uw;
  return ((int64_t)t * H + y) * W + w;
}

// A 64-row tile staged in LDS (bf16, head_dim 128) holds 16 chunks of 16 B
// per row; logical chunk c of the row at position rho inside the tile is
// stored at chunk c ^ chunk_swizzle(rho).  With this map, 16 consecutive rows
// read at one logical chunk, and 4 consecutive rows read as two adjacent
// chunks, both touch distinct LDS banks.
__host__ __device__ inline int chunk_swizzle(int rho) {
  return ((rho & 3) << 2) | ((rho >> 2) & 3);
}

// Work-groups are dispatched to the 8 XCDs round-robin by block id, and each
// XCD has its own L2.  This maps the block id to a logical work unit so that
// XCD x runs the contiguous unit range [x*G/8, (x+1)*G/8): neighbouring units
// (same head, nearby zones, near-identical key lists) then share one L2 and
// walk the same K/V tiles at the same time.
__device__ inline int64_t xcd_unit(int64_t b, int64_t G) {
  const int64_t x = b & 7, i = b >> 3;
  const int64_t per = G >> 3, rem = G & 7;
  return x * per + (x < rem ? x : rem) + i;
}

// Shape id of global block g from the byte array blk_shape, read through its
// aligned 32-bit word so that a uniform index becomes a scalar load (a vector
// byte load would be counted with, and waited for behind, in-flight tile loads).
__device__ inline int block_shape_at(const uint8_t* blk_shape, int64_t g) {
  const uint32_t w = ((const uint32_t*)blk_shape)[g >> 2];
  return (int)((w >> (8 * (g & 3))) & 0xffu);
}

// ---------------------------------------------------------------- numbers
__device__ inline float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// round to nearest even (finite inputs)
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- workspace
struct PlanDev {
  // sizes
  int T, H, W, heads, D, dtype, Z;
  int64_t N;
  // stage 1
  float* vstats;       // [heads][Z][5]
  float* astats;       // [Z][4]
  uint8_t* shape_id;   // [heads][Z]
  int32_t* zone_base;  // [heads][Z]   first local block id of each zone
  int32_t* nblk;       // [heads]
  int64_t* blk_off;    // [heads+1]
  // stage 2/3
  int32_t* blk_start;  // [Gmax]  permuted row of the block's first token (within head)
  uint8_t* blk_shape;  // [Gmax]
  int32_t* blk_head;   // [Gmax]
  float* qbar;         // [Gmax][D]
  float* kbar;
  uint16_t* qgrid;     // [Gmax][D] bf16 integers: high part of the two-level grid
  uint16_t* kgrid;
  uint16_t* qlo;       // [Gmax][D] bf16 integers: low part (x ~ 2^E (hi + 2^-8 lo))
  uint16_t* klo;
  int32_t* qexp;       // [Gmax]
  int32_t* kexp;
  int32_t* blk_org;    // [Gmax]  original token of the block's first row (within head)
  // stage two's re-layout (relayout): K and V in block-contiguous order, each
  // row's 16-byte chunks swizzled (chunk c of row p at c ^ chunk_swizzle(p & 63))
  int relayout;
  uint16_t* kp;        // [heads][N][128] or null
  uint16_t* vp;
  // selection
  float* scores;       // [maxblk][maxblk] scratch for one head
  int32_t* row_cnt;    // [Gmax]
  uint32_t* row_key;   // [Gmax] threshold key
  int32_t* row_tie;    // [Gmax] ties at the threshold key to take (lowest index first)
  int64_t* row_ptr;    // [Gmax+1]
  int32_t* col_idx;    // [cap]
  int64_t* colt_ptr;   // [Gmax+1]
  int32_t* colt_idx;   // [cap]
  int32_t* colt_cnt;   // [Gmax] scratch
  int32_t* chunk_cnt;  // [(maxblk/64+1) * maxblk] scratch: per (row tile, column) counts
  int32_t* chunk_cost; // [(maxblk/64+1) * maxblk] scratch: per (row tile, column) volumes
  unsigned long long* selmask;  // [maxblk][maxblk/64] one head's selection, a bit per pair
  unsigned long long* volm;     // [3][maxblk/64] one head's blocks by volume class
  int64_t* row_cost;   // [Gmax] B_i * sum_{j in S_i} B_j
  int64_t* counters;   // [8]: [0] nnz running total
  int64_t cap;
  // dK/dV work units, per head longest walk first (backward plans)
  int32_t* korder;     // [heads][N/128]
  int64_t* colt_cost;  // [Gmax] B_j * sum_{i: j in S_i} B_i
  int32_t* sync;       // [128] start counters of the persistent dK/dV kernel
  int kv_persist;      // dK/dV launch: ordered persistent (dense selections) or per unit
  // shot-cut-aware temporal zones (cut_threshold > 0)
  double* cut_part;    // [T][heads] frame-difference energy per head
  double* cut_energy;  // [T] mean energy per frame
  uint8_t* cuts;       // [T] 1 where a shot cut starts
  int32_t* zt_cap;     // [T/8] longest block edge in time per temporal row of zones
};

}  // namespace prism

// error helpers
#define PRISM_HIP(x)                        \
  do {                                      \
    hipError_t e_ = (x);                    \
    if (e_ != hipSuccess) return PRISM_EDEVICE; \
  } while (0)
