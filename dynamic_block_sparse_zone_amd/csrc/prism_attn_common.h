// Device pieces shared by the sparse-attention kernels (forward, dK/dV, dQ):
// the walk over selected key blocks, the LDS tile ring and its fragment reads.
//
// Tiles.  A 64-row tile is 64 consecutive rows of one block in the
// block-contiguous order of the plan, and every block is a whole number of
// tiles.  Either its rows are gathered straight from the caller's
// [heads][N][128] bf16 tensors (K, V, and in the backward Q, dO) through the
// closed-form block -> token map (block_row_offset from the block's first
// token), or they come from re-laid copies in block-contiguous order (stage
// two's re-layout), where a tile is one contiguous 16 KB run.  Each lane
// moves one 16-byte chunk per load and picks the chunk so that LDS row rho
// holds logical chunk c at c ^ chunk_swizzle(rho) (the copies store their
// rows that way already); a row is 256 contiguous bytes in HBM, and a
// wave's load covers four whole rows.
//
// Ring.  A work-group keeps kRing tile slots in LDS with kRing - 1 tiles in
// flight.  Every step issues exactly one tile (past the end of the lists it
// re-reads the last real tile into a slot that is never computed on), so
// the number of loads issued after tile j is fixed and a single
// s_waitcnt vmcnt(n) says tile j has landed; a bare s_barrier then says
// every wave has its share and is done with tile j - 1, whose slot is
// refilled.  The tile loads go straight from HBM to LDS and their LDS
// addresses are passed as opaque offsets: they carry no object identity, so
// the compiler adds no conservative full drain of its own before LDS reads.
#pragma once
#include "prism_common.h"
#include <utility>

namespace prism {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// (1, 1) in bf16: a v_dot2 against it sums a packed pair
static constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

constexpr int kTile = 64 * 128 * 2;  // bytes of one 64-row bf16 tile
constexpr int kRing = 4;             // tile slots per ring

// s_waitcnt immediates: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt at
// their maxima (no wait on them)
__host__ __device__ constexpr int wait_vm(int n) {
  return 0x0F70 | (n & 15) | ((n >> 4) << 14);
}

// s_waitcnt immediate for lgkmcnt(0) alone (vmcnt and expcnt at their maxima)
constexpr int kWaitLgkm0 = 0xC07F;

// LDS byte offset of a shared-memory object, opaque to alias analysis
__device__ inline uint32_t lds_offset(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}
// Direct HBM -> LDS loads in the buffer (MUBUF) form: 64 lanes x 16 B (or
// x 4 B) from byte offset `voff` (per lane) of buffer `rs` to LDS offset `o`.
// The buffer form is used rather than the global one because the compiler
// counts a global (FLAT) load to LDS as a possible LDS access too, and then
// turns every LDS-read wait into a full drain.
__device__ inline __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  // raw buffer, no stride, range-checked against `bytes`
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t o) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)(uintptr_t)o, 16, voff, 0, 0, 0);
}
__device__ inline void dma4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t o) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)(uintptr_t)o, 4, voff, 0, 0, 0);
}

// Byte offset, in one head's original [N][128] bf16 rows, of the 16-byte
// chunk that LDS slot `slot` (0..1023: tile row slot >> 4, stored chunk
// slot & 15) takes for tile t of a block of shape sid whose first token is
// org.
__device__ inline uint32_t tile_src16(uint32_t org, int sid, int t, uint32_t slot, int H,
                                      int W) {
  const uint32_t rho = slot >> 4;
  const uint32_t c = (slot & 15u) ^ (uint32_t)chunk_swizzle((int)rho);
  return (org + block_row_offset(sid, 64u * t + rho, H, W)) * 256u + c * 16u;
}
// Byte offset of row rho (0..63) of that tile in a per-token [N] float array.
__device__ inline uint32_t tile_src4(uint32_t org, int sid, int t, uint32_t rho, int H, int W) {
  return (org + block_row_offset(sid, 64u * t + rho, H, W)) * 4u;
}

// Tile sources of the two layouts.  Gathered (kRelaid false): base is the
// block's first token and rows come through the block -> token map.
// Re-laid: base is the block's first permuted row in a copy whose rows are
// in block-contiguous order with their chunks already swizzled, so LDS slot
// `slot` takes byte slot * 16 of the tile's contiguous 16 KB run.
template <bool kRelaid>
__device__ inline uint32_t tile_src(uint32_t base, int sid, int t, uint32_t slot, int H, int W) {
  if constexpr (kRelaid)
    return (base + 64u * t) * 256u + slot * 16u;
  else
    return tile_src16(base, sid, t, slot, H, W);
}
template <bool kRelaid>
__device__ inline uint32_t col_src(uint32_t base, int sid, int t, uint32_t rho, int H, int W) {
  if constexpr (kRelaid)
    return (base + 64u * t + rho) * 4u;
  else
    return tile_src4(base, sid, t, rho, H, W);
}

// Per-lane byte offsets inside a swizzled 64-row tile (row stride 256 B).
// ro[kk]: the 16-byte chunk 2kk + hl of row l32 -- the MFMA operand whose
// rows are the tile's rows (row l32 + 32 adds 8192).  to[db][0/1]: the two
// 8-byte transposed reads that give the operand whose rows are the channels
// 32db.., with k = 16 tile rows in the order {16c+4hl+0..3, 16c+8+4hl+0..3}
// (rows 16c.. add 4096 c).  The swizzle depends on a row's low four bits
// only, so these constants cover every read and the rest folds into
// instruction offsets.
__device__ inline void row_offsets(int lane, uint32_t (&ro)[8]) {
  const int l32 = lane & 31, hl = lane >> 5;
  const int sw = chunk_swizzle(l32);
#pragma unroll
  for (int kk = 0; kk < 8; kk++) ro[kk] = l32 * 256 + (((2 * kk + hl) ^ sw) << 4);
}
__device__ inline void tr_offsets(int lane, uint32_t (&to)[4][2]) {
  const int rA = 4 * (lane >> 5) + ((lane & 15) >> 2), rB = rA + 8;
  const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int off = 8 * (lane & 1);
#pragma unroll
  for (int db = 0; db < 4; db++) {
    to[db][0] = rA * 256 + (((4 * db + cl) ^ chunk_swizzle(rA)) << 4) + off;
    to[db][1] = rB * 256 + (((4 * db + cl) ^ chunk_swizzle(rB)) << 4) + off;
  }
}
__device__ inline bf16x8 ld_frag(const char* p) {
  return __builtin_bit_cast(bf16x8, *(const uint4*)p);
}
__device__ inline bf16x8 ld_tfrag(const char* pa, const char* pb) {
  s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pa);
  s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pb);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// f(std::integral_constant<int, t>{}) for t = 0 .. n-1 in order: the slot
// index is a constant inside f, so register arrays indexed by it stay in
// registers (a plain loop of this size is not always unrolled)
template <class F, int... Ts>
__device__ inline void unrolled_impl(F&& f, std::integer_sequence<int, Ts...>) {
  (f(std::integral_constant<int, Ts>{}), ...);
}
template <int n, class F>
__device__ inline void unrolled(F&& f) {
  unrolled_impl(f, std::make_integer_sequence<int, n>{});
}

// two floats to packed bf16, one v_cvt_pk_bf16_f32 (round to nearest even)
__device__ inline uint32_t pk2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// chunk `chunk` (16 B, 8 channels) of row `row` of an [rows][128] bf16 tensor
__device__ inline bf16x8 row_chunk(const uint16_t* buf, int64_t row, int chunk) {
  return __builtin_bit_cast(bf16x8, *(const uint4*)(buf + row * 128 + chunk * 8));
}

// The same walk with plain (scalar) loads, for the dQ kernel, where it runs
// faster: with the vector-memory walk below, using a list value loaded a
// step earlier also waits for the tile loads issued before it, which takes
// one of the two tiles that ring keeps in flight.
// Merged walk over up to four ascending block lists (the lists of the
// query blocks of one work unit, or of its key blocks in the key-major
// transpose): yields each block once, with a bit mask of the lists that
// hold it.
struct UnionIterS {
  const int32_t* col;
  int64_t a[4], e[4];
  int head[4];
  __device__ void init(const int32_t* c, int nl) {
    col = c;
#pragma unroll
    for (int i = 0; i < 4; i++) head[i] = (i < nl && a[i] < e[i]) ? col[a[i]] : 0x7fffffff;
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

// The 64-row tiles of the blocks of a merged walk, in order (scalar loads):
// per tile the block's first token, its shape id and the tile's index in it.
struct TileIterS {
  UnionIterS U;
  const int32_t* blk_org;
  const uint8_t* blk_shape;
  int64_t hoff;
  uint32_t org_;
  int sid_;
  __device__ uint32_t org() const { return org_; }
  __device__ int sid() const { return sid_; }
  int t, nt, mask;
  bool valid;
  // lists ptr[g0 + i] .. ptr[g0 + i + 1] for i < nl
  __device__ void init(const int64_t* ptr, const int32_t* col, int64_t g0, int nl,
                       const int32_t* borg, const uint8_t* bsh, int64_t off) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int64_t g = g0 + (i < nl ? i : 0);
      U.a[i] = ptr[g];
      U.e[i] = ptr[g + 1];
    }
    U.init(col, nl);
    blk_org = borg;
    blk_shape = bsh;
    hoff = off;
    valid = true;
    t = 0;
    nt = 0;
    advance();
  }
  __device__ void advance() {
    if (valid && t + 1 < nt) {
      t++;
      return;
    }
    int j;
    valid = U.next(j, mask);
    if (valid) {
      org_ = (uint32_t)blk_org[hoff + j];
      sid_ = block_shape_at(blk_shape, hoff + j);
      nt = d_shapes[sid_].volume >> 6;
      t = 0;
    }
  }
};

// The 64-row tiles of the blocks of a merged walk over up to four ascending
// block lists (the lists of the query blocks of one work unit, or of its key
// blocks in the key-major transpose), in block order; each block comes once,
// with a bit mask of the lists that hold it.
//
// The list entries, block first tokens and shape ids are read with buffer
// (vector memory) loads whose values are only needed a step later (the next
// head of a list, the next tile's rows and the block's tile count), so their latency
// hides behind the tile in between; scalar loads would share the counter of
// the LDS reads, and every LDS wait of the tile would then wait for them too.
// The loaded values stay in vector registers (the load offsets carry an
// opaque per-lane zero, so that the compiler does not move them to scalar
// registers at once, which would wait for the load, and with it for every
// earlier tile load) and are read out with readfirstlane where they are used.
struct TileIter {
  __amdgpu_buffer_rsrc_t rcol, rorg, rshape;
  int a[4], e[4];  // list positions relative to the first list's start
  int opq;
  int head_v[4];         // next entry of each list (0x7fffffff: exhausted)
  int org_v, sid_v;      // the current block's first token and shape id
  int t, mask;
  bool valid;
  // lists ptr[g0 + i] .. ptr[g0 + i + 1] for i < nl (consecutive, so one
  // buffer covers them); block j's first token and shape id at
  // borg[off + j], bsh[off + j]
  __device__ void init(const int64_t* ptr, const int32_t* col, int64_t g0, int nl,
                       const int32_t* borg, const uint8_t* bsh, int64_t off) {
    asm volatile("v_mov_b32 %0, 0" : "=v"(opq));
    const int64_t base = ptr[g0];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      a[i] = i < nl ? (int)(ptr[g0 + i] - base) : 0;
      e[i] = i < nl ? (int)(ptr[g0 + i + 1] - base) : 0;
    }
    rcol = buffer_of(col + base, (uint32_t)(ptr[g0 + nl] - base) * 4u);
    rorg = buffer_of(borg + off, 0xffffffffu);
    rshape = buffer_of(bsh + off, 0xffffffffu);
#pragma unroll
    for (int i = 0; i < 4; i++) head_v[i] = a[i] < e[i] ? load_col(i) : 0x7fffffff;
    valid = true;
    t = 0;
    sid_v = 0;  // one tile: the first advance moves to the first block
    advance();
  }
  __device__ int load_col(int i) const {
    return __builtin_amdgcn_raw_buffer_load_b32(rcol, a[i] * 4 + opq, 0, 0);
  }
  // shape ids are ordered by volume: 0..6 are 64 rows, 7..12 128, 13..15 256
  __device__ int tiles() const {
    const int sid = __builtin_amdgcn_readfirstlane(sid_v);
    return sid < 7 ? 1 : sid < 13 ? 2 : 4;
  }
  // the current block's first token and shape id
  __device__ uint32_t org() const { return (uint32_t)__builtin_amdgcn_readfirstlane(org_v); }
  __device__ int sid() const { return __builtin_amdgcn_readfirstlane(sid_v); }
  __device__ void advance() {
    if (valid && t + 1 < tiles()) {
      t++;
      return;
    }
    int head[4];
#pragma unroll
    for (int i = 0; i < 4; i++) head[i] = __builtin_amdgcn_readfirstlane(head_v[i]);
    int best = head[0];
#pragma unroll
    for (int i = 1; i < 4; i++) best = head[i] < best ? head[i] : best;
    valid = best != 0x7fffffff;
    if (!valid) return;
    mask = 0;
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (head[i] == best) {
        mask |= 1 << i;
        a[i]++;
        head_v[i] = a[i] < e[i] ? load_col(i) : 0x7fffffff;
      }
    org_v = __builtin_amdgcn_raw_buffer_load_b32(rorg, best * 4 + opq, 0, 0);
    sid_v = __builtin_amdgcn_raw_buffer_load_b8(rshape, best + opq, 0, 0);
    t = 0;
  }
};

// Persistent work loop (the dK/dV kernel).  A launch has one work-group per
// compute unit.  The work-groups of one XCD (blockIdx % 8: the
// hardware deals work-groups to the XCDs in turn) share that XCD's contiguous
// part of the unit order -- per head, units by walk length, longest first --
// and take its units in generations of gridDim.x / 8.  A generation starts
// together: each work-group adds one to its XCD's counter and polls it, with
// a bounded number of polls, until the whole generation has arrived.  The
// wait only aligns start times, never a result, so the walks of a generation
// (near-equal lengths, mostly the same tiles) pass over their shared tiles
// close together and the XCD's L2 serves the repeats.
constexpr int kStartPolls = 4000;
struct UnitLoop {
  int xg, wgi, per_x, ngen;
  int64_t p0, p1;
  __device__ explicit UnitLoop(int64_t total) {
    xg = blockIdx.x & 7;
    wgi = blockIdx.x >> 3;
    per_x = gridDim.x >= 8 ? gridDim.x >> 3 : 1;  // (a per-unit launch may be smaller)
    p0 = xg * total / 8;
    p1 = (xg + 1) * total / 8;
    ngen = (int)((p1 - p0 + per_x - 1) / per_x);
  }
  // the unit (head * upH + index) of generation gen, or -1
  __device__ int64_t unit(const int32_t* order, int64_t upH, int gen) const {
    const int64_t p = p0 + (int64_t)gen * per_x + wgi;
    if (p >= p1) return -1;
    return (p / upH) * upH + order[p];
  }
  __device__ void start(int32_t* sync, int gen) const {
    if (threadIdx.x == 0) {
      int32_t* c = sync + xg * 16;
      __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int target = per_x * (gen + 1);
      for (int i = 0; i < kStartPolls &&
                      __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target;
           i++)
        __builtin_amdgcn_s_sleep(8);
    }
    __syncthreads();
  }
};

}  // namespace prism
