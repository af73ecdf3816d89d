// Plan stages of Prism's dynamic sparse attention on gfx950 (paper.rainbus.top,
// "方法步骤详情", stages one to three; formulas of xyznot.com/id, "Metode" 1-3):
// zone statistics, indicator / volume / shape, re-layout and pooling, block
// scores, Top-k U Top-p selection and the key-major transpose of the lists.
//
// Every quantity that decides a shape or a selected block is computed in fp32
// in one fixed order (compiled with -ffp-contract=off; fused multiply-add
// only where written as fmaf), so the plan is reproducible bit for bit.
#include "prism_attn_common.h"
#include "prism_kernels.h"
#include <vector>

namespace prism {

// ============================================================ K1: zone stats
// One wave per (head, zone).  Lane l owns channels [l*CPL, l*CPL + CPL).
// Token rows are read 64 lanes wide (one row per load instruction).

template <int DT, int CPL>
struct RowVal;  // one lane's CPL channels of one token row, kept packed

template <>
struct RowVal<1, 2> {  // bf16 x2
  uint32_t v;
  __device__ static RowVal load(const void* base, int64_t e) {
    RowVal r;
    r.v = __builtin_nontemporal_load((const uint32_t*)((const uint16_t*)base + e));
    return r;
  }
  __device__ float get(int k) const {
    return k ? __uint_as_float(v & 0xffff0000u) : __uint_as_float(v << 16);
  }
};
template <>
struct RowVal<1, 1> {
  uint32_t v;
  __device__ static RowVal load(const void* base, int64_t e) {
    RowVal r;
    r.v = ((const uint16_t*)base)[e];
    return r;
  }
  __device__ float get(int) const { return __uint_as_float(v << 16); }
};
template <>
struct RowVal<0, 1> {
  float v;
  __device__ static RowVal load(const void* base, int64_t e) {
    RowVal r;
    r.v = ((const float*)base)[e];
    return r;
  }
  __device__ float get(int) const { return v; }
};
template <>
struct RowVal<0, 2> {
  float2 v;
  __device__ static RowVal load(const void* base, int64_t e) {
    RowVal r;
    r.v = *(const float2*)((const float*)base + e);
    return r;
  }
  __device__ float get(int k) const { return k ? v.y : v.x; }
};

__device__ inline float var8(const float* p) {
  float mu = p[0];
#pragma unroll
  for (int i = 1; i < 8; i++) mu = mu + p[i];
  mu = mu * 0.125f;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    float d = p[i] - mu;
    acc = __builtin_fmaf(d, d, acc);
  }
  return acc * 0.125f;
}

// sum over the 64 lanes: for offsets 32..1 each lane adds the value of lane^offset
__device__ inline float lane_butterfly_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = x + __shfl_xor(x, off, 64);
  return x;
}

template <int DT, int CPL>
__global__ __launch_bounds__(64) void k_zone_stats(const void* __restrict__ v, int H, int W,
                                                   int Z, int64_t N, float* __restrict__ out) {
  constexpr int D = 64 * CPL;
  const int lane = threadIdx.x;
  const int hm = blockIdx.x;
  const int h = hm / Z, m = hm - h * Z;
  const int zH = H >> 3, zW = W >> 3;
  const int mt = m / (zH * zW), rem = m - mt * (zH * zW);
  const int mh = rem / zW, mw = rem - mh * zW;
  const int64_t base = (int64_t)h * N * D + (int64_t)lane * CPL;

  // per-frame profile means and frame-difference means, one slot per lane
  __shared__ float sPT[8][CPL][64], sDM[7][CPL][64];
  RowVal<DT, CPL> cur[64], nxt[64];
  float PH[8][CPL], PW[8][CPL], sv[CPL], within[CPL];

  // bf16 with 128 channels: a frame's 64 token rows (256 B each) travel
  // HBM -> LDS as 16 direct loads of 1 KB (16 B per lane, four rows per
  // load), two frames in flight; each lane then reads its two channels of
  // every row back from LDS.  Other layouts load each row straight into
  // registers, 4 or 8 B per lane.
  constexpr bool kDma = DT == 1 && CPL == 2;
  __shared__ __attribute__((aligned(16))) uint32_t sbuf[kDma ? 2 : 1][64][64];
  const __amdgpu_buffer_rsrc_t rsv =
      buffer_of((const uint16_t*)v + (int64_t)h * N * D, (uint32_t)(N * D * 2));
  const uint32_t lbuf = lds_offset(sbuf);
  auto row_of = [&](int t, int r) {  // token of row r (y = r / 8, w = r % 8) of frame t
    return ((int64_t)((mt << 3) + t) * H + ((mh << 3) + (r >> 3))) * W + (mw << 3) + (r & 7);
  };
  auto stage = [&](int t) {  // frame t into buffer t % 2
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int r = 4 * i + (lane >> 4);
      dma16(rsv, (uint32_t)(row_of(t, r) * D * 2 + (lane & 15) * 16),
            lbuf + (uint32_t)((t & 1) * 16384 + i * 1024));
    }
  };
  auto read_slice = [&](int t, RowVal<DT, CPL>* dst) {
    if constexpr (kDma) {
#pragma unroll
      for (int r = 0; r < 64; r++) dst[r].v = sbuf[t & 1][r][lane];
    }
  };

  auto load_slice = [&](int t, RowVal<DT, CPL>* dst) {
#pragma unroll
    for (int y = 0; y < 8; y++) {
      int64_t n0 = ((int64_t)((mt << 3) + t) * H + ((mh << 3) + y)) * W + (mw << 3);
#pragma unroll
      for (int w = 0; w < 8; w++) dst[y * 8 + w] = RowVal<DT, CPL>::load(v, base + (n0 + w) * D);
    }
  };

  if constexpr (kDma) {
    stage(0);
    stage(1);
    __builtin_amdgcn_s_waitcnt(wait_vm(16));
    asm volatile("" ::: "memory");
    read_slice(0, cur);
  } else {
    load_slice(0, cur);
  }
#pragma unroll 1
  for (int t = 0; t < 8; t++) {
    const bool more = t < 7;
    if constexpr (kDma) {
      // frame t's buffer is free once its reads have landed: it takes frame t + 2
      if (t + 2 < 8) {
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        asm volatile("" ::: "memory");
        stage(t + 2);
      }
    } else {
      if (more) load_slice(t + 1, nxt);
    }
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      float Lw[8], Cy[8];
#pragma unroll
      for (int y = 0; y < 8; y++) {
        float a = cur[y * 8].get(k);
#pragma unroll
        for (int w = 1; w < 8; w++) a = a + cur[y * 8 + w].get(k);
        Lw[y] = a;
      }
#pragma unroll
      for (int w = 0; w < 8; w++) {
        float a = cur[w].get(k);
#pragma unroll
        for (int y = 1; y < 8; y++) a = a + cur[y * 8 + w].get(k);
        Cy[w] = a;
      }
      float ss = Lw[0];
#pragma unroll
      for (int y = 1; y < 8; y++) ss = ss + Lw[y];
      const float mref = ss * 0.015625f;
      sPT[t][k][lane] = mref;
#pragma unroll
      for (int y = 0; y < 8; y++) PH[y][k] = (t == 0) ? Lw[y] : PH[y][k] + Lw[y];
#pragma unroll
      for (int w = 0; w < 8; w++) PW[w][k] = (t == 0) ? Cy[w] : PW[w][k] + Cy[w];
      // spatial variance of frame t
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 64; i++) {
        float d = cur[i].get(k) - mref;
        acc = __builtin_fmaf(d, d, acc);
      }
      float vt = acc * 0.015625f;
      sv[k] = (t == 0) ? vt : sv[k] + vt;
      // frame difference t -> t+1
      if (more) {
        if constexpr (kDma) {
          if (k == 0) {
            // frame t + 1 has landed (frame t + 2 may still be in flight)
            if (t + 2 < 8)
              __builtin_amdgcn_s_waitcnt(wait_vm(16));
            else
              __builtin_amdgcn_s_waitcnt(wait_vm(0));
            asm volatile("" ::: "memory");
            read_slice(t + 1, nxt);
          }
        }
        float s = nxt[0].get(k) - cur[0].get(k);
#pragma unroll
        for (int i = 1; i < 64; i++) s = s + (nxt[i].get(k) - cur[i].get(k));
        float dmt = s * 0.015625f;
        sDM[t][k][lane] = dmt;
        float a2 = 0.0f;
#pragma unroll
        for (int i = 0; i < 64; i++) {
          float e = (nxt[i].get(k) - cur[i].get(k)) - dmt;
          a2 = __builtin_fmaf(e, e, a2);
        }
        float dv = a2 * 0.015625f;
        within[k] = (t == 0) ? dv : within[k] + dv;
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 64; i++) cur[i] = nxt[i];
    }
  }
  float PT[8][CPL], dm[7][CPL];
#pragma unroll
  for (int k = 0; k < CPL; k++) {
#pragma unroll
    for (int t = 0; t < 8; t++) PT[t][k] = sPT[t][k][lane];
#pragma unroll
    for (int t = 0; t < 7; t++) dm[t][k] = sDM[t][k][lane];
  }

  float st[5][CPL];
#pragma unroll
  for (int k = 0; k < CPL; k++) {
    float ph[8], pw[8], pt[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      pt[i] = PT[i][k];
      ph[i] = PH[i][k] * 0.015625f;
      pw[i] = PW[i][k] * 0.015625f;
    }
    st[0][k] = var8(pt);
    st[1][k] = var8(ph);
    st[2][k] = var8(pw);
    st[3][k] = sv[k] * 0.125f;
    float wv = within[k] / 7.0f;
    float mu = dm[0][k];
#pragma unroll
    for (int i = 1; i < 7; i++) mu = mu + dm[i][k];
    mu = mu / 7.0f;
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 7; i++) {
      float e = dm[i][k] - mu;
      a = __builtin_fmaf(e, e, a);
    }
    st[4][k] = wv + a / 7.0f;
  }
  const float invD = 1.0f / (float)D;
#pragma unroll
  for (int s = 0; s < 5; s++) {
    float x = st[s][0];
#pragma unroll
    for (int k = 1; k < CPL; k++) x = x + st[s][k];
    x = lane_butterfly_sum(x);
    if (lane == 0) out[(int64_t)hm * 5 + s] = x * invD;
  }
}

// ============================================================ K1b: audio stats
// One thread per zone over the [N] float32 map: axis-profile variances and the
// zone mean, with the same fixed order as the video statistics (D = 1).
__global__ __launch_bounds__(64) void k_audio_stats(const float* __restrict__ a, int H, int W,
                                                    int Z, float* __restrict__ out) {
  int m = blockIdx.x * 64 + threadIdx.x;
  if (m >= Z) return;
  const int zH = H >> 3, zW = W >> 3;
  const int mt = m / (zH * zW), rem = m - mt * (zH * zW);
  const int mh = rem / zW, mw = rem - mh * zW;
  auto X = [&](int t, int y, int w) {
    return a[((int64_t)((mt << 3) + t) * H + ((mh << 3) + y)) * W + ((mw << 3) + w)];
  };
  float PT[8], PH[8], PW[8];
  for (int t = 0; t < 8; t++) {
    float ss = 0.0f;
    for (int y = 0; y < 8; y++) {
      float l = X(t, y, 0);
      for (int w = 1; w < 8; w++) l = l + X(t, y, w);
      ss = (y == 0) ? l : ss + l;
      PH[y] = (t == 0) ? l : PH[y] + l;
    }
    for (int w = 0; w < 8; w++) {
      float c = X(t, 0, w);
      for (int y = 1; y < 8; y++) c = c + X(t, y, w);
      PW[w] = (t == 0) ? c : PW[w] + c;
    }
    PT[t] = ss * 0.015625f;
  }
  for (int i = 0; i < 8; i++) {
    PH[i] = PH[i] * 0.015625f;
    PW[i] = PW[i] * 0.015625f;
  }
  float mu = PT[0];
  for (int i = 1; i < 8; i++) mu = mu + PT[i];
  out[m * 4 + 0] = var8(PT);
  out[m * 4 + 1] = var8(PH);
  out[m * 4 + 2] = var8(PW);
  out[m * 4 + 3] = mu * 0.125f;
}

// ============================================================ K2: shapes
__device__ inline void ratio3(const float* x, float* r) {
  float s = (x[0] + x[1]) + x[2];
  if (s > 0.0f) {
    r[0] = x[0] / s;
    r[1] = x[1] / s;
    r[2] = x[2] / s;
  } else {
    r[0] = r[1] = r[2] = 1.0f / 3.0f;
  }
}

// Candidate a strictly nearer than b to l*(g) in log2 space.  Since the
// coordinates of l* and of every candidate (log2 of its edges) sum to log2 B,
// |l* - e|^2 = const + sum e_d^2 + sum e_d log2 g_d; "a nearer" is therefore
// prod g_d^(ea_d - eb_d) < 2^(|eb|^2 - |ea|^2).  Each side is a product of at
// most two fp32 values times a power of two, exact in fp64.
__device__ inline bool shape_nearer(const float* g, int a, int b) {
  const Shape& A = d_shapes[a];
  const Shape& Bs = d_shapes[b];
  int ea[3] = {A.log2_bt, A.log2_bh, A.log2_bw};
  int eb[3] = {Bs.log2_bt, Bs.log2_bh, Bs.log2_bw};
  int qa = ea[0] * ea[0] + ea[1] * ea[1] + ea[2] * ea[2];
  int qb = eb[0] * eb[0] + eb[1] * eb[1] + eb[2] * eb[2];
  double lhs = 1.0, rhs = 1.0;
#pragma unroll
  for (int d = 0; d < 3; d++) {
    int k = ea[d] - eb[d];
    double gd = (double)g[d];
    if (k >= 1) lhs = lhs * gd;
    if (k >= 2) lhs = lhs * gd;
    if (k <= -1) rhs = rhs * gd;
    if (k <= -2) rhs = rhs * gd;
  }
  rhs = ldexp(rhs, qb - qa);
  return lhs < rhs;
}

__device__ inline int volume_tier(float rr, float rmax, float tau128, float tau256,
                                  uint32_t mask) {
  int B;
  if (!(rmax > 0.0f)) {
    B = 256;
  } else {
    float rho = rr / rmax;
    B = (rho >= tau128) ? 64 : (rho >= tau256) ? 128 : 256;
  }
  int bit = B == 64 ? 0 : B == 128 ? 1 : 2;
  if (mask & (1u << bit)) return B;
  for (int dist = 1; dist <= 2; dist++) {
    if (bit - dist >= 0 && (mask & (1u << (bit - dist)))) return 64 << (bit - dist);
    if (bit + dist <= 2 && (mask & (1u << (bit + dist)))) return 64 << (bit + dist);
  }
  return B;
}

__device__ inline float block_max(float v, float* sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); i++) r = fmaxf(r, sh[i]);
  return r;
}

// One block of 256 threads per head.
__global__ __launch_bounds__(256) void k_shapes(const float* __restrict__ vstats,
                                                const float* __restrict__ astats, int have_audio,
                                                int Z, float eps, float tau128, float tau256,
                                                uint32_t vmask, int fixed_id,
                                                uint8_t* __restrict__ shape_id,
                                                int32_t* __restrict__ zone_base,
                                                int32_t* __restrict__ nblk) {
  __shared__ float sh[8];
  __shared__ int scan[256];
  const int h = blockIdx.x;
  float am = 0.0f, rm = 0.0f;
  for (int m = threadIdx.x; m < Z; m += 256) {
    if (have_audio) am = fmaxf(am, astats[m * 4 + 3]);
    const float* s = vstats + ((int64_t)h * Z + m) * 5;
    rm = fmaxf(rm, s[3] + s[4]);
  }
  const float amax = block_max(am, sh);
  const float rmax = block_max(rm, sh);
  int carry = 0;
  for (int m0 = 0; m0 < Z; m0 += 256) {
    int m = m0 + threadIdx.x;
    int nb = 0;
    if (m < Z) {
      const float* s = vstats + ((int64_t)h * Z + m) * 5;
      int id, B;
      if (fixed_id >= 0) {
        id = fixed_id;
        B = d_shapes[id].volume;
      } else {
        float r[3], g[3];
        ratio3(s, r);
        if (have_audio && amax > 0.0f) {
          float abar = astats[m * 4 + 3] / amax;
          float va[3];
          ratio3(astats + m * 4, va);
#pragma unroll
          for (int d = 0; d < 3; d++) {
            float c = abar * va[d];
            g[d] = (r[d] + c) + eps;
          }
        } else {
#pragma unroll
          for (int d = 0; d < 3; d++) g[d] = r[d] + eps;
        }
        B = volume_tier(s[3] + s[4], rmax, tau128, tau256, vmask);
        int first = shape_first(B), cnt = shape_count(B);
        id = first;
        for (int c = first + 1; c < first + cnt; c++)
          if (shape_nearer(g, c, id)) id = c;
      }
      shape_id[(int64_t)h * Z + m] = (uint8_t)id;
      nb = 512 / B;
    }
    // exclusive block scan of nb
    scan[threadIdx.x] = nb;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      int v = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    if (m < Z) zone_base[(int64_t)h * Z + m] = carry + scan[threadIdx.x] - nb;
    carry += scan[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) nblk[h] = carry;
}

// ============================================================ K4: re-layout + pooling
// One block of 512 threads (8 waves) per (head, zone); wave w owns permuted
// rows [64w, 64w+64) of the zone.  K and V rows are copied to the permuted
// buffers; Q and K are summed per 64-row tile (rows in permuted order), then
// per block (tiles in order), scaled by 1/B and written with their integer
// grid: q_c = rint(x_c 2^-E), E = exponent(max_c |x_c|) - 8.
template <int DT, int CPL, bool SWZ>
__global__ __launch_bounds__(512) void k_permute_pool(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v, int H,
    int W, int Z, int64_t N, const uint8_t* __restrict__ shape_id,
    const int32_t* __restrict__ zone_base, const int64_t* __restrict__ blk_off,
    void* __restrict__ kp, void* __restrict__ vp, int32_t* __restrict__ blk_start,
    uint8_t* __restrict__ blk_shape, int32_t* __restrict__ blk_head, float* __restrict__ qbar,
    float* __restrict__ kbar, uint16_t* __restrict__ qgrid, uint16_t* __restrict__ kgrid,
    int32_t* __restrict__ qexp, int32_t* __restrict__ kexp) {
  constexpr int D = 64 * CPL;
  constexpr int ES = DT == 1 ? 2 : 4;  // element size
  __shared__ float tsum[2][8][D];
  const int hm = blockIdx.x;
  const int h = hm / Z, m = hm - h * Z;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sid = shape_id[hm];
  const Shape sh = d_shapes[sid];
  const int B = sh.volume;
  const int64_t hb = (int64_t)h * N;
  float aq[CPL], ak[CPL];
  for (int i = 0; i < 64; i++) {
    const int r = wv * 64 + i;
    const int64_t n = token_of(sh, m, r, H, W);
    const int64_t src = (hb + n) * D + lane * CPL;
    RowVal<DT, CPL> rq = RowVal<DT, CPL>::load(q, src);
    RowVal<DT, CPL> rk = RowVal<DT, CPL>::load(k, src);
    RowVal<DT, CPL> rv = RowVal<DT, CPL>::load(v, src);
#pragma unroll
    for (int c = 0; c < CPL; c++) {
      aq[c] = (i == 0) ? rq.get(c) : aq[c] + rq.get(c);
      ak[c] = (i == 0) ? rk.get(c) : ak[c] + rk.get(c);
    }
    const int64_t p = (int64_t)m * 512 + r;  // permuted row within the head
    int64_t dst_byte;
    if (SWZ) {  // bf16, D = 128: 4 bytes per lane inside chunk lane/4
      int rho = (int)(p & 63);
      int chunk = (lane >> 2) ^ chunk_swizzle(rho);
      dst_byte = ((hb + p) * D) * 2 + chunk * 16 + (lane & 3) * 4;
    } else {
      dst_byte = ((hb + p) * D + lane * CPL) * ES;
    }
    constexpr int VB = CPL * ES;  // bytes per lane
    if (VB == 4) {
      *(uint32_t*)((char*)kp + dst_byte) = *(const uint32_t*)((const char*)k + src * ES);
      *(uint32_t*)((char*)vp + dst_byte) = *(const uint32_t*)((const char*)v + src * ES);
    } else if (VB == 2) {
      *(uint16_t*)((char*)kp + dst_byte) = *(const uint16_t*)((const char*)k + src * ES);
      *(uint16_t*)((char*)vp + dst_byte) = *(const uint16_t*)((const char*)v + src * ES);
    } else {
      *(uint2*)((char*)kp + dst_byte) = *(const uint2*)((const char*)k + src * ES);
      *(uint2*)((char*)vp + dst_byte) = *(const uint2*)((const char*)v + src * ES);
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; c++) {
    tsum[0][wv][lane * CPL + c] = aq[c];
    tsum[1][wv][lane * CPL + c] = ak[c];
  }
  __syncthreads();
  const int nb = 512 / B;
  if (wv < nb) {
    const int tpb = B / 64;
    const int64_t g = blk_off[h] + zone_base[hm] + wv;
    if (lane == 0) {
      blk_start[g] = m * 512 + wv * B;
      blk_shape[g] = (uint8_t)sid;
      blk_head[g] = h;
    }
    const float invB = 1.0f / (float)B;
#pragma unroll
    for (int which = 0; which < 2; which++) {
      float x[CPL];
      float mx = 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; c++) {
        float s = tsum[which][wv * tpb][lane * CPL + c];
        for (int t = 1; t < tpb; t++) s = s + tsum[which][wv * tpb + t][lane * CPL + c];
        x[c] = s * invB;
        mx = fmaxf(mx, fabsf(x[c]));
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      int e = 0;
      if (mx > 0.0f) {
        frexpf(mx, &e);
        e -= 8;
      }
      float* xb = which ? kbar : qbar;
      uint16_t* gr = which ? kgrid : qgrid;
#pragma unroll
      for (int c = 0; c < CPL; c++) {
        xb[g * D + lane * CPL + c] = x[c];
        float qv = mx > 0.0f ? rintf(ldexpf(x[c], -e)) : 0.0f;
        gr[g * D + lane * CPL + c] = (uint16_t)(__float_as_uint(qv) >> 16);  // exact: |qv| <= 256
      }
      if (lane == 0) (which ? kexp : qexp)[g] = e;
    }
  }
}

// ============================================================ K5: block scores
// s_ij = ldexp(I_ij, Ei + Ej) * fl(1/sqrt D), I_ij = integer dot product of the
// grid rows, exact in fp32 on the bf16 MFMA (|I| <= 2^23).
// Block of 256 threads covers 128 x 128 scores; each wave 64 x 64.
template <int D>
__global__ __launch_bounds__(256) void k_block_scores(const uint16_t* __restrict__ qgrid,
                                                      const uint16_t* __restrict__ kgrid,
                                                      const int32_t* __restrict__ qexp,
                                                      const int32_t* __restrict__ kexp,
                                                      int64_t g0, int n, float cD,
                                                      float* __restrict__ scores) {
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i0 = blockIdx.y * 128 + (wv >> 1) * 64;
  const int j0 = blockIdx.x * 128 + (wv & 1) * 64;
  const int hl = lane >> 5, l32 = lane & 31;
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[a][b][r] = 0.0f;
#pragma unroll
  for (int kk = 0; kk < D / 16; kk++) {
    bf16x8 af[2], bfr[2];
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
      int i = i0 + rb * 32 + l32;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (i < n) u = *(const uint4*)(qgrid + (g0 + i) * D + kk * 16 + hl * 8);
      af[rb] = __builtin_bit_cast(bf16x8, u);
      int j = j0 + rb * 32 + l32;
      uint4 w = make_uint4(0, 0, 0, 0);
      if (j < n) w = *(const uint4*)(kgrid + (g0 + j) * D + kk * 16 + hl * 8);
      bfr[rb] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 2; b++)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
  }
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int b = 0; b < 2; b++) {
      int j = j0 + b * 32 + l32;
      if (j >= n) continue;
      int ej = kexp[g0 + j];
#pragma unroll
      for (int r = 0; r < 16; r++) {
        int i = i0 + a * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
        if (i < n) {
          float s = ldexpf(acc[a][b][r], qexp[g0 + i] + ej) * cD;
          scores[(int64_t)i * n + j] = (s == 0.0f) ? 0.0f : s;
        }
      }
    }
}

// ============================================================ K6: selection
// Order-preserving map of fp32 to uint32 (larger float -> larger key).
__device__ inline uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key2f(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// 2^x for x <= 0: x = k + f with k = rint(x), |f| <= 1/2, 2^f from its
// degree-7 Taylor series in f ln 2 (Horner, fused multiply-add); the
// coefficients are (ln 2)^n / n! rounded to fp32.
__device__ inline float exp2_taylor(float x) {
  if (!(x > -100.0f)) return 0.0f;
  float kf = rintf(x);
  float f = x - kf;
  float p = 0.000015252733804059840280f;
  p = __builtin_fmaf(p, f, 0.00015403530393381609954f);
  p = __builtin_fmaf(p, f, 0.0013333558146428443423f);
  p = __builtin_fmaf(p, f, 0.0096181291076284771620f);
  p = __builtin_fmaf(p, f, 0.055504108664821579953f);
  p = __builtin_fmaf(p, f, 0.24022650695910071233f);
  p = __builtin_fmaf(p, f, 0.69314718055994530942f);
  p = __builtin_fmaf(p, f, 1.0f);
  return ldexpf(p, (int)kf);
}

// softmax weight of a score in 2^-32 units relative to the row maximum
__device__ inline uint64_t weight_of(float s, float smax) {
  const float LOG2E = 1.44269504088896340736f;
  float x = (s - smax) * LOG2E;
  float y = exp2_taylor(x);
  return (uint64_t)(y * 4294967296.0f);
}

__device__ inline int bucket_of(float s, float smax) {
  const float LOG2E = 1.44269504088896340736f;
  float x = (s - smax) * LOG2E;  // same rounding as weight_of: monotone in s
  float b = -x * 8.0f;
  return b >= 255.0f ? 255 : (int)b;
}

template <typename T>
__device__ inline T block_sum(T v, T* sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  T r = sh[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); i++) r += sh[i];
  __syncthreads();
  return r;
}

constexpr int kSelThreads = 256;
// longest score row (key blocks of a head) the selection kernels stage in LDS
constexpr int kSelLdsMax = 16384;
// floats of LDS a staged row takes (rounded up to whole 64-lane pieces)
__host__ __device__ inline int sel_row_floats(int n) { return (n + 63) / 64 * 64; }
// block volume of a shape id (ids are ordered by volume: 0..6 are 64,
// 7..12 are 128, 13..15 are 256)
__device__ inline int volume_of_id(int sid) { return sid < 7 ? 64 : sid < 13 ? 128 : 256; }

// One score row (n <= kSelLdsMax floats) into LDS: every wave issues its
// 256-byte pieces as direct HBM->LDS loads, all in flight at once, then one
// wait and a barrier.  Lanes past n read zeros (range-checked buffer) into
// the unused tail of `dst`.
__device__ inline void stage_row(const float* row, int n, float* dst) {
  const __amdgpu_buffer_rsrc_t rs = buffer_of(row, (uint32_t)n * 4u);
  const uint32_t o = lds_offset(dst);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  for (int j0 = wv * 64; j0 < n; j0 += kSelThreads)
    dma4(rs, (uint32_t)(j0 + lane) * 4u, o + (uint32_t)j0 * 4u);
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  __syncthreads();
}

// Shared state of the row selection: per-wave digit histograms (count and
// integer weight) of one radix level, and the scan scratch.
struct SelShared {
  uint32_t cnt[kSelThreads / 64][256];
  unsigned long long wt[kSelThreads / 64][256];
  unsigned long long red64[kSelThreads / 64];
  unsigned long long wstar;
  float redf[kSelThreads / 64], redn[kSelThreads / 64];
  int pick;
};

// inclusive scan over the block (kSelThreads threads) of one u64 per thread
__device__ inline unsigned long long block_incl_scan(unsigned long long v,
                                                     unsigned long long* sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    unsigned long long u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) sh[wv] = v;
  __syncthreads();
  unsigned long long before = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; w++) before += w < wv ? sh[w] : 0ull;
  __syncthreads();
  return before + v;
}

// Sources of a row's scores for the selection passes: src.each(f) calls f
// on every score of this thread's share of the row (elements tid + 256 e).
// LdsRow reads a row staged in LDS eight elements at a time, all eight reads
// in flight before any is used (one at a time, every element paid the LDS
// latency); GlobalRow reads a row of any length from HBM on every pass.
struct LdsRow {
  const float* row;
  int n;
  template <class F>
  __device__ void each(F f) const {
    constexpr int kBatch = 8;
    for (int j0 = threadIdx.x; j0 < n; j0 += kBatch * kSelThreads) {
      float v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; k++) {
        const int j = j0 + k * kSelThreads;
        v[k] = row[j < n ? j : j0];
      }
#pragma unroll
      for (int k = 0; k < kBatch; k++)
        if (j0 + k * kSelThreads < n) f(v[k]);
    }
  }
};
struct GlobalRow {
  const float* row;
  int n;
  template <class F>
  __device__ void each(F f) const {
    for (int j = threadIdx.x; j < n; j += kSelThreads) f(row[j]);
  }
};

// One level of the selection: `cls(s)` gives an element's digit (0..255,
// larger digits earlier in the selection order) or -1 when the element is
// not a candidate of this level.  Builds the digit histogram (counts, and
// integer weights when `by_weight`), then walks the digits from the largest
// down and returns the digit at which the running total (weight, else
// count) first reaches `need`; *above_c / *above_w get the count and weight
// of the candidates with a larger digit.  The row is visited through `src`
// (LdsRow or GlobalRow).
template <class Src, class Cls>
__device__ int select_level(const Src& src, Cls cls, float smax, bool by_weight,
                            unsigned long long need, SelShared& S, uint32_t* above_c,
                            unsigned long long* above_w, unsigned long long p32 = 0) {
  const int wv = threadIdx.x >> 6;
  for (int b = threadIdx.x; b < (kSelThreads / 64) * 256; b += blockDim.x) {
    (&S.cnt[0][0])[b] = 0;
    (&S.wt[0][0])[b] = 0ull;
  }
  __syncthreads();
  src.each([&](float s) {
    const int d = cls(s);
    if (d >= 0) {
      atomicAdd(&S.cnt[wv][d], 1u);
      if (by_weight) atomicAdd(&S.wt[wv][d], (unsigned long long)weight_of(s, smax));
    }
  });
  __syncthreads();
  // one wave picks the digit: lane l owns digits 255 - 4l - q (q = 0..3,
  // selection order), one wave scan of its count and weight totals gives
  // every digit's running totals
  if (wv == 0) {
    const int lane = threadIdx.x & 63;
    unsigned long long c[4], w[4], sc = 0, sw = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int d = 255 - 4 * lane - q;
      c[q] = 0;
      w[q] = 0;
#pragma unroll
      for (int k = 0; k < kSelThreads / 64; k++) {
        c[q] += S.cnt[k][d];
        w[q] += S.wt[k][d];
      }
      sc += c[q];
      sw += w[q];
    }
    unsigned long long ic = sc, iw = sw;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned long long uc = __shfl_up(ic, off, 64), uw = __shfl_up(iw, off, 64);
      if (lane >= off) {
        ic += uc;
        iw += uw;
      }
    }
    if (p32) {
      // first level of the Top-p select: the histogram total is the row's
      // weight Z, and the target W* = ceil(p32 Z / 2^32) (no overflow: p32 <= 2^32)
      const unsigned long long Z = __shfl(iw, 63, 64);
      const unsigned long long zh = Z >> 32, zl = Z & 0xffffffffull;
      need = p32 * zh + ((p32 * zl + 0xffffffffull) >> 32);
      if (lane == 0) S.wstar = need;
    }
    // running totals before this lane's first digit; the crossing digit is
    // the first whose running total reaches `need` (if none does, digit 0)
    unsigned long long rc = ic - sc, rw = iw - sw;
    int pick = -1;
    unsigned long long pc = 0, pw = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const unsigned long long before = by_weight ? rw : rc;
      const unsigned long long m = by_weight ? w[q] : c[q];
      if (pick < 0 && before < need && before + m >= need) {
        pick = 255 - 4 * lane - q;
        pc = rc;
        pw = rw;
      }
      rc += c[q];
      rw += w[q];
    }
    const bool found = __ballot(pick >= 0) != 0ull;
    if (lane == 63 && !found) {
      pick = 0;
      pc = rc - c[3];
      pw = rw - w[3];
    }
    if (pick >= 0) {
      S.pick = pick;
      S.red64[0] = pc;
      S.red64[1] = pw;
    }
  }
  __syncthreads();
  const int d = S.pick;
  *above_c = (uint32_t)S.red64[0];
  *above_w = by_weight ? S.red64[1] : 0ull;
  __syncthreads();
  return d;
}

// Exact select: the order key K of the element at which the running total in
// selection order (score descending) first reaches `need`, with the count
// and weight of the elements whose key is larger.  The levels take the
// order keys relative to the row's smallest key, 8 bits at a time from the
// top of the row's key range (rel = key - kmin orders the elements like the
// keys; a row's scores lie in a narrow range, so the top bytes of the raw
// keys would be one or two values, every level's histogram one or two bins,
// and its LDS atomics would serialise).  With p32 != 0 the target is the
// Top-p weight W* of the row, formed from the first level's total; it is
// returned in *need_out.
template <class Src>
__device__ uint32_t exact_select(const Src& src, float smax, float smin, bool by_weight,
                                 unsigned long long need, SelShared& S, uint32_t* above_c,
                                 unsigned long long* above_w, unsigned long long p32 = 0,
                                 unsigned long long* need_out = nullptr) {
  const uint32_t kmin = f2key(smin);
  const uint32_t span = f2key(smax) - kmin;
  uint32_t prefix = 0, ac = 0;
  unsigned long long aw = 0;
  bool first = true;
  // (a row of equal keys still takes one level, which forms W*)
  for (int hi = span ? 32 - __builtin_clz(span) : 1; hi > 0;) {
    const int lo = hi > 8 ? hi - 8 : 0;
    const uint64_t pre = (uint64_t)prefix >> hi;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    uint32_t c;
    unsigned long long w;
    const unsigned long long rest = need - (by_weight ? aw : (unsigned long long)ac);
    const int d = select_level(
        src,
        [&](float s) {
          const uint32_t rel = f2key(s) - kmin;
          return ((uint64_t)rel >> hi) == pre ? (int)((rel >> lo) & dmask) : -1;
        },
        smax, by_weight, rest, S, &c, &w, first ? p32 : 0ull);
    if (first && p32) need = S.wstar;
    first = false;
    prefix |= (uint32_t)d << lo;
    ac += c;
    aw += w;
    hi = lo;
  }
  if (need_out) *need_out = need;
  *above_c = ac;
  *above_w = aw;
  return kmin + prefix;
}

// Per query block row: count of selected key blocks, the threshold key and
// the number of threshold-key ties to take.  S_i = first max(k, L*) keys in
// the order (score desc, index asc), L* = shortest prefix whose integer
// softmax weights reach ceil(p 2^32) Z / 2^32 (Z = row total).  Both
// positions are found exactly by radix selects over the order keys (equal
// keys carry equal weights, so a prefix of the order is "every key above K
// and the first t copies of K").
template <bool kLds>
__global__ __launch_bounds__(kSelThreads) void k_select_count(
    const float* __restrict__ scores, int n, int64_t g0, int k_count, float k_frac, float p,
    int32_t* __restrict__ row_cnt, uint32_t* __restrict__ row_key,
    int32_t* __restrict__ row_tie) {
  __shared__ SelShared S;
  const int i = blockIdx.x;
  const int64_t g = g0 + i;
  int64_t kk = k_count;
  if (k_frac > 0.0f) kk = (int64_t)ceil((double)k_frac * (double)n);
  if (kk > n) kk = n;
  if (kk < 0) kk = 0;
  if (p >= 1.0f) {  // every block
    if (threadIdx.x == 0) {
      row_cnt[g] = n;
      row_key[g] = 0u;
      row_tie[g] = 0;
    }
    return;
  }
  // the row is read from HBM once: into LDS (n floats of dynamic shared
  // memory) when it fits, and every later pass runs over that copy; longer
  // rows are read from HBM on every pass
  const float* grow = scores + (int64_t)i * n;
  extern __shared__ __attribute__((aligned(16))) float srow_dyn[];
  if (kLds) stage_row(grow, n, srow_dyn);
  const LdsRow rr{srow_dyn, n};
  const GlobalRow gr{grow, n};
  // the row's maximum and minimum
  float mx = -INFINITY, mn = INFINITY;
  auto minmax = [&](float s) {
    mx = fmaxf(mx, s);
    mn = fminf(mn, s);
  };
  if (kLds)
    rr.each(minmax);
  else
    gr.each(minmax);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    mn = fminf(mn, __shfl_xor(mn, off, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    S.redf[threadIdx.x >> 6] = mx;
    S.redn[threadIdx.x >> 6] = mn;
  }
  __syncthreads();
  float smax = S.redf[0], smin = S.redn[0];
  for (int w = 1; w < kSelThreads / 64; w++) {
    smax = fmaxf(smax, S.redf[w]);
    smin = fminf(smin, S.redn[w]);
  }
  __syncthreads();
  auto select = [&](bool by_weight, unsigned long long need, uint32_t* ac,
                    unsigned long long* aw, unsigned long long p32,
                    unsigned long long* need_out) {
    return kLds ? exact_select(rr, smax, smin, by_weight, need, S, ac, aw, p32, need_out)
                : exact_select(gr, smax, smin, by_weight, need, S, ac, aw, p32, need_out);
  };

  int64_t L = 0;
  uint32_t keyP = 0, caP = 0;
  if (p > 0.0f) {
    // W* = ceil(ceil(p 2^32) Z / 2^32) with Z the row's total weight
    const unsigned long long P32 = (unsigned long long)ceil((double)p * 4294967296.0);
    unsigned long long wa, Wstar;
    keyP = select(true, 0ull, &caP, &wa, P32, &Wstar);
    const unsigned long long wk = weight_of(key2f(keyP), smax);
    L = (int64_t)caP + (int64_t)((Wstar - wa + wk - 1) / wk);
  }
  int64_t nsel = kk > L ? kk : L;
  if (nsel > n) nsel = n;
  uint32_t keyL = 0xffffffffu;
  int64_t tieL = 0;
  if (nsel > 0 && nsel == L) {
    // the L*-th element of the order carries the crossing key itself
    keyL = keyP;
    tieL = L - (int64_t)caP;
  } else if (nsel > 0) {
    uint32_t ca;
    unsigned long long wa;
    keyL = select(false, (unsigned long long)nsel, &ca, &wa, 0ull, nullptr);
    tieL = nsel - (int64_t)ca;
  }
  if (threadIdx.x == 0) {
    row_cnt[g] = (int32_t)nsel;
    row_key[g] = keyL;
    row_tie[g] = (int32_t)tieL;
  }
}

// Exclusive scan of a head's row counts into row_ptr (base = running total in
// counters[0]); one block of 1024 threads.
__global__ __launch_bounds__(1024) void k_scan_rows(const int32_t* __restrict__ cnt, int n,
                                                    int64_t g0, int64_t* __restrict__ ptr,
                                                    int64_t* __restrict__ counters,
                                                    int last) {
  __shared__ int64_t sh[1024];
  int64_t carry = counters[0];
  for (int i0 = 0; i0 < n; i0 += 1024) {
    int i = i0 + threadIdx.x;
    int64_t v = i < n ? cnt[g0 + i] : 0;
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int64_t a = threadIdx.x >= off ? sh[threadIdx.x - off] : 0;
      __syncthreads();
      sh[threadIdx.x] += a;
      __syncthreads();
    }
    if (i < n) ptr[g0 + i] = carry + sh[threadIdx.x] - v;
    carry += sh[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    counters[0] = carry;
    if (last) ptr[g0 + n] = carry;
  }
}

// Emit each row's selected key blocks in ascending index order; also the
// row's attention cost B_i * sum_j B_j.
// exclusive prefix over the block of one int per thread (kSelThreads threads)
__device__ inline int block_excl_scan_i32(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(x, off, 64);
    if (lane >= off) x += u;
  }
  if (lane == 63) sh[wv] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; w++) {
    before += w < wv ? sh[w] : 0;
    tot += sh[w];
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Writes the selected key blocks of each row in ascending order, given the
// threshold key K and the number of K-ties to take.  Thread t takes the
// contiguous segment [tC, tC + C) of the row (C <= 64, in registers): one
// prefix over the ties and one over the selected counts place every thread's
// output.  With the row staged in LDS, the output is compacted into that
// same buffer and stored contiguously.
template <bool kLds>
__global__ __launch_bounds__(kSelThreads) void k_select_fill(
    const float* __restrict__ scores, int n, int64_t g0, const int32_t* __restrict__ row_cnt,
    const uint32_t* __restrict__ row_key, const int32_t* __restrict__ row_tie,
    const int64_t* __restrict__ row_ptr, int64_t cap, const uint8_t* __restrict__ blk_shape,
    int32_t* __restrict__ col_idx, int64_t* __restrict__ row_cost) {
  extern __shared__ __attribute__((aligned(16))) float srow_dyn[];
  __shared__ int sh[kSelThreads / 64];
  __shared__ int64_t sh_cost[kSelThreads / 64];
  const int i = blockIdx.x;
  const int64_t g = g0 + i;
  const float* grow = scores + (int64_t)i * n;
  // the head's shape ids (key blocks g0 .. g0 + n - 1) follow the row in
  // LDS: the aligned words that cover them, moved in the same wait
  const uint8_t* sshape = nullptr;
  if (kLds) {
    const int64_t w0 = g0 >> 2;
    const int nw = (int)(((g0 + n + 3) >> 2) - w0);
    uint32_t* dst = (uint32_t*)(srow_dyn + sel_row_floats(n));
    const __amdgpu_buffer_rsrc_t rs = buffer_of(blk_shape + w0 * 4, (uint32_t)nw * 4u);
    const uint32_t o = lds_offset(dst);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    for (int j0 = wv * 64; j0 < nw; j0 += kSelThreads)
      dma4(rs, (uint32_t)(j0 + lane) * 4u, o + (uint32_t)j0 * 4u);
    sshape = (const uint8_t*)dst + (g0 & 3);
    stage_row(grow, n, srow_dyn);
  }
  const float* row = kLds ? (const float*)srow_dyn : grow;
  const uint32_t K = row_key[g];
  const int tie = row_tie[g];
  const int64_t base = row_ptr[g];
  const bool fits = base + row_cnt[g] <= cap;
  const int C = (n + kSelThreads - 1) / kSelThreads;  // <= 64 on the LDS path
  const int j0 = min(n, (int)threadIdx.x * C), j1 = min(n, j0 + C);
  int total = 0;
  int64_t cost = 0;
  if (kLds) {
    uint32_t key[kSelLdsMax / kSelThreads];
    int ties = 0;
#pragma unroll
    for (int e = 0; e < kSelLdsMax / kSelThreads; e++) {
      key[e] = j0 + e < j1 ? f2key(row[j0 + e]) : 0u;
      ties += (j0 + e < j1 && key[e] == K) ? 1 : 0;
    }
    int unused;
    const int tie0 = block_excl_scan_i32(ties, sh, &unused);
    int nsel = 0;
    uint64_t selm = 0;  // bit e: element j0 + e selected
#pragma unroll
    for (int e = 0, t = tie0; e < kSelLdsMax / kSelThreads; e++) {
      const bool in = j0 + e < j1;
      const bool sel = in && (key[e] > K || (key[e] == K && t < tie));
      t += (in && key[e] == K) ? 1 : 0;
      if (sel) {
        nsel++;
        selm |= 1ull << e;
        cost += volume_of_id(sshape[j0 + e]);
      }
    }
    int pos = block_excl_scan_i32(nsel, sh, &total);
    // every thread holds its keys in registers: the row buffer takes the output
    int32_t* sout = (int32_t*)srow_dyn;
    while (selm) {
      const int e = __builtin_ctzll(selm);
      selm &= selm - 1;
      sout[pos++] = j0 + e;
    }
    __syncthreads();
    if (fits)
      for (int e = threadIdx.x; e < total; e += blockDim.x) col_idx[base + e] = sout[e];
  } else {
    int ties = 0;
    for (int j = j0; j < j1; j++) ties += f2key(row[j]) == K;
    int unused;
    const int tie0 = block_excl_scan_i32(ties, sh, &unused);
    int nsel = 0;
    for (int j = j0, t = tie0; j < j1; j++) {
      const uint32_t key = f2key(row[j]);
      const bool sel = key > K || (key == K && t < tie);
      t += key == K;
      if (sel) {
        nsel++;
        cost += volume_of_id(block_shape_at(blk_shape, g0 + j));
      }
    }
    int pos = block_excl_scan_i32(nsel, sh, &total);
    for (int j = j0, t = tie0; j < j1; j++) {
      const uint32_t key = f2key(row[j]);
      const bool sel = key > K || (key == K && t < tie);
      t += key == K;
      if (sel && fits) col_idx[base + pos] = j;
      pos += sel;
    }
  }
  const int64_t c = block_sum<int64_t>(cost, sh_cost);
  if (threadIdx.x == 0) row_cost[g] = c * (int64_t)d_shapes[block_shape_at(blk_shape, g)].volume;
}

// Key-major transpose of one head's lists, by tiles of 64 query rows x 256
// key columns.  A work-group takes 64 rows and a part of kTrPart columns:
// each row's start in that part is found by one binary search, then every
// 256-column tile is built as one 64-bit row mask per column (one wave per
// row walks the row's sorted list with coalesced reads; LDS atomic ORs set
// the bits).  The counting pass stores popcounts per (row tile, column); the
// fill pass rebuilds the masks and writes each column's rows in ascending
// order at its offset, one column per store instruction of a wave.  No global atomics, and the result does not depend on
// the order of the ORs.
constexpr int kTrRows = 64;
constexpr int kTrCols = 256;
constexpr int kTrPart = 2048;

template <bool kFill>
__global__ __launch_bounds__(kTrCols) void k_colt_tiles(
    const int64_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int n, int64_t g0,
    const int64_t* __restrict__ colt_ptr, int32_t* __restrict__ tile_cnt,
    int32_t* __restrict__ colt_idx) {
  __shared__ int64_t cur[kTrRows], fin[kTrRows];
  __shared__ unsigned long long mask[kTrCols];
  __shared__ int64_t cpos[kTrCols];
  const int rt = blockIdx.x;
  const int i0 = rt * kTrRows, nrows = min(kTrRows, n - i0);
  const int c0 = blockIdx.y * kTrPart, c1 = min(n, c0 + kTrPart);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (threadIdx.x < kTrRows && (int)threadIdx.x < nrows) {
    // first entry of the row at or after column c0
    const int r = threadIdx.x;
    int64_t lo = row_ptr[g0 + i0 + r], hi = row_ptr[g0 + i0 + r + 1];
    fin[r] = hi;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (col_idx[mid] < c0)
        lo = mid + 1;
      else
        hi = mid;
    }
    cur[r] = lo;
  }
  __syncthreads();
  for (int t0 = c0; t0 < c1; t0 += kTrCols) {
    const int t1 = min(c1, t0 + kTrCols);
    mask[threadIdx.x] = 0ull;
    __syncthreads();
    for (int r = wv; r < nrows; r += kTrCols / 64) {
      int64_t c = cur[r];
      const int64_t e = fin[r];
      while (true) {
        const int64_t idx = c + lane;
        const int col = idx < e ? col_idx[idx] : 0x7fffffff;
        const bool in = col < t1;  // a prefix of the lanes: the list is sorted
        if (in) atomicOr(&mask[col - t0], 1ull << r);
        const int m = __popcll(__ballot(in));
        c += m;
        if (m < 64) break;
      }
      if (lane == 0) cur[r] = c;
    }
    __syncthreads();
    const int col = t0 + threadIdx.x;
    if (!kFill) {
      if (col < t1) tile_cnt[(int64_t)rt * n + col] = __popcll(mask[threadIdx.x]);
    } else {
      // each column's rows go out as one store of a wave: lane r writes row
      // i0 + r at its rank among the column's rows, so a column's run is
      // written by consecutive lanes to consecutive addresses
      if (col < t1) cpos[threadIdx.x] = colt_ptr[g0 + col] + tile_cnt[(int64_t)rt * n + col];
      __syncthreads();
      for (int cc = wv; cc < t1 - t0; cc += kTrCols / 64) {
        const unsigned long long m = mask[cc];
        if ((m >> lane) & 1ull)
          colt_idx[cpos[cc] + __popcll(m & ((1ull << lane) - 1ull))] = i0 + lane;
      }
    }
    __syncthreads();
  }
}

// per column: turn the row-tile counts into output positions relative to the
// column's start (at most n, so they fit in 32 bits at any nnz), and the
// column's total
__global__ void k_colt_offsets(int n, int nch, int32_t* __restrict__ chunk_cnt,
                               int32_t* __restrict__ colt_cnt) {
  int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  int32_t run = 0;
  for (int c = 0; c < nch; c++) {
    int32_t t = chunk_cnt[(int64_t)c * n + j];
    chunk_cnt[(int64_t)c * n + j] = run;
    run += t;
  }
  colt_cnt[j] = run;
}

// key-major scan: counts per column -> pointers (reuses k_scan_rows on colt_cnt)

// first global block id of each head (prefix over heads of N_blk)
__global__ void k_blk_off(const int32_t* __restrict__ nblk, int heads, int64_t* __restrict__ off) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    int64_t a = 0;
    for (int h = 0; h < heads; h++) {
      off[h] = a;
      a += nblk[h];
    }
    off[heads] = a;
  }
}

// original token of every permuted row, [heads][N]
__global__ void k_perm_map(const uint8_t* __restrict__ shape_id, int H, int W, int Z,
                           int64_t N, int heads, int32_t* __restrict__ out) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= (int64_t)heads * N) return;
  int h = (int)(i / N);
  int64_t p = i - (int64_t)h * N;
  int m = (int)(p >> 9), r = (int)(p & 511);
  out[i] = (int32_t)token_of(d_shapes[shape_id[(int64_t)h * Z + m]], m, r, H, W);
}

__global__ __launch_bounds__(256) void k_sum_i64(const int64_t* __restrict__ in, int64_t n,
                                                 int64_t* __restrict__ out) {
  __shared__ int64_t sh[4];
  int64_t s = 0;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += in[i];
  s = block_sum<int64_t>(s, sh);
  if (threadIdx.x == 0) *out = s;
}

// ============================================================ unit order
// The dK/dV kernel's work units (128 key rows) are taken in an order of their
// own: per head, by the length of the unit's walk, longest first (ties by
// unit index).  Units that run side by side then walk lists of nearly equal
// length, which over a dense-ish selection name mostly the same tiles, and
// start and end together.

// Cost of each key block's key-major list in token pairs, B_j * sum_i B_i
// (the transpose of the rows' cost); one wave per block.
__global__ __launch_bounds__(256) void k_colt_cost(const int64_t* __restrict__ colt_ptr,
                                                   const int32_t* __restrict__ colt_idx,
                                                   int64_t g0, int n,
                                                   const uint8_t* __restrict__ blk_shape,
                                                   int64_t* __restrict__ colt_cost) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= n) return;
  const int64_t g = g0 + j;
  int64_t c = 0;
  for (int64_t e = colt_ptr[g] + lane; e < colt_ptr[g + 1]; e += 64)
    c += volume_of_id(block_shape_at(blk_shape, g0 + colt_idx[e]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
  if (lane == 0) colt_cost[g] = c * (int64_t)volume_of_id(block_shape_at(blk_shape, g));
}

// One work-group per head: the walk length of every unit of U rows (the
// longest list among the unit's blocks, in 64-row tiles: cost / B / 64),
// keyed ((16383 - min(tiles, 16383)) << 17 | unit) and sorted ascending by a
// bitonic sort in LDS.  Heads with more units than the LDS holds keep the
// identity order.
constexpr int kOrderMax = 32768;
template <int U>
__global__ __launch_bounds__(1024) void k_unit_order(const uint8_t* __restrict__ shape_id,
                                                     const int32_t* __restrict__ zone_base,
                                                     const int64_t* __restrict__ blk_off,
                                                     const int64_t* __restrict__ cost, int Z,
                                                     int64_t N, int32_t* __restrict__ order) {
  __shared__ uint32_t key[kOrderMax];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int upH = (int)(N / U);
  int32_t* out = order + (int64_t)h * upH;
  if (upH > kOrderMax) {
    for (int u = tid; u < upH; u += 1024) out[u] = u;
    return;
  }
  int np = 1;
  while (np < upH) np <<= 1;
  const int64_t hoff = blk_off[h];
  for (int u = tid; u < np; u += 1024) {
    uint32_t k = 0xffffffffu;
    if (u < upH) {
      const int64_t r0 = (int64_t)u * U;
      const int m = (int)(r0 >> 9);
      const int B = d_shapes[shape_id[(int64_t)h * Z + m]].volume;
      const int first = zone_base[(int64_t)h * Z + m] + (int)(r0 & 511) / B;
      const int cnt = B >= U ? 1 : U / B;
      int64_t w = 0;
      for (int c = 0; c < cnt; c++) w = max(w, cost[hoff + first + c] / B);
      const int t = (int)min<int64_t>(w >> 6, 16383);
      k = ((uint32_t)(16383 - t) << 17) | (uint32_t)u;
    }
    key[u] = k;
  }
  __syncthreads();
  for (int k2 = 2; k2 <= np; k2 <<= 1)
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < np; i += 1024) {
        const int ij = i ^ j;
        if (ij > i) {
          const uint32_t a = key[i], b = key[ij];
          if ((a > b) == ((i & k2) == 0)) {
            key[i] = b;
            key[ij] = a;
          }
        }
      }
      __syncthreads();
    }
  for (int u = tid; u < upH; u += 1024) out[u] = (int32_t)(key[u] & 0x1ffffu);
}

// ============================================================ launchers
bool launch_unit_order_k(const PlanDev& P, const std::vector<int64_t>& off, hipStream_t st) {
  for (int h = 0; h < P.heads; h++) {
    const int n = (int)(off[h + 1] - off[h]);
    if (n > 0)
      hipLaunchKernelGGL(k_colt_cost, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st,
                         P.colt_ptr, P.colt_idx, off[h], n, P.blk_shape, P.colt_cost);
  }
  hipLaunchKernelGGL(k_unit_order<128>, dim3(P.heads), dim3(1024), 0, st, P.shape_id,
                     P.zone_base, P.blk_off, P.colt_cost, P.Z, P.N, P.korder);
  return hipGetLastError() == hipSuccess;
}


bool launch_blk_off(const PlanDev& P, hipStream_t st) {
  hipLaunchKernelGGL(k_blk_off, dim3(1), dim3(64), 0, st, P.nblk, P.heads, P.blk_off);
  return hipGetLastError() == hipSuccess;
}

bool launch_perm_map(const PlanDev& P, int32_t* out, hipStream_t st) {
  int64_t tot = (int64_t)P.heads * P.N;
  hipLaunchKernelGGL(k_perm_map, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st,
                     P.shape_id, P.H, P.W, P.Z, P.N, P.heads, out);
  return hipGetLastError() == hipSuccess;
}

bool launch_sum_i64(const int64_t* in, int64_t n, int64_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_sum_i64, dim3(1), dim3(256), 0, st, in, n, out);
  return hipGetLastError() == hipSuccess;
}

bool launch_zone_stats(const void* v, int dtype, int D, int H, int W, int Z, int heads,
                       int64_t N, float* out, hipStream_t st) {
  dim3 grid(heads * Z), block(64);
  if (dtype == PRISM_BF16 && D == 128)
    hipLaunchKernelGGL((k_zone_stats<1, 2>), grid, block, 0, st, v, H, W, Z, N, out);
  else if (dtype == PRISM_BF16 && D == 64)
    hipLaunchKernelGGL((k_zone_stats<1, 1>), grid, block, 0, st, v, H, W, Z, N, out);
  else if (dtype == PRISM_F32 && D == 64)
    hipLaunchKernelGGL((k_zone_stats<0, 1>), grid, block, 0, st, v, H, W, Z, N, out);
  else if (dtype == PRISM_F32 && D == 128)
    hipLaunchKernelGGL((k_zone_stats<0, 2>), grid, block, 0, st, v, H, W, Z, N, out);
  else
    return false;
  return hipGetLastError() == hipSuccess;
}

bool launch_audio_stats(const float* a, int H, int W, int Z, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_audio_stats, dim3((Z + 63) / 64), dim3(64), 0, st, a, H, W, Z, out);
  return hipGetLastError() == hipSuccess;
}

bool launch_shapes(const PlanDev& P, int have_audio, const prism_config& c, int fixed_id,
                   hipStream_t st) {
  hipLaunchKernelGGL(k_shapes, dim3(P.heads), dim3(256), 0, st, P.vstats, P.astats, have_audio,
                     P.Z, c.eps, c.tau128, c.tau256, c.volume_mask, fixed_id, P.shape_id,
                     P.zone_base, P.nblk);
  return hipGetLastError() == hipSuccess;
}

bool launch_permute_pool(const PlanDev& P, const void* q, const void* k, const void* v,
                         hipStream_t st) {
  dim3 grid(P.heads * P.Z), block(512);
#define PP_ARGS                                                                           \
  q, k, v, P.H, P.W, P.Z, P.N, P.shape_id, P.zone_base, P.blk_off, P.kp, P.vp, P.blk_start, \
      P.blk_shape, P.blk_head, P.qbar, P.kbar, P.qgrid, P.kgrid, P.qexp, P.kexp
  if (P.dtype == PRISM_BF16 && P.D == 128)
    hipLaunchKernelGGL((k_permute_pool<1, 2, true>), grid, block, 0, st, PP_ARGS);
  else if (P.dtype == PRISM_BF16 && P.D == 64)
    hipLaunchKernelGGL((k_permute_pool<1, 1, false>), grid, block, 0, st, PP_ARGS);
  else if (P.dtype == PRISM_F32 && P.D == 64)
    hipLaunchKernelGGL((k_permute_pool<0, 1, false>), grid, block, 0, st, PP_ARGS);
  else if (P.dtype == PRISM_F32 && P.D == 128)
    hipLaunchKernelGGL((k_permute_pool<0, 2, false>), grid, block, 0, st, PP_ARGS);
  else
    return false;
#undef PP_ARGS
  return hipGetLastError() == hipSuccess;
}

bool launch_block_scores(const PlanDev& P, int64_t g0, int n, float* out, hipStream_t st) {
  if (n <= 0) return true;
  float cD = (float)(1.0 / sqrt((double)P.D));
  dim3 grid((n + 127) / 128, (n + 127) / 128), block(256);
  if (P.D == 128)
    hipLaunchKernelGGL((k_block_scores<128>), grid, block, 0, st, P.qgrid, P.kgrid, P.qexp,
                       P.kexp, g0, n, cD, out);
  else
    hipLaunchKernelGGL((k_block_scores<64>), grid, block, 0, st, P.qgrid, P.kgrid, P.qexp,
                       P.kexp, g0, n, cD, out);
  return hipGetLastError() == hipSuccess;
}

// dynamic LDS of the staged row: n floats, rounded up to whole 64-float
// pieces of the staging loads
static unsigned sel_lds_bytes(int n) { return (unsigned)(sel_row_floats(n) * 4); }
// the fill kernel also stages the words that cover the head's n shape ids
static unsigned sel_fill_lds_bytes(int n) {
  return sel_lds_bytes(n) + (unsigned)(((n + 3) / 4 + 1 + 63) / 64 * 64 * 4);
}

bool launch_select(const PlanDev& P, int64_t g0, int n, const prism_config& c, int last,
                   hipStream_t st) {
  const bool lds = n <= kSelLdsMax;
  if (n > 0) {
    if (lds)
      hipLaunchKernelGGL(k_select_count<true>, dim3(n), dim3(kSelThreads), sel_lds_bytes(n), st,
                         P.scores, n, g0, c.top_k, c.top_k_frac, c.top_p, P.row_cnt, P.row_key,
                         P.row_tie);
    else
      hipLaunchKernelGGL(k_select_count<false>, dim3(n), dim3(kSelThreads), 0, st, P.scores, n,
                         g0, c.top_k, c.top_k_frac, c.top_p, P.row_cnt, P.row_key, P.row_tie);
  }
  hipLaunchKernelGGL(k_scan_rows, dim3(1), dim3(1024), 0, st, P.row_cnt, n, g0, P.row_ptr,
                     P.counters, last);
  if (n > 0) {
    if (lds)
      hipLaunchKernelGGL(k_select_fill<true>, dim3(n), dim3(kSelThreads), sel_fill_lds_bytes(n),
                         st,
                         P.scores, n, g0, P.row_cnt, P.row_key, P.row_tie, P.row_ptr, P.cap,
                         P.blk_shape, P.col_idx, P.row_cost);
    else
      hipLaunchKernelGGL(k_select_fill<false>, dim3(n), dim3(kSelThreads), 0, st, P.scores, n,
                         g0, P.row_cnt, P.row_key, P.row_tie, P.row_ptr, P.cap, P.blk_shape,
                         P.col_idx, P.row_cost);
  }
  return hipGetLastError() == hipSuccess;
}

bool launch_transpose(const PlanDev& P, int64_t g0, int n, int last, hipStream_t st) {
  if (n <= 0) return true;
  const int nrt = (n + kTrRows - 1) / kTrRows;
  const dim3 grid((unsigned)nrt, (unsigned)((n + kTrPart - 1) / kTrPart));
  hipLaunchKernelGGL(k_colt_tiles<false>, grid, dim3(kTrCols), 0, st, P.row_ptr, P.col_idx, n,
                     g0, P.colt_ptr, P.chunk_cnt, P.colt_idx);
  hipLaunchKernelGGL(k_colt_offsets, dim3((n + 255) / 256), dim3(256), 0, st, n, nrt,
                     P.chunk_cnt, P.colt_cnt + g0);
  hipLaunchKernelGGL(k_scan_rows, dim3(1), dim3(1024), 0, st, P.colt_cnt, n, g0, P.colt_ptr,
                     P.counters + 1, last);
  hipLaunchKernelGGL(k_colt_tiles<true>, grid, dim3(kTrCols), 0, st, P.row_ptr, P.col_idx, n,
                     g0, P.colt_ptr, P.chunk_cnt, P.colt_idx);
  return hipGetLastError() == hipSuccess;
}

}  // namespace prism
