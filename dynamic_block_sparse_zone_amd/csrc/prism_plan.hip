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

// ---- Shape mappings other than b ~ g^(-1/2), the ablations the pages name
// (paper.rainbus.top "技术新颖性", Table 10): alpha in b ~ g^(-alpha),
// isotropic, softmax, rank and entropy mappings.  Each gives a target point l
// in log2 space with sum_d l_d = log2 B:
//   power(alpha): l_d = -alpha log2 g_d + (S + alpha sum_d log2 g_d) / 3
//   isotropic:    l_d = S / 3
//   softmax:      l_d = S softmax(-g)_d
//   rank:         l_d = S / 3 + rank_d - 1  (rank 0: the largest g_d; equal
//                 values rank the earlier axis first)
//   entropy:      l_d = S i_d / sum i,  i_d = -ln(g_d / sum g)
// and the shape is the candidate of volume B nearest to l (squared
// Euclidean distance, a later candidate replaces the best only when strictly
// nearer).  Evaluated in fp64 with plain operations in a fixed order and the
// logarithm and exponential written below, so the decisions are reproducible.
constexpr double kLn2 = 0.69314718055994530942;
constexpr double kInvLn2 = 1.4426950408889634074;

// x = m 2^e with m in [1, 2), exactly
__device__ inline double mant_exp(double x, int* e) {
  const double m = frexp(x, e);
  *e -= 1;
  return m * 2.0;
}
// ln m for m in [1, 2): 2 atanh(z), z = (m - 1) / (m + 1), by the odd series
// 2 z sum_{k=0..16} z^(2k) / (2k + 1) in Horner form
__device__ inline double ln_mantissa(double m) {
  const double z = (m - 1.0) / (m + 1.0);
  const double z2 = z * z;
  double s = 1.0 / 33.0;
  for (int k = 15; k >= 0; k--) s = s * z2 + 1.0 / (double)(2 * k + 1);
  return (2.0 * z) * s;
}
__device__ inline double log2_w(double x) {
  int e;
  const double m = mant_exp(x, &e);
  return (double)e + ln_mantissa(m) * kInvLn2;
}
__device__ inline double ln_w(double x) {
  int e;
  const double m = mant_exp(x, &e);
  return (double)e * kLn2 + ln_mantissa(m);
}
// e^x = 2^k 2^f, k = rint(x log2 e), 2^f by its Taylor series in f ln 2 to
// degree 14 (coefficients (ln 2)^n / n! by the recurrence c_n = c_{n-1} ln2 / n)
__device__ inline double exp_w(double x) {
  const double y = x * kInvLn2;
  const double k = rint(y);
  const double f = y - k;
  double c[15];
  c[0] = 1.0;
  for (int n = 1; n < 15; n++) c[n] = c[n - 1] * kLn2 / (double)n;
  double p = c[14];
  for (int n = 13; n >= 0; n--) p = p * f + c[n];
  return ldexp(p, (int)k);
}

__device__ inline void map_target(const float* g, int B, int map, float alpha, double* l) {
  const double S = B == 64 ? 6.0 : B == 128 ? 7.0 : 8.0;
  if (map == PRISM_MAP_POWER) {
    const double a = (double)alpha;
    double L[3];
    for (int d = 0; d < 3; d++) L[d] = log2_w((double)g[d]);
    const double Ls = (L[0] + L[1]) + L[2];
    const double c = (S + a * Ls) / 3.0;
    for (int d = 0; d < 3; d++) l[d] = (-a) * L[d] + c;
  } else if (map == PRISM_MAP_ISOTROPIC) {
    for (int d = 0; d < 3; d++) l[d] = S / 3.0;
  } else if (map == PRISM_MAP_SOFTMAX) {
    double gm = (double)g[0];
    for (int d = 1; d < 3; d++) gm = (double)g[d] < gm ? (double)g[d] : gm;
    double w[3];
    for (int d = 0; d < 3; d++) w[d] = exp_w(gm - (double)g[d]);
    const double ws = (w[0] + w[1]) + w[2];
    for (int d = 0; d < 3; d++) l[d] = S * (w[d] / ws);
  } else if (map == PRISM_MAP_RANK) {
    for (int d = 0; d < 3; d++) {
      int r = 0;
      for (int e = 0; e < 3; e++) r += (g[e] > g[d] || (g[e] == g[d] && e < d)) ? 1 : 0;
      l[d] = S / 3.0 + (double)(r - 1);
    }
  } else {  // PRISM_MAP_ENTROPY
    const double gs = ((double)g[0] + (double)g[1]) + (double)g[2];
    const double lgs = ln_w(gs);
    double inf[3];
    for (int d = 0; d < 3; d++) inf[d] = lgs - ln_w((double)g[d]);
    const double is = (inf[0] + inf[1]) + inf[2];
    for (int d = 0; d < 3; d++) l[d] = S * (inf[d] / is);
  }
}

__device__ inline int nearest_mapped(const float* g, int B, int map, float alpha) {
  double l[3];
  map_target(g, B, map, alpha, l);
  const int first = shape_first(B), cnt = shape_count(B);
  int best = first;
  double bestd = 0.0;
  for (int c = first; c < first + cnt; c++) {
    const Shape& s = d_shapes[c];
    const double d0 = l[0] - (double)s.log2_bt;
    const double d1 = l[1] - (double)s.log2_bh;
    const double d2 = l[2] - (double)s.log2_bw;
    const double dist = (d0 * d0 + d1 * d1) + d2 * d2;
    if (c == first || dist < bestd) {
      best = c;
      bestd = dist;
    }
  }
  return best;
}

// The same choices restricted to candidates with b_T <= cap (a zone that a
// shot cut splits in time).
__device__ inline int nearest_capped(const float* g, int B, int map, float alpha, int cap) {
  const int first = shape_first(B), cnt = shape_count(B);
  int best = -1;
  if (map == PRISM_MAP_POWER && alpha == 0.5f) {
    for (int c = first; c < first + cnt; c++)
      if (d_shapes[c].bt <= cap && (best < 0 || shape_nearer(g, c, best))) best = c;
    return best;
  }
  double l[3];
  map_target(g, B, map, alpha, l);
  double bestd = 0.0;
  for (int c = first; c < first + cnt; c++) {
    const Shape& s = d_shapes[c];
    if (s.bt > cap) continue;
    const double d0 = l[0] - (double)s.log2_bt;
    const double d1 = l[1] - (double)s.log2_bh;
    const double d2 = l[2] - (double)s.log2_bw;
    const double dist = (d0 * d0 + d1 * d1) + d2 * d2;
    if (best < 0 || dist < bestd) {
      best = c;
      bestd = dist;
    }
  }
  return best;
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
                                                uint32_t vmask, int fixed_id, int map,
                                                float alpha, const int32_t* __restrict__ zt_cap,
                                                int zones_per_t,
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
        const int cap = zt_cap ? zt_cap[m / zones_per_t] : 8;
        if (cap < 8) {
          // a shot cut inside the zone: blocks no longer in time than cap
          // (b_T = 2 allows at most 128 tokens)
          if (cap == 2 && B > 128) B = 128;
          id = nearest_capped(g, B, map, alpha, cap);
        } else if (map == PRISM_MAP_POWER && alpha == 0.5f) {
          int first = shape_first(B), cnt = shape_count(B);
          id = first;
          for (int c = first + 1; c < first + cnt; c++)
            if (shape_nearer(g, c, id)) id = c;
        } else {
          id = nearest_mapped(g, B, map, alpha);
        }
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

// ============================================================ K4: block table + pooling
// One block of 512 threads (8 waves) per (head, zone); wave w owns the rows
// [64w, 64w+64) of the zone in block-contiguous order (the re-layout of
// stage two, which no kernel materialises: attention gathers each block's
// rows from the original layout through the block -> token map).  Q and K are
// summed per 64-row tile (rows in that order), then per block (tiles in
// order), scaled by 1/B and written with their integer grid:
// q_c = rint(x_c 2^-E), E = exponent(max_c |x_c|) - 8.  Each block's first
// row, first token and shape go to the block table.
template <int DT, int CPL>
__global__ __launch_bounds__(512) void k_pool(
    const void* __restrict__ q, const void* __restrict__ k, int H, int W, int Z, int64_t N,
    const uint8_t* __restrict__ shape_id, const int32_t* __restrict__ zone_base,
    const int64_t* __restrict__ blk_off, int32_t* __restrict__ blk_start,
    int32_t* __restrict__ blk_org, uint8_t* __restrict__ blk_shape,
    int32_t* __restrict__ blk_head, float* __restrict__ qbar, float* __restrict__ kbar,
    uint16_t* __restrict__ qgrid, uint16_t* __restrict__ kgrid, uint16_t* __restrict__ qlo,
    uint16_t* __restrict__ klo, int32_t* __restrict__ qexp, int32_t* __restrict__ kexp) {
  constexpr int D = 64 * CPL;
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
#pragma unroll
    for (int c = 0; c < CPL; c++) {
      aq[c] = (i == 0) ? rq.get(c) : aq[c] + rq.get(c);
      ak[c] = (i == 0) ? rk.get(c) : ak[c] + rk.get(c);
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
      blk_org[g] = (int32_t)token_of(sh, m, wv * B, H, W);
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
      uint16_t* grl = which ? klo : qlo;
#pragma unroll
      for (int c = 0; c < CPL; c++) {
        xb[g * D + lane * CPL + c] = x[c];
        // two-level grid: x ~ 2^E (hi + 2^-8 lo), hi in [-256, 256],
        // lo in [-128, 128], both exact in bf16
        const float y = mx > 0.0f ? ldexpf(x[c], -e) : 0.0f;
        const float hi = rintf(y);
        const float lo = rintf(ldexpf(y - hi, 8));
        gr[g * D + lane * CPL + c] = (uint16_t)(__float_as_uint(hi) >> 16);
        grl[g * D + lane * CPL + c] = (uint16_t)(__float_as_uint(lo) >> 16);
      }
      if (lane == 0) (which ? kexp : qexp)[g] = e;
    }
  }
}

// ============================================================ K4b: re-layout
// Stage two's re-layout (paper.rainbus.top "方法步骤详情", stage two): rows
// of two [heads][N][128] bf16 tensors copied into block-contiguous order
// (permuted row p of a head takes its token token_of(p)), each row's 16-byte
// chunks stored swizzled (chunk c of row p at c ^ chunk_swizzle(p & 63)), so
// that an attention tile is one contiguous 16 KB run that lands in LDS as
// it is.  With fa given, two [heads][N] float columns follow the same order.
// 16 lanes per row (one chunk each), 32 rows per work-group of 512 threads.
__global__ __launch_bounds__(512) void k_relayout(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
    const float* __restrict__ fa, const float* __restrict__ fb,
    const uint8_t* __restrict__ shape_id, int H, int W, int Z, int64_t N, int64_t rows,
    uint16_t* __restrict__ ap, uint16_t* __restrict__ bp, float* __restrict__ fap,
    float* __restrict__ fbp) {
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 4);
  if (row >= rows) return;
  const int c = threadIdx.x & 15;
  const int h = (int)(row / N);
  const int64_t p = row - (int64_t)h * N;
  const int m = (int)(p >> 9);
  const int64_t src = (int64_t)h * N + token_of(d_shapes[shape_id[(int64_t)h * Z + m]], m,
                                                (int)(p & 511), H, W);
  const int dc = c ^ chunk_swizzle((int)(p & 63));
  *(uint4*)(ap + row * 128 + dc * 8) = *(const uint4*)(a + src * 128 + c * 8);
  *(uint4*)(bp + row * 128 + dc * 8) = *(const uint4*)(b + src * 128 + c * 8);
  if (fa && c == 0) {
    fap[row] = fa[src];
    fbp[row] = fb[src];
  }
}

// ============================================================ K5: block scores
// s_ij = Qbar_i . Kbar_j / sqrt(D) on the two-level grid x ~ 2^E (hi + 2^-8 lo):
// the integer dot products I_hh = hi.hi, I_x = hi_i.lo_j + lo_i.hi_j and
// I_ll = lo.lo are exact on the bf16 MFMA (every partial sum is an integer
// below 2^24), J = 2^16 I_hh + 2^8 I_x + I_ll is formed exactly (in fp64),
// and s = fl32(fl32(J) 2^(Ei + Ej - 16)) * fl(1/sqrt D), J rounded once.
// A work-group of four waves covers 128 x 128 scores: the hi and lo grids of
// its 128 key blocks are staged once in LDS (16-byte chunks swizzled by row,
// so that 16 consecutive rows read at one chunk touch distinct banks), and
// each wave holds its 32 query blocks' fragments in registers and walks the
// four 32-key tiles.
template <int D>
__global__ __launch_bounds__(256, 2) void k_block_scores(
    const uint16_t* __restrict__ qgrid, const uint16_t* __restrict__ kgrid,
    const uint16_t* __restrict__ qlo, const uint16_t* __restrict__ klo,
    const int32_t* __restrict__ qexp, const int32_t* __restrict__ kexp, int64_t g0, int n,
    float cD, float* __restrict__ scores) {
  constexpr int C = D / 8;    // 16-byte chunks per row
  constexpr int KK = D / 16;  // MFMA steps over the channels
  __shared__ uint4 ksh[128 * C], ksl[128 * C];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5, l32 = lane & 31;
  const int j0 = blockIdx.x * 128, i0 = blockIdx.y * 128 + wv * 32;
  for (int idx = tid; idx < 128 * C; idx += 256) {
    const int r = idx / C, c = idx % C;
    uint4 vh = make_uint4(0, 0, 0, 0), vl = vh;
    if (j0 + r < n) {
      vh = *(const uint4*)(kgrid + (g0 + j0 + r) * D + c * 8);
      vl = *(const uint4*)(klo + (g0 + j0 + r) * D + c * 8);
    }
    const int pc = r * C + (c ^ (r & (C - 1)));
    ksh[pc] = vh;
    ksl[pc] = vl;
  }
  // this wave's query blocks as MFMA A operands (row l32, channels
  // 16kk + 8hl .. + 7) and the exponents of the rows this lane's outputs hold
  const int ia = i0 + l32;
  bf16x8 qh[KK], ql[KK];
#pragma unroll
  for (int kk = 0; kk < KK; kk++) {
    uint4 uh = make_uint4(0, 0, 0, 0), ul = uh;
    if (ia < n) {
      uh = *(const uint4*)(qgrid + (g0 + ia) * D + kk * 16 + hl * 8);
      ul = *(const uint4*)(qlo + (g0 + ia) * D + kk * 16 + hl * 8);
    }
    qh[kk] = __builtin_bit_cast(bf16x8, uh);
    ql[kk] = __builtin_bit_cast(bf16x8, ul);
  }
  int qe[16];
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int i = i0 + (r >> 2) * 8 + hl * 4 + (r & 3);
    qe[r] = i < n ? qexp[g0 + i] : 0;
  }
  __syncthreads();
  if (i0 >= n) return;
  for (int b = 0; b < 4 && j0 + 32 * b < n; b++) {
    const int jr = 32 * b + l32;  // the lane's key row in the staged tile
    f32x16 hh, hx, ll;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      hh[r] = 0.0f;
      hx[r] = 0.0f;
      ll[r] = 0.0f;
    }
#pragma unroll
    for (int kk = 0; kk < KK; kk++) {
      const int pc = jr * C + ((2 * kk + hl) ^ (jr & (C - 1)));
      const bf16x8 kh = __builtin_bit_cast(bf16x8, ksh[pc]);
      const bf16x8 kl = __builtin_bit_cast(bf16x8, ksl[pc]);
      hh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh[kk], kh, hh, 0, 0, 0);
      hx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh[kk], kl, hx, 0, 0, 0);
      hx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ql[kk], kh, hx, 0, 0, 0);
      ll = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ql[kk], kl, ll, 0, 0, 0);
    }
    const int j = j0 + jr;
    if (j >= n) continue;
    const int ej = kexp[g0 + j];
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int i = i0 + (r >> 2) * 8 + hl * 4 + (r & 3);
      if (i < n) {
        // J = 2^16 I_hh + 2^8 I_x + I_ll: each product is an integer below
        // 2^25 held exactly in fp32, and |J| < 2^42, so the fp64 sum is J
        // exactly and is rounded once to fp32
        const double J = __builtin_fma((double)hh[r], 65536.0,
                                       __builtin_fma((double)hx[r], 256.0, (double)ll[r]));
        const float s = ldexpf((float)J, qe[r] + ej - 16) * cD;
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

// The same value without a branch (the series is evaluated for every x and
// the result replaced by 0 below the cut-off), for unrolled loops.
__device__ inline float exp2_taylor_sel(float x) {
  const float kf = rintf(x);
  const float f = x - kf;
  float p = 0.000015252733804059840280f;
  p = __builtin_fmaf(p, f, 0.00015403530393381609954f);
  p = __builtin_fmaf(p, f, 0.0013333558146428443423f);
  p = __builtin_fmaf(p, f, 0.0096181291076284771620f);
  p = __builtin_fmaf(p, f, 0.055504108664821579953f);
  p = __builtin_fmaf(p, f, 0.24022650695910071233f);
  p = __builtin_fmaf(p, f, 0.69314718055994530942f);
  p = __builtin_fmaf(p, f, 1.0f);
  const float r = ldexpf(p, x > -100.0f ? (int)kf : 0);
  return x > -100.0f ? r : 0.0f;
}

// (u64)(y 2^32) for 0 <= y <= 1 (the exp2 of a non-positive argument): the
// product is exact and below 2^32 unless y = 1, so a truncating 32-bit
// conversion gives the same integer
__device__ inline unsigned long long weight_bits(float y) {
  const float t = y * 4294967296.0f;
  return t >= 4294967296.0f ? (1ull << 32) : (unsigned long long)(uint32_t)t;
}

// softmax weight of a score in 2^-32 units relative to the row maximum
__device__ inline uint64_t weight_of(float s, float smax) {
  const float LOG2E = 1.44269504088896340736f;
  float x = (s - smax) * LOG2E;
  float y = exp2_taylor(x);
  return (uint64_t)(y * 4294967296.0f);
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
// block volume of a shape id (ids are ordered by volume: 0..6 are 64,
// 7..12 are 128, 13..15 are 256)
__device__ inline int volume_of_id(int sid) { return sid < 7 ? 64 : sid < 13 ? 128 : 256; }

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

// The row's scores for the radix select below: src.each(f) calls f on every
// score of this thread's share of the row (elements tid + 256 e), read from
// HBM on every pass.
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
// (a GlobalRow).
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
  const float* grow = scores + (int64_t)i * n;
  const GlobalRow gr{grow, n};
  // the row's maximum and minimum
  float mx = -INFINITY, mn = INFINITY;
  auto minmax = [&](float s) {
    mx = fmaxf(mx, s);
    mn = fminf(mn, s);
  };
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
    return exact_select(gr, smax, smin, by_weight, need, S, ac, aw, p32, need_out);
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
// counters[0]); one block of 1024 threads, each taking a contiguous segment:
// its sum, one block scan of the sums, then the segment's pointers.
__global__ __launch_bounds__(1024) void k_scan_rows(const int32_t* __restrict__ cnt, int n,
                                                    int64_t g0, int64_t* __restrict__ ptr,
                                                    int64_t* __restrict__ counters,
                                                    int last) {
  __shared__ int64_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (n + 1023) / 1024;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  int64_t s = 0;
  for (int i = i0; i < i1; i++) s += cnt[g0 + i];
  int64_t x = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t u = __shfl_up(x, off, 64);
    if (lane >= off) x += u;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  int64_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 16; w++) {
    before += w < wv ? wsum[w] : 0;
    total += wsum[w];
  }
  const int64_t base = counters[0];
  int64_t run = base + before + x - s;
  for (int i = i0; i < i1; i++) {
    ptr[g0 + i] = run;
    run += cnt[g0 + i];
  }
  __syncthreads();  // every thread has read counters[0]
  if (tid == 0) {
    counters[0] = base + total;
    if (last) ptr[g0 + n] = base + total;
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

// Writes the selected key blocks of each row (rows longer than the register
// path holds) in ascending order, given the threshold key K and the number
// of K-ties to take, with the row's attention cost B_i * sum_j B_j.  Thread
// t takes the contiguous segment [tC, tC + C) of the row: one prefix over
// the ties and one over the selected counts place every thread's output.
__global__ __launch_bounds__(kSelThreads) void k_select_fill(
    const float* __restrict__ scores, int n, int64_t g0, const int32_t* __restrict__ row_cnt,
    const uint32_t* __restrict__ row_key, const int32_t* __restrict__ row_tie,
    const int64_t* __restrict__ row_ptr, int64_t cap, const uint8_t* __restrict__ blk_shape,
    int32_t* __restrict__ col_idx, int64_t* __restrict__ row_cost) {
  __shared__ int sh[kSelThreads / 64];
  __shared__ int64_t sh_cost[kSelThreads / 64];
  const int i = blockIdx.x;
  const int64_t g = g0 + i;
  const float* row = scores + (int64_t)i * n;
  const uint32_t K = row_key[g];
  const int tie = row_tie[g];
  const int64_t base = row_ptr[g];
  const bool fits = base + row_cnt[g] <= cap;
  const int C = (n + kSelThreads - 1) / kSelThreads;
  const int j0 = min(n, (int)threadIdx.x * C), j1 = min(n, j0 + C);
  int total = 0;
  int64_t cost = 0;
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
  const int64_t c = block_sum<int64_t>(cost, sh_cost);
  if (threadIdx.x == 0) row_cost[g] = c * (int64_t)d_shapes[block_shape_at(blk_shape, g)].volume;
}

// ---- rows of up to kSelRegMax blocks: the selection from registers
// A work-group of kSelMT threads takes one row; thread t holds the elements
// t + kSelMT e (e < kSelPer) as order keys relative to the row's smallest
// key (a score is recovered exactly from its key, so the integer softmax
// weight is formed from it where needed, as weight_of forms it).  Slots past the
// row's end hold copies of its last element: they leave the row's extremes
// alone, the histogram passes skip them (they fill the slabs past
// n / kSelMT, a uniform test, and part of one slab), and the mask drops their
// bits; in index order they come after every real element.  The selects take 11-bit digits from the top of the row's key range; a level's
// histogram packs count << 47 | integer weight per digit into one u64 (a row
// of at most 16384 blocks has fewer than 2^15 elements and a weight total
// below 2^47, so both fields stay exact): one LDS atomic per candidate.  The
// threshold key and tie count are those of the radix select over the row
// above; the row's selection leaves as a bit mask (word w: blocks
// 64 w .. 64 w + 63, bit b: block 64 w + b).
constexpr int kSelRegMax = 16384;
constexpr int kSelMT = 512;                      // threads per row
constexpr int kSelMW = kSelMT / 64;              // waves per row
constexpr int kSelPer = kSelRegMax / kSelMT;     // elements per thread
constexpr int kSelBits = 11;
constexpr int kSelBins = 1 << kSelBits;
constexpr int kSelQ = kSelBins / kSelMT;         // digits per thread in the scan
constexpr int kCntShift = 47;
constexpr unsigned long long kWtMask = (1ull << kCntShift) - 1ull;

// The levels alternate between two histograms (and scan / result slots):
// a level clears the other one while it fills its own, so a level takes
// three barriers.
struct SelSharedR {
  unsigned long long hist[2][kSelBins];
  unsigned long long wsum[2][kSelMW];
  unsigned long long above[2], fallback[2], wstar;
  int pick[2];
  uint32_t kmin[kSelMW], kmax[kSelMW];
  int isum[kSelMW];
  int trank[kSelPer * kSelMW];
};

// exclusive scan over a kSelMT-thread block of one value per thread, and the
// block total; without `reuse` the trailing barrier is left out (the caller
// does not write `sh` again before a later barrier)
template <typename T, bool reuse = true>
__device__ inline T row_excl_scan(T v, T* sh, T* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  T x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T u = __shfl_up(x, off, 64);
    if (lane >= off) x += u;
  }
  if (lane == 63) sh[wv] = x;
  __syncthreads();
  T before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelMW; w++) {
    before += w < wv ? sh[w] : (T)0;
    tot += sh[w];
  }
  if (reuse) __syncthreads();
  *total = tot;
  return before + x - v;
}

// Per query block row (n <= kSelRegMax): the same count, threshold key and
// tie count as k_select_count, and the row's selection mask (wd words).
__global__ __launch_bounds__(kSelMT) __attribute__((amdgpu_waves_per_eu(4))) void k_select_mask(
    const float* __restrict__ scores, int n, int64_t g0, int k_count, float k_frac, float p,
    int32_t* __restrict__ row_cnt, uint32_t* __restrict__ row_key,
    int32_t* __restrict__ row_tie, unsigned long long* __restrict__ mask, int wd) {
  __shared__ SelSharedR S;
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t g = g0 + i;
  int64_t kk = k_count;
  if (k_frac > 0.0f) kk = (int64_t)ceil((double)k_frac * (double)n);
  if (kk > n) kk = n;
  if (kk < 0) kk = 0;
  // the row, 2 KB per slab (coalesced), as order keys; slots past its end
  // copy element n - 1
  const float* grow = scores + (int64_t)i * n;
  // slabs 0 .. nfull - 1 are whole; slab nfull holds the lanes tid < n % kSelMT
  const int nfull = __builtin_amdgcn_readfirstlane(n / kSelMT);
  const bool tail = tid < n % kSelMT;
  uint32_t rel[kSelPer];
#pragma unroll
  for (int e = 0; e < kSelPer; e++) rel[e] = f2key(grow[min(tid + e * kSelMT, n - 1)]);
  // the row's smallest and largest order keys
  uint32_t kmn = rel[0], kmx = rel[0];
#pragma unroll
  for (int e = 1; e < kSelPer; e++) {
    kmn = min(kmn, rel[e]);
    kmx = max(kmx, rel[e]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, off, 64));
    kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, off, 64));
  }
  if (lane == 0) {
    S.kmin[wv] = kmn;
    S.kmax[wv] = kmx;
  }
  // the first level's histogram and result slot start clear
#pragma unroll
  for (int q = 0; q < kSelQ; q++) S.hist[0][tid + q * kSelMT] = 0ull;
  if (tid == 0) S.pick[0] = -1;
  __syncthreads();
  uint32_t kmin = S.kmin[0], kmax = S.kmax[0];
#pragma unroll
  for (int w = 1; w < kSelMW; w++) {
    kmin = min(kmin, S.kmin[w]);
    kmax = max(kmax, S.kmax[w]);
  }
  const float smax = key2f(kmax);
  const uint32_t span = kmax - kmin;
#pragma unroll
  for (int e = 0; e < kSelPer; e++) rel[e] -= kmin;
  // integer softmax weight of the element of relative key r (its score is
  // recovered exactly from the key, kb = kmin): weight_of's value
  const uint32_t kbase = __builtin_amdgcn_readfirstlane(kmin);
  auto wt = [&](uint32_t r, uint32_t kb) -> unsigned long long {
    const float s = key2f(r + kb);
    return weight_bits(exp2_taylor_sel((s - smax) * 1.44269504088896340736f));
  };

  // one level: histogram of the digits (rel >> lo) & dmask of the
  // candidates (the bits of rel from hi up equal those of `pre`; every
  // element when `all`), then the digit, from the top, at which the running
  // total (weight, else count) first reaches `need` (digit 0 if none does),
  // with the packed totals of the larger digits.  With p32 the target is the
  // Top-p weight W*, formed from the level's total.  hist[cur] is clear on
  // entry; hist[cur ^ 1] is cleared for the next level.
  int cur = 0;
  auto level = [&](int hi, int lo, uint32_t pre, bool all, bool by_weight,
                   unsigned long long need, unsigned long long p32,
                   unsigned long long* above) -> int {
    unsigned long long* H = S.hist[cur];
#pragma unroll
    for (int q = 0; q < kSelQ; q++) S.hist[cur ^ 1][tid + q * kSelMT] = 0ull;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    const uint32_t hmask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
    pre &= hmask;
    // an opaque copy per level: the weights are formed inside the level
    // rather than hoisted out of the level loop (32 more u64 live)
    uint32_t kb = kbase;
    asm volatile("" : "+s"(kb));
    // (each weight is formed from a copy made at its use, so that it is not
    // computed ahead for every element)
    auto add = [&](uint32_t r) {
      asm volatile("" : "+v"(r));
      unsigned long long inc = 1ull << kCntShift;
      if (by_weight) inc += wt(r, kb);
      atomicAdd(&H[(r >> lo) & dmask], inc);
    };
    // slabs past the row's end (whole slabs of padding copies: a uniform
    // branch) are skipped, and in the one partial slab only the lanes before
    // the end take part
#pragma unroll
    for (int e = 0; e < kSelPer; e++) {
      if (e > nfull) break;
      if (e == nfull && !tail) continue;
      if (all || (rel[e] & hmask) == pre) add(rel[e]);
    }
    __syncthreads();
    // every thread has read the previous level's result slot
    if (tid == 0) S.pick[cur ^ 1] = -1;
    // thread t owns the digits kSelBins - 1 - kSelQ t - q, in selection order
    unsigned long long v[kSelQ], sum = 0;
#pragma unroll
    for (int q = 0; q < kSelQ; q++) {
      v[q] = H[kSelBins - 1 - kSelQ * tid - q];
      sum += v[q];
    }
    unsigned long long total;
    unsigned long long run =
        row_excl_scan<unsigned long long, false>(sum, S.wsum[cur], &total);
    if (p32) {
      const unsigned long long Z = total & kWtMask;
      const unsigned long long zh = Z >> 32, zl = Z & 0xffffffffull;
      need = p32 * zh + ((p32 * zl + 0xffffffffull) >> 32);
      if (tid == 0) S.wstar = need;
    }
#pragma unroll
    for (int q = 0; q < kSelQ; q++) {
      const unsigned long long before = by_weight ? (run & kWtMask) : (run >> kCntShift);
      const unsigned long long m = by_weight ? (v[q] & kWtMask) : (v[q] >> kCntShift);
      if (before < need && before + m >= need) {
        S.pick[cur] = kSelBins - 1 - kSelQ * tid - q;
        S.above[cur] = run;
      }
      // (the totals above digit 0, the answer when no digit reaches need)
      if (kSelBins - 1 - kSelQ * tid - q == 0) S.fallback[cur] = run;
      run += v[q];
    }
    __syncthreads();
    int d = S.pick[cur];
    if (d < 0) {
      d = 0;
      *above = S.fallback[cur];
    } else {
      *above = S.above[cur];
    }
    cur ^= 1;
    return d;
  };
  // exact select: the order key at which the running total in selection
  // order first reaches `need`, with the count and weight of larger keys
  auto select = [&](bool by_weight, unsigned long long need, unsigned long long p32,
                    uint32_t* ac, unsigned long long* aw,
                    unsigned long long* need_out) -> uint32_t {
    uint32_t prefix = 0;
    unsigned long long ab = 0;
    bool first = true;
    for (int hi = span ? 32 - __builtin_clz(span) : 1; hi > 0;) {
      const int lo = hi > kSelBits ? hi - kSelBits : 0;
      const unsigned long long done = by_weight ? (ab & kWtMask) : (ab >> kCntShift);
      unsigned long long a;
      const int d = level(hi, lo, prefix, first, by_weight, need - done,
                          first ? p32 : 0ull, &a);
      if (first && p32) need = S.wstar;
      first = false;
      prefix |= (uint32_t)d << lo;
      ab += a;
      hi = lo;
    }
    if (need_out) *need_out = need;
    *ac = (uint32_t)(ab >> kCntShift);
    *aw = ab & kWtMask;
    return kmin + prefix;
  };

  int64_t nsel = n;
  uint32_t keyL = 0u;
  int64_t tieL = 0;
  if (p < 1.0f) {
    int64_t L = 0;
    uint32_t keyP = 0, caP = 0;
    if (p > 0.0f) {
      const unsigned long long P32 = (unsigned long long)ceil((double)p * 4294967296.0);
      unsigned long long wa, Wstar;
      keyP = select(true, 0ull, P32, &caP, &wa, &Wstar);
      const unsigned long long wk = weight_of(key2f(keyP), smax);
      L = (int64_t)caP + (int64_t)((Wstar - wa + wk - 1) / wk);
    }
    nsel = kk > L ? kk : L;
    if (nsel > n) nsel = n;
    keyL = 0xffffffffu;
    tieL = 0;
    if (nsel > 0 && nsel == L) {
      keyL = keyP;
      tieL = L - (int64_t)caP;
    } else if (nsel > 0) {
      uint32_t ca;
      unsigned long long wa;
      keyL = select(false, (unsigned long long)nsel, 0ull, &ca, &wa, nullptr);
      tieL = nsel - (int64_t)ca;
    }
  }
  if (tid == 0) {
    row_cnt[g] = (int32_t)nsel;
    row_key[g] = keyL;
    row_tie[g] = (int32_t)tieL;
  }

  // the mask: every key above keyL and the first tieL copies of keyL in
  // index order (index j = kSelMT e + 64 wave + lane); all of the row when
  // p >= 1, none when nothing is selected.  Padding copies of keyL rank
  // after every real one, so the first tieL copies are real.
  const int mode = p >= 1.0f ? 2 : nsel == 0 ? 0 : 1;
  const uint32_t Kr = keyL - kmin;  // keyL relative to the row's smallest key (mode 1)
  int teq = 0;
  if (mode == 1) {
#pragma unroll
    for (int e = 0; e < kSelPer; e++) teq += rel[e] == Kr ? 1 : 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) teq += __shfl_xor(teq, off, 64);
  if (lane == 0) S.isum[wv] = teq;
  __syncthreads();
  int tall = 0;
#pragma unroll
  for (int w = 0; w < kSelMW; w++) tall += S.isum[w];
  // only some copies of keyL are taken: their ranks in index order
  const bool split = mode == 1 && tieL < tall;
  if (split) {
#pragma unroll
    for (int e = 0; e < kSelPer; e++) {
      const unsigned long long b = __ballot(rel[e] == Kr);
      if (lane == 0) S.trank[e * kSelMW + wv] = __popcll(b);
    }
    __syncthreads();
    int unused;
    const int x = tid < kSelPer * kSelMW ? S.trank[tid] : 0;
    const int ex = row_excl_scan<int>(x, S.isum, &unused);
    if (tid < kSelPer * kSelMW) S.trank[tid] = ex;
    __syncthreads();
  }
  unsigned long long word = 0;
#pragma unroll
  for (int e = 0; e < kSelPer; e++) {
    bool sel = false;
    if (mode == 2) {
      sel = true;
    } else if (mode == 1) {
      const bool eq = rel[e] == Kr;
      sel = rel[e] > Kr;
      if (split) {
        const unsigned long long b = __ballot(eq);
        const int rank = S.trank[e * kSelMW + wv] +
                         (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        sel = sel || (eq && rank < tieL);
      } else {
        sel = sel || eq;
      }
    }
    const unsigned long long b = __ballot(sel);
    if (lane == e) word = b;
  }
  // lane e (< kSelPer) holds the word of slab e and this wave: blocks
  // j0 .. j0 + 63, j0 = kSelMT e + 64 wave; the bits of j >= n are dropped
  const int w = kSelMW * lane + wv;
  const int lim = n - (kSelMT * lane + 64 * wv);
  if (lim < 64) word &= lim <= 0 ? 0ull : (1ull << lim) - 1ull;
  if (lane < kSelPer && w < wd) mask[(int64_t)i * wd + w] = word;
}

// Per head: masks of the blocks of each volume class (64, 128, 256 rows),
// word w covering blocks 64 w .. 64 w + 63 (one wave per word).
__global__ __launch_bounds__(256) void k_vol_masks(const uint8_t* __restrict__ blk_shape,
                                                   int64_t g0, int n, int wd,
                                                   unsigned long long* __restrict__ volm) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= wd) return;
  const int j = 64 * w + lane;
  const int vol = j < n ? volume_of_id(block_shape_at(blk_shape, g0 + j)) : 0;
  const unsigned long long m64 = __ballot(vol == 64), m128 = __ballot(vol == 128),
                           m256 = __ballot(vol == 256);
  if (lane == 0) {
    volm[w] = m64;
    volm[wd + w] = m128;
    volm[2 * wd + w] = m256;
  }
}

// sum of the volumes of the blocks set in word m of mask word index w
__device__ inline int64_t masked_volume(unsigned long long m, const unsigned long long* volm,
                                        int wd, int w) {
  return 64 * (int64_t)__popcll(m & volm[w]) + 128 * (int64_t)__popcll(m & volm[wd + w]) +
         256 * (int64_t)__popcll(m & volm[2 * wd + w]);
}

// Each row's selected key blocks in ascending order from its mask, and the
// row's attention cost B_i * sum_{j in S_i} B_j.  Thread t takes word t
// (wd <= 256): one prefix over the words' popcounts places every thread's
// output in LDS, which is then stored contiguously.
__global__ __launch_bounds__(kSelThreads) void k_select_emit(
    const unsigned long long* __restrict__ mask, int wd, int64_t g0,
    const int64_t* __restrict__ row_ptr, int64_t cap, const unsigned long long* __restrict__ volm,
    const uint8_t* __restrict__ blk_shape, int32_t* __restrict__ col_idx,
    int64_t* __restrict__ row_cost) {
  // block indices of a register-path row are below kSelRegMax <= 2^16: 16 bits
  // each, so that 32 KB of LDS leaves room for four work-groups per CU
  static_assert(kSelRegMax <= 65536, "16-bit list staging");
  __shared__ uint16_t sout[kSelRegMax];
  __shared__ int sh[kSelThreads / 64];
  __shared__ int64_t sh_cost[kSelThreads / 64];
  const int i = blockIdx.x, tid = threadIdx.x;
  const int64_t g = g0 + i;
  unsigned long long m = tid < wd ? mask[(int64_t)i * wd + tid] : 0ull;
  const int64_t cost = tid < wd ? masked_volume(m, volm, wd, tid) : 0;
  int total;
  int pos = block_excl_scan_i32(__popcll(m), sh, &total);
  while (m) {
    sout[pos++] = (uint16_t)(64 * tid + __builtin_ctzll(m));
    m &= m - 1;
  }
  __syncthreads();
  const int64_t base = row_ptr[g];
  if (base + total <= cap)
    for (int e = tid; e < total; e += kSelThreads) col_idx[base + e] = sout[e];
  const int64_t c = block_sum<int64_t>(cost, sh_cost);
  if (tid == 0) row_cost[g] = c * (int64_t)volume_of_id(block_shape_at(blk_shape, g));
}

// The mask of a row from its ascending list (rows longer than the register
// path holds): thread t builds the words t, t + 256, ..; a word's entries
// are found by a binary search for its first block.  A row whose list did
// not fit the workspace gets an empty mask.
__global__ __launch_bounds__(kSelThreads) void k_list_mask(
    const int64_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t g0,
    int wd, int64_t cap, unsigned long long* __restrict__ mask) {
  const int i = blockIdx.x;
  const int64_t a = row_ptr[g0 + i], e = row_ptr[g0 + i + 1];
  const bool ok = e <= cap;
  for (int w = threadIdx.x; w < wd; w += kSelThreads) {
    unsigned long long word = 0;
    if (ok) {
      int64_t lo = a, hi = e;
      while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (col_idx[mid] < 64 * w)
          lo = mid + 1;
        else
          hi = mid;
      }
      for (int64_t q = lo; q < e && col_idx[q] < 64 * w + 64; q++)
        word |= 1ull << (col_idx[q] - 64 * w);
    }
    mask[(int64_t)i * wd + w] = word;
  }
}

// Key-major transpose of one head's selection masks, by tiles of 64 query
// rows x 64 key columns: lane r holds row i0 + r's mask word of the tile,
// and one ballot per column gives that column's rows.  The counting pass
// stores per (row tile, column) the column's row count and the sum of those
// rows' volumes; the fill pass writes each column's rows of the tile in
// ascending order at the column's offset, one store instruction per column.
// No atomics: the result does not depend on the schedule.  Positions past
// the workspace's capacity are not written (the plan then reports it).
constexpr int kMtWords = 4;  // column words per wave
template <bool kFill>
__global__ __launch_bounds__(256) void k_mask_tr(
    const unsigned long long* __restrict__ mask, int wd, int n, int64_t g0,
    const unsigned long long* __restrict__ volm, const int64_t* __restrict__ colt_ptr,
    int32_t* __restrict__ tile_cnt, int32_t* __restrict__ tile_cost, int64_t cap,
    int32_t* __restrict__ colt_idx) {
  const int rt = blockIdx.x, i0 = rt * 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = i0 + lane;
  const int cw0 = (blockIdx.y * 4 + wv) * kMtWords;
  for (int k = 0; k < kMtWords; k++) {
    const int c = cw0 + k;
    if (c >= wd) break;
    const unsigned long long m = row < n ? mask[(int64_t)row * wd + c] : 0ull;
    const int col = 64 * c + lane;
    if (!kFill) {
      unsigned long long cm = 0;
#pragma unroll
      for (int b = 0; b < 64; b++) {
        const unsigned long long bal = __ballot((m >> b) & 1ull);
        if (lane == b) cm = bal;
      }
      if (col < n) {
        tile_cnt[(int64_t)rt * n + col] = __popcll(cm);
        tile_cost[(int64_t)rt * n + col] = (int32_t)masked_volume(cm, volm, wd, rt);
      }
    } else {
      const int64_t cpos = col < n ? colt_ptr[g0 + col] + tile_cnt[(int64_t)rt * n + col] : 0;
      const uint32_t plo = (uint32_t)cpos, phi = (uint32_t)(cpos >> 32);
#pragma unroll
      for (int b = 0; b < 64; b++) {
        const bool bit = (m >> b) & 1ull;
        const unsigned long long bal = __ballot(bit);
        if (bal == 0ull) continue;
        const int64_t base = (int64_t)(((uint64_t)__builtin_amdgcn_readlane(phi, b) << 32) |
                                       (uint32_t)__builtin_amdgcn_readlane(plo, b));
        const int64_t pos = base + __builtin_amdgcn_mbcnt_hi(
                                       (uint32_t)(bal >> 32),
                                       __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (bit && pos < cap) colt_idx[pos] = row;
      }
    }
  }
}

// per column: turn the row-tile counts into output positions relative to the
// column's start (at most n, so they fit in 32 bits at any nnz), the
// column's total, and its cost B_j * sum_{i: j in S_i} B_i.  64 columns per
// work-group, four threads per column, each over a quarter of the row tiles.
__global__ __launch_bounds__(256) void k_colt_offsets(int n, int nch, int64_t g0,
                                                      int32_t* __restrict__ chunk_cnt,
                                                      const int32_t* __restrict__ chunk_cost,
                                                      const uint8_t* __restrict__ blk_shape,
                                                      int32_t* __restrict__ colt_cnt,
                                                      int64_t* __restrict__ colt_cost) {
  __shared__ int32_t part[4][64];
  __shared__ int64_t pcost[4][64];
  const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + c;
  const int r0 = q * nch / 4, r1 = (q + 1) * nch / 4;
  int32_t s = 0;
  int64_t cost = 0;
  if (j < n)
    for (int r = r0; r < r1; r++) {
      s += chunk_cnt[(int64_t)r * n + j];
      cost += chunk_cost[(int64_t)r * n + j];
    }
  part[q][c] = s;
  pcost[q][c] = cost;
  __syncthreads();
  int32_t run = 0;
  for (int k = 0; k < q; k++) run += part[k][c];
  if (j >= n) return;
  for (int r = r0; r < r1; r++) {
    const int32_t t = chunk_cnt[(int64_t)r * n + j];
    chunk_cnt[(int64_t)r * n + j] = run;
    run += t;
  }
  if (q == 3) {
    colt_cnt[g0 + j] = run;
    const int64_t tc = pcost[0][c] + pcost[1][c] + pcost[2][c] + pcost[3][c];
    colt_cost[g0 + j] = tc * (int64_t)volume_of_id(block_shape_at(blk_shape, g0 + j));
  }
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
bool launch_unit_order_k(const PlanDev& P, hipStream_t st) {
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

// ============================================================ shot cuts
// Shot-cut-aware temporal zones (paper.rainbus.top "独立分析的弱点" (1)):
// the frame-difference energy e_t = mean over heads, tokens of the frame and
// channels of (V_t - V_{t-1})^2, a cut where e_t > kappa * mean_t e_t, and
// per temporal row of zones the longest block edge in time that keeps the
// blocks off the cut (the largest power of two dividing the cut's offset in
// the zone, at least 2; 8 without a cut).
//
// One block of 256 threads per (frame t >= 1, head): frame t of head h is
// the contiguous run of H*W*D elements at (h*N + t*H*W)*D.  Each thread reads
// both frames in 16-byte vectors (a fixed strided set of them) and keeps four
// fp64 partial sums, element e of a vector going to sum e % 4, in order; then
// the four in order and a fixed tree over the threads.
__device__ inline void energy_add(double (&s)[4], int k, float a, float b) {
  const double d = (double)a - (double)b;
  s[k] = s[k] + d * d;
}
template <int DT>
__global__ __launch_bounds__(256) void k_frame_energy(const void* __restrict__ v, int64_t N,
                                                      int64_t HW, int D, int heads,
                                                      double* __restrict__ part) {
  __shared__ double red[256];
  const int t = blockIdx.x + 1, h = blockIdx.y;
  const int64_t fe = HW * D;
  const int64_t cur = ((int64_t)h * N + (int64_t)t * HW) * D;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  if (DT == 1) {
    // D is a multiple of 8, so each frame is a whole number of 16-byte vectors
    const uint4* pa = (const uint4*)((const uint16_t*)v + cur);
    const uint4* pb = (const uint4*)((const uint16_t*)v + cur - fe);
    const int64_t nv = fe / 8;
#pragma unroll 4
    for (int64_t i = threadIdx.x; i < nv; i += 256) {
      const uint4 x = pa[i], y = pb[i];
      const uint32_t xa[4] = {x.x, x.y, x.z, x.w}, ya[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int q = 0; q < 4; q++) {
        energy_add(s, (2 * q) & 3, __uint_as_float(xa[q] << 16), __uint_as_float(ya[q] << 16));
        energy_add(s, (2 * q + 1) & 3, __uint_as_float(xa[q] & 0xffff0000u),
                   __uint_as_float(ya[q] & 0xffff0000u));
      }
    }
  } else {
    const float4* pa = (const float4*)((const float*)v + cur);
    const float4* pb = (const float4*)((const float*)v + cur - fe);
    const int64_t nv = fe / 4;
#pragma unroll 4
    for (int64_t i = threadIdx.x; i < nv; i += 256) {
      const float4 x = pa[i], y = pb[i];
      energy_add(s, 0, x.x, y.x);
      energy_add(s, 1, x.y, y.y);
      energy_add(s, 2, x.z, y.z);
      energy_add(s, 3, x.w, y.w);
    }
  }
  red[threadIdx.x] = ((s[0] + s[1]) + s[2]) + s[3];
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] = red[threadIdx.x] + red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[(int64_t)t * heads + h] = red[0];
}

// One block: thread t sums frame t's heads in order (frames t, t + 256, ...),
// then thread 0 takes the mean over frames, the cut decisions and the
// per-row caps.
__global__ __launch_bounds__(256) void k_cuts(const double* __restrict__ part, int T, int heads,
                                              double denom, float kappa,
                                              double* __restrict__ energy,
                                              uint8_t* __restrict__ cuts,
                                              int32_t* __restrict__ zt_cap) {
  for (int t = threadIdx.x; t < T; t += blockDim.x) {
    double e = 0.0;
    if (t > 0)
      for (int h = 0; h < heads; h++) e = e + part[(int64_t)t * heads + h];
    energy[t] = e / denom;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  double mean = 0.0;
  for (int t = 1; t < T; t++) mean = mean + energy[t];
  mean = T > 1 ? mean / (double)(T - 1) : 0.0;
  cuts[0] = 0;
  for (int t = 1; t < T; t++) cuts[t] = (kappa > 0.0f && energy[t] > (double)kappa * mean) ? 1 : 0;
  for (int zt = 0; zt < T / 8; zt++) {
    int cap = 8;
    for (int c = 1; c < 8; c++) {
      if (!cuts[8 * zt + c]) continue;
      int p = c & (-c);
      p = p < 2 ? 2 : p;
      cap = p < cap ? p : cap;
    }
    zt_cap[zt] = cap;
  }
}

bool launch_cuts(const PlanDev& P, const void* v, float kappa, hipStream_t st) {
  const int64_t HW = (int64_t)P.H * P.W;
  if (P.T > 1) {
    dim3 grid((unsigned)(P.T - 1), (unsigned)P.heads), block(256);
    if (P.dtype == PRISM_BF16)
      hipLaunchKernelGGL((k_frame_energy<1>), grid, block, 0, st, v, P.N, HW, P.D, P.heads,
                         P.cut_part);
    else
      hipLaunchKernelGGL((k_frame_energy<0>), grid, block, 0, st, v, P.N, HW, P.D, P.heads,
                         P.cut_part);
  }
  const double denom = ((double)P.heads * (double)HW) * (double)P.D;
  hipLaunchKernelGGL(k_cuts, dim3(1), dim3(256), 0, st, P.cut_part, P.T, P.heads, denom, kappa,
                     P.cut_energy, P.cuts, P.zt_cap);
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
                     P.Z, c.eps, c.tau128, c.tau256, c.volume_mask, fixed_id, c.shape_map,
                     c.alpha, c.cut_threshold > 0.0f ? P.zt_cap : nullptr,
                     (P.H / 8) * (P.W / 8), P.shape_id,
                     P.zone_base, P.nblk);
  return hipGetLastError() == hipSuccess;
}

bool launch_pool(const PlanDev& P, const void* q, const void* k, hipStream_t st) {
  dim3 grid(P.heads * P.Z), block(512);
#define PP_ARGS                                                                          \
  q, k, P.H, P.W, P.Z, P.N, P.shape_id, P.zone_base, P.blk_off, P.blk_start, P.blk_org, \
      P.blk_shape, P.blk_head, P.qbar, P.kbar, P.qgrid, P.kgrid, P.qlo, P.klo, P.qexp, P.kexp
  if (P.dtype == PRISM_BF16 && P.D == 128)
    hipLaunchKernelGGL((k_pool<1, 2>), grid, block, 0, st, PP_ARGS);
  else if (P.dtype == PRISM_BF16 && P.D == 64)
    hipLaunchKernelGGL((k_pool<1, 1>), grid, block, 0, st, PP_ARGS);
  else if (P.dtype == PRISM_F32 && P.D == 64)
    hipLaunchKernelGGL((k_pool<0, 1>), grid, block, 0, st, PP_ARGS);
  else if (P.dtype == PRISM_F32 && P.D == 128)
    hipLaunchKernelGGL((k_pool<0, 2>), grid, block, 0, st, PP_ARGS);
  else
    return false;
#undef PP_ARGS
  return hipGetLastError() == hipSuccess;
}

bool launch_relayout(const PlanDev& P, const void* a, const void* b, const float* fa,
                     const float* fb, uint16_t* ap, uint16_t* bp, float* fap, float* fbp,
                     hipStream_t st) {
  if (!(P.dtype == PRISM_BF16 && P.D == 128)) return false;
  const int64_t rows = P.heads * P.N;
  hipLaunchKernelGGL(k_relayout, dim3((unsigned)((rows + 31) / 32)), dim3(512), 0, st,
                     (const uint16_t*)a, (const uint16_t*)b, fa, fb, P.shape_id, P.H, P.W, P.Z,
                     P.N, rows, ap, bp, fap, fbp);
  return hipGetLastError() == hipSuccess;
}

bool launch_block_scores(const PlanDev& P, int64_t g0, int n, float* out, hipStream_t st) {
  if (n <= 0) return true;
  float cD = (float)(1.0 / sqrt((double)P.D));
  dim3 grid((n + 127) / 128, (n + 127) / 128), block(256);
  if (P.D == 128)
    hipLaunchKernelGGL((k_block_scores<128>), grid, block, 0, st, P.qgrid, P.kgrid, P.qlo,
                       P.klo, P.qexp, P.kexp, g0, n, cD, out);
  else
    hipLaunchKernelGGL((k_block_scores<64>), grid, block, 0, st, P.qgrid, P.kgrid, P.qlo,
                       P.klo, P.qexp, P.kexp, g0, n, cD, out);
  return hipGetLastError() == hipSuccess;
}

// mask words per row of a head of n blocks
static int mask_words(int n) { return (n + 63) / 64; }

bool launch_select(const PlanDev& P, int64_t g0, int n, const prism_config& c, int last,
                   hipStream_t st) {
  const int wd = mask_words(n);
  if (n > 0)
    hipLaunchKernelGGL(k_vol_masks, dim3((unsigned)((wd + 3) / 4)), dim3(256), 0, st,
                       P.blk_shape, g0, n, wd, P.volm);
  if (n > 0 && n <= kSelRegMax) {
    hipLaunchKernelGGL(k_select_mask, dim3(n), dim3(kSelMT), 0, st, P.scores, n, g0,
                       c.top_k, c.top_k_frac, c.top_p, P.row_cnt, P.row_key, P.row_tie,
                       P.selmask, wd);
    hipLaunchKernelGGL(k_scan_rows, dim3(1), dim3(1024), 0, st, P.row_cnt, n, g0, P.row_ptr,
                       P.counters, last);
    hipLaunchKernelGGL(k_select_emit, dim3(n), dim3(kSelThreads), 0, st, P.selmask, wd, g0,
                       P.row_ptr, P.cap, P.volm, P.blk_shape, P.col_idx, P.row_cost);
  } else {
    if (n > 0)
      hipLaunchKernelGGL(k_select_count, dim3(n), dim3(kSelThreads), 0, st, P.scores, n, g0,
                         c.top_k, c.top_k_frac, c.top_p, P.row_cnt, P.row_key, P.row_tie);
    hipLaunchKernelGGL(k_scan_rows, dim3(1), dim3(1024), 0, st, P.row_cnt, n, g0, P.row_ptr,
                       P.counters, last);
    if (n > 0) {
      hipLaunchKernelGGL(k_select_fill, dim3(n), dim3(kSelThreads), 0, st, P.scores, n, g0,
                         P.row_cnt, P.row_key, P.row_tie, P.row_ptr, P.cap, P.blk_shape,
                         P.col_idx, P.row_cost);
      if (c.need_backward)
        hipLaunchKernelGGL(k_list_mask, dim3(n), dim3(kSelThreads), 0, st, P.row_ptr,
                           P.col_idx, g0, wd, P.cap, P.selmask);
    }
  }
  return hipGetLastError() == hipSuccess;
}

bool launch_transpose(const PlanDev& P, int64_t g0, int n, int last, hipStream_t st) {
  if (n <= 0) return true;
  const int wd = mask_words(n);
  const dim3 grid((unsigned)wd, (unsigned)((wd + 4 * kMtWords - 1) / (4 * kMtWords)));
  hipLaunchKernelGGL(k_mask_tr<false>, grid, dim3(256), 0, st, P.selmask, wd, n, g0, P.volm,
                     P.colt_ptr, P.chunk_cnt, P.chunk_cost, P.cap, P.colt_idx);
  hipLaunchKernelGGL(k_colt_offsets, dim3((n + 63) / 64), dim3(256), 0, st, n, wd, g0,
                     P.chunk_cnt, P.chunk_cost, P.blk_shape, P.colt_cnt, P.colt_cost);
  hipLaunchKernelGGL(k_scan_rows, dim3(1), dim3(1024), 0, st, P.colt_cnt, n, g0, P.colt_ptr,
                     P.counters + 1, last);
  hipLaunchKernelGGL(k_mask_tr<true>, grid, dim3(256), 0, st, P.selmask, wd, n, g0, P.volm,
                     P.colt_ptr, P.chunk_cnt, P.chunk_cost, P.cap, P.colt_idx);
  return hipGetLastError() == hipSuccess;
}

}  // namespace prism
