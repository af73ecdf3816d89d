/*
 * prism_oracle.c -- plain, slow CPU oracle for Prism's dynamic block-sparse
 * video self-attention ("Prism: Dynamic Sparse Attention for Native 2K Joint
 * Video-Audio Generation Model Training", arXiv 2610.05416).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with
 * the GPU library; both are written independently from the pages' formulas
 * plus the canonical readings listed in the design notes.
 *
 * Sources (page / section):
 *   [ID]  xyznot.com/id  "Metode" 1-3: sigma^2_{v,d}, r_{v,d}; g_d; B(m) via
 *         tau_128 / tau_256; l*_d in log2 space; S_i = TopK U TopP.
 *   [ZH]  paper.rainbus.top "方法步骤详情" (Algorithm 1, five stages): eps=1e-4,
 *         first layer g = r + eps, rho = spatial var + frame-difference var,
 *         max-normalised; 16 candidates, edges {2,4,8}; block-contiguous
 *         re-layout into 64-token tiles; P_i = softmax(Qbar Kbar^T / sqrt(D));
 *         online-softmax attention over S_i only; inverse permutation.
 *   [ZH-N] same page "技术新颖性": discrete decisions detached, gradients only
 *         through the selected blocks.
 *
 * Precision: every quantity that feeds a discrete decision (block volume,
 * block shape, selected key blocks) is computed in fp32 in one fixed,
 * written order (fused multiply-add only where written as fmaf), so that an
 * independent implementation can reproduce it bit for bit.  Attention and its
 * gradients are computed in fp64 with a plain two-pass softmax.
 *
 * Compile: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL 1

/* ------------------------------------------------------------------ */
/* element loads: dtype 0 = fp32, 1 = bf16 (raw uint16)                */
/* ------------------------------------------------------------------ */
static inline float ld(const void* x, int dtype, int64_t i) {
  if (dtype == 0) return ((const float*)x)[i];
  uint32_t u = ((uint32_t)((const uint16_t*)x)[i]) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------------ */
/* candidate block shapes [ZH]: edges in {2,4,8}, product B in          */
/* {64,128,256}; ids in order of B, then lexicographic (bT,bH,bW).      */
/* ------------------------------------------------------------------ */
static int cand_n = 0;
static int cand[16][4]; /* bT, bH, bW, B */

static void build_candidates(void) {
  if (cand_n) return;
  static const int edges[3] = {2, 4, 8};
  static const int vols[3] = {64, 128, 256};
  int n = 0;
  for (int vi = 0; vi < 3; vi++)
    for (int a = 0; a < 3; a++)
      for (int b = 0; b < 3; b++)
        for (int c = 0; c < 3; c++)
          if (edges[a] * edges[b] * edges[c] == vols[vi]) {
            cand[n][0] = edges[a];
            cand[n][1] = edges[b];
            cand[n][2] = edges[c];
            cand[n][3] = vols[vi];
            n++;
          }
  cand_n = n;
}

int orc_candidates(int32_t* out) {
  build_candidates();
  for (int i = 0; i < cand_n; i++)
    for (int j = 0; j < 4; j++) out[4 * i + j] = cand[i][j];
  return cand_n;
}

static int ilog2i(int x) {
  int e = 0;
  while ((1 << e) < x) e++;
  return e;
}

/* ------------------------------------------------------------------ */
/* fixed-order reductions                                              */
/* ------------------------------------------------------------------ */

/* Sum over channels: channel c belongs to lane c / (D/64) of 64 lanes; each
 * lane first adds its own channels in ascending order, then the 64 lane
 * partials are combined by a butterfly: for offsets 32,16,8,4,2,1 every lane
 * l takes (its value) + (value of lane l xor offset). */
static float channel_sum(const float* s, int D) {
  float lane[64], nxt[64];
  int cpl = D / 64;
  for (int l = 0; l < 64; l++) {
    float a = s[l * cpl];
    for (int k = 1; k < cpl; k++) a = a + s[l * cpl + k];
    lane[l] = a;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    for (int l = 0; l < 64; l++) nxt[l] = lane[l] + lane[l ^ off];
    memcpy(lane, nxt, sizeof(lane));
  }
  return lane[0];
}

/* population variance of 8 profile samples, two-pass [ID] eq. for sigma^2 */
static float var8(const float* p) {
  float mu = p[0];
  for (int i = 1; i < 8; i++) mu = mu + p[i];
  mu = mu * 0.125f;
  float acc = 0.0f;
  for (int i = 0; i < 8; i++) {
    float d = p[i] - mu;
    acc = fmaf(d, d, acc);
  }
  return acc * 0.125f;
}

/* Per-channel zone statistics of one 8x8x8 zone (x indexed [t][y][w]).
 * out[0..2] = directional variance of the axis profiles along T, H, W
 *             ([ID] sigma^2_{v,d}: the profile along axis d averages the
 *             other two axes; its 8 samples are centred on their own mean);
 * out[3]    = intra-zone spatial variance: per frame t the variance over the
 *             64 (h,w) positions, averaged over the 8 frames [ZH];
 * out[4]    = temporal frame-difference variance: the variance of the 7x64
 *             differences x[t+1]-x[t], written as the mean within-pair
 *             variance plus the variance of the 7 pair means (the two are
 *             equal in exact arithmetic) [ZH].                            */
static void zone_channel_stats(const float x[8][8][8], float out[5]) {
  float Lw[8][8], Cy[8][8], PT[8], PH[8], PW[8];
  for (int t = 0; t < 8; t++) {
    for (int y = 0; y < 8; y++) {
      float a = x[t][y][0];
      for (int w = 1; w < 8; w++) a = a + x[t][y][w];
      Lw[t][y] = a;
    }
    for (int w = 0; w < 8; w++) {
      float a = x[t][0][w];
      for (int y = 1; y < 8; y++) a = a + x[t][y][w];
      Cy[t][w] = a;
    }
    float ss = Lw[t][0];
    for (int y = 1; y < 8; y++) ss = ss + Lw[t][y];
    PT[t] = ss * 0.015625f;
  }
  for (int y = 0; y < 8; y++) {
    float a = Lw[0][y];
    for (int t = 1; t < 8; t++) a = a + Lw[t][y];
    PH[y] = a * 0.015625f;
  }
  for (int w = 0; w < 8; w++) {
    float a = Cy[0][w];
    for (int t = 1; t < 8; t++) a = a + Cy[t][w];
    PW[w] = a * 0.015625f;
  }
  out[0] = var8(PT);
  out[1] = var8(PH);
  out[2] = var8(PW);

  /* spatial variance per frame, mean over frames */
  float sv = 0.0f;
  for (int t = 0; t < 8; t++) {
    float m = PT[t];
    float acc = 0.0f;
    for (int y = 0; y < 8; y++)
      for (int w = 0; w < 8; w++) {
        float d = x[t][y][w] - m;
        acc = fmaf(d, d, acc);
      }
    float vt = acc * 0.015625f;
    sv = (t == 0) ? vt : sv + vt;
  }
  out[3] = sv * 0.125f;

  /* frame-difference variance */
  float dm[7], within = 0.0f;
  for (int t = 0; t < 7; t++) {
    float dd[64];
    for (int y = 0; y < 8; y++)
      for (int w = 0; w < 8; w++) dd[y * 8 + w] = x[t + 1][y][w] - x[t][y][w];
    float s = dd[0];
    for (int i = 1; i < 64; i++) s = s + dd[i];
    dm[t] = s * 0.015625f;
    float acc = 0.0f;
    for (int i = 0; i < 64; i++) {
      float e = dd[i] - dm[t];
      acc = fmaf(e, e, acc);
    }
    float dv = acc * 0.015625f;
    within = (t == 0) ? dv : within + dv;
  }
  within = within / 7.0f;
  float mu = dm[0];
  for (int t = 1; t < 7; t++) mu = mu + dm[t];
  mu = mu / 7.0f;
  float acc = 0.0f;
  for (int t = 0; t < 7; t++) {
    float e = dm[t] - mu;
    acc = fmaf(e, e, acc);
  }
  out[4] = within + acc / 7.0f;
}

/* ------------------------------------------------------------------ */
/* stage 1a: video zone statistics [ID] 1, [ZH] stage one               */
/* out[h][m][5] = sigma2_T, sigma2_H, sigma2_W, SV, TV (channel means)   */
/* ------------------------------------------------------------------ */
int orc_zone_stats(const void* v, int dtype, int T, int H, int W, int heads, int D,
                   float* out) {
  if (T % 8 || H % 8 || W % 8 || (D != 64 && D != 128)) return OR_EINVAL;
  int zT = T / 8, zH = H / 8, zW = W / 8, Z = zT * zH * zW;
  int64_t N = (int64_t)T * H * W;
#pragma omp parallel for schedule(dynamic)
  for (int64_t hm = 0; hm < (int64_t)heads * Z; hm++) {
    int h = (int)(hm / Z), m = (int)(hm % Z);
    int mt = m / (zH * zW), mh = (m / zW) % zH, mw = m % zW;
    float per_c[5][128];
    float x[8][8][8];
    for (int c = 0; c < D; c++) {
      for (int t = 0; t < 8; t++)
        for (int y = 0; y < 8; y++)
          for (int w = 0; w < 8; w++) {
            int64_t n = ((int64_t)(mt * 8 + t) * H + (mh * 8 + y)) * W + (mw * 8 + w);
            x[t][y][w] = ld(v, dtype, ((int64_t)h * N + n) * D + c);
          }
      float st[5];
      zone_channel_stats(x, st);
      for (int s = 0; s < 5; s++) per_c[s][c] = st[s];
    }
    float invD = 1.0f / (float)D; /* exact: D is a power of two */
    for (int s = 0; s < 5; s++) out[hm * 5 + s] = channel_sum(per_c[s], D) * invD;
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* stage 1b: audio statistics from the A->V norm map a[t][h][w]  [ID] 1  */
/* out[m][4] = directional variances along T,H,W and the zone mean.      */
/* ------------------------------------------------------------------ */
int orc_audio_stats(const float* a, int T, int H, int W, float* out) {
  if (T % 8 || H % 8 || W % 8) return OR_EINVAL;
  int zT = T / 8, zH = H / 8, zW = W / 8, Z = zT * zH * zW;
#pragma omp parallel for schedule(static)
  for (int m = 0; m < Z; m++) {
    int mt = m / (zH * zW), mh = (m / zW) % zH, mw = m % zW;
    float x[8][8][8];
    for (int t = 0; t < 8; t++)
      for (int y = 0; y < 8; y++)
        for (int w = 0; w < 8; w++)
          x[t][y][w] = a[((int64_t)(mt * 8 + t) * H + (mh * 8 + y)) * W + (mw * 8 + w)];
    float st[5];
    zone_channel_stats(x, st);
    /* zone mean = mean of the temporal profile (same fixed order as var8) */
    float Lw, ss, PT[8];
    for (int t = 0; t < 8; t++) {
      ss = 0.0f;
      for (int y = 0; y < 8; y++) {
        Lw = x[t][y][0];
        for (int w = 1; w < 8; w++) Lw = Lw + x[t][y][w];
        ss = (y == 0) ? Lw : ss + Lw;
      }
      PT[t] = ss * 0.015625f;
    }
    float mu = PT[0];
    for (int i = 1; i < 8; i++) mu = mu + PT[i];
    out[m * 4 + 0] = st[0];
    out[m * 4 + 1] = st[1];
    out[m * 4 + 2] = st[2];
    out[m * 4 + 3] = mu * 0.125f;
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* stage 1c/1d: indicator g_d, volume B, shape                          */
/* ------------------------------------------------------------------ */

/* ratio x_d / (x_T + x_H + x_W); an all-zero triple gives 1/3 each */
static void ratio3(const float* x, float* r) {
  float s = (x[0] + x[1]) + x[2];
  if (s > 0.0f) {
    r[0] = x[0] / s;
    r[1] = x[1] / s;
    r[2] = x[2] / s;
  } else {
    r[0] = r[1] = r[2] = 1.0f / 3.0f;
  }
}

/* Continuous optimum in log2 space [ID] 2:
 *   l*_d = -1/2 log2 g_d + 1/3 (S + 1/2 (log2 g_T + log2 g_H + log2 g_W)). */
void orc_lstar(const float* g, int B, double* l) {
  double S = (double)ilog2i(B);
  double lg[3] = {log2((double)g[0]), log2((double)g[1]), log2((double)g[2])};
  double c = (S + 0.5 * (lg[0] + lg[1] + lg[2])) / 3.0;
  for (int d = 0; d < 3; d++) l[d] = -0.5 * lg[d] + c;
}

/* Is candidate a strictly nearer to l* than candidate b (Euclidean, [ID] 2)?
 * Because sum_d l*_d = S = sum_d e_d for every candidate e = log2(b),
 *   |l* - e|^2 = const + sum_d e_d^2 + sum_d e_d log2 g_d,
 * so a is nearer iff  prod_d g_d^(ea_d - eb_d) < 2^(|eb|^2 - |ea|^2).
 * Exponent differences lie in [-2,2] and sum to zero, so each side is a
 * product of at most two fp32 numbers times a power of two: exact in fp64,
 * and the comparison is the exact comparison of the real distances. */
static int nearer(const float* g, int a, int b) {
  int ea[3], eb[3];
  int qa = 0, qb = 0;
  for (int d = 0; d < 3; d++) {
    ea[d] = ilog2i(cand[a][d]);
    eb[d] = ilog2i(cand[b][d]);
    qa += ea[d] * ea[d];
    qb += eb[d] * eb[d];
  }
  double lhs = 1.0, rhs = 1.0;
  for (int d = 0; d < 3; d++) {
    int k = ea[d] - eb[d];
    for (; k > 0; k--) lhs = lhs * (double)g[d];
    for (; k < 0; k++) rhs = rhs * (double)g[d];
  }
  rhs = ldexp(rhs, qb - qa);
  return lhs < rhs;
}

/* nearest candidate of volume B to l*(g); exact ties go to the lower id */
int orc_nearest_shape(const float* g, int B) {
  build_candidates();
  int best = -1;
  for (int i = 0; i < cand_n; i++) {
    if (cand[i][3] != B) continue;
    if (best < 0 || nearer(g, i, best)) best = i;
  }
  return best;
}

/* ------------------------------------------------------------------ */
/* Shape-mapping variants.  paper.rainbus.top "技术新颖性" (ablation of     */
/* Table 10) names b_d ~ g_d^(-alpha) with alpha in {1/3, 1/2, 2},        */
/* Softmax, Rank and Entropy mappings and an Isotropic baseline, without  */
/* formulas; the readings below (listed in the design notes) give each a  */
/* target point l in log2 space with sum_d l_d = S = log2 B, and the      */
/* shape is the candidate of volume B nearest to l (Euclidean, ties to    */
/* the lower id), as for alpha = 1/2 [ID] 2.                              */
/*   power(alpha): l_d = -alpha log2 g_d + (S + alpha sum log2 g) / 3     */
/*   isotropic:    l_d = S / 3                                            */
/*   softmax:      l_d = S softmax(-g)_d                                  */
/*   rank:         l_d = S / 3 + rank_d - 1, rank_d = 0 for the largest   */
/*                 g (ties: earlier axis first)                           */
/*   entropy:      l_d = S i_d / sum i, i_d = -ln(g_d / sum g) (the       */
/*                 self-information of each axis' share of g)             */
/* alpha = 1/2 keeps the exact product-form test above.  Every other      */
/* target is evaluated in fp64 with plain operations in the written      */
/* order, with the logarithm and exponential below, so that an           */
/* independent implementation reproduces the decisions bit for bit.      */
/* ------------------------------------------------------------------ */
#define MAP_POWER 0
#define MAP_ISOTROPIC 1
#define MAP_SOFTMAX 2
#define MAP_RANK 3
#define MAP_ENTROPY 4

static const double W_LN2 = 0.69314718055994530942;
static const double W_INV_LN2 = 1.4426950408889634074;

/* x = m 2^e with m in [1, 2), exactly */
static double split_pow2(double x, int* e) {
  double m = frexp(x, e); /* [0.5, 1) */
  *e -= 1;
  return m * 2.0;
}

/* ln m for m in [1, 2): z = (m - 1) / (m + 1), ln m = 2 atanh z =
 * 2 z sum_{k=0}^{16} z^(2k) / (2k + 1), Horner in z^2. */
static double ln_mant(double m) {
  double z = (m - 1.0) / (m + 1.0);
  double z2 = z * z;
  double s = 1.0 / 33.0;
  for (int k = 15; k >= 0; k--) s = s * z2 + 1.0 / (double)(2 * k + 1);
  return (2.0 * z) * s;
}

double orc_wlog2(double x) {
  int e;
  double m = split_pow2(x, &e);
  return (double)e + ln_mant(m) * W_INV_LN2;
}

double orc_wln(double x) {
  int e;
  double m = split_pow2(x, &e);
  return (double)e * W_LN2 + ln_mant(m);
}

/* e^x: y = x log2 e, k = rint(y), f = y - k in [-1/2, 1/2],
 * 2^f = sum_{n=0}^{14} (f ln 2)^n / n! with c_n = c_{n-1} ln2 / n, Horner. */
double orc_wexp(double x) {
  double y = x * W_INV_LN2;
  double k = rint(y);
  double f = y - k;
  double cn[15];
  cn[0] = 1.0;
  for (int n = 1; n < 15; n++) cn[n] = cn[n - 1] * W_LN2 / (double)n;
  double p = cn[14];
  for (int n = 13; n >= 0; n--) p = p * f + cn[n];
  return ldexp(p, (int)k);
}

/* target point l (fp64) of a mapping; 0 on success */
int orc_map_target(const float* g, int B, int map, float alpha, double* l) {
  double S = (double)ilog2i(B);
  if (map == MAP_POWER) {
    double a = (double)alpha;
    double L[3] = {orc_wlog2((double)g[0]), orc_wlog2((double)g[1]), orc_wlog2((double)g[2])};
    double Ls = (L[0] + L[1]) + L[2];
    double c = (S + a * Ls) / 3.0;
    for (int d = 0; d < 3; d++) l[d] = (-a) * L[d] + c;
  } else if (map == MAP_ISOTROPIC) {
    for (int d = 0; d < 3; d++) l[d] = S / 3.0;
  } else if (map == MAP_SOFTMAX) {
    double gm = (double)g[0];
    for (int d = 1; d < 3; d++)
      if ((double)g[d] < gm) gm = (double)g[d];
    double w[3];
    for (int d = 0; d < 3; d++) w[d] = orc_wexp(gm - (double)g[d]); /* exp(-g_d) / exp(-min g) */
    double ws = (w[0] + w[1]) + w[2];
    for (int d = 0; d < 3; d++) l[d] = S * (w[d] / ws);
  } else if (map == MAP_RANK) {
    for (int d = 0; d < 3; d++) {
      int r = 0;
      for (int e = 0; e < 3; e++)
        if (g[e] > g[d] || (g[e] == g[d] && e < d)) r++;
      l[d] = S / 3.0 + (double)(r - 1);
    }
  } else if (map == MAP_ENTROPY) {
    double gs = ((double)g[0] + (double)g[1]) + (double)g[2];
    double lgs = orc_wln(gs);
    double inf[3];
    for (int d = 0; d < 3; d++) inf[d] = lgs - orc_wln((double)g[d]);
    double is = (inf[0] + inf[1]) + inf[2];
    for (int d = 0; d < 3; d++) l[d] = S * (inf[d] / is);
  } else {
    return OR_EINVAL;
  }
  return OR_OK;
}

/* nearest candidate of volume B to the mapping's target; exact ties go to
 * the lower id.  power with alpha = 1/2 is the exact test above. */
int orc_nearest_shape_map(const float* g, int B, int map, float alpha) {
  build_candidates();
  if (map == MAP_POWER && alpha == 0.5f) return orc_nearest_shape(g, B);
  double l[3];
  if (orc_map_target(g, B, map, alpha, l) != OR_OK) return -1;
  int best = -1;
  double bestd = 0.0;
  for (int i = 0; i < cand_n; i++) {
    if (cand[i][3] != B) continue;
    double d0 = l[0] - (double)ilog2i(cand[i][0]);
    double d1 = l[1] - (double)ilog2i(cand[i][1]);
    double d2 = l[2] - (double)ilog2i(cand[i][2]);
    double dist = (d0 * d0 + d1 * d1) + d2 * d2;
    if (best < 0 || dist < bestd) {
      best = i;
      bestd = dist;
    }
  }
  return best;
}

/* nearest candidate of volume B with b_T <= cap (a zone split by a shot
 * cut); the same comparisons as without the cap, over fewer candidates */
static int orc_nearest_capped(const float* g, int B, int map, float alpha, int cap) {
  build_candidates();
  int best = -1;
  if (map == MAP_POWER && alpha == 0.5f) {
    for (int i = 0; i < cand_n; i++) {
      if (cand[i][3] != B || cand[i][0] > cap) continue;
      if (best < 0 || nearer(g, i, best)) best = i;
    }
    return best;
  }
  double l[3];
  if (orc_map_target(g, B, map, alpha, l) != OR_OK) return -1;
  double bestd = 0.0;
  for (int i = 0; i < cand_n; i++) {
    if (cand[i][3] != B || cand[i][0] > cap) continue;
    double d0 = l[0] - (double)ilog2i(cand[i][0]);
    double d1 = l[1] - (double)ilog2i(cand[i][1]);
    double d2 = l[2] - (double)ilog2i(cand[i][2]);
    double dist = (d0 * d0 + d1 * d1) + d2 * d2;
    if (best < 0 || dist < bestd) {
      best = i;
      bestd = dist;
    }
  }
  return best;
}

/* Volume tier from rho = rho_raw / max rho_raw [ZH]:
 * rho >= tau128 -> 64, else rho >= tau256 -> 128, else 256.
 * A head whose zones all have zero density takes 256 everywhere.
 * Volumes outside volume_mask (bit0=64, bit1=128, bit2=256) move to the
 * nearest allowed volume, the smaller one on a tie. */
static int volume_of(float rho_raw, float rho_max, float tau128, float tau256,
                     uint32_t mask) {
  int B;
  if (!(rho_max > 0.0f)) {
    B = 256;
  } else {
    float rho = rho_raw / rho_max;
    B = (rho >= tau128) ? 64 : (rho >= tau256) ? 128 : 256;
  }
  int bit = ilog2i(B) - 6;
  if (mask & (1u << bit)) return B;
  for (int dist = 1; dist <= 2; dist++) {
    if (bit - dist >= 0 && (mask & (1u << (bit - dist)))) return 64 << (bit - dist);
    if (bit + dist <= 2 && (mask & (1u << (bit + dist)))) return 64 << (bit + dist);
  }
  return B;
}

/* vstats [heads][Z][5] from orc_zone_stats; astats [Z][4] or NULL (first
 * layer).  Writes shape ids [heads][Z]; optional g [heads][Z][3] and
 * volume [heads][Z]. fixed_id >= 0 forces one shape everywhere; otherwise
 * map / alpha select the shape mapping (MAP_POWER with alpha = 1/2 is the
 * pages' method). */
static int orc_nearest_capped(const float* g, int B, int map, float alpha, int cap);

int orc_shapes(const float* vstats, const float* astats, int heads, int Z, float eps,
               float tau128, float tau256, uint32_t volume_mask, int fixed_id, int map,
               float alpha, const int32_t* zt_cap, int zones_per_t, uint8_t* shape_id,
               float* g_out, int32_t* vol_out) {
  build_candidates();
  if (fixed_id >= cand_n) return OR_EINVAL;
  if (map < MAP_POWER || map > MAP_ENTROPY) return OR_EINVAL;
  if ((volume_mask & 7u) == 0) return OR_EINVAL;
  /* audio coupling abar = zone mean / max zone mean (0 if all zero) */
  float amax = 0.0f;
  if (astats)
    for (int m = 0; m < Z; m++)
      if (astats[m * 4 + 3] > amax) amax = astats[m * 4 + 3];
  for (int h = 0; h < heads; h++) {
    float rmax = 0.0f;
    for (int m = 0; m < Z; m++) {
      const float* s = vstats + ((int64_t)h * Z + m) * 5;
      float rr = s[3] + s[4];
      if (rr > rmax) rmax = rr;
    }
    for (int m = 0; m < Z; m++) {
      const float* s = vstats + ((int64_t)h * Z + m) * 5;
      float r[3], g[3];
      ratio3(s, r);
      if (astats && amax > 0.0f) {
        float abar = astats[m * 4 + 3] / amax;
        float va[3];
        ratio3(astats + m * 4, va);
        for (int d = 0; d < 3; d++) g[d] = (r[d] + abar * va[d]) + eps;
      } else {
        for (int d = 0; d < 3; d++) g[d] = r[d] + eps;
      }
      int id, B;
      if (fixed_id >= 0) {
        id = fixed_id;
        B = cand[id][3];
      } else {
        B = volume_of(s[3] + s[4], rmax, tau128, tau256, volume_mask);
        int cap = zt_cap ? zt_cap[m / zones_per_t] : 8;
        if (cap >= 8) {
          id = orc_nearest_shape_map(g, B, map, alpha);
        } else {
          /* a shot cut inside the zone: at most 128 tokens when b_T = 2 */
          if (cap == 2 && B > 128) B = 128;
          id = orc_nearest_capped(g, B, map, alpha, cap);
        }
      }
      shape_id[(int64_t)h * Z + m] = (uint8_t)id;
      if (g_out)
        for (int d = 0; d < 3; d++) g_out[((int64_t)h * Z + m) * 3 + d] = g[d];
      if (vol_out) vol_out[(int64_t)h * Z + m] = B;
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* stage 2: zone-aware re-layout [ZH] stage two                          */
/* Zone m occupies permuted rows [512 m, 512 m + 512) of its head; inside */
/* it the blocks follow in raster order over the block grid (bw fastest), */
/* and each block's tokens in raster order (t, h, w).                     */
/* ------------------------------------------------------------------ */
static int64_t token_of(int T, int H, int W, int shape, int m, int r) {
  (void)T;
  int zH = H / 8, zW = W / 8;
  int mt = m / (zH * zW), mh = (m / zW) % zH, mw = m % zW;
  int bT = cand[shape][0], bH = cand[shape][1], bW = cand[shape][2], B = cand[shape][3];
  int nbH = 8 / bH, nbW = 8 / bW;
  int jl = r / B, u = r % B;
  int jt = jl / (nbH * nbW), jh = (jl / nbW) % nbH, jw = jl % nbW;
  int ut = u / (bH * bW), uh = (u / bW) % bH, uw = u % bW;
  int t = mt * 8 + jt * bT + ut, y = mh * 8 + jh * bH + uh, w = mw * 8 + jw * bW + uw;
  return ((int64_t)t * H + y) * W + w;
}

/* perm[h][p] = original token index of permuted position p */
int orc_perm_map(const uint8_t* shape_id, int T, int H, int W, int heads, int32_t* perm) {
  build_candidates();
  int Z = (T / 8) * (H / 8) * (W / 8);
  int64_t N = (int64_t)T * H * W;
  for (int h = 0; h < heads; h++)
    for (int m = 0; m < Z; m++)
      for (int r = 0; r < 512; r++)
        perm[(int64_t)h * N + 512 * m + r] =
            (int32_t)token_of(T, H, W, shape_id[(int64_t)h * Z + m], m, r);
  return OR_OK;
}

/* block table: blk_off[h] = first global block id of head h (heads+1
 * entries); per global block its start row (permuted order) and volume. */
int orc_block_table(const uint8_t* shape_id, int heads, int Z, int64_t* blk_off,
                    int32_t* blk_start, int32_t* blk_len) {
  build_candidates();
  int64_t g = 0;
  for (int h = 0; h < heads; h++) {
    blk_off[h] = g;
    for (int m = 0; m < Z; m++) {
      int B = cand[shape_id[(int64_t)h * Z + m]][3];
      for (int j = 0; j < 512 / B; j++) {
        if (blk_start) blk_start[g] = 512 * m + j * B;
        if (blk_len) blk_len[g] = B;
        g++;
      }
    }
  }
  blk_off[heads] = g;
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* stage 3a: block mean pooling [ZH] stage three (Qbar_i, Kbar_j)       */
/* per channel: each 64-token tile summed in permuted order, tile sums   */
/* added in order, times 1/B.                                            */
/* ------------------------------------------------------------------ */
int orc_pool(const void* x, int dtype, int T, int H, int W, int heads, int D,
             const uint8_t* shape_id, const int64_t* blk_off, float* xbar) {
  build_candidates();
  int Z = (T / 8) * (H / 8) * (W / 8);
  int64_t N = (int64_t)T * H * W;
#pragma omp parallel for schedule(dynamic)
  for (int64_t hm = 0; hm < (int64_t)heads * Z; hm++) {
    int h = (int)(hm / Z), m = (int)(hm % Z);
    int shape = shape_id[hm];
    int B = cand[shape][3];
    int64_t g0 = blk_off[h];
    for (int mm = 0; mm < m; mm++) g0 += 512 / cand[shape_id[(int64_t)h * Z + mm]][3];
    for (int j = 0; j < 512 / B; j++) {
      float* out = xbar + (g0 + j) * D;
      for (int c = 0; c < D; c++) {
        float blk = 0.0f;
        for (int tile = 0; tile < B / 64; tile++) {
          float ts = 0.0f;
          for (int u = 0; u < 64; u++) {
            int r = j * B + tile * 64 + u;
            int64_t n = token_of(T, H, W, shape, m, r);
            float val = ld(x, dtype, ((int64_t)h * N + n) * D + c);
            ts = (u == 0) ? val : ts + val;
          }
          blk = (tile == 0) ? ts : blk + ts;
        }
        out[c] = blk * (1.0f / (float)B);
      }
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* stage 3b: block scores on an exact integer grid, then Top-k U Top-p   */
/* ------------------------------------------------------------------ */

/* Each pooled row x is written on a two-level integer grid,
 *   x_c ~ 2^E (hi_c + 2^-8 lo_c),
 * E chosen so that max_c |x_c| 2^-E lies in [128, 256):
 *   hi_c = rint(x_c 2^-E)            in [-256, 256]
 *   lo_c = rint((x_c 2^-E - hi_c) 2^8) in [-128, 128]
 * (the subtraction is exact), so x is seen to about 17 significant bits and
 * every product of grid values is an integer the matrix cores sum exactly.
 * A zero row has E = 0, hi = lo = 0. */
int orc_quantize(const float* xbar, int64_t rows, int D, float* qgrid, float* qlo, int32_t* E) {
  for (int64_t i = 0; i < rows; i++) {
    const float* x = xbar + i * D;
    float mx = 0.0f;
    for (int c = 0; c < D; c++)
      if (fabsf(x[c]) > mx) mx = fabsf(x[c]);
    int e = 0;
    if (mx > 0.0f) {
      frexpf(mx, &e); /* mx = f 2^e, f in [0.5, 1) */
      e -= 8;
    }
    E[i] = e;
    for (int c = 0; c < D; c++) {
      float y = mx > 0.0f ? ldexpf(x[c], -e) : 0.0f;
      float hi = rintf(y);
      qgrid[i * D + c] = hi;
      if (qlo) qlo[i * D + c] = rintf(ldexpf(y - hi, 8));
    }
  }
  return OR_OK;
}

/* scores s_ij = Qbar_i . Kbar_j / sqrt(D) of query row i against the n key
 * rows on the two-level grid: with the integer dot products I_hh = hi.hi,
 * I_x = hi_i.lo_j + lo_i.hi_j and I_ll = lo.lo,
 *   J = 2^16 I_hh + 2^8 I_x + I_ll   (exact, |J| < 2^41)
 * and s = fl32(fl32(J) 2^(Ei + Ej - 16)) * fl32(1/sqrt D), fl32(J) rounded
 * once to nearest (J is exact in fp64). */
int orc_score_row(const float* qrow, const float* qlo, int32_t Ei, const float* kgrid,
                  const float* klo, const int32_t* Ek, int64_t n, int D, float* s) {
  float cD = (float)(1.0 / sqrt((double)D));
  for (int64_t j = 0; j < n; j++) {
    int64_t Ihh = 0, Ix = 0, Ill = 0;
    for (int c = 0; c < D; c++) {
      int64_t qh = (int64_t)qrow[c], ql = (int64_t)qlo[c];
      int64_t kh = (int64_t)kgrid[j * D + c], kl = (int64_t)klo[j * D + c];
      Ihh += qh * kh;
      Ix += qh * kl + ql * kh;
      Ill += ql * kl;
    }
    int64_t J = Ihh * 65536 + Ix * 256 + Ill;
    float v = ldexpf((float)(double)J, Ei + Ek[j] - 16) * cD;
    s[j] = (v == 0.0f) ? 0.0f : v;
  }
  return OR_OK;
}

/* 2^x for x <= 0: x = k + f with k = rint(x), |f| <= 1/2, and 2^f from its
 * Taylor series sum_n (f ln2)^n / n! to degree 7 (Horner, fused multiply-
 * add); coefficients are (ln 2)^n / n! rounded to fp32. */
float orc_exp2(float x) {
  static const float c[8] = {1.0f,
                             0.69314718055994530942f,
                             0.24022650695910071233f,
                             0.055504108664821579953f,
                             0.0096181291076284771620f,
                             0.0013333558146428443423f,
                             0.00015403530393381609954f,
                             0.000015252733804059840280f};
  if (!(x > -100.0f)) return 0.0f;
  float k = rintf(x);
  float f = x - k;
  float p = c[7];
  for (int i = 6; i >= 0; i--) p = fmaf(p, f, c[i]);
  return ldexpf(p, (int)k);
}

typedef struct {
  float s;
  int32_t j;
} keyed;

static int by_score_desc(const void* a, const void* b) {
  const keyed* x = (const keyed*)a;
  const keyed* y = (const keyed*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* S_i = TopK(P_i, k) U TopP(P_i, p)  [ID] 3, [ZH] stage three.
 * Keys are ordered by score, descending, ties by lower index.  P_ij is the
 * softmax of the row; for an exact cumulative test each P_ij is held as the
 * integer w_j = floor(2^32 * 2^((s_j - s_max) log2 e)) and the row total is
 * Z = sum_j w_j.  Top-p takes the shortest prefix L of that order with
 * sum_{l<=L} w >= p Z (tested as 2^32 sum >= ceil(p 2^32) Z); both sets are
 * prefixes of one order, so their union is the first max(k, L) keys.  p >= 1
 * selects every key block; p <= 0 leaves Top-k alone.  Indices are written
 * in ascending order; the return value is their count. */
int orc_select_row(const float* s, int64_t n, int64_t k, float p, int32_t* out) {
  if (n <= 0) return 0;
  if (k > n) k = n;
  if (k < 0) k = 0;
  keyed* e = (keyed*)malloc(sizeof(keyed) * n);
  for (int64_t j = 0; j < n; j++) {
    e[j].s = s[j];
    e[j].j = (int32_t)j;
  }
  qsort(e, n, sizeof(keyed), by_score_desc);
  int64_t L = 0;
  if (p >= 1.0f) {
    L = n;
  } else if (p > 0.0f) {
    const float LOG2E = 1.44269504088896340736f;
    float smax = e[0].s;
    uint64_t* w = (uint64_t*)malloc(sizeof(uint64_t) * n);
    uint64_t Z = 0;
    for (int64_t l = 0; l < n; l++) {
      float xx = (e[l].s - smax) * LOG2E;
      float y = orc_exp2(xx);
      w[l] = (uint64_t)(y * 4294967296.0f);
      Z += w[l];
    }
    uint64_t P32 = (uint64_t)ceil((double)p * 4294967296.0);
    unsigned __int128 need = (unsigned __int128)P32 * Z;
    unsigned __int128 cum = 0;
    for (L = 0; L < n;) {
      if (cum >= need) break;
      cum += (unsigned __int128)w[L] << 32;
      L++;
    }
    free(w);
  }
  int64_t cnt = k > L ? k : L;
  for (int64_t l = 0; l < cnt; l++) out[l] = e[l].j;
  qsort(out, cnt, sizeof(int32_t), cmp_i32);
  free(e);
  return (int)cnt;
}

/* ------------------------------------------------------------------ */
/* stages 4-5: attention over the selected blocks, fp64, two-pass        */
/* ([ZH] stage four: attention restricted to the key blocks in S_i; the  */
/* result equals softmax attention with all other keys masked out).      */
/* ------------------------------------------------------------------ */

/* For one query block (head h, global block gi) with selected key blocks
 * sel[0..ns): outputs per query row u (permuted order inside the block)
 * O[u][D], lse[u] (natural log of the softmax normaliser of q.k/sqrt D). */
static void attn_block(const void* q, const void* k, const void* v, int dtype, int64_t N,
                       int D, const int32_t* perm_h, int h, int32_t qstart, int32_t qlen,
                       const int32_t* sel, int ns, const int32_t* blk_start,
                       const int32_t* blk_len, int64_t goff, double* O, double* lse,
                       double* scratch) {
  double scale = 1.0 / sqrt((double)D);
  int64_t nk = 0;
  for (int a = 0; a < ns; a++) nk += blk_len[goff + sel[a]];
  for (int u = 0; u < qlen; u++) {
    int64_t nq = perm_h[qstart + u];
    double qv[128];
    for (int c = 0; c < D; c++) qv[c] = ld(q, dtype, ((int64_t)h * N + nq) * D + c);
    double mx = -INFINITY;
    int64_t idx = 0;
    for (int a = 0; a < ns; a++) {
      int64_t g = goff + sel[a];
      for (int r = 0; r < blk_len[g]; r++) {
        int64_t nk_tok = perm_h[blk_start[g] + r];
        double sc = 0.0;
        for (int c = 0; c < D; c++) sc += qv[c] * ld(k, dtype, ((int64_t)h * N + nk_tok) * D + c);
        sc *= scale;
        scratch[idx++] = sc;
        if (sc > mx) mx = sc;
      }
    }
    double sum = 0.0;
    for (int64_t i = 0; i < nk; i++) sum += exp(scratch[i] - mx);
    double* o = O + (int64_t)u * D;
    for (int c = 0; c < D; c++) o[c] = 0.0;
    idx = 0;
    for (int a = 0; a < ns; a++) {
      int64_t g = goff + sel[a];
      for (int r = 0; r < blk_len[g]; r++) {
        int64_t nk_tok = perm_h[blk_start[g] + r];
        double pr = exp(scratch[idx++] - mx) / sum;
        for (int c = 0; c < D; c++) o[c] += pr * ld(v, dtype, ((int64_t)h * N + nk_tok) * D + c);
      }
    }
    lse[u] = mx + log(sum);
  }
}

/* items: (head, local query block) pairs; sel_ptr/sel_idx: each item's
 * selected key blocks (local ids).  O_out [items][256][D], lse_out
 * [items][256], rows in permuted order within the block. */
int orc_attn_fwd(const void* q, const void* k, const void* v, int dtype, int64_t N, int D,
                 const int32_t* perm, const int64_t* blk_off, const int32_t* blk_start,
                 const int32_t* blk_len, int nitems, const int32_t* item_head,
                 const int32_t* item_blk, const int64_t* sel_ptr, const int32_t* sel_idx,
                 double* O_out, double* lse_out) {
#pragma omp parallel for schedule(dynamic)
  for (int it = 0; it < nitems; it++) {
    int h = item_head[it];
    int64_t g = blk_off[h] + item_blk[it];
    int ns = (int)(sel_ptr[it + 1] - sel_ptr[it]);
    int64_t nk = 0;
    for (int a = 0; a < ns; a++) nk += blk_len[blk_off[h] + sel_idx[sel_ptr[it] + a]];
    double* scratch = (double*)malloc(sizeof(double) * (nk + 1));
    attn_block(q, k, v, dtype, N, D, perm + (int64_t)h * N, h, blk_start[g], blk_len[g],
               sel_idx + sel_ptr[it], ns, blk_start, blk_len, blk_off[h],
               O_out + (int64_t)it * 256 * D, lse_out + (int64_t)it * 256, scratch);
    free(scratch);
  }
  return OR_OK;
}

/* Gradients with the plan held constant [ZH-N]: with s = q.k/sqrt D over the
 * selected keys, P = softmax, dP = dO.v, Delta = sum_m P dP,
 * dS = P (dP - Delta):  dQ = sum_m dS k / sqrt D,  dK = sum_n dS q / sqrt D,
 * dV = sum_n P dO.  Keys outside S_i get no gradient from row n. */

/* per query row: scores, P and Delta of one query block */
static void row_softmax_grad(const void* q, const void* k, const void* v, const void* dO,
                             int dtype, int64_t N, int D, const int32_t* perm_h, int h,
                             int64_t nq, const int32_t* sel, int ns, const int32_t* blk_start,
                             const int32_t* blk_len, int64_t goff, double* P, double* dP,
                             double* delta) {
  double scale = 1.0 / sqrt((double)D);
  double qv[128], dov[128];
  for (int c = 0; c < D; c++) {
    qv[c] = ld(q, dtype, ((int64_t)h * N + nq) * D + c);
    dov[c] = ld(dO, dtype, ((int64_t)h * N + nq) * D + c);
  }
  int64_t idx = 0;
  double mx = -INFINITY;
  for (int a = 0; a < ns; a++) {
    int64_t g = goff + sel[a];
    for (int r = 0; r < blk_len[g]; r++) {
      int64_t nk = perm_h[blk_start[g] + r];
      double sc = 0.0, dp = 0.0;
      for (int c = 0; c < D; c++) {
        sc += qv[c] * ld(k, dtype, ((int64_t)h * N + nk) * D + c);
        dp += dov[c] * ld(v, dtype, ((int64_t)h * N + nk) * D + c);
      }
      P[idx] = sc * scale;
      dP[idx] = dp;
      if (P[idx] > mx) mx = P[idx];
      idx++;
    }
  }
  double sum = 0.0;
  for (int64_t i = 0; i < idx; i++) sum += exp(P[i] - mx);
  double dl = 0.0;
  for (int64_t i = 0; i < idx; i++) {
    P[i] = exp(P[i] - mx) / sum;
    dl += P[i] * dP[i];
  }
  *delta = dl;
}

/* dQ for query-block items: dq_out [items][256][D] */
int orc_attn_bwd_q(const void* q, const void* k, const void* v, const void* dO, int dtype,
                   int64_t N, int D, const int32_t* perm, const int64_t* blk_off,
                   const int32_t* blk_start, const int32_t* blk_len, int nitems,
                   const int32_t* item_head, const int32_t* item_blk, const int64_t* sel_ptr,
                   const int32_t* sel_idx, double* dq_out) {
  double scale = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(dynamic)
  for (int it = 0; it < nitems; it++) {
    int h = item_head[it];
    int64_t goff = blk_off[h];
    int64_t g = goff + item_blk[it];
    const int32_t* sel = sel_idx + sel_ptr[it];
    int ns = (int)(sel_ptr[it + 1] - sel_ptr[it]);
    int64_t nk = 0;
    for (int a = 0; a < ns; a++) nk += blk_len[goff + sel[a]];
    double* P = (double*)malloc(sizeof(double) * (nk + 1));
    double* dP = (double*)malloc(sizeof(double) * (nk + 1));
    const int32_t* perm_h = perm + (int64_t)h * N;
    for (int u = 0; u < blk_len[g]; u++) {
      int64_t nq = perm_h[blk_start[g] + u];
      double delta;
      row_softmax_grad(q, k, v, dO, dtype, N, D, perm_h, h, nq, sel, ns, blk_start, blk_len,
                       goff, P, dP, &delta);
      double* out = dq_out + ((int64_t)it * 256 + u) * D;
      for (int c = 0; c < D; c++) out[c] = 0.0;
      int64_t idx = 0;
      for (int a = 0; a < ns; a++) {
        int64_t gk = goff + sel[a];
        for (int r = 0; r < blk_len[gk]; r++) {
          int64_t nkt = perm_h[blk_start[gk] + r];
          double ds = P[idx] * (dP[idx] - delta) * scale;
          for (int c = 0; c < D; c++) out[c] += ds * ld(k, dtype, ((int64_t)h * N + nkt) * D + c);
          idx++;
        }
      }
    }
    free(P);
    free(dP);
  }
  return OR_OK;
}

/* dK, dV for key-block items.  row_ptr/col_idx: the full selection of every
 * query block (global block ids index row_ptr; col ids are local);
 * tq_ptr/tq_idx: for each item the local query blocks whose S_i holds it.
 * dk_out, dv_out [items][256][D]. */
int orc_attn_bwd_kv(const void* q, const void* k, const void* v, const void* dO, int dtype,
                    int64_t N, int D, const int32_t* perm, const int64_t* blk_off,
                    const int32_t* blk_start, const int32_t* blk_len, const int64_t* row_ptr,
                    const int32_t* col_idx, int nitems, const int32_t* item_head,
                    const int32_t* item_blk, const int64_t* tq_ptr, const int32_t* tq_idx,
                    double* dk_out, double* dv_out) {
  double scale = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(dynamic)
  for (int it = 0; it < nitems; it++) {
    int h = item_head[it];
    int64_t goff = blk_off[h];
    int jb = item_blk[it];
    int64_t gj = goff + jb;
    const int32_t* perm_h = perm + (int64_t)h * N;
    double* dk = dk_out + (int64_t)it * 256 * D;
    double* dv = dv_out + (int64_t)it * 256 * D;
    memset(dk, 0, sizeof(double) * 256 * D);
    memset(dv, 0, sizeof(double) * 256 * D);
    for (int64_t a = tq_ptr[it]; a < tq_ptr[it + 1]; a++) {
      int ib = tq_idx[a];
      int64_t gi = goff + ib;
      const int32_t* sel = col_idx + row_ptr[gi];
      int ns = (int)(row_ptr[gi + 1] - row_ptr[gi]);
      int64_t nk = 0, off = -1;
      for (int b = 0; b < ns; b++) {
        if (sel[b] == jb) off = nk;
        nk += blk_len[goff + sel[b]];
      }
      if (off < 0) continue; /* not selected: no gradient */
      double* P = (double*)malloc(sizeof(double) * (nk + 1));
      double* dP = (double*)malloc(sizeof(double) * (nk + 1));
      for (int u = 0; u < blk_len[gi]; u++) {
        int64_t nq = perm_h[blk_start[gi] + u];
        double delta;
        row_softmax_grad(q, k, v, dO, dtype, N, D, perm_h, h, nq, sel, ns, blk_start, blk_len,
                         goff, P, dP, &delta);
        for (int r = 0; r < blk_len[gj]; r++) {
          double pr = P[off + r];
          double ds = pr * (dP[off + r] - delta) * scale;
          for (int c = 0; c < D; c++) {
            dk[(int64_t)r * D + c] += ds * ld(q, dtype, ((int64_t)h * N + nq) * D + c);
            dv[(int64_t)r * D + c] += pr * ld(dO, dtype, ((int64_t)h * N + nq) * D + c);
          }
        }
      }
      free(P);
      free(dP);
    }
  }
  return OR_OK;
}

/* All gradients of one head by walking every query row once: for row n of
 * query block i, P and dP over the keys of S_i, Delta = sum_m P dP; then
 * dQ_n = sum_m dS k_m / sqrt D and, for each selected key m,
 * dK_m += dS q_n / sqrt D, dV_m += P dO_n.  row_ptr/col_idx hold the full
 * selection (global block ids index row_ptr).  dq, dk, dv: [N][D] in the
 * original token order. */
int orc_attn_bwd_head(const void* q, const void* k, const void* v, const void* dO, int dtype,
                      int64_t N, int D, const int32_t* perm, const int64_t* blk_off,
                      const int32_t* blk_start, const int32_t* blk_len, const int64_t* row_ptr,
                      const int32_t* col_idx, int h, double* dq, double* dk, double* dv) {
  double scale = 1.0 / sqrt((double)D);
  const int32_t* perm_h = perm + (int64_t)h * N;
  int64_t goff = blk_off[h];
  int nblk = (int)(blk_off[h + 1] - blk_off[h]);
  memset(dq, 0, sizeof(double) * N * D);
  memset(dk, 0, sizeof(double) * N * D);
  memset(dv, 0, sizeof(double) * N * D);
#pragma omp parallel
  {
    double* lk = (double*)calloc((size_t)N * D, sizeof(double));
    double* lv = (double*)calloc((size_t)N * D, sizeof(double));
#pragma omp for schedule(dynamic)
    for (int i = 0; i < nblk; i++) {
      int64_t gi = goff + i;
      const int32_t* sel = col_idx + row_ptr[gi];
      int ns = (int)(row_ptr[gi + 1] - row_ptr[gi]);
      int64_t nk = 0;
      for (int a = 0; a < ns; a++) nk += blk_len[goff + sel[a]];
      double* P = (double*)malloc(sizeof(double) * (nk + 1));
      double* dP = (double*)malloc(sizeof(double) * (nk + 1));
      for (int u = 0; u < blk_len[gi]; u++) {
        int64_t nq = perm_h[blk_start[gi] + u];
        double delta;
        row_softmax_grad(q, k, v, dO, dtype, N, D, perm_h, h, nq, sel, ns, blk_start, blk_len,
                         goff, P, dP, &delta);
        int64_t idx = 0;
        for (int a = 0; a < ns; a++) {
          int64_t gk = goff + sel[a];
          for (int r = 0; r < blk_len[gk]; r++) {
            int64_t nkt = perm_h[blk_start[gk] + r];
            double pr = P[idx], ds = P[idx] * (dP[idx] - delta) * scale;
            for (int c = 0; c < D; c++) {
              dq[nq * D + c] += ds * ld(k, dtype, ((int64_t)h * N + nkt) * D + c);
              lk[nkt * D + c] += ds * ld(q, dtype, ((int64_t)h * N + nq) * D + c);
              lv[nkt * D + c] += pr * ld(dO, dtype, ((int64_t)h * N + nq) * D + c);
            }
            idx++;
          }
        }
      }
      free(P);
      free(dP);
    }
#pragma omp critical
    {
      for (int64_t e = 0; e < N * D; e++) {
        dk[e] += lk[e];
        dv[e] += lv[e];
      }
    }
    free(lk);
    free(lv);
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* The A->V norm map consumed by the next layer's stage one             */
/* (paper.rainbus.top "双分支视频-音频 DiT 与跨模态交叉注意力": the video  */
/* hidden state takes audio information through h_hat =                  */
/* CrossAttn(h, K_a, V_a), and the L2 norm of that output at each video  */
/* position measures how much audio it absorbed; "核心方法": the norms    */
/* of one layer are cached for the next).  Reading: h_hat of token n is  */
/* the concatenation over heads of softmax(q_{h,n} K_a,h^T / sqrt D)     */
/* V_a,h (before any output projection), and a_n = ||h_hat_n||_2.       */
/* fp64, two-pass softmax.  For each listed token: norm_out[i] and, if   */
/* o_out is not NULL, o_out[i][heads][D].                               */
/* ------------------------------------------------------------------ */
int orc_av_cross(const void* q, const void* ka, const void* va, int dtype, int heads, int64_t N,
                 int64_t Na, int D, int ntok, const int64_t* tokens, double* norm_out,
                 double* o_out) {
  if (Na <= 0 || D > 128) return OR_EINVAL;
  double scale = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(dynamic)
  for (int it = 0; it < ntok; it++) {
    int64_t n = tokens[it];
    double* s = (double*)malloc(sizeof(double) * Na);
    double ss = 0.0;
    for (int h = 0; h < heads; h++) {
      double qv[128], o[128];
      for (int c = 0; c < D; c++) {
        qv[c] = ld(q, dtype, ((int64_t)h * N + n) * D + c);
        o[c] = 0.0;
      }
      double mx = -INFINITY;
      for (int64_t m = 0; m < Na; m++) {
        double acc = 0.0;
        for (int c = 0; c < D; c++) acc += qv[c] * ld(ka, dtype, ((int64_t)h * Na + m) * D + c);
        s[m] = acc * scale;
        if (s[m] > mx) mx = s[m];
      }
      double sum = 0.0;
      for (int64_t m = 0; m < Na; m++) sum += exp(s[m] - mx);
      for (int64_t m = 0; m < Na; m++) {
        double p = exp(s[m] - mx) / sum;
        for (int c = 0; c < D; c++) o[c] += p * ld(va, dtype, ((int64_t)h * Na + m) * D + c);
      }
      for (int c = 0; c < D; c++) {
        ss += o[c] * o[c];
        if (o_out) o_out[((int64_t)it * heads + h) * D + c] = o[c];
      }
    }
    norm_out[it] = sqrt(ss);
    free(s);
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Shot-cut-aware temporal zone boundaries (paper.rainbus.top            */
/* "独立分析的弱点" (1): detect shot cuts from frame differences and force */
/* the macro-zones to split there).  Readings:                            */
/*  - the frame-difference energy of frame t >= 1 is                      */
/*    e_t = mean over heads, the H x W tokens and the channels of         */
/*    (V_t - V_{t-1})^2 (fp64); a cut starts frame t when                 */
/*    e_t > kappa * mean_{t'} e_{t'} (kappa = the cut threshold, 0: off);  */
/*  - a zone of frames [8 zt, 8 zt + 8) with a cut at offset c (1..7)     */
/*    splits there: its blocks may not be longer in time than the largest */
/*    power of two dividing c (at least 2, the shortest edge a candidate  */
/*    has, so an odd offset leaves one 2-frame block row across the cut); */
/*    the cap is the smallest over the zone's cuts, and the zone's volume */
/*    drops to the largest volume that has a candidate within the cap     */
/*    (b_T = 2 allows at most 128).                                       */
/* cuts[t] = 1 where a cut starts (cuts[0] = 0); energy[t] = e_t (e_0 = 0) */
/* ------------------------------------------------------------------ */
int orc_detect_cuts(const void* v, int dtype, int T, int H, int W, int heads, int D,
                    float kappa, uint8_t* cuts, double* energy) {
  int64_t N = (int64_t)T * H * W, HW = (int64_t)H * W;
  energy[0] = 0.0;
#pragma omp parallel for schedule(static)
  for (int t = 1; t < T; t++) {
    double s = 0.0;
    for (int h = 0; h < heads; h++)
      for (int64_t p = 0; p < HW; p++)
        for (int c = 0; c < D; c++) {
          double a = ld(v, dtype, ((int64_t)h * N + (int64_t)t * HW + p) * D + c);
          double b = ld(v, dtype, ((int64_t)h * N + (int64_t)(t - 1) * HW + p) * D + c);
          s += (a - b) * (a - b);
        }
    energy[t] = s / ((double)heads * (double)HW * (double)D);
  }
  double mean = 0.0;
  for (int t = 1; t < T; t++) mean += energy[t];
  mean = T > 1 ? mean / (double)(T - 1) : 0.0;
  cuts[0] = 0;
  for (int t = 1; t < T; t++) cuts[t] = (kappa > 0.0f && energy[t] > (double)kappa * mean) ? 1 : 0;
  return OR_OK;
}

/* largest b_T allowed in each temporal zone row zt (8 = no cut inside) */
int orc_cut_caps(const uint8_t* cuts, int T, int32_t* cap) {
  for (int zt = 0; zt < T / 8; zt++) {
    int c_cap = 8;
    for (int c = 1; c < 8; c++) {
      if (!cuts[8 * zt + c]) continue;
      int p = c & (-c); /* largest power of two dividing c */
      if (p < 2) p = 2;
      if (p < c_cap) c_cap = p;
    }
    cap[zt] = c_cap;
  }
  return OR_OK;
}
