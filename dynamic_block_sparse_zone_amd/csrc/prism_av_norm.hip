// The A->V norm map: the audio-to-video cross-attention of the video tokens
// over the audio tokens, h_hat = CrossAttn(h, K_a, V_a), with the L2 norm of
// each video position's output, a_n = ||h_hat_n||_2, computed in the
// epilogue (paper.rainbus.top "双分支视频-音频 DiT 与跨模态交叉注意力": the
// norm measures how much audio a position absorbed; "核心方法": the norms of
// one layer are cached and guide the block shapes of the next).  The map is
// the av_norm input of the next layer's prism_plan_create.
//
// gfx950 design (bf16, head_dim 128): dense attention (every audio key),
// the same MFMA tiling as the sparse forward -- 8 waves x 32 video rows per
// work-group, S^T = K_a Q^T so that each lane holds one row's scores, online
// softmax in the log2 domain, O^T += V_a^T P^T with the transposed V_a
// fragments read by ds_read_b64_tr_b16 -- over 64-row audio tiles double
// buffered in LDS.  The work-group walks the heads in order for its rows and
// keeps each row's sum of squares in a register, so the norm over heads and
// channels needs no atomics and no scratch, and is deterministic.  K_a and
// V_a of all heads (a few MB) stay in L2.
#include "prism_attn_common.h"
#include "prism_kernels.h"

namespace prism {

constexpr int kAvRows = 256;
constexpr int kAvWaves = kAvRows / 32;

__global__ __launch_bounds__(kAvWaves * 64, 1) void k_av_cross(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ka,
    const uint16_t* __restrict__ va, int heads, int64_t N, int Na, float c_log2,
    uint16_t* __restrict__ o, float* __restrict__ norm) {
  __shared__ __attribute__((aligned(16))) char ringK[2 * kTile];
  __shared__ __attribute__((aligned(16))) char ringV[2 * kTile];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int64_t n = (int64_t)blockIdx.x * kAvRows + wv * 32 + l32;  // this lane's video token
  uint32_t ro[8], to[4][2];
  row_offsets(lane, ro);
  tr_offsets(lane, to);
  const uint32_t lK = lds_offset(ringK), lV = lds_offset(ringV);
  const int ntile = Na >> 6;
  float ss = 0.0f;  // sum over heads of this lane's channels of h_hat^2

  for (int h = 0; h < heads; h++) {
    const __amdgpu_buffer_rsrc_t rsK =
        buffer_of(ka + (int64_t)h * Na * 128, (uint32_t)Na * 256u);
    const __amdgpu_buffer_rsrc_t rsV =
        buffer_of(va + (int64_t)h * Na * 128, (uint32_t)Na * 256u);
    // audio tile t of K_a and V_a into slot b: wave w fills the 1 KB pieces
    // w, w + 8 of each, LDS row rho holding logical chunk c at c ^ swizzle
    auto stage = [&](int b, int t) {
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const uint32_t piece = i * 512 + wvu * 64;
        const uint32_t slot = piece + lane, rho = slot >> 4;
        const uint32_t c = (slot & 15u) ^ (uint32_t)chunk_swizzle((int)rho);
        const uint32_t src = ((uint32_t)t * 64u + rho) * 256u + c * 16u;
        dma16(rsK, src, lK + b * kTile + piece * 16);
        dma16(rsV, src, lV + b * kTile + piece * 16);
      }
    };
    const uint16_t* qrow = q + ((int64_t)h * N + n) * 128;
    bf16x8 qf[8];
#pragma unroll
    for (int kk = 0; kk < 8; kk++)
      qf[kk] = __builtin_bit_cast(bf16x8, *(const uint4*)(qrow + kk * 16 + hl * 8));
    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[db][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    __syncthreads();  // every wave is done with the slots of the previous head
    stage(0, 0);
    for (int t = 0; t < ntile; t++) {
      // tile t has landed for every wave, and every wave is done with tile
      // t - 1, whose slot takes tile t + 1
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
      __syncthreads();
      if (t + 1 < ntile) stage((t + 1) & 1, t + 1);
      const char* sk = ringK + (t & 1) * kTile;
      const char* sv = ringV + (t & 1) * kTile;
      f32x16 st[2];
#pragma unroll
      for (int i = 0; i < 16; i++)
        st[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            ld_frag(sk + (i & 1) * 8192 + ro[i >> 1]), qf[i >> 1],
            i < 2 ? f32x16{} : st[i & 1], 0, 0, 0);
      float mx = st[0][0];
#pragma unroll
      for (int r = 1; r < 16; r++) mx = fmaxf(mx, st[0][r]);
#pragma unroll
      for (int r = 0; r < 16; r++) mx = fmaxf(mx, st[1][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mt = mx * c_log2;
      if (mt > m_run) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - mt);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
          for (int r = 0; r < 16; r++) acc[db][r] *= alpha;
        m_run = mt;
      }
      const float negm = -m_run;
      bf16x8 pb[4];
#pragma unroll
      for (int c = 0; c < 4; c++) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int r = 8 * (c & 1) + 2 * e;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[c >> 1][r], c_log2, negm));
          const float p1 =
              __builtin_amdgcn_exp2f(__builtin_fmaf(st[c >> 1][r + 1], c_log2, negm));
          pk[e] = pk2(p0, p1);
          l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e]), kOnes2,
                                                  l_run, false);
        }
        pb[c] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
      }
#pragma unroll
      for (int tt = 0; tt < 16; tt++)
        acc[tt & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            ld_tfrag(sv + (tt >> 2) * 4096 + to[tt & 3][0], sv + (tt >> 2) * 4096 + to[tt & 3][1]),
            pb[tt >> 2], acc[tt & 3], 0, 0, 0);
    }
    // this head's output row: lane holds channels 32db + 8jj + 4hl + 0..3
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.0f / l_tot;
    uint16_t* orow = o ? o + ((int64_t)h * N + n) * 128 : nullptr;
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          y[e] = acc[db][4 * jj + e] * inv;
          ss = __builtin_fmaf(y[e], y[e], ss);
        }
        if (orow) {
          uint2 u;
          u.x = pk2(y[0], y[1]);
          u.y = pk2(y[2], y[3]);
          *(uint2*)(orow + 32 * db + 8 * jj + 4 * hl) = u;
        }
      }
  }
  const float tot = ss + __shfl_xor(ss, 32, 64);
  if (hl == 0) norm[n] = sqrtf(tot);
}

bool launch_av_cross(const void* q, const void* ka, const void* va, int heads, int64_t N,
                     int Na, void* o, float* norm, hipStream_t st) {
  dim3 grid((unsigned)(N / kAvRows)), block(kAvWaves * 64);
  const float c_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  hipLaunchKernelGGL(k_av_cross, grid, block, 0, st, (const uint16_t*)q, (const uint16_t*)ka,
                     (const uint16_t*)va, heads, N, Na, c_log2, (uint16_t*)o, norm);
  return hipGetLastError() == hipSuccess;
}

}  // namespace prism
