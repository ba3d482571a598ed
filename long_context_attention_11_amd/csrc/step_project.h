// One-token projection step (T = 1, bf16), shared by its own kernel and by the launch that
// runs it beside the top-k threshold pass.
//
// Source: reading notes "DeepSeekV4技术报告阅读笔记" §2.3.1 eqs. 9-10 (the per-token projections the
// compressor folds).
#pragma once

#include "csa_internal.h"

namespace csa {

// One 16-row x 16-column output tile per workgroup of 16 waves (1024 threads).  The waves split
// K in sixteen; each loads its weight rows straight into MFMA operands (PS_DEPTH steps per
// round: at d = 4096 one round, so every load is in flight at once), and the sixteen partial
// tiles are summed through LDS in a fixed order.  The result goes directly into the sequence's
// projection-state slot for the token (pos0[b] % S), where the fold reads it, so there is no
// separate split-K reduction or state copy.
constexpr int PS_DEPTH = 8;
constexpr int PS_WAVES = 16;

struct ProjectStepArgs {
  const uint16_t* H;      // [M][K] bf16
  const uint16_t* wkv;    // [nkv][K] bf16
  const uint16_t* widx;   // [NP - nkv][K] bf16
  int nkv, M, NP, K;
  const int32_t* pos0;    // [M]
  int S;                  // state rows
  float* state;           // [M][S][NP]
};

// Tile (bx, by) = output columns 16 bx .. +15, rows 16 by .. +15.  red: LDS [PS_WAVES][256].
__device__ __forceinline__ void project_step_tile(const ProjectStepArgs& a, int bx, int by,
                                                  float (*red)[256]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const int n0 = bx * 16, m0 = by * 16;
  const int K = a.K;
  const int kq = K / PS_WAVES;                // this wave's share of K (a multiple of 32)
  const int kb = wave * kq + fg * 8;
  const uint16_t* arow = a.H + (size_t)min(m0 + fr, a.M - 1) * K + kb;
  const int n = min(n0 + fr, a.NP - 1);
  const uint16_t* brow = (n < a.nkv ? a.wkv + (size_t)n * K : a.widx + (size_t)(n - a.nkv) * K) + kb;
  const int nsteps = kq / 32;
  uint4 ra[PS_DEPTH], rb[PS_DEPTH];
#pragma unroll
  for (int i = 0; i < PS_DEPTH; ++i) {
    const int k = min(i, nsteps - 1) * 32;
    ra[i] = *reinterpret_cast<const uint4*>(arow + k);
    rb[i] = *reinterpret_cast<const uint4*>(brow + k);
  }
  f32x4 acc = {0, 0, 0, 0};
  for (int s0 = 0; s0 < nsteps; s0 += PS_DEPTH) {
#pragma unroll
    for (int i = 0; i < PS_DEPTH; ++i) {
      // a step past the end reloads the last one and is not accumulated
      const bool live = s0 + i < nsteps;
      const bf16x8 A = __builtin_bit_cast(bf16x8, ra[i]);
      const bf16x8 Bv = __builtin_bit_cast(bf16x8, rb[i]);
      const f32x4 nxt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bv, acc, 0, 0, 0);
      acc = live ? nxt : acc;
      const int k = min(s0 + i + PS_DEPTH, nsteps - 1) * 32;
      ra[i] = *reinterpret_cast<const uint4*>(arow + k);
      rb[i] = *reinterpret_cast<const uint4*>(brow + k);
    }
  }
  // D layout: lane holds column fr, rows 4*fg + e
#pragma unroll
  for (int e = 0; e < 4; ++e) red[wave][(4 * fg + e) * 16 + fr] = acc[e];
  __syncthreads();
  if (tid >= 256) return;
  const int row = tid >> 4, col = tid & 15;
  float v = red[0][tid];
#pragma unroll
  for (int w = 1; w < PS_WAVES; ++w) v += red[w][tid];
  const int b = m0 + row, nn = n0 + col;
  if (b < a.M && nn < a.NP) a.state[((size_t)b * a.S + (a.pos0[b] % a.S)) * a.NP + nn] = v;
}

// Host: the arguments for a one-token step of cache c (defined with the compressor).
ProjectStepArgs project_step_args(const csa_dims& d, const csa_weights& w, const csa_cache& c,
                                  const void* H, const int32_t* pos0);

inline int project_step_grid_x(int NP) { return (NP + 15) / 16; }
inline int project_step_grid_y(int M) { return (M + 15) / 16; }

}  // namespace csa
