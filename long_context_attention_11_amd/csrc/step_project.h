// One-token projection step (T = 1, bf16), shared by its own kernel and by the launch that
// runs it beside the top-k threshold pass.
//
// Source: reading notes "DeepSeekV4技术报告阅读笔记" §2.3.1 eqs. 9-10 (the per-token projections the
// compressor folds).
#pragma once

#include "csa_internal.h"

namespace csa {

// One 16-row x 16-column output tile per workgroup of NW waves (NW = 16: 1024 threads; NW = 4:
// the 256-thread launches).  K is split in PS_WAVES = 16 slices, PS_WAVES / NW per wave, each
// accumulated on its own (its weight rows loaded straight into MFMA operands, PS_DEPTH steps
// per round: at d = 4096 one round per slice, every load of the round in flight at once); the
// sixteen partial tiles are summed through LDS in a fixed order, so the result does not depend
// on NW.  It goes directly into the sequence's projection-state slot for the token
// (pos0[b] % S), where the fold reads it, so there is no separate split-K reduction or state
// copy.
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
template <int NW>
__device__ __forceinline__ void project_step_tile(const ProjectStepArgs& a, int bx, int by,
                                                  float (*red)[256]) {
  static_assert(PS_WAVES % NW == 0, "slices per wave");
  constexpr int SL = PS_WAVES / NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const int n0 = bx * 16, m0 = by * 16;
  const int K = a.K;
  const int kq = K / PS_WAVES;                // one slice of K (a multiple of 32)
  const int nsteps = kq / 32;
  const int n = min(n0 + fr, a.NP - 1);
  const uint16_t* arow0 = a.H + (size_t)min(m0 + fr, a.M - 1) * K + fg * 8;
  const uint16_t* brow0 = (n < a.nkv ? a.wkv + (size_t)n * K : a.widx + (size_t)(n - a.nkv) * K) + fg * 8;
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) {
    const int slice = wave * SL + sl;
    const uint16_t* arow = arow0 + slice * kq;
    const uint16_t* brow = brow0 + slice * kq;
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
        if (s0 + PS_DEPTH < nsteps) {   // uniform
          const int k = min(s0 + i + PS_DEPTH, nsteps - 1) * 32;
          ra[i] = *reinterpret_cast<const uint4*>(arow + k);
          rb[i] = *reinterpret_cast<const uint4*>(brow + k);
        }
      }
    }
    // D layout: lane holds column fr, rows 4*fg + e
#pragma unroll
    for (int e = 0; e < 4; ++e) red[slice][(4 * fg + e) * 16 + fr] = acc[e];
  }
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
