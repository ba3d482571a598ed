// One-token projection step (T = 1, bf16), shared by its own kernel and by the launch that
// runs it beside the top-k threshold pass.
//
// Source: reading notes "DeepSeekV4技术报告阅读笔记" §2.3.1 eqs. 9-10 (the per-token projections the
// compressor folds).
#pragma once

#include "csa_internal.h"

namespace csa {

// The work is cut into wave-sized units so that it spreads over every CU (one CU streams
// only some 25 GB/s from HBM, so a launch needs all of them): a unit is TILES 16-column
// output tiles x one of PU_SLICES slices of K, for one 16-row tile of tokens, and its partial
// sums go to part[slice][row][col].  The fold adds the PU_SLICES partials in slice order (so
// the result is deterministic) and also writes the summed row into the projection state.
// Each lane reads 32 contiguous bytes per pair of K steps: lane group g takes elements
// 16g .. 16g+15 of each 64-element pair, the first eight for the pair's first MFMA step and
// the rest for its second, on both operands alike, so the four lane groups together read
// whole 128-byte lines of the 16 rows.  The tiles of a unit share the token operand.
constexpr int PU_SLICES = 16;   // slices of K (partial sums per output)
constexpr int PU_PAIRS = 4;     // 64-element pairs per load round

struct ProjectStepArgs {
  const uint16_t* H;      // [M][K] bf16
  const uint16_t* wkv;    // [nkv][K] bf16
  const uint16_t* widx;   // [NP - nkv][K] bf16
  int nkv, M, NP, K;      // K a multiple of 64 * PU_SLICES
  float* part;            // [PU_SLICES][M][NP]
};

__host__ __device__ inline int project_col_groups(int NP, int tiles) { return ((NP + 15) / 16 + tiles - 1) / tiles; }
inline int project_units(int NP, int M, int tiles) { return project_col_groups(NP, tiles) * PU_SLICES * ((M + 15) / 16); }

// Unit u (one wave): column group u % G, slice (u / G) % PU_SLICES, row tile u / (G PU_SLICES).
template <int TILES>
__device__ __forceinline__ void project_unit(const ProjectStepArgs& a, int u) {
  const int lane = threadIdx.x & 63, fr = lane & 15, fg = lane >> 4;
  const int ncg = project_col_groups(a.NP, TILES), px = (a.NP + 15) / 16;
  const int cg = u % ncg, sl = (u / ncg) % PU_SLICES, rt = u / (ncg * PU_SLICES);
  const int K = a.K, kq = K / PU_SLICES, npair = kq / 64;
  const uint16_t* arow = a.H + (size_t)min(16 * rt + fr, a.M - 1) * K + sl * kq + 16 * fg;
  const uint16_t* brow[TILES];
#pragma unroll
  for (int c = 0; c < TILES; ++c) {
    const int n = min(16 * min(cg * TILES + c, px - 1) + fr, a.NP - 1);
    brow[c] = (n < a.nkv ? a.wkv + (size_t)n * K : a.widx + (size_t)(n - a.nkv) * K) + sl * kq + 16 * fg;
  }
  f32x4 acc[TILES];
#pragma unroll
  for (int c = 0; c < TILES; ++c) acc[c] = f32x4{0, 0, 0, 0};
  for (int p0 = 0; p0 < npair; p0 += PU_PAIRS) {
    // a pair past the end reloads the last one and is not accumulated
    uint4 ra[2 * PU_PAIRS], rb[TILES][2 * PU_PAIRS];
#pragma unroll
    for (int p = 0; p < PU_PAIRS; ++p) {
      const int k = 64 * min(p0 + p, npair - 1);
      ra[2 * p] = *reinterpret_cast<const uint4*>(arow + k);
      ra[2 * p + 1] = *reinterpret_cast<const uint4*>(arow + k + 8);
#pragma unroll
      for (int c = 0; c < TILES; ++c) {
        rb[c][2 * p] = *reinterpret_cast<const uint4*>(brow[c] + k);
        rb[c][2 * p + 1] = *reinterpret_cast<const uint4*>(brow[c] + k + 8);
      }
    }
#pragma unroll
    for (int p = 0; p < PU_PAIRS; ++p) {
      const bool live = p0 + p < npair;
#pragma unroll
      for (int c = 0; c < TILES; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4 nxt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, ra[2 * p + h]), __builtin_bit_cast(bf16x8, rb[c][2 * p + h]), acc[c], 0, 0, 0);
          acc[c] = live ? nxt : acc[c];
        }
    }
  }
  // D layout: lane holds column fr, rows 4*fg + e
#pragma unroll
  for (int c = 0; c < TILES; ++c) {
    const int tile = cg * TILES + c, col = 16 * tile + fr;
    if (tile < px && col < a.NP) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + 4 * fg + e;
        if (row < a.M) a.part[((size_t)sl * a.M + row) * a.NP + col] = acc[c][e];
      }
    }
  }
}

// Host: the arguments for a one-token step of cache c (defined with the compressor); part
// holds project_part_bytes.
ProjectStepArgs project_step_args(const csa_dims& d, const csa_weights& w, const csa_cache& c,
                                  const void* H, float* part);

}  // namespace csa
