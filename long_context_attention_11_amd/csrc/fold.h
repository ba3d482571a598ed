// The compressor's softmax fold and row finalisation, shared by the fold kernel and by the
// launch that runs a one-token fold beside the final top-k pass.
//
// Sources: reading notes "DeepSeekV4技术报告阅读笔记" (zouxinn.github.io) §2.3.1 eqs. 11-12 (CSA
// fold), §2.4.1 eqs. 22-23 (HCA fold), §2.5.1-2.5.2 (RMSNorm, partial RoPE); PaperTrace "02 ·
// DeepSeek-V4: 压缩注意力撑起 1M 上下文" §2.5 (RoPE dims in BF16, the rest FP8).
#pragma once

#include "csa_internal.h"
#include "step_project.h"

namespace csa {

struct FoldArgs {
  const float* P;        // [B*T][NP] summed projections, or null: all in the state ring
  const float* part;     // T = 1: [PU_SLICES][B][NP] partial projections of the new token
                         // (then also written, summed, into the state ring), or null
  int B;
  float* state;          // [B][S][NP]
  int S, NP;
  int T, m, dual, c, r, cI;
  const int32_t* pos0;
  const float* bias;     // CSA [2][m][c], HCA [m][c]
  const float* bias_idx; // CSA [2][m][cI]
  const float* gamma;    // [c] or null
  float eps;
  double log2_base;
  int kv_fmt, idx_fmt;
  int cap, win_cap, rowB;
  uint8_t* kv;
  uint8_t* ki;
  uint8_t* win;
  int32_t* win_pos;
  int32_t* n_entries;
};

// Maximum of the bit patterns of non-negative floats (ordered as the floats are).
struct MaxBits { __device__ int operator()(int a, int b) const { return max(a, b); } };

// Projection value of token j (global position) in column col of sequence b.
// PART (one-token steps, a.part set): earlier tokens come from the state ring and the new
// token from its partial sums, added in slice order.  Otherwise tokens of the chunk come from
// P (or, with P null, everything from the state ring).
template <bool PART>
__device__ __forceinline__ float proj(const FoldArgs& a, int b, int p0, int j, int col) {
  if constexpr (PART) {
    if (j == p0) {
      float v = 0.f;
#pragma unroll
      for (int s = 0; s < PU_SLICES; ++s) v += a.part[((size_t)s * a.B + b) * a.NP + col];
      return v;
    }
  } else {
    if (a.P && j >= p0) return a.P[((size_t)b * a.T + (j - p0)) * a.NP + col];
  }
  return a.state[((size_t)b * a.S + (j % a.S)) * a.NP + col];
}

// Softmax fold of one column (reading notes eqs. 11-12 / 22-23).
//   CSA: logits Z^a_{mi+r} + B^a_r and Z^b_{m(i-1)+r} + B^b_r (b half absent for i = 0),
//        values C^a and C^b.  HCA: logits Z_{mi+r} + B_r over the m rows of block i.
// colC/colZ name the projection columns of the a path; b-path columns are +boff.
template <bool PART>
__device__ __forceinline__ float fold_column(const FoldArgs& a, int b, int p0, int i, int colCa, int colZa,
                             int boff, const float* Ba, const float* Bb, int bstride_col,
                             int u) {
  const int m = a.m;
  const int ja = m * i, jb = m * (i - 1);
  const bool has_b = a.dual && i > 0;
  float mx = -INFINITY;
  for (int r = 0; r < m; ++r) mx = fmaxf(mx, proj<PART>(a, b, p0, ja + r, colZa) + Ba[r * bstride_col + u]);
  if (has_b)
    for (int r = 0; r < m; ++r)
      mx = fmaxf(mx, proj<PART>(a, b, p0, jb + r, colZa + boff) + Bb[r * bstride_col + u]);
  float den = 0.f, num = 0.f;
  for (int r = 0; r < m; ++r) {
    float e = expf(proj<PART>(a, b, p0, ja + r, colZa) + Ba[r * bstride_col + u] - mx);
    den += e;
    num = fmaf(e, proj<PART>(a, b, p0, ja + r, colCa), num);
  }
  if (has_b)
    for (int r = 0; r < m; ++r) {
      float e = expf(proj<PART>(a, b, p0, jb + r, colZa + boff) + Bb[r * bstride_col + u] - mx);
      den += e;
      num = fmaf(e, proj<PART>(a, b, p0, jb + r, colCa + boff), num);
    }
  return num / den;
}

// Sum over a block of NW waves (NW >= 4); the first four partial sums are added in the same
// order whatever NW is (the rest hold zeros in the 1024-thread launch), so the result does
// not depend on the block size.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = red[0] + red[1] + red[2] + red[3];
#pragma unroll
  for (int i = 4; i < NW; ++i) s += red[i];
  return s;
}

// RMSNorm over c columns (each thread holds columns 2t, 2t+1), RoPE at pos on the last r
// columns, then store the row in its format.  Threads with 2t >= c hold zeros.
template <int NW>
__device__ __forceinline__ void finalize_store(const FoldArgs& a, float x0, float x1, int64_t pos,
                                               uint8_t* dst, float* red) {
  const int t = threadIdx.x, u = 2 * t;
  const bool act = u < a.c;
  float ss = block_sum<NW>(act ? x0 * x0 + x1 * x1 : 0.f, red);
  float inv = 1.0f / sqrtf(ss / (float)a.c + a.eps);
  if (!act) return;
  float g0 = a.gamma ? a.gamma[u] : 1.f, g1 = a.gamma ? a.gamma[u + 1] : 1.f;
  float y0 = g0 * (x0 * inv), y1 = g1 * (x1 * inv);
  const int rs = a.c - a.r;
  if (u >= rs) {
    float cs, sn;
    rope_cos_sin(pos, (u - rs) >> 1, a.r, a.log2_base, cs, sn);
    float z0 = y0 * cs - y1 * sn, z1 = y0 * sn + y1 * cs;
    y0 = z0;
    y1 = z1;
  }
  if (a.kv_fmt == CSA_FMT_F32) {
    float2 v = make_float2(y0, y1);
    *reinterpret_cast<float2*>(dst + 4 * u) = v;
  } else if (u < rs) {
    uint32_t code = f32_to_e4m3(y0) | (f32_to_e4m3(y1) << 8);
    *reinterpret_cast<uint16_t*>(dst + u) = (uint16_t)code;
  } else {
    uint32_t bits = f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16);
    *reinterpret_cast<uint32_t*>(dst + rs + 2 * (u - rs)) = bits;
  }
}

// Block (slot, b) of the fold: slot < T the raw window row of token pos0[b] + slot, otherwise
// the entry slot - T past pos0[b] / m (when its block completes in this chunk).  Threads hold
// columns 2t, 2t + 1; a block of NW waves (NW >= 4; those past the c columns hold zeros).
// red: LDS [NW].
template <int NW, bool PART>
__device__ __forceinline__ void fold_block(const FoldArgs& a, int slot, int b, float* red) {
  const int t = threadIdx.x;
  const int p0 = a.pos0[b];
  const int u = 2 * t;
  const int nfold = a.T + a.T / a.m + 1;
  if (PART && slot >= nfold) {
    // the new token's summed projections (512 columns per block) into its state slot
    const int c0 = 512 * (slot - nfold);
    float* dst = a.state + ((size_t)b * a.S + (p0 % a.S)) * a.NP;
    for (int col = c0 + t; col < min(c0 + 512, a.NP); col += 64 * NW) dst[col] = proj<PART>(a, b, p0, p0, col);
    return;
  }
  if (slot < a.T) {
    // raw window row of token j = p0 + slot: a-path row (HCA: C), finalized at position j.
    const int j = p0 + slot;
    if (slot == 0 && t == 0) a.n_entries[b] = min(a.cap, (p0 + a.T) / a.m);
    if (slot < a.T - a.win_cap) return;  // an older token of this chunk the ring cannot keep
    const int ws = j % a.win_cap;
    float x0 = 0.f, x1 = 0.f;
    if (u < a.c) {
      x0 = proj<PART>(a, b, p0, j, u);
      x1 = proj<PART>(a, b, p0, j, u + 1);
    }
    uint8_t* dst = a.win + ((size_t)b * a.win_cap + ws) * a.rowB;
    finalize_store<NW>(a, x0, x1, j, dst, red);
    if (t == 0) a.win_pos[(size_t)b * a.win_cap + ws] = j;
    return;
  }
  const int i = p0 / a.m + (slot - a.T);
  if (a.m * (i + 1) > p0 + a.T || i >= a.cap) return;  // block not complete in this chunk
  // main KV entry: columns C^a at 0, C^b at c, Z^a at 2c, Z^b at 3c (HCA: C at 0, Z at c)
  float x0 = 0.f, x1 = 0.f;
  if (u < a.c) {
    if (a.dual) {
      x0 = fold_column<PART>(a, b, p0, i, u, 2 * a.c + u, a.c, a.bias, a.bias + a.m * a.c, a.c, u);
      x1 = fold_column<PART>(a, b, p0, i, u + 1, 2 * a.c + u + 1, a.c, a.bias, a.bias + a.m * a.c, a.c, u + 1);
    } else {
      x0 = fold_column<PART>(a, b, p0, i, u, a.c + u, 0, a.bias, a.bias, a.c, u);
      x1 = fold_column<PART>(a, b, p0, i, u + 1, a.c + u + 1, 0, a.bias, a.bias, a.c, u + 1);
    }
  }
  uint8_t* dst = a.kv + ((size_t)b * a.cap + i) * a.rowB;
  finalize_store<NW>(a, x0, x1, (int64_t)a.m * i, dst, red);
  // indexer key: same fold with its own columns and biases; stored as folded
  if (a.dual && u < a.cI) {
    const int base = 4 * a.c;
    const float* BIa = a.bias_idx;
    const float* BIb = a.bias_idx + a.m * a.cI;
    float k0 = fold_column<PART>(a, b, p0, i, base + u, base + 2 * a.cI + u, a.cI, BIa, BIb, a.cI, u);
    float k1 = fold_column<PART>(a, b, p0, i, base + u + 1, base + 2 * a.cI + u + 1, a.cI, BIa, BIb, a.cI, u + 1);
    if (a.idx_fmt == CSA_FMT_F32) {
      float* kd = reinterpret_cast<float*>(a.ki) + ((size_t)b * a.cap + i) * a.cI;
      kd[u] = k0;
      kd[u + 1] = k1;
    } else if (a.idx_fmt == CSA_FMT_MXFP4) {
      // a block of 32 dims is the 16 threads of one DPP row: its largest magnitude sets the
      // scale, then each thread encodes its two elements into one byte
      const float amax = __int_as_float(row_allreduce(__float_as_int(fmaxf(fabsf(k0), fabsf(k1))), MaxBits()));
      int e = 0;
      if (amax > 0.f) {
        int ex;
        frexpf(amax, &ex);   // amax = f 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
        e = min(127, max(-127, ex - 1 - 2));
      }
      const size_t krow = (size_t)a.cI / 2 + a.cI / 32;
      uint8_t* kseq = a.ki + (size_t)b * a.cap * krow;
      kseq[(size_t)i * (a.cI / 2) + t] = (uint8_t)(e2m1_code(ldexpf(k0, -e)) | (e2m1_code(ldexpf(k1, -e)) << 4));
      if ((t & 15) == 0) kseq[(size_t)a.cap * (a.cI / 2) + (size_t)i * (a.cI / 32) + (t >> 4)] = (uint8_t)(e + 127);
    } else {
      uint8_t* kd = a.ki + ((size_t)b * a.cap + i) * a.cI;
      *reinterpret_cast<uint16_t*>(kd + u) = (uint16_t)(f32_to_e4m3(k0) | (f32_to_e4m3(k1) << 8));
    }
  }
}


// Host: the arguments of a fold of T tokens per sequence of cache c (P: summed projections of
// the chunk, or null when the projections sit in the state ring; part: with T = 1 and P null,
// the new token's partial projections, or null when it too is in the state ring).
FoldArgs fold_args(const csa_dims& d, const csa_weights& w, const csa_cache& c, int32_t T,
                   const int32_t* pos0, const float* P, const float* part = nullptr);
// Blocks per sequence: T raw rows, T/m + 1 entry slots, and with part the state writers.
inline int fold_grid_x(const FoldArgs& a) { return a.T + a.T / a.m + 1 + (a.part ? (a.NP + 511) / 512 : 0); }

}  // namespace csa
