// The compressor's softmax fold and row finalisation, shared by the fold kernel and by the
// launch that runs a one-token fold beside the final top-k pass.
//
// Sources: reading notes "DeepSeekV4技术报告阅读笔记" (zouxinn.github.io) §2.3.1 eqs. 11-12 (CSA
// fold), §2.4.1 eqs. 22-23 (HCA fold), §2.5.1-2.5.2 (RMSNorm, partial RoPE); PaperTrace "02 ·
// DeepSeek-V4: 压缩注意力撑起 1M 上下文" §2.5 (RoPE dims in BF16, the rest FP8) and §6.4
// (CSA2: single-path fold without bias, index keys from the entry, FP4 main KV).
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
  const float* bias;     // CSA [2][m][c], HCA [m][c], CSA2 null (no bias)
  const float* bias_idx; // CSA [2][m][cI]
  const void* w_ik;      // CSA2: [cI][c] projection of the normalised entry onto its key
  int act_f32;           // w_ik in float32 (else bfloat16)
  int keys_entry;        // CSA2: the index key is projected from the entry
  const float* gamma;    // [c] or null
  float eps;
  double log2_base;
  int kv_fmt, idx_fmt;
  int cap, win_cap, rowB;
  RowMap rm;             // where entry i of a sequence lives in kv and ki
  uint8_t* kv;
  uint8_t* ki;
  uint8_t* win;
  int32_t* win_pos;
  int32_t* n_entries;
};

// The PU_SLICES partial sums of a one-token projection at p (slice stride `stride` floats),
// added in slice order.  All loads are issued before the first add (the scheduling barrier
// keeps the compiler from interleaving them with the adds, which under register pressure
// it otherwise does, one round of memory latency per slice).
__device__ __forceinline__ float sum_slices(const float* p, size_t stride) {
  float x[PU_SLICES];
#pragma unroll
  for (int sl = 0; sl < PU_SLICES; ++sl) x[sl] = p[sl * stride];
  __builtin_amdgcn_sched_barrier(0);
  float v = 0.f;
#pragma unroll
  for (int sl = 0; sl < PU_SLICES; ++sl) v += x[sl];
  return v;
}

// Maximum of the bit patterns of non-negative floats (ordered as the floats are).
struct MaxBits { __device__ int operator()(int a, int b) const { return max(a, b); } };

// Projection value of token j (global position) in column col of sequence b.
// PART (one-token steps, a.part set): earlier tokens come from the state ring and the new
// token from its partial sums, added in slice order.  Otherwise tokens of the chunk come from
// P (or, with P null, everything from the state ring).
template <bool PART>
__device__ __forceinline__ float proj(const FoldArgs& a, int b, int p0, int j, int col) {
  if constexpr (PART) {
    if (j == p0) return sum_slices(a.part + (size_t)b * a.NP + col, (size_t)a.B * a.NP);
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
  auto bias = [&](const float* B, int r) { return B ? B[r * bstride_col + u] : 0.f; };
  float mx = -INFINITY;
  for (int r = 0; r < m; ++r) mx = fmaxf(mx, proj<PART>(a, b, p0, ja + r, colZa) + bias(Ba, r));
  if (has_b)
    for (int r = 0; r < m; ++r)
      mx = fmaxf(mx, proj<PART>(a, b, p0, jb + r, colZa + boff) + bias(Bb, r));
  float den = 0.f, num = 0.f;
  for (int r = 0; r < m; ++r) {
    float e = expf(proj<PART>(a, b, p0, ja + r, colZa) + bias(Ba, r) - mx);
    den += e;
    num = fmaf(e, proj<PART>(a, b, p0, ja + r, colCa), num);
  }
  if (has_b)
    for (int r = 0; r < m; ++r) {
      float e = expf(proj<PART>(a, b, p0, jb + r, colZa + boff) + bias(Bb, r) - mx);
      den += e;
      num = fmaf(e, proj<PART>(a, b, p0, jb + r, colCa + boff), num);
    }
  return num / den;
}

// The new token's summed projection in column col (its partial sums added in slice order).
__device__ __forceinline__ float new_token_proj(const FoldArgs& a, int b, int col) {
  return sum_slices(a.part + (size_t)b * a.NP + col, (size_t)a.B * a.NP);
}

// The same fold for the entry a one-token step completes (T = 1, partial sums in a.part):
// entry i's block ends at the new token, p0 = M i + M - 1, so its first M - 1 rows and the
// previous block come from the state ring and its last row from the new token's partial
// sums.  step_load issues every load of a column (all but the new token's values, which
// step_finish takes summed, from LDS, or sums itself) before any is used, so they take one
// round of latency instead of one per row: a step completes an entry with one workgroup
// per sequence, and nothing else hides that latency.  The arithmetic is fold_column's, in
// its order.
template <int M>
struct StepCol {
  float za[M], ca[M], zb[M], cb[M];
  int colCa, colZa;
};
template <int M>
__device__ __forceinline__ void step_load(const FoldArgs& a, int b, int i, int colCa, int colZa, int boff,
                                          StepCol<M>& v) {
  const bool has_b = a.dual && i > 0;
  const float* st = a.state + (size_t)b * a.S * a.NP;
  v.colCa = colCa;
  v.colZa = colZa;
#pragma unroll
  for (int r = 0; r < M; ++r) {
    if (r < M - 1) {
      const float* row = st + (size_t)((M * i + r) % a.S) * a.NP;
      v.za[r] = row[colZa];
      v.ca[r] = row[colCa];
    }
    // the previous block's rows (read from a valid row when there is none, then ignored)
    const float* rowb = st + (size_t)((has_b ? M * (i - 1) + r : r) % a.S) * a.NP;
    v.zb[r] = rowb[colZa + boff];
    v.cb[r] = rowb[colCa + boff];
  }
}
// FROM_LDS: the new token's Z and C values are at pz, pc (LDS), else they are summed here; the
// biases (a few KB, cache-resident) are read here.
template <int M, bool FROM_LDS>
__device__ __forceinline__ float step_finish(const FoldArgs& a, int b, int i, StepCol<M>& v, const float* pz,
                                             const float* pc, const float* Ba, const float* Bb, int bstride_col,
                                             int u) {
  const bool has_b = a.dual && i > 0;
  if constexpr (FROM_LDS) {
    v.za[M - 1] = *pz;
    v.ca[M - 1] = *pc;
  } else {
    v.za[M - 1] = new_token_proj(a, b, v.colZa);
    v.ca[M - 1] = new_token_proj(a, b, v.colCa);
  }
  float ba[M], bb[M];
#pragma unroll
  for (int r = 0; r < M; ++r) {
    ba[r] = Ba ? Ba[r * bstride_col + u] : 0.f;
    bb[r] = Bb ? Bb[r * bstride_col + u] : 0.f;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < M; ++r) mx = fmaxf(mx, v.za[r] + ba[r]);
  if (has_b) {
#pragma unroll
    for (int r = 0; r < M; ++r) mx = fmaxf(mx, v.zb[r] + bb[r]);
  }
  float den = 0.f, num = 0.f;
#pragma unroll
  for (int r = 0; r < M; ++r) {
    const float e = expf(v.za[r] + ba[r] - mx);
    den += e;
    num = fmaf(e, v.ca[r], num);
  }
  if (has_b) {
#pragma unroll
    for (int r = 0; r < M; ++r) {
      const float e = expf(v.zb[r] + bb[r] - mx);
      den += e;
      num = fmaf(e, v.cb[r], num);
    }
  }
  return num / den;
}

// The single-path fold (HCA) of columns u and u + 1 for the entry a one-token step completes,
// with any m: rows m i .. m i + m - 2 from the state ring, the last row the new token.  Both
// passes read CH rows at a time with every load of a chunk issued together (one round of
// memory latency per chunk, not per row); the arithmetic is fold_column's, in its order.
__device__ __forceinline__ void fold_pair_rows(const FoldArgs& a, int b, int i, int u, float& x0, float& x1) {
  constexpr int CH = 16;
  const int m = a.m, colZ = a.c + u, colC = u;
  const float* st = a.state + (size_t)b * a.S * a.NP;
  const float* B = a.bias;   // [m][c] or null
  auto bias = [&](int r, int h) { return B ? B[r * a.c + u + h] : 0.f; };
  float zn[2], cn[2];   // the new token (row m - 1)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    zn[h] = new_token_proj(a, b, colZ + h);
    cn[h] = new_token_proj(a, b, colC + h);
  }
  float mx[2] = {-INFINITY, -INFINITY};
  for (int r0 = 0; r0 < m - 1; r0 += CH) {
    float z[2][CH];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int r = min(r0 + q, m - 2);   // past the chunk's end: a repeated row, ignored
      const float* row = st + (size_t)((m * i + r) % a.S) * a.NP;
#pragma unroll
      for (int h = 0; h < 2; ++h) z[h][q] = row[colZ + h] + bias(r, h);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < CH; ++q)
      if (r0 + q < m - 1) {
#pragma unroll
        for (int h = 0; h < 2; ++h) mx[h] = fmaxf(mx[h], z[h][q]);
      }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) mx[h] = fmaxf(mx[h], zn[h] + bias(m - 1, h));
  float den[2] = {0.f, 0.f}, num[2] = {0.f, 0.f};
  for (int r0 = 0; r0 < m - 1; r0 += CH) {
    float z[2][CH], cv[2][CH];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int r = min(r0 + q, m - 2);
      const float* row = st + (size_t)((m * i + r) % a.S) * a.NP;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        z[h][q] = row[colZ + h] + bias(r, h);
        cv[h][q] = row[colC + h];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < CH; ++q)
      if (r0 + q < m - 1) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float e = expf(z[h][q] - mx[h]);
          den[h] += e;
          num[h] = fmaf(e, cv[h][q], num[h]);
        }
      }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float e = expf(zn[h] + bias(m - 1, h) - mx[h]);
    den[h] += e;
    num[h] = fmaf(e, cn[h], num[h]);
  }
  x0 = num[0] / den[0];
  x1 = num[1] / den[1];
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

// MXFP4 encoding of a 32-dim block held by the 16 threads of one DPP row, two dims each:
// the row's largest magnitude sets the scale exponent e (the MX rule: floor(log2 max) - 2,
// 0 for an all-zero block), and each thread's two dims become one byte (first dim in the
// low nibble).  Returns the byte; *e_out the exponent (scale code e + 127).
__device__ __forceinline__ uint8_t mx_encode_pair(float v0, float v1, int* e_out) {
  const float amax = __int_as_float(row_allreduce(__float_as_int(fmaxf(fabsf(v0), fabsf(v1))), MaxBits()));
  int e = 0;
  if (amax > 0.f) {
    int ex;
    frexpf(amax, &ex);   // amax = f 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
    e = min(127, max(-127, ex - 1 - 2));
  }
  *e_out = e;
  return (uint8_t)(e2m1_code(ldexpf(v0, -e)) | (e2m1_code(ldexpf(v1, -e)) << 4));
}

// Byte offsets inside an MXFP4_BF16 row (c = 512, r = 64): RoPE dims first, then the codes
// of dims 0 .. c - r - 1, then one scale code per 32 of them, zero padding to MXR_BYTES.
constexpr int MXR_CODES = 128, MXR_SCALES = 352, MXR_PAD = 366, MXR_BYTES = 384;

// RMSNorm over c columns (each thread holds columns 2t, 2t+1), RoPE at pos on the last r
// columns, then store the row in its format.  Threads with 2t >= c hold zeros.  With ybuf
// set, the normalised row before RoPE is also left there (ybuf[u], c floats of LDS; the
// caller synchronises before reading it).
template <int NW>
__device__ __forceinline__ void finalize_store(const FoldArgs& a, float x0, float x1, int64_t pos,
                                               uint8_t* dst, float* red, float* ybuf = nullptr) {
  const int t = threadIdx.x, u = 2 * t;
  const bool act = u < a.c;
  float ss = block_sum<NW>(act ? x0 * x0 + x1 * x1 : 0.f, red);
  float inv = 1.0f / sqrtf(ss / (float)a.c + a.eps);
  if (!act) return;
  float g0 = a.gamma ? a.gamma[u] : 1.f, g1 = a.gamma ? a.gamma[u + 1] : 1.f;
  float y0 = g0 * (x0 * inv), y1 = g1 * (x1 * inv);
  if (ybuf) {
    ybuf[u] = y0;
    ybuf[u + 1] = y1;
  }
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
  } else if (a.kv_fmt == CSA_FMT_MXFP4_BF16) {
    if (u < rs) {
      // dims 32k .. 32k + 31 are the 16 threads of DPP row k (rs is a multiple of 32)
      int e;
      dst[MXR_CODES + t] = mx_encode_pair(y0, y1, &e);
      if ((t & 15) == 0) dst[MXR_SCALES + (t >> 4)] = (uint8_t)(e + 127);
      if (t == 0) {
        *reinterpret_cast<uint16_t*>(dst + MXR_PAD) = 0;
        *reinterpret_cast<uint4*>(dst + MXR_PAD + 2) = make_uint4(0u, 0u, 0u, 0u);
      }
    } else {
      const uint32_t bits = f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16);
      *reinterpret_cast<uint32_t*>(dst + 2 * (u - rs)) = bits;
    }
  } else if (u < rs) {
    uint32_t code = f32_to_e4m3(y0) | (f32_to_e4m3(y1) << 8);
    *reinterpret_cast<uint16_t*>(dst + u) = (uint16_t)code;
  } else {
    uint32_t bits = f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16);
    *reinterpret_cast<uint32_t*>(dst + rs + 2 * (u - rs)) = bits;
  }
}

// Keys 2t and 2t + 1 of entry i of sequence b, stored in the index format (2t < cI; pair t
// is held by a thread whose lane is t modulo 64, so that a DPP row holds a 32-dim block).
__device__ __forceinline__ void store_key_pair(const FoldArgs& a, int b, int i, int t, float k0, float k1) {
  const int u = 2 * t;
  if (a.idx_fmt == CSA_FMT_F32) {
    float* kd = reinterpret_cast<float*>(a.ki) + row_of(a.rm, b, i) * a.cI;
    kd[u] = k0;
    kd[u + 1] = k1;
  } else if (a.idx_fmt == CSA_FMT_MXFP4) {
    // a block of 32 dims is the 16 threads of one DPP row
    int e;
    const uint8_t byte = mx_encode_pair(k0, k1, &e);
    int64_t oc, os;
    mx_offsets(a.rm, b, i, a.cI / 2, a.cI / 32, oc, os);
    a.ki[oc + t] = byte;
    if ((t & 15) == 0) a.ki[os + (t >> 4)] = (uint8_t)(e + 127);
  } else {
    uint8_t* kd = a.ki + row_of(a.rm, b, i) * a.cI;
    *reinterpret_cast<uint16_t*>(kd + u) = (uint16_t)(f32_to_e4m3(k0) | (f32_to_e4m3(k1) << 8));
  }
}

// CSA2's index key of entry i: K^I = y . W^IK over the normalised entry y (ybuf, before RoPE),
// float32 sums over the c dims in order, two threads per key (halves of the dims, added
// together), then stored in the index format.  kbuf: LDS [cI].  Every thread of the block
// calls it (it synchronises).
template <int NW>
__device__ __forceinline__ void entry_key(const FoldArgs& a, int b, int i, const float* ybuf, float* kbuf) {
  const int t = threadIdx.x;
  __syncthreads();   // ybuf complete
  const int half = a.c / 2;
  for (int o2 = t; o2 < 2 * a.cI; o2 += 64 * NW) {
    const int o = o2 >> 1, h = o2 & 1;
    float acc = 0.f;
    if (a.act_f32) {
      const float* wr = static_cast<const float*>(a.w_ik) + (size_t)o * a.c + h * half;
      for (int v = 0; v < half; ++v) acc = fmaf(ybuf[h * half + v], wr[v], acc);
    } else {
      const uint16_t* wr = static_cast<const uint16_t*>(a.w_ik) + (size_t)o * a.c + h * half;
      if ((reinterpret_cast<uintptr_t>(wr) & 15) == 0 && half % 32 == 0) {
        // 16-byte loads, 32 weights issued at a time; the sum keeps its order
        const float* yb = ybuf + h * half;
        for (int v0 = 0; v0 < half; v0 += 32) {
          uint4 w4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) w4[q] = *reinterpret_cast<const uint4*>(wr + v0 + 8 * q);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t ww[4] = {w4[q].x, w4[q].y, w4[q].z, w4[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int v = v0 + 8 * q + 2 * e;
              acc = fmaf(yb[v], bf16_bits_to_f32(ww[e] & 0xffffu), acc);
              acc = fmaf(yb[v + 1], bf16_bits_to_f32(ww[e] >> 16), acc);
            }
          }
        }
      } else {
        for (int v = 0; v < half; ++v) acc = fmaf(ybuf[h * half + v], bf16_bits_to_f32(wr[v]), acc);
      }
    }
    // pairs (2o, 2o + 1) are adjacent lanes of one wave
    const float other = __shfl_xor(acc, 1);
    if (h == 0) kbuf[o] = acc + other;
  }
  __syncthreads();
  if (2 * t < a.cI) store_key_pair(a, b, i, t, kbuf[2 * t], kbuf[2 * t + 1]);
}

// Block (slot, b) of the fold: slot < T the raw window row of token pos0[b] + slot, otherwise
// the entry slot - T past pos0[b] / m (when its block completes in this chunk).  Threads hold
// columns 2t, 2t + 1; a block of NW waves (NW >= 4; those past the c columns hold zeros).
// red: LDS [NW]; ybuf, kbuf: LDS [c] and [cI] for CSA2's index keys (null where the fold
// never serves a CSA2 layer); pnew: LDS [FOLD_PNEW] or null: with it, a one-token step's
// entry first sums the new token's partial projections of the columns it reads with every
// thread of the block (the blocks of the top-k launch have four times the threads the
// columns need), then folds from LDS.
constexpr int FOLD_PNEW = 2 * 512 + 2 * 128;
template <int NW, bool PART>
__device__ __forceinline__ void fold_block(const FoldArgs& a, int slot, int b, float* red,
                                           float* ybuf = nullptr, float* kbuf = nullptr, float* pnew = nullptr) {
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
  // (a one-token step with m = 4 loads each column's values at once; in blocks of 16 waves
  // the new token's values go through LDS first, and past its size the general fold runs)
  constexpr bool LDS_NEW = NW >= 16;
  const int nnew = 2 * a.c + (a.dual ? 2 * a.cI : 0);
  const bool step4 = PART && a.T == 1 && a.part && a.m == 4 && (!LDS_NEW || (pnew && nnew <= FOLD_PNEW));
  // With threads to spare (the top-k launch's blocks) CSA's index key is folded by threads
  // c/2 .. c/2 + cI/2 - 1 beside the entry's columns, else by threads 0 .. cI/2 - 1 after.
  const bool keys_apart = NW >= 8 && a.dual && 64 * NW >= a.c / 2 + a.cI / 2;   // (NW < 8: never)
  const int kp = keys_apart ? t - a.c / 2 : t;   // this thread's key pair
  const bool has_key = a.dual && kp >= 0 && 2 * kp < a.cI;
  // the new token's values in LDS: C (C^a) at [0, c), Z (Z^a) at [c, 2c), then (CSA) the
  // key's C at [2c, 2c + cI) and Z at [2c + cI, 2c + 2cI)
  float* const pn = LDS_NEW && step4 ? pnew : nullptr;   // uniform
  // the entry's column pair (threads u < c) or key pair (has_key)
  const int uk = 2 * kp, kbase = 4 * a.c;
  const float* BIa = a.bias_idx;
  const float* BIb = a.bias_idx + a.m * a.cI;
  const bool main_cols = u < a.c;
  const bool key_here = keys_apart && has_key && !main_cols;
  if (pn) {
    for (int v = t; v < nnew; v += 64 * NW) {
      int col;
      if (v < 2 * a.c) col = v < a.c ? v : (a.dual ? 2 * a.c : a.c) + (v - a.c);
      else col = 4 * a.c + (v < 2 * a.c + a.cI ? v - 2 * a.c : 2 * a.cI + (v - 2 * a.c - a.cI));
      pn[v] = new_token_proj(a, b, col);
    }
    __syncthreads();
  }
  StepCol<4> s0, s1;
  if (step4 && main_cols) {
    if (a.dual) {
      step_load<4>(a, b, i, u, 2 * a.c + u, a.c, s0);
      step_load<4>(a, b, i, u + 1, 2 * a.c + u + 1, a.c, s1);
    } else {
      step_load<4>(a, b, i, u, a.c + u, 0, s0);
      step_load<4>(a, b, i, u + 1, a.c + u + 1, 0, s1);
    }
  } else if (step4 && key_here) {
    step_load<4>(a, b, i, kbase + uk, kbase + 2 * a.cI + uk, a.cI, s0);
    step_load<4>(a, b, i, kbase + uk + 1, kbase + 2 * a.cI + uk + 1, a.cI, s1);
  }
  auto fold_key = [&]() {
    float k0, k1;
    if (step4) {
      if (!key_here) {
        step_load<4>(a, b, i, kbase + uk, kbase + 2 * a.cI + uk, a.cI, s0);
        step_load<4>(a, b, i, kbase + uk + 1, kbase + 2 * a.cI + uk + 1, a.cI, s1);
      }
      const float* kn = pn + 2 * a.c;   // the key's C, then Z (used with LDS_NEW only)
      k0 = step_finish<4, LDS_NEW>(a, b, i, s0, kn + a.cI + uk, kn + uk, BIa, BIb, a.cI, uk);
      k1 = step_finish<4, LDS_NEW>(a, b, i, s1, kn + a.cI + uk + 1, kn + uk + 1, BIa, BIb, a.cI, uk + 1);
    } else {
      k0 = fold_column<PART>(a, b, p0, i, kbase + uk, kbase + 2 * a.cI + uk, a.cI, BIa, BIb, a.cI, uk);
      k1 = fold_column<PART>(a, b, p0, i, kbase + uk + 1, kbase + 2 * a.cI + uk + 1, a.cI, BIa, BIb, a.cI, uk + 1);
    }
    store_key_pair(a, b, i, kp, k0, k1);
  };
  float x0 = 0.f, x1 = 0.f;
  if (main_cols) {
    if (step4) {
      const float* Bb = a.dual ? a.bias + a.m * a.c : nullptr;
      x0 = step_finish<4, LDS_NEW>(a, b, i, s0, pn + a.c + u, pn + u, a.bias, Bb, a.c, u);
      __builtin_amdgcn_sched_barrier(0);
      x1 = step_finish<4, LDS_NEW>(a, b, i, s1, pn + a.c + u + 1, pn + u + 1, a.bias, Bb, a.c, u + 1);
    } else if (!LDS_NEW && PART && a.T == 1 && a.part && !a.dual) {
      fold_pair_rows(a, b, i, u, x0, x1);   // HCA's one-token step
    } else if (a.dual) {
      x0 = fold_column<PART>(a, b, p0, i, u, 2 * a.c + u, a.c, a.bias, a.bias + a.m * a.c, a.c, u);
      x1 = fold_column<PART>(a, b, p0, i, u + 1, 2 * a.c + u + 1, a.c, a.bias, a.bias + a.m * a.c, a.c, u + 1);
    } else {
      x0 = fold_column<PART>(a, b, p0, i, u, a.c + u, 0, a.bias, a.bias, a.c, u);
      x1 = fold_column<PART>(a, b, p0, i, u + 1, a.c + u + 1, 0, a.bias, a.bias, a.c, u + 1);
    }
  } else if (key_here) {
    fold_key();
  }
  uint8_t* dst = a.kv + row_of(a.rm, b, i) * a.rowB;
  const bool ek = a.keys_entry && ybuf;
  finalize_store<NW>(a, x0, x1, (int64_t)a.m * i, dst, red, ek ? ybuf : nullptr);
  if (ek) {
    entry_key<NW>(a, b, i, ybuf, kbuf);
    return;
  }
  // CSA indexer key: same fold with its own columns and biases; stored as folded
  if (!keys_apart && has_key) fold_key();
}


// Host: the arguments of a fold of T tokens per sequence of cache c (P: summed projections of
// the chunk, or null when the projections sit in the state ring; part: with T = 1 and P null,
// the new token's partial projections, or null when it too is in the state ring).
FoldArgs fold_args(const csa_dims& d, const csa_weights& w, const csa_cache& c, int32_t T,
                   const int32_t* pos0, const float* P, const float* part = nullptr);
// Blocks per sequence: T raw rows, T/m + 1 entry slots, and with part the state writers.
__host__ __device__ inline int fold_grid_x(const FoldArgs& a) { return a.T + a.T / a.m + 1 + (a.part ? (a.NP + 511) / 512 : 0); }

}  // namespace csa
