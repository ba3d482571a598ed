// KV compression for gfx950: projection GEMM, dual-window (or single-path) softmax fold,
// RMSNorm + RoPE finalize and storage rounding, and the projection state carried between
// calls.
//
// Sources: reading notes "DeepSeekV4技术报告阅读笔记" (zouxinn.github.io) §2.3.1 eqs. 9-12
// (CSA fold), §2.4.1 eqs. 20-23 (HCA fold), §2.5.1-2.5.2 (RMSNorm, partial RoPE);
// PaperTrace "02 · DeepSeek-V4: 压缩注意力撑起 1M 上下文" §2.1 (m = 4 worked case), §2.5
// (RoPE dims in BF16, the rest FP8); deep dive "DeepSeek-V4 架构设计深度解析" §3.2 (indexer keys
// use the same compression with a smaller width).
#include "csa_internal.h"
#include "step_project.h"
#include "fold.h"

namespace csa {

// ============================================================================ projection
//
// P[ks][M][NP] = H[M][K-range ks] . Wall[NP][K-range ks]^T, Wall = [w_kv rows; w_idx rows].
// Column order of P (CSA): C^a | C^b | Z^a | Z^b (c each) | the same four of width c_I.
// HCA: C | Z.  Split-K partials are summed by the consumers in a fixed order.

namespace {

constexpr int PJ_BM = 64, PJ_BN = 64, PJ_BK = 64, PJ_LD = PJ_BK + 8;  // LDS row pitch (bf16)

__device__ __forceinline__ const uint16_t* wall_row(const uint16_t* wkv, const uint16_t* widx,
                                                    int nkv, int n, int K) {
  return n < nkv ? wkv + (size_t)n * K : widx + (size_t)(n - nkv) * K;
}

// bf16 MFMA GEMM: 64x64 tile per workgroup, 4 waves each 32x32 (2x2 MFMA 16x16x32 tiles).
__global__ __launch_bounds__(256) void k_project_bf16(const uint16_t* __restrict__ H,
                                                      const uint16_t* __restrict__ wkv,
                                                      const uint16_t* __restrict__ widx, int nkv,
                                                      int M, int NP, int K, int kchunk,
                                                      float* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][PJ_BM * PJ_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][PJ_BN * PJ_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * PJ_BM, n0 = blockIdx.x * PJ_BN, ks = blockIdx.z;
  const int k_begin = ks * kchunk, k_end = min(K, k_begin + kchunk);
  // loader mapping: 64 rows x 64 k per stage = 512 chunks of 8 bf16 (16 B); 2 per thread
  const int lr = tid >> 3, lc = (tid & 7) * 8;  // row 0..31 (+32), col chunk
  const uint16_t* arow[2];
  const uint16_t* brow[2];
  bool aval[2], bval[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int r = lr + 32 * h;
    aval[h] = (m0 + r) < M;
    arow[h] = H + (size_t)min(m0 + r, M - 1) * K;
    bval[h] = (n0 + r) < NP;
    brow[h] = wall_row(wkv, widx, nkv, min(n0 + r, NP - 1), K);
  }
  uint4 ra[2], rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ra[h] = aval[h] ? *reinterpret_cast<const uint4*>(arow[h] + k0 + lc) : make_uint4(0, 0, 0, 0);
      rb[h] = bval[h] ? *reinterpret_cast<const uint4*>(brow[h] + k0 + lc) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<uint4*>(&As[buf][(lr + 32 * h) * PJ_LD + lc]) = ra[h];
      *reinterpret_cast<uint4*>(&Bs[buf][(lr + 32 * h) * PJ_LD + lc]) = rb[h];
    }
  };
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int fr = lane & 15, fg = lane >> 4;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  int buf = 0;
  if (k_begin < k_end) gload(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += PJ_BK) {
    sstore(buf);
    __syncthreads();
    if (k0 + PJ_BK < k_end) gload(k0 + PJ_BK);
#pragma unroll
    for (int kk = 0; kk < PJ_BK; kk += 32) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm + 16 * i + fr) * PJ_LD + kk + fg * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(wn + 16 * j + fr) * PJ_LD + kk + fg * 8]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    buf ^= 1;
  }
  // D layout of a 16x16 MFMA tile: lane holds column (lane & 15), rows 4*(lane >> 4) + e.
  float* Pk = P + (size_t)ks * M * NP;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int col = n0 + wn + 16 * j + fr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int row = m0 + wm + 16 * i + 4 * fg + e;
        if (row < M && col < NP) Pk[(size_t)row * NP + col] = acc[i][j][e];
      }
    }
}

// float32 GEMM on the vector ALUs (fp32 activations): 16x16 outputs per workgroup.
__global__ __launch_bounds__(256) void k_project_f32(const float* __restrict__ H,
                                                     const float* __restrict__ wkv,
                                                     const float* __restrict__ widx, int nkv,
                                                     int M, int NP, int K, float* __restrict__ P) {
  __shared__ float As[16][17], Bs[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int row = blockIdx.y * 16 + ty, col = blockIdx.x * 16 + tx;
  const int brow_n = blockIdx.x * 16 + ty;
  const float* bsrc = brow_n < NP ? (brow_n < nkv ? wkv + (size_t)brow_n * K
                                                  : widx + (size_t)(brow_n - nkv) * K)
                                  : nullptr;
  float acc = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    As[ty][tx] = (row < M && k0 + tx < K) ? H[(size_t)row * K + k0 + tx] : 0.f;
    Bs[ty][tx] = (bsrc && k0 + tx < K) ? bsrc[k0 + tx] : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(As[ty][kk], Bs[tx][kk], acc);
    __syncthreads();
  }
  if (row < M && col < NP) P[(size_t)row * NP + col] = acc;
}

// ============================================================================ fold / finalize

// One-token projection: one unit per 64-thread workgroup.
__global__ __launch_bounds__(64) void k_project_step(ProjectStepArgs a, int units) {
  if ((int)blockIdx.x < units) project_unit<2>(a, blockIdx.x);
}

// grid: x = T raw rows + (T/m + 1) entry slots (+ state writers), y = sequence.  256
// threads, 2 columns each.  EK: index keys projected from the entries (CSA2), a separate
// instance so that the other layers' folds do not carry its registers.
template <bool PART, bool EK>
__global__ __launch_bounds__(256) void k_fold(FoldArgs a) {
  __shared__ float red[4];
  __shared__ float ybuf[EK ? 512 : 1], kbuf[EK ? 512 : 1];   // CSA2's index keys (c, c_I <= 512)
  fold_block<4, PART>(a, blockIdx.x, blockIdx.y, red, EK ? ybuf : nullptr, EK ? kbuf : nullptr);
}

// Keep the projections of the last S tokens of each sequence: slot j % S.
// grid: x = column blocks of 256, y = the last min(T, S) tokens, z = sequence.
__global__ __launch_bounds__(256) void k_state_update(const float* __restrict__ P, int T, int NP,
                                                      int S, const int32_t* __restrict__ pos0,
                                                      float* __restrict__ state) {
  const int b = blockIdx.z;
  const int t = max(0, T - S) + blockIdx.y;
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (t >= T || col >= NP) return;
  const int j = pos0[b] + t;
  state[((size_t)b * S + (j % S)) * NP + col] = P[((size_t)b * T + t) * NP + col];
}

// Sum split-K partials: out[i] = sum_k P[k][i], in a fixed order (deterministic).
__global__ __launch_bounds__(256) void k_reduce_partials(const float* __restrict__ P, int ksplit,
                                                         int64_t n, float* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float4 acc = *reinterpret_cast<const float4*>(P + i);
  for (int k = 1; k < ksplit; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(P + (size_t)k * n + i);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<float4*>(out + i) = acc;
}

// Query metadata of a forward chunk: query b*T + t is sequence b at position pos0[b] + t.
__global__ void k_query_meta(int B, int T, const int32_t* __restrict__ pos0,
                             int32_t* __restrict__ q_seq, int32_t* __restrict__ q_pos) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * T) return;
  const int b = i / T;
  q_seq[i] = b;
  q_pos[i] = pos0[b] + (i - b * T);
}

}  // namespace

hipError_t launch_query_meta(int32_t B, int32_t T, const int32_t* pos0, int32_t* q_seq,
                             int32_t* q_pos, hipStream_t s) {
  const int n = B * T;
  hipLaunchKernelGGL(k_query_meta, dim3((n + 255) / 256), dim3(256), 0, s, B, T, pos0, q_seq, q_pos);
  return hipGetLastError();
}

int32_t state_width(const csa_dims& d) { return d.dual ? 4 * d.c + 4 * d.c_I : 2 * d.c; }
int32_t state_rows(const csa_dims& d) { return d.dual ? 2 * d.m : d.m; }
size_t row_bytes(const csa_dims& d) {
  if (d.kv_fmt == CSA_FMT_F32) return (size_t)4 * d.c;
  if (d.kv_fmt == CSA_FMT_MXFP4_BF16) {
    // bf16 RoPE dims, E2M1 codes and E8M0 scales, padded to whole 128-byte lines
    const size_t n = 2 * (size_t)d.rope_dim + (size_t)(d.c - d.rope_dim) / 2 + (size_t)(d.c - d.rope_dim) / 32;
    return (n + 127) / 128 * 128;
  }
  return (size_t)(d.c - d.rope_dim) + 2 * (size_t)d.rope_dim;
}

int32_t project_ksplit(const csa_dims& d, int32_t M) {
  if (d.act_fmt != CSA_FMT_BF16) return 1;
  // Small M (decode): split K so that enough workgroups stream the weights.
  const int NP = state_width(d);
  const int tiles = ((M + PJ_BM - 1) / PJ_BM) * ((NP + PJ_BN - 1) / PJ_BN);
  int ks = 1;
  while (tiles * ks < 512 && (d.d / (ks * 2)) >= 256 && (d.d % (ks * 2 * PJ_BK)) == 0) ks *= 2;
  return ks;
}

hipError_t launch_project(const csa_dims& d, const csa_weights& w, const void* H, int32_t M,
                          int32_t ksplit, float* P, hipStream_t s) {
  const int NP = state_width(d);
  const int nkv = d.dual ? 4 * d.c : 2 * d.c;
  if (d.act_fmt == CSA_FMT_BF16 && project_gemm_ok(M)) {
    // long chunks: the 128x128-tile GEMM (same partial layout)
    return launch_project_gemm((const uint16_t*)H, (const uint16_t*)w.w_kv, (const uint16_t*)w.w_idx, nkv, M,
                               NP, d.d, ksplit, P, s);
  }
  if (d.act_fmt == CSA_FMT_BF16) {
    dim3 grid((NP + PJ_BN - 1) / PJ_BN, (M + PJ_BM - 1) / PJ_BM, ksplit);
    hipLaunchKernelGGL(k_project_bf16, grid, dim3(256), 0, s, (const uint16_t*)H,
                       (const uint16_t*)w.w_kv, (const uint16_t*)w.w_idx, nkv, M, NP, d.d,
                       d.d / ksplit, P);
  } else {
    dim3 grid((NP + 15) / 16, (M + 15) / 16);
    hipLaunchKernelGGL(k_project_f32, grid, dim3(256), 0, s, (const float*)H,
                       (const float*)w.w_kv, (const float*)w.w_idx, nkv, M, NP, d.d, P);
  }
  return hipGetLastError();
}

bool project_step_ok(const csa_dims& d, int32_t T) {
  return T == 1 && d.act_fmt == CSA_FMT_BF16 && d.d % (64 * PU_SLICES) == 0;
}

size_t project_part_bytes(const csa_dims& d, int32_t B) {
  return (size_t)PU_SLICES * B * state_width(d) * sizeof(float);
}

int32_t project_step_units(const csa_dims& d, int32_t B) { return project_units(state_width(d), B, 2); }

ProjectStepArgs project_step_args(const csa_dims& d, const csa_weights& w, const csa_cache& c,
                                  const void* H, float* part) {
  ProjectStepArgs a;
  a.H = (const uint16_t*)H;
  a.wkv = (const uint16_t*)w.w_kv;
  a.widx = (const uint16_t*)w.w_idx;
  a.nkv = d.dual ? 4 * d.c : 2 * d.c;
  a.M = c.B;
  a.NP = state_width(d);
  a.K = d.d;
  a.part = part;
  return a;
}

hipError_t launch_project_step(const csa_dims& d, const csa_weights& w, const csa_cache& c,
                               const void* H, float* part, hipStream_t s) {
  const ProjectStepArgs a = project_step_args(d, w, c, H, part);
  const int units = project_units(a.NP, a.M, 2);
  hipLaunchKernelGGL(k_project_step, dim3(units), dim3(64), 0, s, a, units);
  return hipGetLastError();
}

FoldArgs fold_args(const csa_dims& d, const csa_weights& w, const csa_cache& c, int32_t T,
                   const int32_t* pos0, const float* P, const float* part) {
  FoldArgs a;
  a.P = P;
  a.part = (T == 1 && !P) ? part : nullptr;
  a.B = c.B;
  a.state = c.state;
  a.S = state_rows(d);
  a.NP = state_width(d);
  a.T = T;
  a.m = d.m;
  a.dual = d.dual;
  a.c = d.c;
  a.r = d.rope_dim;
  a.cI = has_indexer(d) ? d.c_I : 0;
  a.pos0 = pos0;
  a.bias = w.bias;
  a.bias_idx = w.bias_idx;
  a.keys_entry = keys_from_entry(d);
  a.w_ik = a.keys_entry ? w.w_idx : nullptr;
  a.act_f32 = d.act_fmt == CSA_FMT_F32;
  a.gamma = w.gamma_kv;
  a.eps = d.rms_eps;
  a.log2_base = std::log2((double)d.rope_base);
  a.kv_fmt = d.kv_fmt;
  a.idx_fmt = d.idx_fmt;
  a.cap = c.cap;
  a.win_cap = c.win_cap;
  a.rowB = (int)row_bytes(d);
  a.rm = row_map(d, c);
  a.kv = (uint8_t*)c.kv;
  a.ki = (uint8_t*)c.ki;
  a.win = (uint8_t*)c.win;
  a.win_pos = c.win_pos;
  a.n_entries = c.n_entries;
  return a;
}

hipError_t launch_fold(const csa_dims& d, const csa_weights& w, const csa_cache& c, int32_t T,
                       const int32_t* pos0, const float* P, int32_t ksplit, hipStream_t s,
                       const float* part) {
  if (ksplit != 1) return hipErrorInvalidValue;  // partials are summed first
  const FoldArgs a = fold_args(d, w, c, T, pos0, P, part);
  dim3 grid(fold_grid_x(a), c.B);
  if (a.keys_entry) {
    if (a.part) hipLaunchKernelGGL((k_fold<true, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_fold<false, true>), grid, dim3(256), 0, s, a);
  } else {
    if (a.part) hipLaunchKernelGGL((k_fold<true, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_fold<false, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_state_update(const csa_dims& d, const csa_cache& c, int32_t T,
                               const int32_t* pos0, const float* P, int32_t ksplit,
                               hipStream_t s) {
  if (ksplit != 1) return hipErrorInvalidValue;  // partials are summed first
  const int S = state_rows(d), NP = state_width(d);
  dim3 grid((NP + 255) / 256, min(T, S), c.B);
  hipLaunchKernelGGL(k_state_update, grid, dim3(256), 0, s, P, T, NP, S, pos0, c.state);
  return hipGetLastError();
}

hipError_t launch_reduce_partials(const float* P, int32_t ksplit, int64_t n, float* out,
                                  hipStream_t s) {
  // n is a multiple of 4 (NP is a multiple of 4 for every supported layout)
  const int64_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(k_reduce_partials, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     P, ksplit, n, out);
  return hipGetLastError();
}

}  // namespace csa
