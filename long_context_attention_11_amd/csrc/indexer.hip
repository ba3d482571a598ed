// Lightning-indexer scores for gfx950:
//   I_{t,s} = sum_h w_{t,h} * ReLU(q^I_{t,h} . K^I_s),  s < V(t) = min(t / m, n_entries)
// (reading notes "DeepSeekV4技术报告阅读笔记" §2.3.2 eq. 16 and the causal rule after eq. 17;
// deep dive "DeepSeek-V4 架构设计深度解析" §3.2; PaperTrace "02 · DeepSeek-V4" §2.2).
//
// The contraction over c_I runs on bf16 MFMA: E4M3 values widen to bf16 exactly, products
// are exact and accumulate in float32.  (The fp8 MFMA forms accumulate with fewer bits:
// measured errors of ~2^-16 of sum|a_k b_k|, which top-k selection cannot tolerate.)
// The ReLU, the head weight and the sum over heads are fused into the MFMA epilogue.
#include "csa_internal.h"

namespace csa {
namespace {

constexpr int IX_CI = 128;  // indexer key width handled by the MFMA kernel

// Convert 32 E4M3 codes (8 dwords, dims g*32 .. g*32+31 of one row) into four bf16x8
// MFMA operands, one per 32-wide K step: step ks takes codes ks*8 .. ks*8+7.
__device__ __forceinline__ void e4m3x32_to_ops(const uint4& lo, const uint4& hi, bf16x8 op[4]) {
  const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint32_t a0, a1, b0, b1;
    e4m3x4_to_bf16x4(w[2 * ks], a0, a1);
    e4m3x4_to_bf16x4(w[2 * ks + 1], b0, b1);
    uint4 v = make_uint4(a0, a1, b0, b1);
    op[ks] = __builtin_bit_cast(bf16x8, v);
  }
}

// One workgroup = 4 waves; blockIdx.x = group of QPW queries (same sequence), blockIdx.y =
// entry chunk; wave w scans its quarter of the chunk in tiles of 16 entries.
// MFMA mapping (16x16x32 bf16): A = q^I rows (heads), B = K^I rows (entries), contraction
// over c_I.  Lane l holds head/entry (l & 15) and, within each 32-wide K step ks, dims
// g*32 + ks*8 .. +7 with g = l >> 4 -- the same mapping on both operands, so each product
// pairs equal dims.  Output tile: lane l holds entry (l & 15), heads 4g .. 4g+3.
template <int NH, int QPW>
__global__ __launch_bounds__(256) void k_indexer_bf16(
    const uint8_t* __restrict__ qI, const uint16_t* __restrict__ wI,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int Q,
    const uint8_t* __restrict__ ki, int cap, const int32_t* __restrict__ n_entries, int m,
    float* __restrict__ scores, int64_t ld, int chunk) {
  constexpr int HT = NH / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int q0 = blockIdx.x * QPW;
  const int seq = q_seq[q0];
  const int nent = n_entries[seq];
  int V[QPW];
  int Vmax = 0;
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    const int q = q0 + qq;
    V[qq] = q < Q ? max(0, min(q_pos[q] / m, nent)) : 0;
    Vmax = max(Vmax, V[qq]);
  }
  const int c_lo = blockIdx.y * chunk;
  const int c_hi = min(c_lo + chunk, Vmax);
  if (c_lo >= c_hi) return;
  const int per_wave = (chunk / 4 + 15) & ~15;
  const int w_lo = c_lo + wave * per_wave;
  const int w_hi = min(c_hi, w_lo + per_wave);
  if (w_lo >= w_hi) return;

  // A operands (q^I) and head weights, per query, kept in registers.
  bf16x8 A[QPW][HT][4];
  float W[QPW][HT][4];
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    const int q = min(q0 + qq, Q - 1);
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const uint8_t* src = qI + ((size_t)q * NH + ht * 16 + col) * IX_CI + g * 32;
      uint4 lo = *reinterpret_cast<const uint4*>(src);
      uint4 hi = *reinterpret_cast<const uint4*>(src + 16);
      e4m3x32_to_ops(lo, hi, A[qq][ht]);
#pragma unroll
      for (int e = 0; e < 4; ++e) W[qq][ht][e] = bf16_bits_to_f32(wI[(size_t)q * NH + ht * 16 + 4 * g + e]);
    }
  }
  const uint8_t* kbase = ki + (size_t)seq * cap * IX_CI + g * 32;
  // Register ring of DEPTH tiles: the raw bytes of the next DEPTH tiles are in flight while
  // one computes (each tile: 16 entries x 128 B per wave, 32 B per lane).
  constexpr int DEPTH = 4;
  uint4 rlo[DEPTH], rhi[DEPTH];
  auto load_tile = [&](int s0, uint4& lo, uint4& hi) {
    const int s = min(s0 + col, w_hi - 1);
    const uint8_t* src = kbase + (size_t)s * IX_CI;
    lo = load_stream16(src);
    hi = load_stream16(src + 16);
  };
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) load_tile(w_lo + 16 * i, rlo[i], rhi[i]);
  for (int base = w_lo; base < w_hi; base += 16 * DEPTH) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      const int s0 = base + 16 * i;
      if (s0 >= w_hi) break;
      const uint4 clo = rlo[i], chi = rhi[i];
      if (s0 + 16 * DEPTH < w_hi) load_tile(s0 + 16 * DEPTH, rlo[i], rhi[i]);
      bf16x8 B[4];
      e4m3x32_to_ops(clo, chi, B);
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq) {
        float part = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          f32x4 acc = {0, 0, 0, 0};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[qq][ht][ks], B[ks], acc, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) part = fmaf(W[qq][ht][e], fmaxf(acc[e], 0.f), part);
        }
        part += __shfl_xor(part, 16, 64);
        part += __shfl_xor(part, 32, 64);
        const int s = s0 + col;
        if (g == 0 && s < V[qq] && s < w_hi) scores[(size_t)(q0 + qq) * ld + s] = part;
      }
    }
  }
}

// float32 indexer (fp32 formats): one thread per (query, entry).
__global__ __launch_bounds__(256) void k_indexer_f32(
    const float* __restrict__ qI, const float* __restrict__ wI, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int Q, const float* __restrict__ ki, int cap,
    const int32_t* __restrict__ n_entries, int m, int nh, int cI, float* __restrict__ scores,
    int64_t ld) {
  const int q = blockIdx.y;
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= Q) return;
  const int seq = q_seq[q];
  const int V = max(0, min(q_pos[q] / m, n_entries[seq]));
  if (s >= V) return;
  const float* k = ki + ((size_t)seq * cap + s) * cI;
  float acc = 0.f;
  for (int h = 0; h < nh; ++h) {
    const float* qh = qI + ((size_t)q * nh + h) * cI;
    float dot = 0.f;
    for (int u = 0; u < cI; ++u) dot = fmaf(qh[u], k[u], dot);
    acc = fmaf(wI[(size_t)q * nh + h], fmaxf(dot, 0.f), acc);
  }
  scores[(size_t)q * ld + s] = acc;
}

}  // namespace

hipError_t launch_indexer(const csa_dims& d, const csa_cache& c, const void* qI, const void* w,
                          const int32_t* q_seq, const int32_t* q_pos, int32_t Q, float* scores,
                          int64_t ld, hipStream_t s) {
  if (d.idx_fmt == CSA_FMT_F32) {
    dim3 grid((c.cap + 255) / 256, Q);
    hipLaunchKernelGGL(k_indexer_f32, grid, dim3(256), 0, s, (const float*)qI, (const float*)w,
                       q_seq, q_pos, Q, (const float*)c.ki, c.cap, c.n_entries, d.m, d.n_hI,
                       d.c_I, scores, ld);
    return hipGetLastError();
  }
  // E4M3 keys: bf16 MFMA.  One query per group; entry chunks sized to fill the GPU.
  const int chunk = 512;
  dim3 grid(Q, (c.cap + chunk - 1) / chunk);
  switch (d.n_hI) {
    case 64:
      hipLaunchKernelGGL((k_indexer_bf16<64, 1>), grid, dim3(256), 0, s, (const uint8_t*)qI,
                         (const uint16_t*)w, q_seq, q_pos, Q, (const uint8_t*)c.ki, c.cap,
                         c.n_entries, d.m, scores, ld, chunk);
      break;
    case 32:
      hipLaunchKernelGGL((k_indexer_bf16<32, 1>), grid, dim3(256), 0, s, (const uint8_t*)qI,
                         (const uint16_t*)w, q_seq, q_pos, Q, (const uint8_t*)c.ki, c.cap,
                         c.n_entries, d.m, scores, ld, chunk);
      break;
    case 16:
      hipLaunchKernelGGL((k_indexer_bf16<16, 1>), grid, dim3(256), 0, s, (const uint8_t*)qI,
                         (const uint16_t*)w, q_seq, q_pos, Q, (const uint8_t*)c.ki, c.cap,
                         c.n_entries, d.m, scores, ld, chunk);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace csa
