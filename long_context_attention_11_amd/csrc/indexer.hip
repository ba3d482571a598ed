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
  constexpr int DEPTH = 4;
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
  // this wave's entries: tiles of 16 dealt round-robin over the 4 waves of the chunk
  const int c_lo = blockIdx.y * chunk;
  const int c_hi = min(c_lo + chunk, Vmax);
  if (c_lo >= c_hi) return;
  const int w_lo = c_lo + 16 * wave;
  if (w_lo >= c_hi) return;
  const int stride = 64;  // 4 waves x 16 entries

  const uint8_t* kbase = ki + (size_t)seq * cap * IX_CI + g * 32;
  // Prologue: the query operands (q^I rows, head weights) and the first DEPTH tiles of keys
  // are all requested before anything waits, so their latencies overlap.  The ring holds
  // DEPTH tiles (16 entries x 128 B per wave, 32 B per lane); waits count outstanding loads
  // in issue order, so tile 0 is issued first among the keys.
  uint4 araw[QPW][HT][2];
  uint2 wraw[QPW][HT];
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    const int q = min(q0 + qq, Q - 1);
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const uint8_t* src = qI + ((size_t)q * NH + ht * 16 + col) * IX_CI + g * 32;
      araw[qq][ht][0] = *reinterpret_cast<const uint4*>(src);
      araw[qq][ht][1] = *reinterpret_cast<const uint4*>(src + 16);
      wraw[qq][ht] = *reinterpret_cast<const uint2*>(wI + (size_t)q * NH + ht * 16 + 4 * g);
    }
  }
  uint4 rlo[DEPTH], rhi[DEPTH];
  auto load_tile = [&](int s0, uint4& lo, uint4& hi) {
    const int s = min(s0 + col, c_hi - 1);
    const uint8_t* src = kbase + (size_t)s * IX_CI;
    lo = *reinterpret_cast<const uint4*>(src);
    hi = *reinterpret_cast<const uint4*>(src + 16);
  };
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) load_tile(w_lo + stride * i, rlo[i], rhi[i]);
  __builtin_amdgcn_sched_barrier(0);

  bf16x8 A[QPW][HT][4];
  float W[QPW][HT][4];
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      e4m3x32_to_ops(araw[qq][ht][0], araw[qq][ht][1], A[qq][ht]);
      const uint2 w4 = wraw[qq][ht];
      W[qq][ht][0] = bf16_bits_to_f32(w4.x & 0xffffu);
      W[qq][ht][1] = bf16_bits_to_f32(w4.x >> 16);
      W[qq][ht][2] = bf16_bits_to_f32(w4.y & 0xffffu);
      W[qq][ht][3] = bf16_bits_to_f32(w4.y >> 16);
    }
  }
  // Straight-line ring: every wave runs whole rounds of DEPTH tiles.  Loads past the end are
  // clamped to the last entry (same cache line for every lane) and their results discarded,
  // so no load is conditional and the loads of the next round stay in flight while this
  // round's tiles are multiplied.
  const int rounds = (c_hi - w_lo + stride * DEPTH - 1) / (stride * DEPTH);
  int it = 0;
  do {  // rounds >= 1 since w_lo < c_hi
    const int base = w_lo + it * stride * DEPTH;
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      const int s0 = base + stride * i;
      // widen the tile first, then reuse its registers for the load of the next round
      bf16x8 Bop[4];
      e4m3x32_to_ops(rlo[i], rhi[i], Bop);
      load_tile(s0 + stride * DEPTH, rlo[i], rhi[i]);
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq) {
        float part = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          f32x4 acc = {0, 0, 0, 0};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[qq][ht][ks], Bop[ks], acc, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) part = fmaf(W[qq][ht][e], fmaxf(acc[e], 0.f), part);
        }
        part += __shfl_xor(part, 16, 64);
        part += __shfl_xor(part, 32, 64);
        const int s = s0 + col;
        if (g == 0 && s < min(V[qq], c_hi)) scores[(size_t)(q0 + qq) * ld + s] = part;
      }
    }
  } while (++it < rounds);
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
  // E4M3 keys: bf16 MFMA.  One query per group; entry chunks sized so that the grid is about
  // two workgroups (8 waves) per CU, each wave streaming a long run of tiles.
  const int target_wgs = 512;
  const int per_q = std::max(1, target_wgs / std::max(Q, 1));
  int chunk = (c.cap + per_q - 1) / per_q;
  chunk = std::max(256, (chunk + 255) / 256 * 256);
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
