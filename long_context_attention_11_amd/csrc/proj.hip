// The projections around the attention core, for gfx950:
//   query side   c^Q = h W^DQ, q = c^Q W^UQ, q^I = c^Q W^IUQ, w = h W^w
//   output side  the grouped output projection: heads in g consecutive groups, group i's
//                c n_h / g values projected to d_g by its own map, the g results
//                concatenated and projected to d
// (reading notes "DeepSeekV4技术报告阅读笔记" §2.3.2 eqs. 13-15, §2.3.3 eq. 18 and its grouped
// output projection paragraph; deep dive "DeepSeek-V4 架构设计深度解析" stage three for g and
// d_g; PaperTrace "02 · DeepSeek-V4: 压缩注意力撑起 1M 上下文" §1 for Pro's d_c = 1536, from its
// 1536 x 128 x 512 query up-projection, and §2.2 for g and d_g.)
//
// All six maps are plain bf16 GEMMs with float32 accumulation on MFMA.  One kernel serves
// them: 64x64 output tiles, BK = 64 stages double buffered in LDS, a group index (the g
// group maps of the output side run in one launch) and split-K for short inputs, whose
// partials finishing kernels sum in a fixed order.  Weights are stored one row per output
// column ([N][K], K contiguous), the layout the tiles load with 16-byte reads.
#include "csa_internal.h"

namespace csa {
namespace {

constexpr int GM_ROWS = 8192;   // rows per pass of the host loops (bounds the workspace)
constexpr int GM_BIG_M = 256;   // inputs of at least this many rows take the 128x128 tiles
constexpr int GM_WIDE_M = 4096; // ... and of at least this many the 256x256 tiles

struct GemmArgs {
  const uint16_t* A;   // [M][lda]; group z reads columns z * a_zoff .. + K
  int64_t lda, a_zoff;
  const uint16_t* B;   // weight rows n < nb1: B + n * ldb (+ z * b_zstride) ...
  const uint16_t* B2;  // ... rows n >= nb1: B2 + (n - nb1) * ldb
  int nb1;
  int64_t ldb, b_zstride;
  int M, N, K, kchunk, ksplit;
  int n_bf;            // columns n < n_bf are stored to D in bfloat16 (ksplit == 1 only)
  uint16_t* D;
  int64_t ldd, d_zoff;
  float* P;            // columns n >= n_bf: P[ks * p_ks + row * ldp + z * p_zoff + n - n_bf]
  int64_t ldp, p_zoff, p_ks;
};

// blockIdx = (column tile, row tile, z * ksplit + ks).  A workgroup of 4 waves computes a
// BM x BN tile, each wave a (BM/2) x (BN/2) quarter as (BM/32) x (BN/32) MFMA 16x16x32 tiles;
// stages of BK k are double buffered in LDS with rows padded by 8 bf16 (the 16 rows one read
// instruction touches then start in distinct 16-byte bank groups).  64x64 / BK 64 serves short
// inputs; 128x128 / BK 32 reads each operand fragment from LDS once per 4 MFMAs instead of 2.
template <int BM, int BN, int BK>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmArgs g) {
  constexpr int LD = BK + 8;
  constexpr int PR = BK / 8;                 // 16-byte pieces per row of a stage
  constexpr int RPP = 256 / PR;              // rows covered by one pass of the 256 threads
  constexpr int PA = BM / RPP, PB = BN / RPP;
  constexpr int TI = BM / 32, TJ = BN / 32;  // MFMA tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int z = blockIdx.z / g.ksplit, ks = blockIdx.z % g.ksplit;
  const int k_begin = ks * g.kchunk, k_end = min(g.K, k_begin + g.kchunk);
  const int lr = tid / PR, lc = (tid % PR) * 8;
  // Rows past M (columns past N) load the last row (column) again: they only feed outputs
  // past M (N), which are not stored, so every load is unconditional (no branch per load).
  const uint16_t* arow[PA];
  const uint16_t* brow[PB];
#pragma unroll
  for (int h = 0; h < PA; ++h) {
    const int r = lr + RPP * h;
    arow[h] = g.A + (size_t)min(m0 + r, g.M - 1) * g.lda + (size_t)z * g.a_zoff;
  }
#pragma unroll
  for (int h = 0; h < PB; ++h) {
    const int r = lr + RPP * h;
    const int n = min(n0 + r, g.N - 1);
    brow[h] = (n < g.nb1 ? g.B + (size_t)n * g.ldb : g.B2 + (size_t)(n - g.nb1) * g.ldb) +
              (size_t)z * g.b_zstride;
  }
  uint4 ra[PA], rb[PB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < PA; ++h) {
      const uint4 v = *reinterpret_cast<const uint4*>(arow[h] + k0 + lc);
      ra[h] = v;
    }
#pragma unroll
    for (int h = 0; h < PB; ++h) {
      const uint4 v = *reinterpret_cast<const uint4*>(brow[h] + k0 + lc);
      rb[h] = v;
    }
    asm volatile("" ::: "memory");   // compiler-only fence, as in k_gemm_wide
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < PA; ++h) *reinterpret_cast<uint4*>(&As[buf][(lr + RPP * h) * LD + lc]) = ra[h];
#pragma unroll
    for (int h = 0; h < PB; ++h) *reinterpret_cast<uint4*>(&Bs[buf][(lr + RPP * h) * LD + lc]) = rb[h];
  };
  const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (BN / 2);
  const int fr = lane & 15, fg = lane >> 4;
  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  int buf = 0;
  if (k_begin < k_end) gload(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += BK) {
    sstore(buf);
    __syncthreads();
    if (k0 + BK < k_end) gload(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8 a[TI], b[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm + 16 * i + fr) * LD + kk + fg * 8]);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(wn + 16 * j + fr) * LD + kk + fg * 8]);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    buf ^= 1;
  }
  // an MFMA 16x16 result: lane holds column (lane & 15), rows 4 (lane >> 4) + e
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = n0 + wn + 16 * j + fr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm + 16 * i + 4 * fg + e;
        if (row >= g.M || col >= g.N) continue;
        if (col < g.n_bf)
          g.D[(size_t)row * g.ldd + (size_t)z * g.d_zoff + col] = (uint16_t)f32_to_bf16_bits(acc[i][j][e]);
        else
          g.P[(size_t)ks * g.p_ks + (size_t)row * g.ldp + (size_t)z * g.p_zoff + (col - g.n_bf)] = acc[i][j][e];
      }
    }
}

// Long inputs: 256x256 output tiles, 8 waves in a 2 x 4 grid, each wave a 128x64 part as 8 x 4
// MFMA 16x16x32 tiles (128 accumulators per lane, two waves per SIMD).  A stage is BK = 64 deep
// and double buffered in LDS (rows padded by 8 bf16, 147 KB in all, one workgroup per CU).
// The LDS read rate bounds the smaller tiles: each fragment read here feeds 4 (A) or 8 (B)
// MFMAs, so a stage moves 0.5 KB of LDS data per 16x16x32 MFMA (written and read), against
// 0.81 KB on the 128x128 tiles.  Same arguments and stores as k_gemm_bf16; workgroups are
// ordered so that the column tiles of one row tile run on the same XCD (its L2 then holds
// the shared A rows).
template <int BK>
__global__ __launch_bounds__(512) void k_gemm_wide(GemmArgs g) {
  constexpr int BM = 256, BN = 256, LD = BK + 8;
  constexpr int PR = BK / 8;                 // 16-byte pieces per row of a stage
  constexpr int RPP = 512 / PR;              // rows covered by one pass of the 512 threads
  constexpr int PA = BM / RPP, PB = BN / RPP;
  constexpr int TI = 8, TJ = 4;              // MFMA tiles per wave (128 x 64)
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t ncol = gridDim.x, nxy = gridDim.x * gridDim.y;
  const uint32_t L = xcd_logical_id(blockIdx.y * ncol + blockIdx.x, nxy);
  const int m0 = (int)(L / ncol) * BM, n0 = (int)(L % ncol) * BN;
  const int z = blockIdx.z / g.ksplit, ks = blockIdx.z % g.ksplit;
  const int k_begin = ks * g.kchunk, k_end = min(g.K, k_begin + g.kchunk);
  const int lr = tid / PR, lc = (tid % PR) * 8;
  // Rows past M (columns past N) load the last row (column) again: they only feed outputs
  // past M (N), which are not stored, so every load is unconditional (no branch per load).
  const uint16_t* arow[PA];
  const uint16_t* brow[PB];
#pragma unroll
  for (int h = 0; h < PA; ++h) {
    const int r = lr + RPP * h;
    arow[h] = g.A + (size_t)min(m0 + r, g.M - 1) * g.lda + (size_t)z * g.a_zoff;
  }
#pragma unroll
  for (int h = 0; h < PB; ++h) {
    const int r = lr + RPP * h;
    const int n = min(n0 + r, g.N - 1);
    brow[h] = (n < g.nb1 ? g.B + (size_t)n * g.ldb : g.B2 + (size_t)(n - g.nb1) * g.ldb) +
              (size_t)z * g.b_zstride;
  }
  uint4 ra[PA], rb[PB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < PA; ++h) {
      const uint4 v = *reinterpret_cast<const uint4*>(arow[h] + k0 + lc);
      ra[h] = v;
    }
#pragma unroll
    for (int h = 0; h < PB; ++h) {
      const uint4 v = *reinterpret_cast<const uint4*>(brow[h] + k0 + lc);
      rb[h] = v;
    }
    // a compiler-only fence (it waits for nothing): without it the staging registers are
    // kept in private memory, and every load is then waited for as soon as it is issued
    asm volatile("" ::: "memory");
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < PA; ++h) *reinterpret_cast<uint4*>(&As[buf][(lr + RPP * h) * LD + lc]) = ra[h];
#pragma unroll
    for (int h = 0; h < PB; ++h) *reinterpret_cast<uint4*>(&Bs[buf][(lr + RPP * h) * LD + lc]) = rb[h];
  };
  const int wm = (wave >> 2) * 128, wn = (wave & 3) * 64;
  const int fr = lane & 15, fg = lane >> 4;
  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  int buf = 0;
  if (k_begin < k_end) gload(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += BK) {
    sstore(buf);
    __syncthreads();
    if (k0 + BK < k_end) gload(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8 b[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(wn + 16 * j + fr) * LD + kk + fg * 8]);
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&As[buf][(wm + 16 * i + fr) * LD + kk + fg * 8]);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a, acc[i][j], 0, 0, 0);
      }
    }
    buf ^= 1;
  }
  // The weights are the MFMA's first operand, so a 16x16 result holds the tile transposed:
  // lane l has row (l & 15) and the four consecutive columns 4 (l >> 4) + e, stored as one
  // 8-byte (bf16) or 16-byte (fp32) write when the layout allows it.
  const bool vec = g.N % 4 == 0 && g.n_bf % 4 == 0 && g.ldd % 4 == 0 && g.d_zoff % 4 == 0 &&
                   g.ldp % 4 == 0 && g.p_zoff % 4 == 0 && g.p_ks % 4 == 0 &&
                   (reinterpret_cast<uintptr_t>(g.D) & 7) == 0 && (reinterpret_cast<uintptr_t>(g.P) & 15) == 0;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int row = m0 + wm + 16 * i + fr;
      const int c0 = n0 + wn + 16 * j + 4 * fg;
      if (row >= g.M) continue;
      if (vec) {
        if (c0 >= g.N) continue;
        if (c0 < g.n_bf) {
          *reinterpret_cast<uint2*>(g.D + (size_t)row * g.ldd + (size_t)z * g.d_zoff + c0) =
              make_uint2(f32_to_bf16_bits(acc[i][j][0]) | (f32_to_bf16_bits(acc[i][j][1]) << 16),
                         f32_to_bf16_bits(acc[i][j][2]) | (f32_to_bf16_bits(acc[i][j][3]) << 16));
        } else {
          *reinterpret_cast<f32x4*>(g.P + (size_t)ks * g.p_ks + (size_t)row * g.ldp + (size_t)z * g.p_zoff +
                                    (c0 - g.n_bf)) = acc[i][j];
        }
        continue;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = c0 + e;
        if (col >= g.N) continue;
        if (col < g.n_bf)
          g.D[(size_t)row * g.ldd + (size_t)z * g.d_zoff + col] = (uint16_t)f32_to_bf16_bits(acc[i][j][e]);
        else
          g.P[(size_t)ks * g.p_ks + (size_t)row * g.ldp + (size_t)z * g.p_zoff + (col - g.n_bf)] = acc[i][j][e];
      }
    }
}

// Split-K partials of an fp32 block [M][n1 + n2] (row pitch ldp, partial pitch p_ks) summed in
// partial order and stored in bfloat16: columns c < n1 to D1 [M][ldd1], the rest to D2 [M][ldd2].
__global__ __launch_bounds__(256) void k_sum_bf16(const float* __restrict__ P, int ksplit, int64_t p_ks,
                                                  int M, int64_t ldp, int n1, uint16_t* __restrict__ D1,
                                                  int64_t ldd1, int n2, uint16_t* __restrict__ D2,
                                                  int64_t ldd2) {
  const int ncol = n1 + n2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * ncol) return;
  const int r = (int)(i / ncol), c = (int)(i % ncol);
  float s = 0.f;
  for (int k = 0; k < ksplit; ++k) s += P[(size_t)k * p_ks + (size_t)r * ldp + c];
  if (c < n1) D1[(size_t)r * ldd1 + c] = (uint16_t)f32_to_bf16_bits(s);
  else D2[(size_t)r * ldd2 + (c - n1)] = (uint16_t)f32_to_bf16_bits(s);
}

// The query side's finish, one launch: blocks [0, nsum) sum the split-K partials of q (when K
// was split) into bfloat16; the rest store q^I in the indexer's format, one wave per (token,
// head): lane l takes dims 2l, 2l + 1 (partials summed in order), so a block of 32 dims is
// the 16 lanes of one DPP row.  E4M3: [n_hI][c_I] codes per token.  MXFP4: per token n_hI
// rows of c_I / 2 element bytes (dim 2i in the low nibble of byte i), then n_hI rows of
// c_I / 32 scale codes; the block scale is 2^(floor(log2 max|v|) - 2) (1 for an all-zero
// block), the elements the nearest E2M1 values of v / scale, ties to even, saturating at 6.
// Built for c_I = 128 (64 lanes x 2 dims).
__global__ __launch_bounds__(256) void k_finish_q(const float* __restrict__ P, int ksplit, int64_t p_ks, int M,
                                                  int64_t ldp, int nq, uint16_t* __restrict__ q, int nsum,
                                                  const float* __restrict__ PqI, int n_hI, int fmt,
                                                  uint8_t* __restrict__ qI) {
  constexpr int CI = 128;
  if ((int)blockIdx.x < nsum) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * nq) return;
    const int r = (int)(i / nq), c = (int)(i % nq);
    float s = 0.f;
    for (int k = 0; k < ksplit; ++k) s += P[(size_t)k * p_ks + (size_t)r * ldp + c];
    q[(size_t)r * nq + c] = (uint16_t)f32_to_bf16_bits(s);
    return;
  }
  const int wid = ((int)blockIdx.x - nsum) * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wid >= M * n_hI) return;   // uniform per wave
  const int r = wid / n_hI, h = wid % n_hI;
  float v0 = 0.f, v1 = 0.f;
  for (int k = 0; k < ksplit; ++k) {
    const float2 p = *reinterpret_cast<const float2*>(PqI + (size_t)k * p_ks + (size_t)r * ldp + h * CI + 2 * lane);
    v0 += p.x;
    v1 += p.y;
  }
  if (fmt == CSA_FMT_MXFP4) {
    float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    int e = 0;
    if (amax > 0.f) {
      int ex;
      frexpf(amax, &ex);   // amax = f 2^ex with f in [0.5, 1): floor(log2 amax) = ex - 1
      e = min(127, max(-127, ex - 1 - 2));
    }
    const size_t row = (size_t)n_hI * (CI / 2 + CI / 32);
    uint8_t* base = qI + (size_t)r * row;
    base[(size_t)h * (CI / 2) + lane] = (uint8_t)(e2m1_code(ldexpf(v0, -e)) | (e2m1_code(ldexpf(v1, -e)) << 4));
    if ((lane & 15) == 0) base[(size_t)n_hI * (CI / 2) + (size_t)h * (CI / 32) + (lane >> 4)] = (uint8_t)(e + 127);
  } else {
    *reinterpret_cast<uint16_t*>(qI + ((size_t)r * n_hI + h) * CI + 2 * lane) =
        (uint16_t)(f32_to_e4m3(v0) | (f32_to_e4m3(v1) << 8));
  }
}

// Split K for short inputs, so that the weight stream spreads evenly over the 256 CUs (one CU
// streams only ~25 GB/s): the split minimizing the largest per-CU share of tiles, ceil(tiles
// ks / 256) / ks, with ties going to the workgroup count nearest 512 (two per CU: one
// workgroup per CU streams slower, e.g. Pro's 256 group tiles unsplit took 122 us against
// 104 us split in two).  Each K range
// stays a multiple of the 64-deep stage and at least 256 long.  Long inputs (256x256 tiles)
// are not split once their tiles fill half the CUs: there the float32 partials (written and
// summed again: 8 x 8192 x 1600 floats for the Flash latent split 8 ways) cost more than the
// CUs the split would add.
// The 256x256 tiles run one workgroup per CU, so they are taken only where their rounds of 256
// workgroups are at least 80 % full (or there are four or more rounds): 8192 x 2560 makes 320
// tiles, whose second round would leave three CUs in four idle.
int gemm_tile(int M, int N, int Z) {
  if (M >= GM_WIDE_M) {
    const int64_t tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256) * Z;
    const int64_t rounds = (tiles + 255) / 256;
    if (rounds >= 4 || tiles * 5 >= rounds * 256 * 4) return 256;
  }
  return M >= GM_BIG_M ? 128 : 64;
}

int gemm_ksplit(int M, int N, int Z, int K) {
  const int t = gemm_tile(M, N, Z);
  const int tiles = ((M + t - 1) / t) * ((N + t - 1) / t) * Z;
  if (t == 256 && tiles >= 128) return 1;
  int best = 1;
  double best_cost = (double)((tiles + 255) / 256);
  for (int ks = 2; K % (ks * 64) == 0 && K / ks >= 256; ks *= 2) {
    const double cost = (double)((tiles * ks + 255) / 256) / ks;
    const bool tie = cost == best_cost;
    if (cost < best_cost || (tie && std::abs(tiles * ks - 512) < std::abs(tiles * best - 512))) {
      best = ks;
      best_cost = cost;
    }
  }
  return best;
}

// One GEMM plan: output columns [0, n_direct) go to D in bfloat16 when K is not split; the
// rest (or all, when split) go to fp32 partials at P.
struct Plan {
  int ks;
  int n_bf;
  int64_t ldp;      // fp32 columns per row (all groups)
  size_t p_floats;  // partial buffer size
};

Plan plan_of(int M, int N, int Z, int K, int n_direct) {
  Plan p;
  p.ks = gemm_ksplit(M, N, Z, K);
  p.n_bf = p.ks == 1 ? n_direct : 0;
  p.ldp = (int64_t)Z * (N - p.n_bf);
  p.p_floats = (size_t)p.ks * M * p.ldp;
  return p;
}

hipError_t launch_gemm(const GemmArgs& g, int Z, hipStream_t s) {
  const int t = gemm_tile(g.M, g.N, Z);
  dim3 grid((g.N + t - 1) / t, (g.M + t - 1) / t, Z * g.ksplit);
  if (t == 256) hipLaunchKernelGGL((k_gemm_wide<64>), grid, dim3(512), 0, s, g);
  else if (t == 128) hipLaunchKernelGGL((k_gemm_bf16<128, 128, 32>), grid, dim3(256), 0, s, g);
  else hipLaunchKernelGGL((k_gemm_bf16<64, 64, 64>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_sum_bf16(const float* P, int ks, int64_t p_ks, int M, int64_t ldp, int n1, uint16_t* D1,
                           int64_t ldd1, int n2, uint16_t* D2, int64_t ldd2, hipStream_t s) {
  const int64_t n = (int64_t)M * (n1 + n2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_sum_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, P, ks, p_ks, M, ldp, n1, D1,
                     ldd1, n2, D2, ldd2);
  return hipGetLastError();
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Rows of the first and the last pass (the largest partial buffers come from one of them).
template <typename F>
size_t max_over_passes(int32_t T, F f) {
  const int first = std::min<int32_t>(T, GM_ROWS);
  const int last = T % GM_ROWS ? T % GM_ROWS : first;
  return std::max(f(first), f(last));
}

size_t query_ws_rows(const csa_dims& d, int32_t d_c, int M) {
  const int n1 = d_c + (d.dual ? d.n_hI : 0);
  const int n2 = d.n_h * d.c + (d.dual ? d.n_hI * d.c_I : 0);
  const Plan p1 = plan_of(M, n1, 1, d.d, d_c);
  const Plan p2 = plan_of(M, n2, 1, d_c, d.n_h * d.c);
  return align256((size_t)M * d_c * 2) + align256(p1.p_floats * 4) + align256(p2.p_floats * 4);
}

size_t output_ws_rows(const csa_dims& d, int32_t g, int32_t d_g, int M) {
  const Plan p3 = plan_of(M, d_g, g, d.n_h * d.c / g, d_g);
  const Plan p4 = plan_of(M, d.d, 1, g * d_g, d.d);
  return align256((size_t)M * g * d_g * 2) + align256(p3.p_floats * 4) + align256(p4.p_floats * 4);
}

}  // namespace

// The compression projection P[ks][M][NP] = H . [w_kv rows; w_idx rows]^T for inputs of at
// least 256 rows, on the 128x128 tiles (the chunked compress path).
bool project_gemm_ok(int32_t M) { return M >= GM_BIG_M; }

hipError_t launch_project_gemm(const uint16_t* H, const uint16_t* wkv, const uint16_t* widx, int nkv, int M,
                               int NP, int K, int ksplit, float* P, hipStream_t s) {
  GemmArgs g{};
  g.A = H;
  g.lda = K;
  g.B = wkv;
  g.B2 = widx;
  g.nb1 = nkv;
  g.ldb = K;
  g.M = M, g.N = NP, g.K = K, g.ksplit = ksplit, g.kchunk = K / ksplit;
  g.n_bf = 0;
  g.P = P, g.ldp = NP, g.p_ks = (int64_t)M * NP;
  return launch_gemm(g, 1, s);
}

size_t query_project_ws_bytes(const csa_dims& d, int32_t d_c, int32_t T) {
  return max_over_passes(T, [&](int M) { return query_ws_rows(d, d_c, M); });
}

size_t output_project_ws_bytes(const csa_dims& d, int32_t g, int32_t d_g, int32_t T) {
  return max_over_passes(T, [&](int M) { return output_ws_rows(d, g, d_g, M); });
}

hipError_t launch_query_project(const csa_dims& d, const csa_proj_weights& w, const void* h, int32_t T,
                                void* q, void* qI, void* wI, void* ws, hipStream_t s) {
  const int d_c = w.d_c;
  const int nq = d.n_h * d.c, nqI = d.dual ? d.n_hI * d.c_I : 0, nw = d.dual ? d.n_hI : 0;
  const size_t qI_row = d.idx_fmt == CSA_FMT_MXFP4 ? (size_t)d.n_hI * (d.c_I / 2 + d.c_I / 32)
                                                   : (size_t)d.n_hI * d.c_I;
  for (int t0 = 0; t0 < T; t0 += GM_ROWS) {
    const int M = std::min<int>(GM_ROWS, T - t0);
    const Plan p1 = plan_of(M, d_c + nw, 1, d.d, d_c);
    const Plan p2 = plan_of(M, nq + nqI, 1, d_c, nq);
    char* base = static_cast<char*>(ws);
    uint16_t* cQ = reinterpret_cast<uint16_t*>(base);
    float* P1 = reinterpret_cast<float*>(base + align256((size_t)M * d_c * 2));
    float* P2 = reinterpret_cast<float*>(base + align256((size_t)M * d_c * 2) + align256(p1.p_floats * 4));
    // eqs. 13 and 15: [c^Q | w] = h [W^DQ | W^w]
    GemmArgs g1{};
    g1.A = static_cast<const uint16_t*>(h) + (size_t)t0 * d.d;
    g1.lda = d.d;
    g1.B = static_cast<const uint16_t*>(w.w_dq);
    g1.B2 = static_cast<const uint16_t*>(w.w_w);
    g1.nb1 = d_c;
    g1.ldb = d.d;
    g1.M = M, g1.N = d_c + nw, g1.K = d.d, g1.ksplit = p1.ks, g1.kchunk = d.d / p1.ks;
    g1.n_bf = p1.n_bf, g1.D = cQ, g1.ldd = d_c;
    g1.P = P1, g1.ldp = p1.ldp, g1.p_ks = (int64_t)M * p1.ldp;
    hipError_t e = launch_gemm(g1, 1, s);
    if (e != hipSuccess) return e;
    // the partial columns: c^Q (when K was split) then w, one launch
    uint16_t* wout = nw ? static_cast<uint16_t*>(wI) + (size_t)t0 * nw : nullptr;
    if ((e = launch_sum_bf16(P1, p1.ks, g1.p_ks, M, p1.ldp, d_c - p1.n_bf, cQ, d_c, nw, wout, nw, s)) != hipSuccess)
      return e;
    // eqs. 18 and 14: [q | q^I] = c^Q [W^UQ | W^IUQ]
    GemmArgs g2{};
    g2.A = cQ;
    g2.lda = d_c;
    g2.B = static_cast<const uint16_t*>(w.w_uq);
    g2.B2 = static_cast<const uint16_t*>(w.w_iuq);
    g2.nb1 = nq;
    g2.ldb = d_c;
    g2.M = M, g2.N = nq + nqI, g2.K = d_c, g2.ksplit = p2.ks, g2.kchunk = d_c / p2.ks;
    g2.n_bf = p2.n_bf, g2.D = static_cast<uint16_t*>(q) + (size_t)t0 * nq, g2.ldd = nq;
    g2.P = P2, g2.ldp = p2.ldp, g2.p_ks = (int64_t)M * p2.ldp;
    if ((e = launch_gemm(g2, 1, s)) != hipSuccess) return e;
    // q from the partials (when K was split) and q^I in the indexer's format, one launch
    const int nsum = p2.ks > 1 ? (int)(((int64_t)M * nq + 255) / 256) : 0;
    const int nwav = nqI ? (M * d.n_hI + 3) / 4 : 0;
    if (nsum + nwav) {
      hipLaunchKernelGGL(k_finish_q, dim3(nsum + nwav), dim3(256), 0, s, P2, p2.ks, g2.p_ks, M, p2.ldp, nq,
                         static_cast<uint16_t*>(q) + (size_t)t0 * nq, nsum, P2 + (nq - p2.n_bf), d.n_hI,
                         d.idx_fmt, nqI ? static_cast<uint8_t*>(qI) + (size_t)t0 * qI_row : nullptr);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_output_project(const csa_dims& d, const csa_proj_weights& w, const void* o, int32_t T, void* out,
                                 void* ws, hipStream_t s) {
  const int g = w.g, d_g = w.d_g, G = d.n_h * d.c / g, width = d.n_h * d.c;
  for (int t0 = 0; t0 < T; t0 += GM_ROWS) {
    const int M = std::min<int>(GM_ROWS, T - t0);
    const Plan p3 = plan_of(M, d_g, g, G, d_g);
    const Plan p4 = plan_of(M, d.d, 1, g * d_g, d.d);
    char* base = static_cast<char*>(ws);
    uint16_t* mid = reinterpret_cast<uint16_t*>(base);
    float* P3 = reinterpret_cast<float*>(base + align256((size_t)M * g * d_g * 2));
    float* P4 = reinterpret_cast<float*>(base + align256((size_t)M * g * d_g * 2) + align256(p3.p_floats * 4));
    // group i: o[:, i G .. (i + 1) G] W^{O,i}, into columns i d_g .. of the concatenation
    GemmArgs g3{};
    g3.A = static_cast<const uint16_t*>(o) + (size_t)t0 * width;
    g3.lda = width;
    g3.a_zoff = G;
    g3.B = static_cast<const uint16_t*>(w.w_og);
    g3.nb1 = d_g;
    g3.ldb = G;
    g3.b_zstride = (int64_t)d_g * G;
    g3.M = M, g3.N = d_g, g3.K = G, g3.ksplit = p3.ks, g3.kchunk = G / p3.ks;
    g3.n_bf = p3.n_bf, g3.D = mid, g3.ldd = (int64_t)g * d_g, g3.d_zoff = d_g;
    g3.P = P3, g3.ldp = p3.ldp, g3.p_zoff = d_g - p3.n_bf, g3.p_ks = (int64_t)M * p3.ldp;
    hipError_t e = launch_gemm(g3, g, s);
    if (e != hipSuccess) return e;
    if (p3.ks > 1) {
      if ((e = launch_sum_bf16(P3, p3.ks, g3.p_ks, M, p3.ldp, g * d_g, mid, (int64_t)g * d_g, 0, nullptr, 0, s)) !=
          hipSuccess)
        return e;
    }
    // the concatenation to d
    GemmArgs g4{};
    g4.A = mid;
    g4.lda = (int64_t)g * d_g;
    g4.B = static_cast<const uint16_t*>(w.w_o);
    g4.nb1 = d.d;
    g4.ldb = (int64_t)g * d_g;
    g4.M = M, g4.N = d.d, g4.K = g * d_g, g4.ksplit = p4.ks, g4.kchunk = g * d_g / p4.ks;
    g4.n_bf = p4.n_bf, g4.D = static_cast<uint16_t*>(out) + (size_t)t0 * d.d, g4.ldd = d.d;
    g4.P = P4, g4.ldp = p4.ldp, g4.p_ks = (int64_t)M * p4.ldp;
    if ((e = launch_gemm(g4, 1, s)) != hipSuccess) return e;
    if (p4.ks > 1) {
      if ((e = launch_sum_bf16(P4, p4.ks, g4.p_ks, M, p4.ldp, d.d, static_cast<uint16_t*>(out) + (size_t)t0 * d.d,
                               d.d, 0, nullptr, 0, s)) != hipSuccess)
        return e;
    }
  }
  return hipSuccess;
}

}  // namespace csa
