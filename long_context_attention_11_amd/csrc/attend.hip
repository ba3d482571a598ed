// Shared-KV multi-query attention over selected compressed entries plus a sliding window of
// raw rows, with an attention sink, query RMSNorm, partial RoPE and output de-rotation.
//
// Sources: reading notes "DeepSeekV4技术报告阅读笔记" (zouxinn.github.io) eq. 19 / eq. 26
// (one KV head shared by all query heads, K = V), §2.5.1 (RMSNorm on query heads), §2.5.2
// (RoPE on the last 64 dims, output rotated back by the query position), §2.5.3 (window of
// uncompressed tokens), §2.5.4 eq. 27 (sink logit in the softmax denominator); PaperTrace
// "02 · DeepSeek-V4: 压缩注意力撑起 1M 上下文" §2.4 (window rows join the compressed entries in
// one attention).
//
// E4M3/bf16 rows: 64-row tiles are gathered into LDS as bf16 (the E4M3 -> bf16 widening is
// exact) in two layouts, row-major for Q.K and dim-major for P.V, and contracted on bf16
// MFMA with float32 accumulation.  A workgroup (4 waves, 16 heads each) covers 64 heads of
// one query, so every staged row serves 64 heads.  Decode splits a query's rows over several
// workgroups and merges their (max, sum, output) triples in a second kernel.
#include "csa_internal.h"

namespace csa {
namespace {

constexpr int AC = 512, AR = 64, ANOPE = AC - AR, AROWB = ANOPE + 2 * AR;  // 576 B rows
constexpr int ATILE = 64;
constexpr int AK_LD = AC + 8;        // bf16 pitch of the row-major tile (1040 B)
constexpr int AV_LD = ATILE + 8;     // bf16 pitch of the dim-major tile (144 B)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_BIG = -1.0e30f;

struct AttendArgs {
  const uint16_t* q;          // [Q][n_h][512] bf16
  const float* gamma_q;       // [512] or null
  const float* sink;          // [n_h] or null
  const int32_t* q_seq;
  const int32_t* q_pos;
  int Q, n_h;
  const int32_t* idx;         // [Q][k] or null (dense)
  int k;
  const uint8_t* kv;          // [B][cap][576]
  const uint8_t* win;         // [B][win_cap][576]
  const int32_t* win_pos;     // [B][win_cap]
  const int32_t* n_entries;   // [B]
  int cap, win_cap, m, n_win;
  float scale_log2;           // softmax scale * log2(e)
  float eps;
  double log2_base;
  int splits, tiles_per_split;
  uint16_t* out;              // [Q][n_h][512] bf16 (splits == 1)
  float* part_o;              // [Q][n_h][splits][512] (splits > 1)
  float* part_ml;             // [Q][n_h][splits][2]
};

// Row source of row r of a query's key list: entries first (idx order, or 0..V-1 when
// dense), then window positions w0 .. tau.  Returns a byte offset, or -1 if masked.
__device__ __forceinline__ int64_t row_offset(const AttendArgs& a, int q, int seq, int V,
                                              int nsel, int w0, int r) {
  if (r < nsel) {
    int s = a.idx ? a.idx[(size_t)q * a.k + r] : r;
    if (s < 0 || s >= V) return -1;
    return ((int64_t)seq * a.cap + s) * AROWB;
  }
  const int j = w0 + (r - nsel);
  const int slot = j % a.win_cap;
  if (a.win_pos[(size_t)seq * a.win_cap + slot] != j) return -1;
  return ((int64_t)seq * a.win_cap + slot) * AROWB | ((int64_t)1 << 62);  // tag: window ring
}

// Swizzled position of (dim d, row r) in the dim-major tile: 16-byte chunks of a dim's row
// are XOR-permuted by (d >> 3) & 7 so that writers stepping over dims spread across banks.
__device__ __forceinline__ int vt_index(int d, int r) {
  const int chunk = (r >> 3) ^ ((d >> 3) & 7);
  return d * AV_LD + chunk * 8 + (r & 7);
}

// Sum of squares of 8 bf16 values packed in a uint4.
__device__ __forceinline__ float sumsq_bf16x8(const uint4& v) {
  float s = 0.f;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = bf16_bits_to_f32(w[e] & 0xffffu), hi = bf16_bits_to_f32(w[e] >> 16);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}

// Normalise 8 query dims (dim0 .. dim0+7), rotate them to tau when they are RoPE dims, and
// pack them as a bf16 MFMA operand.
__device__ __forceinline__ bf16x8 prep_q8(const uint4& v, float inv, const float* gamma,
                                          int dim0, bool rope, int64_t tau, double log2_base) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int dim = dim0 + 2 * e;
    float y0 = bf16_bits_to_f32(w[e] & 0xffffu) * inv;
    float y1 = bf16_bits_to_f32(w[e] >> 16) * inv;
    if (gamma) {
      y0 *= gamma[dim];
      y1 *= gamma[dim + 1];
    }
    if (rope) {
      float cs, sn;
      rope_cos_sin(tau, (dim - ANOPE) >> 1, AR, log2_base, cs, sn);
      const float z0 = y0 * cs - y1 * sn, z1 = y0 * sn + y1 * cs;
      y0 = z0;
      y1 = z1;
    }
    o[e] = f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16);
  }
  return __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

// Scale 4 output dims (d0 .. d0+3) of one head by 1/L, rotate RoPE dims back by -tau, and
// store them as bf16.
__device__ __forceinline__ void store_out4(const f32x4& o, float invL, uint16_t* orow, int d0,
                                           bool rope, int64_t tau, double log2_base) {
  float y[4] = {o[0] * invL, o[1] * invL, o[2] * invL, o[3] * invL};
  if (rope) {
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      float cs, sn;
      rope_cos_sin(tau, (d0 + e - ANOPE) >> 1, AR, log2_base, cs, sn);
      const float z0 = y[e] * cs + y[e + 1] * sn;  // rotate by -tau
      const float z1 = -y[e] * sn + y[e + 1] * cs;
      y[e] = z0;
      y[e + 1] = z1;
    }
  }
  uint2 pk;
  pk.x = f32_to_bf16_bits(y[0]) | (f32_to_bf16_bits(y[1]) << 16);
  pk.y = f32_to_bf16_bits(y[2]) | (f32_to_bf16_bits(y[3]) << 16);
  *reinterpret_cast<uint2*>(orow + d0) = pk;
}

__global__ __launch_bounds__(256) void k_attend_mfma(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[ATILE * AK_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[AC * AV_LD];
  __shared__ int64_t rowoff[ATILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int nhg = (a.n_h + 63) / 64;
  const uint32_t L = xcd_logical_id(blockIdx.x, gridDim.x);
  const int split = L % a.splits;
  const int rest = L / a.splits;
  const int hg = rest % nhg;
  const int q = rest / nhg;
  const int seq = a.q_seq[q];
  const int tau = a.q_pos[q];
  const int V = max(0, min(tau / a.m, a.n_entries[seq]));
  const int nsel = a.idx ? a.k : V;
  const int w0 = max(0, tau - a.n_win + 1);
  const int nrows = nsel + (tau - w0 + 1);
  const int r_lo = split * a.tiles_per_split * ATILE;
  const int r_hi = min(nrows, r_lo + a.tiles_per_split * ATILE);
  const int h = hg * 64 + wave * 16 + col;   // this lane's head
  const bool head_ok = (hg * 64 + wave * 16) < a.n_h;
  const int hh = min(h, a.n_h - 1);

  // ---- query prep: RMSNorm over 512 dims, RoPE at tau on dims 448..511, round to bf16.
  // B operand of step ks (dims ks*32 .. +31): lane holds dims ks*32 + g*8 .. +7 of head h.
  bf16x8 Qop[16];
  {
    const uint16_t* qrow = a.q + ((size_t)q * a.n_h + hh) * AC;
    uint4 raw[16];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      raw[ks] = *reinterpret_cast<const uint4*>(qrow + ks * 32 + g * 8);
      ss += sumsq_bf16x8(raw[ks]);
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = 1.0f / sqrtf(ss / (float)AC + a.eps);
#pragma unroll
    for (int ks = 0; ks < ANOPE / 32; ++ks)
      Qop[ks] = prep_q8(raw[ks], inv, a.gamma_q, ks * 32 + g * 8, false, tau, a.log2_base);
    Qop[14] = prep_q8(raw[14], inv, a.gamma_q, 14 * 32 + g * 8, true, tau, a.log2_base);
    Qop[15] = prep_q8(raw[15], inv, a.gamma_q, 15 * 32 + g * 8, true, tau, a.log2_base);
  }

  const float sink2 = (a.sink && head_ok) ? a.sink[hh] * LOG2E : NEG_BIG;
  float m_run = a.sink ? sink2 : NEG_BIG;
  float l_run = 0.f;
  f32x4 O[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) O[i] = f32x4{0, 0, 0, 0};

  // staging map: thread covers dim-group dg (8 dims) of rows rsub*16 .. rsub*16+15
  const int dg = tid >> 2, rsub = tid & 3;

  for (int t0 = r_lo; t0 < r_hi; t0 += ATILE) {
    if (tid < ATILE) {
      const int r = t0 + tid;
      rowoff[tid] = r < r_hi ? row_offset(a, q, seq, V, nsel, w0, r) : (int64_t)-1;
    }
    __syncthreads();
    // ---- gather 64 rows x 512 dims into Ks (row-major) and Vt (dim-major), as bf16.
    // Thread: dim-group dg (8 dims) of rows rsub*16 .. +15, in batches of 4 rows.
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      uint32_t colv[4][4];  // 4 rows x 8 bf16
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = rsub * 16 + rb * 4 + rr;
        const int64_t off = rowoff[row];
        uint4 v = make_uint4(0, 0, 0, 0);
        if (off >= 0) {
          const uint8_t* base = ((off >> 62) & 1) ? a.win : a.kv;
          const uint8_t* src = base + (off & (((int64_t)1 << 62) - 1));
          if (dg < ANOPE / 8) {
            uint2 raw = *reinterpret_cast<const uint2*>(src + dg * 8);
            e4m3x4_to_bf16x4(raw.x, v.x, v.y);
            e4m3x4_to_bf16x4(raw.y, v.z, v.w);
          } else {
            v = *reinterpret_cast<const uint4*>(src + ANOPE + (dg - ANOPE / 8) * 16);
          }
        }
        *reinterpret_cast<uint4*>(&Ks[row * AK_LD + dg * 8]) = v;
        colv[rr][0] = v.x;
        colv[rr][1] = v.y;
        colv[rr][2] = v.z;
        colv[rr][3] = v.w;
      }
      // transpose: each of the 8 dims gets 4 consecutive rows (8 bytes)
      const int r0 = rsub * 16 + rb * 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        const uint32_t r01 = ((colv[0][e >> 1] >> sh) & 0xffffu) | (((colv[1][e >> 1] >> sh) & 0xffffu) << 16);
        const uint32_t r23 = ((colv[2][e >> 1] >> sh) & 0xffffu) | (((colv[3][e >> 1] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<uint2*>(&Vt[vt_index(dg * 8 + e, r0)]) = make_uint2(r01, r23);
      }
    }
    __syncthreads();

    if (head_ok) {
      // ---- S^T = K . Q^T for 4 row tiles: lane holds head col, rows 16*rt + 4g + e
      f32x4 S[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        S[rt] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          bf16x8 A = *reinterpret_cast<const bf16x8*>(&Ks[(rt * 16 + col) * AK_LD + ks * 32 + g * 8]);
          S[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Qop[ks], S[rt], 0, 0, 0);
        }
      }
      // ---- online softmax (log2 domain), sink already in m_run
      float mx = NEG_BIG;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rt * 16 + 4 * g + e;
          const bool ok = rowoff[row] >= 0;
          S[rt][e] = ok ? S[rt][e] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, S[rt][e]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      float ls = 0.f;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          S[rt][e] = exp2f(S[rt][e] - m_new);
          ls += S[rt][e];
        }
      ls += __shfl_xor(ls, 16, 64);
      ls += __shfl_xor(ls, 32, 64);
      l_run = l_run * alpha + ls;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < 32; ++i) O[i] *= alpha;
      // ---- O^T += V^T . P^T over 64 rows (2 K steps of 32).  K step kk pairs lane group g's
      // rows {32kk + 4g + e} and {32kk + 16 + 4g + e} (e < 4) on both operands.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint4 pb;
        pb.x = f32_to_bf16_bits(S[2 * kk][0]) | (f32_to_bf16_bits(S[2 * kk][1]) << 16);
        pb.y = f32_to_bf16_bits(S[2 * kk][2]) | (f32_to_bf16_bits(S[2 * kk][3]) << 16);
        pb.z = f32_to_bf16_bits(S[2 * kk + 1][0]) | (f32_to_bf16_bits(S[2 * kk + 1][1]) << 16);
        pb.w = f32_to_bf16_bits(S[2 * kk + 1][2]) | (f32_to_bf16_bits(S[2 * kk + 1][3]) << 16);
        const bf16x8 Bp = __builtin_bit_cast(bf16x8, pb);
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) {
          const int d = dt * 16 + col;
          const uint2 lo = *reinterpret_cast<const uint2*>(&Vt[vt_index(d, kk * 32 + 4 * g)]);
          const uint2 hi = *reinterpret_cast<const uint2*>(&Vt[vt_index(d, kk * 32 + 16 + 4 * g)]);
          const bf16x8 Av = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
          O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Av, Bp, O[dt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  if (!head_ok) return;
  // O[dt][e] holds head col, dim dt*16 + 4g + e.
  if (a.splits == 1) {
    float Lsum = l_run + (a.sink ? exp2f(sink2 - m_run) : 0.f);
    const float invL = Lsum > 0.f ? 1.0f / Lsum : 0.f;
    uint16_t* orow = a.out + ((size_t)q * a.n_h + h) * AC;
#pragma unroll
    for (int dt = 0; dt < ANOPE / 16; ++dt) store_out4(O[dt], invL, orow, dt * 16 + 4 * g, false, tau, a.log2_base);
#pragma unroll
    for (int dt = ANOPE / 16; dt < 32; ++dt) store_out4(O[dt], invL, orow, dt * 16 + 4 * g, true, tau, a.log2_base);
  } else {
    const size_t pidx = ((size_t)q * a.n_h + h) * a.splits + split;
    float* po = a.part_o + pidx * AC;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      *reinterpret_cast<float4*>(po + dt * 16 + 4 * g) = make_float4(O[dt][0], O[dt][1], O[dt][2], O[dt][3]);
    if (g == 0) {
      a.part_ml[pidx * 2] = m_run;
      a.part_ml[pidx * 2 + 1] = l_run;
    }
  }
}

// Merge split partials: one workgroup of 256 threads per (query, head), 2 dims per thread.
__global__ __launch_bounds__(256) void k_attend_combine(AttendArgs a) {
  const int qh = blockIdx.x;
  const int q = qh / a.n_h, h = qh % a.n_h;
  const int tau = a.q_pos[q];
  const float* ml = a.part_ml + (size_t)qh * a.splits * 2;
  const float sink2 = a.sink ? a.sink[h] * LOG2E : NEG_BIG;
  float M = a.sink ? sink2 : NEG_BIG;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, ml[2 * s]);
  float Lsum = a.sink ? exp2f(sink2 - M) : 0.f;
  for (int s = 0; s < a.splits; ++s) Lsum += ml[2 * s + 1] * exp2f(ml[2 * s] - M);
  const float invL = Lsum > 0.f ? 1.0f / Lsum : 0.f;
  const int d = 2 * threadIdx.x;
  float y0 = 0.f, y1 = 0.f;
  const float* po = a.part_o + (size_t)qh * a.splits * AC;
  for (int s = 0; s < a.splits; ++s) {
    const float f = exp2f(ml[2 * s] - M);
    y0 = fmaf(po[(size_t)s * AC + d], f, y0);
    y1 = fmaf(po[(size_t)s * AC + d + 1], f, y1);
  }
  y0 *= invL;
  y1 *= invL;
  if (d >= ANOPE) {
    float cs, sn;
    rope_cos_sin(tau, (d - ANOPE) >> 1, AR, a.log2_base, cs, sn);
    const float z0 = y0 * cs + y1 * sn, z1 = -y0 * sn + y1 * cs;
    y0 = z0;
    y1 = z1;
  }
  *reinterpret_cast<uint32_t*>(a.out + (size_t)qh * AC + d) =
      f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16);
}

// float32 rows (fp32 formats): one workgroup of 64 threads per (query, head); exact
// two-pass softmax over the key list held in LDS.
constexpr int AF_MAXK = 4096;

__global__ __launch_bounds__(64) void k_attend_f32(const float* __restrict__ qv,
                                                   const float* __restrict__ gamma_q,
                                                   const float* __restrict__ sink,
                                                   const int32_t* __restrict__ q_seq,
                                                   const int32_t* __restrict__ q_pos, int n_h,
                                                   const int32_t* __restrict__ idx, int k,
                                                   const float* __restrict__ kv,
                                                   const float* __restrict__ win,
                                                   const int32_t* __restrict__ win_pos,
                                                   const int32_t* __restrict__ n_entries,
                                                   int cap, int win_cap, int m, int n_win, int c,
                                                   int r, float scale, float eps, double log2_base,
                                                   float* __restrict__ out) {
  __shared__ float qs[1024];
  __shared__ float z[AF_MAXK];
  __shared__ const float* rows[AF_MAXK];
  const int qh = blockIdx.x;
  const int q = qh / n_h, h = qh % n_h, t = threadIdx.x;
  const int seq = q_seq[q], tau = q_pos[q];
  const int V = max(0, min(tau / m, n_entries[seq]));
  const int nsel = idx ? k : V;
  const int w0 = max(0, tau - n_win + 1);
  const int nrows = nsel + (tau - w0 + 1);
  // query prep
  const float* qrow = qv + ((size_t)q * n_h + h) * c;
  float ss = 0.f;
  for (int u = t; u < c; u += 64) { float x = qrow[u]; qs[u] = x; ss = fmaf(x, x, ss); }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)c + eps);
  __syncthreads();
  for (int u = 2 * t; u < c; u += 128) {
    float y0 = (gamma_q ? gamma_q[u] : 1.f) * (qs[u] * inv);
    float y1 = (gamma_q ? gamma_q[u + 1] : 1.f) * (qs[u + 1] * inv);
    if (u >= c - r) {
      float cs, sn;
      rope_cos_sin(tau, (u - (c - r)) >> 1, r, log2_base, cs, sn);
      const float z0 = y0 * cs - y1 * sn, z1 = y0 * sn + y1 * cs;
      y0 = z0;
      y1 = z1;
    }
    qs[u] = y0;
    qs[u + 1] = y1;
  }
  __syncthreads();
  // key list and logits
  for (int j = t; j < nrows; j += 64) {
    const float* p = nullptr;
    if (j < nsel) {
      int s = idx ? idx[(size_t)q * k + j] : j;
      if (s >= 0 && s < V) p = kv + ((size_t)seq * cap + s) * c;
    } else {
      const int pos = w0 + (j - nsel);
      const int slot = pos % win_cap;
      if (win_pos[(size_t)seq * win_cap + slot] == pos) p = win + ((size_t)seq * win_cap + slot) * c;
    }
    rows[j] = p;
    float acc = -INFINITY;
    if (p) {
      acc = 0.f;
      for (int u = 0; u < c; ++u) acc = fmaf(qs[u], p[u], acc);
      acc *= scale;
    }
    z[j] = acc;
  }
  __syncthreads();
  float mx = sink ? sink[h] : -INFINITY;
  for (int j = t; j < nrows; j += 64) mx = fmaxf(mx, z[j]);
  mx = wave_max(mx);
  float den = 0.f;
  for (int j = t; j < nrows; j += 64) den += rows[j] ? expf(z[j] - mx) : 0.f;
  den = wave_sum(den);
  if (sink) den += expf(sink[h] - mx);
  __syncthreads();
  for (int j = t; j < nrows; j += 64) z[j] = rows[j] ? expf(z[j] - mx) / den : 0.f;
  __syncthreads();
  float* orow = out + ((size_t)q * n_h + h) * c;
  for (int u = 2 * t; u < c; u += 128) {
    float y0 = 0.f, y1 = 0.f;
    for (int j = 0; j < nrows; ++j) {
      const float* p = rows[j];
      if (!p) continue;
      y0 = fmaf(z[j], p[u], y0);
      y1 = fmaf(z[j], p[u + 1], y1);
    }
    if (u >= c - r) {
      float cs, sn;
      rope_cos_sin(tau, (u - (c - r)) >> 1, r, log2_base, cs, sn);
      const float z0 = y0 * cs + y1 * sn, z1 = -y0 * sn + y1 * cs;
      y0 = z0;
      y1 = z1;
    }
    orow[u] = y0;
    orow[u + 1] = y1;
  }
}

struct SplitPlan {
  int splits, tiles_per_split;
};

SplitPlan plan_splits(const csa_dims& d, int32_t Q, int32_t cap, bool dense) {
  const int max_rows = (dense ? cap : d.top_k) + d.n_win;
  const int ntiles = (max_rows + ATILE - 1) / ATILE;
  const int blocks = Q * ((d.n_h + 63) / 64);
  int target = (512 + blocks - 1) / blocks;
  target = std::max(1, std::min(target, ntiles));
  const int tps = (ntiles + target - 1) / target;
  return {(ntiles + tps - 1) / tps, tps};
}

}  // namespace

size_t attend_workspace_bytes(const csa_dims& d, int32_t Q, int32_t cap) {
  if (d.kv_fmt == CSA_FMT_F32) return 0;
  // a CSA layer may also be attended densely (idx = NULL): size for the larger plan
  const SplitPlan dense = plan_splits(d, Q, cap, true);
  const SplitPlan sparse = d.top_k > 0 ? plan_splits(d, Q, cap, false) : dense;
  const int splits = std::max(dense.splits, sparse.splits);
  if (splits == 1) return 0;
  return (size_t)Q * d.n_h * splits * (AC + 2) * sizeof(float);
}

hipError_t launch_attend(const csa_dims& d, const csa_cache& c, const void* q,
                         const float* gamma_q, const float* sink, const int32_t* q_seq,
                         const int32_t* q_pos, int32_t Q, const int32_t* idx, void* out,
                         void* ws, hipStream_t s) {
  const float scale = d.scale > 0.f ? d.scale : 1.0f / sqrtf((float)d.c);
  if (d.kv_fmt == CSA_FMT_F32) {
    hipLaunchKernelGGL(k_attend_f32, dim3(Q * d.n_h), dim3(64), 0, s, (const float*)q, gamma_q,
                       sink, q_seq, q_pos, d.n_h, idx, d.top_k, (const float*)c.kv,
                       (const float*)c.win, c.win_pos, c.n_entries, c.cap, c.win_cap, d.m,
                       d.n_win, d.c, d.rope_dim, scale, d.rms_eps, std::log2((double)d.rope_base),
                       (float*)out);
    return hipGetLastError();
  }
  AttendArgs a;
  a.q = (const uint16_t*)q;
  a.gamma_q = gamma_q;
  a.sink = sink;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.Q = Q;
  a.n_h = d.n_h;
  a.idx = idx;
  a.k = d.top_k;
  a.kv = (const uint8_t*)c.kv;
  a.win = (const uint8_t*)c.win;
  a.win_pos = c.win_pos;
  a.n_entries = c.n_entries;
  a.cap = c.cap;
  a.win_cap = c.win_cap;
  a.m = d.m;
  a.n_win = d.n_win;
  a.scale_log2 = scale * LOG2E;
  a.eps = d.rms_eps;
  a.log2_base = std::log2((double)d.rope_base);
  SplitPlan p = plan_splits(d, Q, c.cap, idx == nullptr);
  a.splits = p.splits;
  a.tiles_per_split = p.tiles_per_split;
  a.out = (uint16_t*)out;
  a.part_o = (float*)ws;
  a.part_ml = p.splits > 1 ? (float*)ws + (size_t)Q * d.n_h * p.splits * AC : nullptr;
  const int nhg = (d.n_h + 63) / 64;
  hipLaunchKernelGGL(k_attend_mfma, dim3(Q * nhg * p.splits), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(k_attend_combine, dim3(Q * d.n_h), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
