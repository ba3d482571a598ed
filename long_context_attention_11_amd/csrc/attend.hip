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
// E4M3/bf16 rows: 32-row tiles are gathered into LDS as bf16 (the E4M3 -> bf16 widening is
// exact) in two layouts, row-major for Q.K and dim-major for P.V, and contracted on bf16
// MFMA with float32 accumulation.  A workgroup (8 waves) covers 64 heads of one query, so
// every staged row serves 64 heads.  Decode splits a query's rows over several workgroups
// and merges their (max, sum, output) triples in a second kernel.
#include <type_traits>

#include "csa_internal.h"

namespace csa {
namespace {

constexpr int AC = 512, AR = 64, ANOPE = AC - AR, AROWB = ANOPE + 2 * AR;  // 576 B rows
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
  uint16_t* part_o;           // [Q][n_h][splits][512] bf16 (splits > 1)
  float* part_ml;             // [Q][n_h][splits][2]
};

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

// Normalise 8 query dims (dim0 .. dim0+7) with weights gamma (a table of 512), rotate them to
// tau when they are RoPE dims (cos/sin of pair j at cs[2j], cs[2j+1]), and return them as
// packed bf16.
__device__ __forceinline__ uint4 prep_q8(const uint4& v, float inv, const float* gamma, int dim0,
                                         const float* cs) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const float4 g0 = *reinterpret_cast<const float4*>(gamma + dim0);
  const float4 g1 = *reinterpret_cast<const float4*>(gamma + dim0 + 4);
  const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  const bool rope = dim0 >= ANOPE;
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float y0 = bf16_bits_to_f32(w[e] & 0xffffu) * inv * gm[2 * e];
    float y1 = bf16_bits_to_f32(w[e] >> 16) * inv * gm[2 * e + 1];
    if (rope) {
      const int j = (dim0 + 2 * e - ANOPE) >> 1;
      const float c = cs[2 * j], sn = cs[2 * j + 1];
      const float z0 = y0 * c - y1 * sn, z1 = y0 * sn + y1 * c;
      y0 = z0;
      y1 = z1;
    }
    o[e] = pack_bf16x2(y0, y1);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Scale 4 output dims (d0 .. d0+3) of one head by 1/L, rotate RoPE dims back by -tau (table
// cs as above), and store them as bf16.
__device__ __forceinline__ void store_out4(const f32x4& o, float invL, uint16_t* orow, int d0,
                                           const float* cs) {
  float y[4] = {o[0] * invL, o[1] * invL, o[2] * invL, o[3] * invL};
  if (d0 >= ANOPE) {
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const int j = (d0 + e - ANOPE) >> 1;
      const float c = cs[2 * j], sn = cs[2 * j + 1];
      const float z0 = y[e] * c + y[e + 1] * sn;  // rotate by -tau
      const float z1 = -y[e] * sn + y[e + 1] * c;
      y[e] = z0;
      y[e + 1] = z1;
    }
  }
  *reinterpret_cast<uint2*>(orow + d0) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
}

// One workgroup = 8 waves = 64 heads of one query over a range of 32-row tiles.
// Wave w: heads 16*(w & 3) .. +15 (hq), dims 256*(w >> 2) .. +255 (half).  Q.K is split over
// the pair's halves of the contraction and summed through LDS in a fixed order, so both
// waves of a pair hold identical scores, maxima and sums; each then accumulates P.V for its
// own 256 output dims.  The next tile's rows are loaded into registers while the current one
// computes.
constexpr int T2 = 32;               // rows per tile
constexpr int AT_MAX_ROWS = 4096;    // rows one workgroup covers (their indices sit in LDS)
constexpr int K2_LD = AC + 8;        // bf16 pitch of the row-major tile (1040 B)
constexpr int V2_LD = T2 + 8;        // bf16 pitch of the dim-major tile (80 B)

// (dim d, row r) in the dim-major tile: the four 16-byte chunks of a dim's row are XOR-permuted
// by (d >> 3) & 3, so writers stepping over dim groups spread over the banks.
__device__ __forceinline__ int vt2_index(int d, int r) {
  return d * V2_LD + (((r >> 3) ^ ((d >> 3) & 3)) << 3) + (r & 7);
}

__global__ __launch_bounds__(512) void k_attend_mfma(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[T2 * K2_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[AC * V2_LD];
  __shared__ __attribute__((aligned(16))) f32x4 Sx[8][2][64];   // partial S per wave
  __shared__ __attribute__((aligned(16))) float gam[AC];
  __shared__ int rowok[2][T2];
  __shared__ int ridx[AT_MAX_ROWS];   // entry index of each of this workgroup's entry rows
  __shared__ float rope_cs[AR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int hq = wave & 3, half = wave >> 2;
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
  const int r_lo = split * a.tiles_per_split * T2;
  const int r_hi = min(nrows, r_lo + a.tiles_per_split * T2);
  const int h = hg * 64 + hq * 16 + col;   // this lane's head
  const bool head_ok = (hg * 64 + hq * 16) < a.n_h;
  const int hh = min(h, a.n_h - 1);
  const int dbase = half * 256;            // this wave's output dims

  // ---- loads are issued in the order they are needed (the wait counter retires them in
  // order): this workgroup's entry indices (to LDS, so that no gather waits on an index
  // load), the query norm weights, then the query rows.
  const int e_hi = min(r_hi, nsel);
  // A wave loads the indices of exactly the rows it gathers (rows 4*wave .. 4*wave+3 of each
  // tile): lane l of batch i takes tile (64i + l) / 4, row (64i + l) % 4.  The wave reads
  // them back itself, so no barrier is needed before the first gathers.
  constexpr int IPT = AT_MAX_ROWS / 512;   // index loads per thread
  int rid[IPT];
  auto rid_row = [&](int i) { const int f = 64 * i + lane; return r_lo + (f >> 2) * T2 + wave * 4 + (f & 3); };
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int r = rid_row(i);
    rid[i] = a.idx ? a.idx[(size_t)q * a.k + min(r, a.k - 1)] : r;
  }
  float4 gq = make_float4(1.f, 1.f, 1.f, 1.f);
  const int gu = (tid & 127) * 4;
  if (a.gamma_q) gq = *reinterpret_cast<const float4*>(a.gamma_q + gu);
  // every lane holds all 512 dims of its head in 16 chunks (needed for the norm); this wave
  // keeps its 8 for the operands
  const uint16_t* qrow = a.q + ((size_t)q * a.n_h + hh) * AC;
  uint4 raw[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) raw[ks] = *reinterpret_cast<const uint4*>(qrow + ks * 32 + g * 8);

#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int r = rid_row(i);
    if (r < e_hi) ridx[r - r_lo] = rid[i];
  }

  // ---- staging map: thread covers dim-group dg (8 dims) of rows 4*rq .. 4*rq+3 of a tile
  // (rq = wave, so a wave's row references are uniform across its lanes)
  const int dg = tid & 63, rq = tid >> 6;
  const bool nope_group = dg < ANOPE / 8;
  // byte offset of this group's 16-byte load: 8 E4M3 dims (the next 8 bytes are unused), or
  // 8 bf16 RoPE dims
  const int col_off = nope_group ? dg * 8 : ANOPE + (dg - ANOPE / 8) * 16;
  // Row r of the key list: entries first (idx order, or 0..V-1 when dense), then window
  // positions w0 .. tau.  Two tiles of rows are in flight ahead of the one being computed.
  // Every row issues its loads unconditionally (masked rows read entry row 0 of the cache)
  // so that the compiler's wait counts stay exact; a window row is valid only if its ring
  // slot still holds its position, read alongside it.
  uint4 pre[2][4];
  int wpos[2][4], want[2][4];
  bool rok[2][4], rwin[2][4];
  const uint8_t* kvseq = a.kv + (size_t)seq * a.cap * AROWB;
  const uint8_t* winseq = a.win + (size_t)seq * a.win_cap * AROWB;
  const int32_t* wpseq = a.win_pos + (size_t)seq * a.win_cap;
  auto gather = [&](int t0, auto bconst) {
    constexpr int b = decltype(bconst)::value;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = t0 + rq * 4 + rr;
      const bool in = r < r_hi, ent = r < nsel;
      const int s = ridx[min(max(r - r_lo, 0), AT_MAX_ROWS - 1)];
      const bool ok_e = in && ent && s >= 0 && s < V;
      const int j = w0 + (r - nsel);
      const int slot = (ent ? 0 : j) % a.win_cap;
      const uint8_t* src = ent ? kvseq + (size_t)(ok_e ? s : 0) * AROWB
                               : (in ? winseq + (size_t)slot * AROWB : kvseq);
      pre[b][rr] = *reinterpret_cast<const uint4*>(src + col_off);
      wpos[b][rr] = wpseq[slot];
      want[b][rr] = j;
      rwin[b][rr] = !ent;
      rok[b][rr] = ent ? ok_e : in;
    }
  };
  gather(r_lo, std::integral_constant<int, 0>{});
  gather(r_lo + T2, std::integral_constant<int, 1>{});

  if (tid < AR / 2) rope_cos_sin(tau, tid, AR, a.log2_base, rope_cs[2 * tid], rope_cs[2 * tid + 1]);
  if (tid < 128) *reinterpret_cast<float4*>(&gam[gu]) = gq;
  lds_barrier();

  // ---- query prep: RMSNorm over 512 dims, RoPE at tau on dims 448..511, bf16.  B operand of
  // step ks (dims dbase + ks*32 .. +31): lane holds dims dbase + ks*32 + g*8 .. +7 of head h.
  bf16x8 Qop[8];
  {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) ss += sumsq_bf16x8(raw[ks]);
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = 1.0f / sqrtf(ss / (float)AC + a.eps);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int dim0 = dbase + ks * 32 + g * 8;
      const uint4 pk = prep_q8(half ? raw[8 + ks] : raw[ks], inv, gam, dim0, rope_cs);
      Qop[ks] = __builtin_bit_cast(bf16x8, pk);
    }
  }

  const float sink2 = (a.sink && head_ok) ? a.sink[hh] * LOG2E : NEG_BIG;
  float m_run = a.sink ? sink2 : NEG_BIG;
  float l_run = 0.f;
  f32x4 O[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) O[i] = f32x4{0, 0, 0, 0};

  // One tile; b (the register/LDS buffer of its rows) is a compile-time constant so that
  // the row buffers stay in registers.
  auto tile = [&](int t0, auto bconst) {
    constexpr int b = decltype(bconst)::value;
      // ---- convert the prefetched rows; write Ks (row-major) and Vt (dim-major)
      uint4 v[4];
  #pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const bool ok = rok[b][rr] && (!rwin[b][rr] || wpos[b][rr] == want[b][rr]);
        uint32_t x0, x1, x2, x3;
        e4m3x4_to_bf16x4(pre[b][rr].x, x0, x1);
        e4m3x4_to_bf16x4(pre[b][rr].y, x2, x3);
        uint4 o = nope_group ? make_uint4(x0, x1, x2, x3) : pre[b][rr];
        if (!ok) o = make_uint4(0u, 0u, 0u, 0u);
        v[rr] = o;
        *reinterpret_cast<uint4*>(&Ks[(rq * 4 + rr) * K2_LD + dg * 8]) = o;
        if (dg == 0) rowok[b][rq * 4 + rr] = ok ? 1 : 0;
      }
  #pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a0 = reinterpret_cast<const uint32_t*>(&v[0])[w];
        const uint32_t a1 = reinterpret_cast<const uint32_t*>(&v[1])[w];
        const uint32_t a2 = reinterpret_cast<const uint32_t*>(&v[2])[w];
        const uint32_t a3 = reinterpret_cast<const uint32_t*>(&v[3])[w];
        const uint2 lo = make_uint2(__builtin_amdgcn_perm(a1, a0, 0x05040100u), __builtin_amdgcn_perm(a3, a2, 0x05040100u));
        const uint2 hi = make_uint2(__builtin_amdgcn_perm(a1, a0, 0x07060302u), __builtin_amdgcn_perm(a3, a2, 0x07060302u));
        *reinterpret_cast<uint2*>(&Vt[vt2_index(dg * 8 + 2 * w, rq * 4)]) = lo;
        *reinterpret_cast<uint2*>(&Vt[vt2_index(dg * 8 + 2 * w + 1, rq * 4)]) = hi;
      }
      lds_barrier();
      // the tile after next, into the row buffers just consumed
      gather(t0 + 2 * T2, bconst);

      // ---- partial S^T = K . Q^T over this wave's 256 dims, 2 row tiles
      f32x4 S[2];
  #pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        S[rt] = f32x4{0, 0, 0, 0};
  #pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 A = *reinterpret_cast<const bf16x8*>(&Ks[(rt * 16 + col) * K2_LD + dbase + ks * 32 + g * 8]);
          S[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Qop[ks], S[rt], 0, 0, 0);
        }
        Sx[wave][rt][lane] = S[rt];
      }
      lds_barrier();
      // full scores: half 0 + half 1, the same order in both waves of the pair
  #pragma unroll
      for (int rt = 0; rt < 2; ++rt) S[rt] = Sx[hq][rt][lane] + Sx[hq + 4][rt][lane];

      // ---- online softmax (log2 domain), sink already in m_run; lane holds head col, rows
      // 16*rt + 4g + e
      float mx = NEG_BIG;
  #pragma unroll
      for (int rt = 0; rt < 2; ++rt)
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = rowok[b][rt * 16 + 4 * g + e] != 0;
          S[rt][e] = ok ? S[rt][e] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, S[rt][e]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      float ls = 0.f;
  #pragma unroll
      for (int rt = 0; rt < 2; ++rt)
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          S[rt][e] = exp2f(S[rt][e] - m_new);
          ls += S[rt][e];
        }
      ls += __shfl_xor(ls, 16, 64);
      ls += __shfl_xor(ls, 32, 64);
      l_run = l_run * alpha + ls;
      m_run = m_new;
      if (t0 != r_lo && __any(alpha != 1.0f)) {  // O is zero on the first tile; skip when no max moved
  #pragma unroll
        for (int i = 0; i < 16; ++i) O[i] *= alpha;
      }
      // ---- O^T += V^T . P^T over the 32 rows (one K step): lane group g pairs rows
      // {4g + e} and {16 + 4g + e} (e < 4) on both operands
      uint4 pb;
      pb.x = pack_bf16x2(S[0][0], S[0][1]);
      pb.y = pack_bf16x2(S[0][2], S[0][3]);
      pb.z = pack_bf16x2(S[1][0], S[1][1]);
      pb.w = pack_bf16x2(S[1][2], S[1][3]);
      const bf16x8 Bp = __builtin_bit_cast(bf16x8, pb);
  #pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        const int d = dbase + dt * 16 + col;
        const uint2 lo = *reinterpret_cast<const uint2*>(&Vt[vt2_index(d, 4 * g)]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&Vt[vt2_index(d, 16 + 4 * g)]);
        const bf16x8 Av = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Av, Bp, O[dt], 0, 0, 0);
      }
    lds_barrier();
  };
  // tiles go in pairs (a pair's second tile may be past the end: fully masked, it changes
  // nothing)
  for (int t0 = r_lo; t0 < r_hi; t0 += 2 * T2) {
    tile(t0, std::integral_constant<int, 0>{});
    tile(t0 + T2, std::integral_constant<int, 1>{});
  }

  if (!head_ok) return;
  // O[dt][e] holds head col, dim dbase + dt*16 + 4g + e.
  if (a.splits == 1) {
    const float Lsum = l_run + (a.sink ? exp2f(sink2 - m_run) : 0.f);
    const float invL = Lsum > 0.f ? 1.0f / Lsum : 0.f;
    uint16_t* orow = a.out + ((size_t)q * a.n_h + h) * AC;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) store_out4(O[dt], invL, orow, dbase + dt * 16 + 4 * g, rope_cs);
  } else {
    const size_t pidx = ((size_t)q * a.n_h + h) * a.splits + split;
    // unnormalised partial output, rounded to bf16 (the final output is bf16 as well)
    uint16_t* po = a.part_o + pidx * AC;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
      *reinterpret_cast<uint2*>(po + dbase + dt * 16 + 4 * g) =
          make_uint2(pack_bf16x2(O[dt][0], O[dt][1]), pack_bf16x2(O[dt][2], O[dt][3]));
    if (g == 0 && half == 0) {
      a.part_ml[pidx * 2] = m_run;
      a.part_ml[pidx * 2 + 1] = l_run;
    }
  }
}

// Merge split partials: one workgroup of 256 threads per (query, head), 2 dims per thread.
// Splits are taken 8 at a time (all loads of a chunk in flight), merged with a running max.
constexpr int COMB_MAX = 128;  // most splits a plan uses

__global__ __launch_bounds__(256) void k_attend_combine(AttendArgs a) {
  const int qh = blockIdx.x;
  const int q = qh / a.n_h, h = qh % a.n_h;
  const int tau = a.q_pos[q];
  const int d = 2 * threadIdx.x;
  const float* ml = a.part_ml + (size_t)qh * a.splits * 2;
  const uint16_t* po = a.part_o + (size_t)qh * a.splits * AC + d;
  const float sink2 = a.sink ? a.sink[h] * LOG2E : NEG_BIG;
  float M = a.sink ? sink2 : NEG_BIG;
  float Lsum = a.sink ? 1.0f : 0.f;   // the sink's term exp2(sink2 - M) with M = sink2
  float y0 = 0.f, y1 = 0.f;
  for (int s0 = 0; s0 < a.splits; s0 += 8) {
    float2 mls[8], ov[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = min(s0 + i, a.splits - 1);
      mls[i] = *reinterpret_cast<const float2*>(ml + 2 * s);
      const uint32_t pk = *reinterpret_cast<const uint32_t*>(po + (size_t)s * AC);
      ov[i] = make_float2(bf16_bits_to_f32(pk & 0xffffu), bf16_bits_to_f32(pk >> 16));
    }
    float Mc = M;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (s0 + i < a.splits) Mc = fmaxf(Mc, mls[i].x);
    const float r = exp2f(M - Mc);
    Lsum *= r;
    y0 *= r;
    y1 *= r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (s0 + i >= a.splits) break;
      const float f = exp2f(mls[i].x - Mc);
      Lsum = fmaf(mls[i].y, f, Lsum);
      y0 = fmaf(ov[i].x, f, y0);
      y1 = fmaf(ov[i].y, f, y1);
    }
    M = Mc;
  }
  const float invL = Lsum > 0.f ? 1.0f / Lsum : 0.f;
  y0 *= invL;
  y1 *= invL;
  if (d >= ANOPE) {
    float cs, sn;
    rope_cos_sin(tau, (d - ANOPE) >> 1, AR, a.log2_base, cs, sn);
    const float z0 = y0 * cs + y1 * sn, z1 = -y0 * sn + y1 * cs;
    y0 = z0;
    y1 = z1;
  }
  *reinterpret_cast<uint32_t*>(a.out + (size_t)qh * AC + d) = pack_bf16x2(y0, y1);
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

// Rows of a query are split over workgroups: about one workgroup per CU (each holds ~94 KB
// of LDS), but at least AT_MIN_TILES tiles each, so that the two-tile gather prefetch runs
// ahead of the compute and fewer partial outputs go through memory.
constexpr int AT_MIN_TILES = 2;

SplitPlan plan_splits(const csa_dims& d, int32_t Q, int32_t cap, bool dense) {
  const int64_t max_rows = (int64_t)(dense ? cap : d.top_k) + d.n_win;
  const int ntiles = (int)((max_rows + T2 - 1) / T2);
  const int blocks = Q * ((d.n_h + 63) / 64);
  int target = (256 + blocks - 1) / blocks;
  target = std::max(1, std::min(std::min(target, ntiles), COMB_MAX));
  int tps = std::max((ntiles + target - 1) / target, std::min(AT_MIN_TILES, ntiles));
  tps = std::min(tps, AT_MAX_ROWS / T2);
  return {(ntiles + tps - 1) / tps, tps};
}

}  // namespace

int64_t attend_max_rows() { return (int64_t)COMB_MAX * AT_MAX_ROWS; }

// which: 0 = sparse (idx given; CSA only), 1 = dense (idx = NULL), 2 = the larger of the two
// (a CSA layer may be attended either way when the caller does not say).
size_t attend_workspace_bytes(const csa_dims& d, int32_t Q, int32_t cap, int which) {
  if (d.kv_fmt == CSA_FMT_F32) return 0;
  int splits = 1;
  if (which != 0 || d.top_k <= 0) splits = std::max(splits, plan_splits(d, Q, cap, true).splits);
  if (which != 1 && d.top_k > 0) splits = std::max(splits, plan_splits(d, Q, cap, false).splits);
  if (splits == 1) return 0;
  const size_t po = ((size_t)Q * d.n_h * splits * AC * sizeof(uint16_t) + 255) / 256 * 256;
  return po + (size_t)Q * d.n_h * splits * 2 * sizeof(float);
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
  a.part_o = (uint16_t*)ws;
  const size_t po = ((size_t)Q * d.n_h * p.splits * AC * sizeof(uint16_t) + 255) / 256 * 256;
  a.part_ml = p.splits > 1 ? (float*)((char*)ws + po) : nullptr;
  const int nhg = (d.n_h + 63) / 64;
  hipLaunchKernelGGL(k_attend_mfma, dim3(Q * nhg * p.splits), dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(k_attend_combine, dim3(Q * d.n_h), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
