// Lightning-indexer scores for gfx950:
//   I_{t,s} = sum_h w_{t,h} * ReLU(q^I_{t,h} . K^I_s),  s < V(t) = min(t / m, n_entries)
// (reading notes "DeepSeekV4技术报告阅读笔记" §2.3.2 eq. 16 and the causal rule after eq. 17;
// deep dive "DeepSeek-V4 架构设计深度解析" §3.2; PaperTrace "02 · DeepSeek-V4" §2.2).
//
// With E4M3 keys and queries the contraction over c_I runs on bf16 MFMA: E4M3 values widen to
// bf16 exactly, products are exact and accumulate in float32.  (The fp8 MFMA forms accumulate
// with fewer bits: measured errors of ~2^-16 of sum|a_k b_k|, which top-k selection cannot
// tolerate.)  With MXFP4 keys and queries (the FP4 indexer path, PaperTrace §3.3) the
// codes and scales go to the block-scaled FP4 MFMA as stored.  Its float32 result is the
// exact dot whenever that fits a float32 significand, which the block scales decide: each
// tile checks them, and a tile whose (head, key) pairs could overflow the significand
// contracts each 32-element block on its own and adds the four exact block terms in float64.
// The ReLU, the head weight and the sum over heads are fused into the MFMA epilogue; the FP4
// path sums in float64 and stores the BF16 score rounded once.
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

// One block-scaled 16x16x128 MFMA over E2M1 operands (OCP MX FP4): lane l supplies row
// (l & 15), elements 32g .. 32g+31 with g = l >> 4 (16 bytes, element 2i in the low nibble of
// byte i) and that block's E8M0 scale code; the result lane l holds column (l & 15), rows
// 4g .. 4g+3.  Products of E2M1 values are exact, and so is the sum whenever it fits a
// float32 significand (it does when the scales of a row pair lie within a few octaves).
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma_fp4(const uint4& a, int sa, const uint4& b, int sb) {
  const i32x8 av = {(int32_t)a.x, (int32_t)a.y, (int32_t)a.z, (int32_t)a.w, 0, 0, 0, 0};
  const i32x8 bv = {(int32_t)b.x, (int32_t)b.y, (int32_t)b.z, (int32_t)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, f32x4{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, sa,
                                                          0, sb);
}

// When the 16x16x128 FP4 MFMA's float32 result is exact.  A 32-element block's sum of E2M1
// products is an integer multiple of 2^-2 below 32 * 36 (|product| <= 6 * 6), scaled by the
// product of the two block scales 2^p_b, p_b = (code_q - 127) + (code_k - 127).  In units of
// 2^(min_b p_b - 2) the four-block sum stays below 4 * 4608 * 2^D, D = max_b p_b - min_b p_b,
// which fits the 24-bit float32 significand for D <= 9; gfx950 then returns it exactly.  D is
// at most the query head's code spread plus the key's.
constexpr int FP4_EXACT_SPREAD = 9;

// Largest minus smallest of the four scale codes of one row, where lane group g (l >> 4) holds
// block g's code and the 16 lanes of a group hold 16 rows (the layout of an FP4 MFMA operand).
__device__ __forceinline__ int code_spread(int code) {
  int mx = code, mn = code;
  int o = __float_as_int(lane_xor16(__int_as_float(mx)));
  int p = __float_as_int(lane_xor16(__int_as_float(mn)));
  mx = max(mx, o);
  mn = min(mn, p);
  o = __float_as_int(lane_xor32(__int_as_float(mx)));
  p = __float_as_int(lane_xor32(__int_as_float(mn)));
  return max(mx, o) - min(mn, p);
}

// ReLU of an MFMA result as one integer max on its bits: negative floats (and -0) are
// negative integers.  (fmaxf would first canonicalize its operand, a second instruction.)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// The value of the lane 32 (16) apart, for a float64.
__device__ __forceinline__ double lane_xor32_d(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const float lo = lane_xor32(__uint_as_float((uint32_t)u)), hi = lane_xor32(__uint_as_float((uint32_t)(u >> 32)));
  return __builtin_bit_cast(double, (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32));
}
__device__ __forceinline__ double lane_xor16_d(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const float lo = lane_xor16(__uint_as_float((uint32_t)u)), hi = lane_xor16(__uint_as_float((uint32_t)(u >> 32)));
  return __builtin_bit_cast(double, (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32));
}

// The nearest bfloat16 to a float64 (ties to even), rounded once: with x = f 2^e, f in
// [0.5, 1), the value keeps rint(f 2^8) 2^(e - 8), which float32 holds exactly.
__device__ __forceinline__ uint16_t bf16_nearest_from_f64(double x) {
  int e;
  const double f = frexp(x, &e);
  const float v = (float)ldexp(rint(ldexp(f, 8)), e - 8);
  return (uint16_t)(__float_as_uint(v) >> 16);
}

// Head sum of one query's MFMA tile with its weights, for the BF16 scores of the FP4 path:
// the products of a bf16 weight and an exact float32 dot are exact in float64, and so is
// their sum for these magnitudes; the score is rounded once, at the store.
template <int HT>
__device__ __forceinline__ double head_sum_f64(const uint4 (&qa)[HT], const int (&qs)[HT],
                                               const double (&W)[HT][4], const uint4& b, int bs) {
  double part = 0.0;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const f32x4 acc = mfma_fp4(qa[ht], qs[ht], b, bs);
#pragma unroll
    for (int e = 0; e < 4; ++e) part = fma(W[ht][e], (double)relu(acc[e]), part);
  }
  return part;
}

// One workgroup = 4 waves; blockIdx.x = group of QPW queries (same sequence), blockIdx.y =
// entry chunk; wave w scans its quarter of the chunk in tiles of 16 entries.
// MFMA mapping (16x16x32 bf16): A = q^I rows (heads), B = K^I rows (entries), contraction
// over c_I.  Lane l holds head/entry (l & 15) and, within each 32-wide K step ks, dims
// g*32 + ks*8 .. +7 with g = l >> 4 -- the same mapping on both operands, so each product
// pairs equal dims.  Output tile: lane l holds entry (l & 15), heads 4g .. 4g+3.
struct IndexerArgs {
  const uint8_t* qI;
  const uint16_t* wI;
  const int32_t* q_seq;
  const int32_t* q_pos;
  int Q;
  const uint8_t* ki;
  int cap;
  const int32_t* n_entries;
  int m;
  void* scores;           // float32, or bfloat16 with MXFP4
  int64_t ld;
  int chunk;
  RowMap rm;              // where a sequence's keys live (contiguous or paged)
};

// Paged keys in the decode bodies: a wave scans tiles s0 = w_lo + 64 j, each inside one page
// (pages hold a multiple of 16 entries and tiles start at multiples of 16).  A tile past the
// end reads the last 16-aligned tile's entries instead (s is clamped to c_hi - 1), so tile j
// is found at t0 = min(s0, (c_hi - 1) & ~15).  Lane j of the wave looks up tile j's page and
// the row of t0 in it once, before any key is requested; a key row is then two lane reads
// and an add.  (The chunk is capped so that a wave's tiles, prefetched ones past the end
// included, number at most 64.)
struct WavePages {
  int page, r0;
};
__device__ __forceinline__ WavePages wave_pages(const RowMap& rm, int seq, int w_lo, int c_hi, int lane) {
  if (!rm.bt) return {0, 0};
  const int t0 = min(w_lo + 64 * lane, (c_hi - 1) & ~15);
  return {page_of(rm, seq, t0), t0 % rm.epp};
}
// Entry s of the tile at s0: the first row of its group (a sequence's cap rows, or a page's
// epp rows) and its row within the group.
__device__ __forceinline__ void tile_loc(const RowMap& rm, int seq, const WavePages& wp, int w_lo, int c_hi,
                                         int s0, int s, int64_t& g0, int& r) {
  if (!rm.bt) {
    g0 = (int64_t)seq * rm.cap;
    r = s;
    return;
  }
  const int j = __builtin_amdgcn_readfirstlane((s0 - w_lo) >> 6);
  const int t0 = min(s0, (c_hi - 1) & ~15);
  g0 = (int64_t)__builtin_amdgcn_readlane(wp.page, j) * rm.epp;
  r = __builtin_amdgcn_readlane(wp.r0, j) + (s - t0);
}

// The part of a workgroup's work every indexer body shares: its queries' visible ranges and
// the wave's first tile of the chunk.  Returns false when the wave has nothing to score.
template <int QPW>
__device__ __forceinline__ bool indexer_range(const IndexerArgs& ia, int bx, int by, int wave, int& seq,
                                              int (&V)[QPW], int& c_hi, int& w_lo) {
  const int q0 = bx * QPW;
  seq = ia.q_seq ? ia.q_seq[q0] : q0;
  const int nent = ia.n_entries[seq];
  int Vmax = 0;
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    const int q = q0 + qq;
    V[qq] = q < ia.Q ? max(0, min(ia.q_pos[q] / ia.m, nent)) : 0;
    Vmax = max(Vmax, V[qq]);
  }
  // this wave's entries: tiles of 16 dealt round-robin over the 4 waves of the chunk
  const int c_lo = by * ia.chunk;
  c_hi = min(c_lo + ia.chunk, Vmax);
  w_lo = c_lo + 16 * wave;
  return c_lo < c_hi && w_lo < c_hi;
}

// E4M3 keys and queries.  Workgroup (bx, by): queries bx * QPW .. +QPW-1 against entry chunk by.
template <int NH, int QPW>
__device__ __forceinline__ void indexer_bf16_body(const IndexerArgs& ia, int bx, int by) {
  const uint8_t* __restrict__ qI = ia.qI;
  const uint16_t* __restrict__ wI = ia.wI;
  const int Q = ia.Q;
  const uint8_t* __restrict__ ki = ia.ki;
  float* __restrict__ scores = static_cast<float*>(ia.scores);
  const int64_t ld = ia.ld;
  constexpr int HT = NH / 16;
  constexpr int DEPTH = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int q0 = bx * QPW;
  int seq, V[QPW], c_hi, w_lo;
  // contiguous keys: the first ring goes out as soon as the sequence is known, bounded by the
  // chunk and the capacity; the visible count (one more dependent load) bounds the rest
  const bool spec = ia.rm.bt == nullptr;
  if (spec) {
    seq = ia.q_seq ? ia.q_seq[q0] : q0;
    const int c_lo = by * ia.chunk;
    c_hi = min(c_lo + ia.chunk, ia.cap);
    w_lo = c_lo + 16 * wave;
    if (w_lo >= c_hi) return;
  } else if (!indexer_range<QPW>(ia, bx, by, wave, seq, V, c_hi, w_lo)) {
    return;
  }
  const int stride = 64;  // 4 waves x 16 entries

  const WavePages wp = wave_pages(ia.rm, seq, w_lo, c_hi, lane);
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
  uint4 rk[DEPTH][2];
  auto load_tile = [&](int s0, uint4 (&r)[2]) {
    const int s = min(s0 + col, c_hi - 1);
    int64_t g0;
    int ri;
    tile_loc(ia.rm, seq, wp, w_lo, c_hi, s0, s, g0, ri);
    const uint8_t* src = ki + (g0 + ri) * IX_CI + g * 32;
    r[0] = *reinterpret_cast<const uint4*>(src);
    r[1] = *reinterpret_cast<const uint4*>(src + 16);
  };
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) load_tile(w_lo + stride * i, rk[i]);
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
  if (spec) {
    int sq, wl;
    if (!indexer_range<QPW>(ia, bx, by, wave, sq, V, c_hi, wl)) return;
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
      e4m3x32_to_ops(rk[i][0], rk[i][1], Bop);
      load_tile(s0 + stride * DEPTH, rk[i]);
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
          for (int e = 0; e < 4; ++e) part = fmaf(W[qq][ht][e], relu(acc[e]), part);
        }
        // lane groups summed as (g + g^2) + (g^1 + g^3), the order the tiled kernel uses
        part += lane_xor32(part);
        part += lane_xor16(part);
        const int s = s0 + col;
        if (g == 0 && s < min(V[qq], c_hi)) scores[(size_t)(q0 + qq) * ld + s] = part;
      }
    }
  } while (++it < rounds);
}

// MXFP4 keys and queries, with the same work split and ring as indexer_bf16_body.  A
// sequence's keys are cap rows of 64 element bytes, then cap rows of 4 scale codes; a query's
// q^I is NH rows of 64 element bytes, then NH rows of 4 scale codes.  Lane group g reads
// block g of a row (16 element bytes and one scale code), which is exactly the lane's share
// of a block-scaled MFMA operand, so the codes go to the matrix cores as loaded: one
// 16x16x128 MFMA per head tile covers all 128 dims.  Scores are bfloat16.
// The same head sum for a tile whose block scales may span more octaves than a float32 sum
// holds: block blk is contracted alone (the key operand's other blocks zeroed; zeroing the
// query operand instead would be loop-invariant, and the compiler would keep all sixteen
// masked copies live), where its sum is exact, and the dot is the float64 sum of the four
// block terms in block order.
template <int HT>
__device__ __forceinline__ double head_sum_f64_blocks(const uint4 (&qa)[HT], const int (&qs)[HT],
                                                      const double (&W)[HT][4], const uint4& b, int bs,
                                                      int g) {
  // (scheduling fences keep one head tile's MFMAs in flight at a time: the path is rare, and
  // hoisting all of them would raise the register use of the common path around it)
  uint4 bm[4];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) bm[blk] = g == blk ? b : make_uint4(0u, 0u, 0u, 0u);
  double part = 0.0;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) acc[blk] = mfma_fp4(qa[ht], qs[ht], bm[blk], bs);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double dot = (((double)acc[0][e] + (double)acc[1][e]) + (double)acc[2][e]) + (double)acc[3][e];
      part = fma(W[ht][e], fmax(dot, 0.0), part);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  return part;
}

// Largest scale-code spread over a query's NH heads (every lane of the wave gets it).
template <int HT>
__device__ __forceinline__ int query_code_spread(const int (&qs)[HT]) {
  int sp = 0;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) sp = max(sp, code_spread(qs[ht]));
  return wave_allreduce(sp, [](int x, int y) { return max(x, y); });
}

template <int NH, int QPW>
__device__ __forceinline__ void indexer_fp4_body(const IndexerArgs& ia, int bx, int by) {
  constexpr int KC = IX_CI / 2, KS = IX_CI / 32;  // element bytes, scale codes per row
  constexpr int HT = NH / 16;
  constexpr int DEPTH = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int q0 = bx * QPW;
  int seq, V[QPW], c_hi, w_lo;
  // contiguous keys: the first ring goes out before the entry count is known, as in
  // indexer_bf16_body
  const bool spec = ia.rm.bt == nullptr;
  if (spec) {
    seq = ia.q_seq ? ia.q_seq[q0] : q0;
    const int c_lo = by * ia.chunk;
    c_hi = min(c_lo + ia.chunk, ia.cap);
    w_lo = c_lo + 16 * wave;
    if (w_lo >= c_hi) return;
  } else if (!indexer_range<QPW>(ia, bx, by, wave, seq, V, c_hi, w_lo)) {
    return;
  }
  const int stride = 64;  // 4 waves x 16 entries
  uint16_t* __restrict__ scores = static_cast<uint16_t*>(ia.scores);

  const WavePages wp = wave_pages(ia.rm, seq, w_lo, c_hi, lane);
  // a group of n rows (a sequence's cap, or a page's epp) holds n rows of element bytes, then
  // n rows of scale codes
  const int64_t gn = ia.rm.bt ? ia.rm.epp : ia.cap;
  uint4 qa[QPW][HT];
  int qs[QPW][HT];
  uint2 wraw[QPW][HT];
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    const int q = min(q0 + qq, ia.Q - 1);
    const uint8_t* qrow = ia.qI + (size_t)q * NH * (KC + KS);
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 16 + col;
      qa[qq][ht] = *reinterpret_cast<const uint4*>(qrow + h * KC + g * 16);
      qs[qq][ht] = qrow[NH * KC + h * KS + g];
      wraw[qq][ht] = *reinterpret_cast<const uint2*>(ia.wI + (size_t)q * NH + ht * 16 + 4 * g);
    }
  }
  uint4 kc[DEPTH];
  int ks[DEPTH];
  auto load_tile = [&](int s0, uint4& c, int& sc) {
    const int s = min(s0 + col, c_hi - 1);
    int64_t g0;
    int r;
    tile_loc(ia.rm, seq, wp, w_lo, c_hi, s0, s, g0, r);
    const uint8_t* grp = ia.ki + g0 * (KC + KS);
    c = *reinterpret_cast<const uint4*>(grp + r * KC + g * 16);
    sc = grp[gn * KC + r * KS + g];
  };
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) load_tile(w_lo + stride * i, kc[i], ks[i]);
  __builtin_amdgcn_sched_barrier(0);

  double W[QPW][HT][4];
  int sq[QPW];
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const uint2 w4 = wraw[qq][ht];
      W[qq][ht][0] = bf16_bits_to_f32(w4.x & 0xffffu);
      W[qq][ht][1] = bf16_bits_to_f32(w4.x >> 16);
      W[qq][ht][2] = bf16_bits_to_f32(w4.y & 0xffffu);
      W[qq][ht][3] = bf16_bits_to_f32(w4.y >> 16);
    }
    sq[qq] = query_code_spread<HT>(qs[qq]);
  }
  if (spec) {
    int sq2, wl;
    if (!indexer_range<QPW>(ia, bx, by, wave, sq2, V, c_hi, wl)) return;
  }
  const int rounds = (c_hi - w_lo + stride * DEPTH - 1) / (stride * DEPTH);
  int it = 0;
  do {  // rounds >= 1 since w_lo < c_hi
    const int base = w_lo + it * stride * DEPTH;
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      const int s0 = base + stride * i;
      const uint4 b = kc[i];
      const int bs = ks[i];
      load_tile(s0 + stride * DEPTH, kc[i], ks[i]);
      const int sk = code_spread(bs);
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq) {
        // wave-uniform: every (head, key) pair of the tile sums exactly in float32
        const bool fast = __ballot(sq[qq] + sk > FP4_EXACT_SPREAD) == 0;
        double part = fast ? head_sum_f64<HT>(qa[qq], qs[qq], W[qq], b, bs)
                           : head_sum_f64_blocks<HT>(qa[qq], qs[qq], W[qq], b, bs, g);
        part += lane_xor32_d(part);
        part += lane_xor16_d(part);
        const int s = s0 + col;
        if (g == 0 && s < min(V[qq], c_hi)) scores[(size_t)(q0 + qq) * ia.ld + s] = bf16_nearest_from_f64(part);
      }
    }
  } while (++it < rounds);
}

template <int NH, int QPW>
__global__ __launch_bounds__(256) void k_indexer_bf16(IndexerArgs ia) {
  indexer_bf16_body<NH, QPW>(ia, blockIdx.x, blockIdx.y);
}

template <int NH, int QPW>
__global__ __launch_bounds__(256) void k_indexer_fp4(IndexerArgs ia) {
  indexer_fp4_body<NH, QPW>(ia, blockIdx.x, blockIdx.y);
}

// Prefill-shaped indexer: a workgroup of 8 waves scores IT_Q = 16 queries of ONE sequence
// (2 per wave) against that sequence's entries [e_lo, e_hi).  Keys are shared by every query
// of the tile, so they are staged once through LDS (256-entry stages, double buffered, four
// 16-byte loads per thread per stage, widened to bf16 once while staging) instead of being
// fetched and widened per query.  Each wave keeps its two queries' q^I (64 heads, widened to
// bf16) in registers; per 16-entry tile it reads the keys from LDS and runs 2 x 4 head tiles
// x 4 K-steps of bf16 MFMA, with the same operand mapping and epilogue order as
// k_indexer_bf16 (so the scores are identical).
constexpr int IT_Q = 16;        // queries per workgroup
constexpr int IT_STAGE = 256;   // entries per LDS stage (one barrier per 16 tiles)
constexpr int IT_LD = 272;      // LDS bytes per entry row: 128 dims in bf16 + 16 pad (spreads the banks)

// With CAND the kernel also thresholds its own scores: before the main pass it scores a
// sample of IT_SMP entries shared by the tile's queries (IT_SMP_RUNS evenly spaced runs of 64
// below the smallest visible count of the tile), writes those scores to their places in the
// rows, reads each query's sample back and takes its r-th largest, r chosen so that about
// IT_TARGET of the row's V scores are expected at or above it (every score passes when
// V <= TOPK_FINAL_CAND).  The main pass then appends, besides storing every score, the
// entries at or above the threshold to the query's list for this workgroup's segment of the
// row (wave ballots, index order).  The lists of all segments hold every score at or above one
// threshold, an upper set of the row, so when they hold at least k entries they hold the top k.
constexpr int IT_SMP_RUNS = 16, IT_SMP = IT_SMP_RUNS * 64;
constexpr int IT_TARGET = 3072;
constexpr int IT_STAGE_CAND = 128;   // the thresholding kernel's stage (its registers fit no larger)

template <bool CAND, int STG>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_indexer_tile(
    const uint8_t* __restrict__ qI, const uint16_t* __restrict__ wI,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int Q,
    const uint8_t* __restrict__ ki, RowMap rm, const int32_t* __restrict__ n_entries, int m,
    float* __restrict__ scores, int64_t ld, int chunk, CandLists cl) {
  constexpr int NH = 64, HT = NH / 16;
  static_assert(IT_SMP % STG == 0, "the sample is whole stages");
  __shared__ __align__(16) uint8_t kbuf[2][STG * IT_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int qt0 = blockIdx.x * IT_Q;
  const int seq = q_seq ? q_seq[qt0] : qt0;
  const int nent = n_entries[seq];
  // visible entries of the tile's queries (clamped duplicates past Q store nothing); the
  // smallest and largest over the real ones
  int Vmax = 0, Vmin = 0x7fffffff;
  for (int i = 0; i < IT_Q; ++i) {
    const int q = min(qt0 + i, Q - 1);
    const int v = max(0, min(q_pos[q] / m, nent));
    Vmax = max(Vmax, v);
    if (qt0 + i < Q) Vmin = min(Vmin, v);
  }
  const int seg = blockIdx.y, nseg = gridDim.y;
  if constexpr (CAND) {
    if (seg == 0 && tid < IT_Q && qt0 + tid < Q) cl.vis[qt0 + tid] = max(0, min(q_pos[qt0 + tid] / m, nent));
  }
  const int e_lo = seg * chunk;
  const int e_hi = min(e_lo + chunk, Vmax);
  if (e_lo >= e_hi) {  // uniform over the workgroup
    if constexpr (CAND) {
      if (tid < IT_Q && qt0 + tid < Q) cl.cnt[(size_t)(qt0 + tid) * nseg + seg] = 0;
    }
    return;
  }

  int V[2];
  bf16x8 A[2][HT][4];
  float W[2][HT][4];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int qr = qt0 + 2 * wave + qq;
    const int q = min(qr, Q - 1);
    V[qq] = qr < Q ? max(0, min(q_pos[q] / m, nent)) : 0;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const uint8_t* src = qI + ((size_t)q * NH + ht * 16 + col) * IX_CI + g * 32;
      e4m3x32_to_ops(*reinterpret_cast<const uint4*>(src), *reinterpret_cast<const uint4*>(src + 16),
                     A[qq][ht]);
      const uint2 w4 = *reinterpret_cast<const uint2*>(wI + (size_t)q * NH + ht * 16 + 4 * g);
      W[qq][ht][0] = bf16_bits_to_f32(w4.x & 0xffffu);
      W[qq][ht][1] = bf16_bits_to_f32(w4.x >> 16);
      W[qq][ht][2] = bf16_bits_to_f32(w4.y & 0xffffu);
      W[qq][ht][3] = bf16_bits_to_f32(w4.y >> 16);
    }
  }

  // stage loader: thread t moves dims 8p .. 8p+7 and 64+8p .. 64+8p+7 (p = t % 8) of entry
  // t / 8 of the stage, widened to bf16; the 8 threads of an entry write two contiguous
  // 128-byte runs, which keeps the LDS writes free of bank conflicts
  // (a paged cache costs one block-table read per entry, hidden behind a stage of MFMAs).
  // entry_of maps a position in the pass (st * STG + ...) to the entry it scores.
  const int le = tid >> 3, lp = (tid & 7) * 8;
  constexpr int RPT = STG / 64;  // entries per thread per stage
  auto gload = [&](auto entry_of, int st, uint4 (&v)[RPT]) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int e = entry_of(st * STG + 64 * r + le);
      const uint8_t* src = ki + row_of(rm, seq, e) * IX_CI + lp;
      const uint2 a = *reinterpret_cast<const uint2*>(src);
      const uint2 b = *reinterpret_cast<const uint2*>(src + 64);
      v[r] = make_uint4(a.x, a.y, b.x, b.y);
    }
  };
  auto lstore = [&](int buf, const uint4 (&v)[RPT]) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      uint32_t b[8];
      e4m3x4_to_bf16x4(v[r].x, b[0], b[1]);
      e4m3x4_to_bf16x4(v[r].y, b[2], b[3]);
      e4m3x4_to_bf16x4(v[r].z, b[4], b[5]);
      e4m3x4_to_bf16x4(v[r].w, b[6], b[7]);
      uint8_t* dst = &kbuf[buf][(64 * r + le) * IT_LD + 2 * lp];
      *reinterpret_cast<uint4*>(dst) = make_uint4(b[0], b[1], b[2], b[3]);
      *reinterpret_cast<uint4*>(dst + 128) = make_uint4(b[4], b[5], b[6], b[7]);
    }
  };
  // Scores of the 64 entries of one sub-stage (kb) for this wave's two queries: lane (col, g)
  // receives entry 16 g + col's.
  auto score_sub = [&](const uint8_t* kb, float (&tot)[2]) {
    // per lane partial head sums: part[t][qq] for tile t of the sub-stage, query qq (the
    // lane's 4 heads of each head tile); reduced over the 4 lane groups once per 64 entries
    float part[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // dims g*32 + ks*8 .. +7 (the mapping e4m3x32_to_ops gives the q^I operands)
      const uint8_t* row = kb + (t * 16 + col) * IT_LD + g * 64;
      bf16x8 Bop[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) Bop[ks] = *reinterpret_cast<const bf16x8*>(row + 16 * ks);
      // K-step outermost: the 8 accumulators are independent, so consecutive MFMAs never
      // wait on each other's results
      f32x4 acc[2][HT];
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[qq][ht] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
            acc[qq][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[qq][ht][ks], Bop[ks], acc[qq][ht], 0, 0, 0);
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        float p = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int e = 0; e < 4; ++e) p = fmaf(W[qq][ht][e], relu(acc[qq][ht][e]), p);
        part[t][qq] = p;
      }
    }
    // Reduce-scatter over the lane groups g = lane >> 4: after the exchange with lane ^ 32
    // a lane keeps tiles {0,1} (g < 2) or {2,3}; after lane ^ 16 it keeps tile g.  Lane
    // (col, g) then holds entry t*16 + col of tile t = g, summed over all 64 heads.
    const bool hi2 = g >= 2, odd = g & 1;
    float r1[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const float keep = hi2 ? part[2 + j][qq] : part[j][qq];
        const float send = hi2 ? part[j][qq] : part[2 + j][qq];
        r1[j][qq] = keep + lane_xor32(send);
      }
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const float keep = odd ? r1[1][qq] : r1[0][qq];
      const float send = odd ? r1[0][qq] : r1[1][qq];
      tot[qq] = keep + lane_xor16(send);
    }
  };
  uint4 nxt[RPT];
  auto main_entry = [&](int v) { return min(e_lo + v, e_hi - 1); };

  // ---- CAND: the sample and the thresholds (thr = 0 takes every score)
  uint32_t thr[2] = {0u, 0u};
  int ccount[2] = {0, 0};
  if constexpr (CAND) {
    int vbig = 0;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) vbig = max(vbig, V[qq]);
    const bool need = __syncthreads_or(vbig > TOPK_FINAL_CAND) != 0;
    const int span = max(Vmin - 64, 0);
    auto sample_entry = [&](int v) {
      return min((int)((int64_t)(v >> 6) * span / (IT_SMP_RUNS - 1)) + (v & 63), Vmax - 1);
    };
    if (need) {   // uniform
      gload(sample_entry, 0, nxt);
      lstore(0, nxt);
      __syncthreads();
      for (int st = 0; st < IT_SMP / STG; ++st) {
        if (st + 1 < IT_SMP / STG) gload(sample_entry, st + 1, nxt);
#pragma unroll
        for (int sub = 0; sub < RPT; ++sub) {
          float tot[2];
          score_sub(kbuf[st & 1] + sub * 64 * IT_LD, tot);
          // the sample scores go to their places in the rows (the main pass stores the same
          // values there again), from where this wave reads them back
          const int e = sample_entry(st * STG + sub * 64 + g * 16 + col);
#pragma unroll
          for (int qq = 0; qq < 2; ++qq)
            if (qt0 + 2 * wave + qq < Q) scores[(size_t)(qt0 + 2 * wave + qq) * ld + e] = tot[qq];
        }
        if (st + 1 < IT_SMP / STG) lstore((st + 1) & 1, nxt);
        __syncthreads();
      }
      // the wave's own stores are complete and visible to its lanes before they are read back
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q = qt0 + 2 * wave + qq;
        if (V[qq] <= TOPK_FINAL_CAND) continue;   // uniform: every score passes
        uint32_t kk[IT_SMP / 64];
#pragma unroll
        for (int i = 0; i < IT_SMP / 64; ++i) kk[i] = score_key(scores[(size_t)q * ld + sample_entry(lane + 64 * i)]);
        const int r = min(IT_SMP, max(1, (int)(((int64_t)IT_TARGET * IT_SMP + V[qq] - 1) / V[qq])));
        // the largest key t with at least r sample keys >= t: the sample's r-th largest
        uint32_t lo = 0u, hi = 0xffffffffu;
        while (lo < hi) {   // uniform
          const uint32_t mid = lo + ((hi - lo) >> 1) + 1u;
          int cnt = 0;
#pragma unroll
          for (int i = 0; i < IT_SMP / 64; ++i) cnt += __popcll(__ballot(kk[i] >= mid));
          if (cnt >= r) lo = mid;
          else hi = mid - 1u;
        }
        thr[qq] = __builtin_amdgcn_readfirstlane(lo);
      }
    }
  }

  // ---- main pass over the segment's entries
  const int nst = (e_hi - e_lo + STG - 1) / STG;
  gload(main_entry, 0, nxt);
  lstore(0, nxt);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) gload(main_entry, st + 1, nxt);
#pragma unroll
    for (int sub = 0; sub < RPT; ++sub) {
      float tot[2];
      score_sub(kbuf[st & 1] + sub * 64 * IT_LD, tot);
      // the 64 lanes store one contiguous run of 64 scores per query
      const int s = e_lo + st * STG + sub * 64 + g * 16 + col;
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const bool vis = s < min(V[qq], e_hi);
        if (vis) scores[(size_t)(qt0 + 2 * wave + qq) * ld + s] = tot[qq];
        if constexpr (CAND) {
          const uint32_t key = score_key(tot[qq]);
          const bool pass = vis && key >= thr[qq];
          const uint64_t bal = __ballot(pass);
          if (pass) {
            const int pos = ccount[qq] + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            if (pos < cl.cs) {
              const size_t at = ((size_t)(qt0 + 2 * wave + qq) * nseg + seg) * cl.cs + pos;
              cl.idx[at] = s;
              cl.key[at] = key;
            }
          }
          ccount[qq] = __builtin_amdgcn_readfirstlane(ccount[qq] + (int)__popcll(bal));
        }
      }
    }
    if (st + 1 < nst) lstore((st + 1) & 1, nxt);
    __syncthreads();
  }
  if constexpr (CAND) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
      if (lane == 0 && qt0 + 2 * wave + qq < Q) cl.cnt[(size_t)(qt0 + 2 * wave + qq) * nseg + seg] = ccount[qq];
  }
}

// Prefill-shaped MXFP4 indexer: the work split of k_indexer_tile (8 waves, IT_Q = 16 queries of
// one sequence, 2 per wave), with the keys kept in MXFP4 all the way to the matrix cores.  A
// stage of IF_STAGE entries is copied to LDS as stored (one 16-byte load of element bytes per
// thread; the first IF_STAGE threads also move an entry's 4 scale codes), double buffered.
// Per 16-entry tile a lane reads its block of the entry (16 bytes and the scale code) and
// runs one block-scaled 16x16x128 MFMA per head tile and query; the head sum is the FP4
// decode kernel's (float64, scores rounded once to bfloat16), reduced over lane groups as
// in k_indexer_tile so that 64 lanes store 64 contiguous scores.
constexpr int IF_STAGE = 128;  // entries per LDS stage
constexpr int IF_RS = 80;      // LDS bytes per entry row: 64 element bytes + 16 pad, so the 16
                               // rows a read touches start in 16 distinct 16-byte bank groups

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_indexer_tile_fp4(
    const uint8_t* __restrict__ qI, const uint16_t* __restrict__ wI,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int Q,
    const uint8_t* __restrict__ ki, RowMap rm, const int32_t* __restrict__ n_entries, int m,
    uint16_t* __restrict__ scores, int64_t ld, int chunk) {
  constexpr int NH = 64, HT = NH / 16, KC = IX_CI / 2, KS = IX_CI / 32;
  __shared__ __align__(16) uint8_t kbuf[2][IF_STAGE * IF_RS];
  __shared__ __align__(16) uint8_t sbuf[2][IF_STAGE * KS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int qt0 = blockIdx.x * IT_Q;
  const int seq = q_seq ? q_seq[qt0] : qt0;
  const int nent = n_entries[seq];
  int Vmax = 0;
  for (int i = 0; i < IT_Q; ++i) {
    const int q = min(qt0 + i, Q - 1);
    Vmax = max(Vmax, max(0, min(q_pos[q] / m, nent)));
  }
  const int e_lo = blockIdx.y * chunk;
  const int e_hi = min(e_lo + chunk, Vmax);
  if (e_lo >= e_hi) return;  // uniform over the workgroup

  int V[2];
  uint4 qa[2][HT];
  int qs[2][HT];
  double W[2][HT][4];
  int sq[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int qr = qt0 + 2 * wave + qq;
    const int q = min(qr, Q - 1);
    V[qq] = qr < Q ? max(0, min(q_pos[q] / m, nent)) : 0;
    const uint8_t* qrow = qI + (size_t)q * NH * (KC + KS);
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 16 + col;
      qa[qq][ht] = *reinterpret_cast<const uint4*>(qrow + h * KC + g * 16);
      qs[qq][ht] = qrow[NH * KC + h * KS + g];
      const uint2 w4 = *reinterpret_cast<const uint2*>(wI + (size_t)q * NH + ht * 16 + 4 * g);
      W[qq][ht][0] = bf16_bits_to_f32(w4.x & 0xffffu);
      W[qq][ht][1] = bf16_bits_to_f32(w4.x >> 16);
      W[qq][ht][2] = bf16_bits_to_f32(w4.y & 0xffffu);
      W[qq][ht][3] = bf16_bits_to_f32(w4.y >> 16);
    }
    sq[qq] = query_code_spread<HT>(qs[qq]);
  }

  // stage loader: thread t moves element bytes 16 (t % 4) .. +15 of entry t / 4 of the stage;
  // threads t < IF_STAGE also move entry t's scale codes (clamped past the end, unused there)
  const int le = tid >> 2, lp = (tid & 3) * 16;
  auto gload = [&](int st, uint4& v, uint32_t& sv) {
    const int e = min(e_lo + st * IF_STAGE + le, e_hi - 1);
    int64_t oc, os;
    mx_offsets(rm, seq, e, KC, KS, oc, os);
    v = *reinterpret_cast<const uint4*>(ki + oc + lp);
    if (tid < IF_STAGE) {
      const int es = min(e_lo + st * IF_STAGE + tid, e_hi - 1);
      mx_offsets(rm, seq, es, KC, KS, oc, os);
      sv = *reinterpret_cast<const uint32_t*>(ki + os);
    }
  };
  auto lstore = [&](int buf, const uint4& v, uint32_t sv) {
    *reinterpret_cast<uint4*>(&kbuf[buf][le * IF_RS + lp]) = v;
    if (tid < IF_STAGE) *reinterpret_cast<uint32_t*>(&sbuf[buf][tid * KS]) = sv;
  };
  const int nst = (e_hi - e_lo + IF_STAGE - 1) / IF_STAGE;
  uint4 nv;
  uint32_t ns = 0;
  gload(0, nv, ns);
  lstore(0, nv, ns);
  __syncthreads();
  // A unit is (tile t of the stage, query qq), u = 2t + qq.  Software pipeline over the
  // units: the MFMAs of unit u + 1 are issued before the epilogue of unit u, so the matrix
  // cores run while the vector ALUs sum the heads (the epilogue is the larger part).
  constexpr int NT = IF_STAGE / 16, NU = 2 * NT;
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) gload(st + 1, nv, ns);
    const uint8_t* kb = kbuf[st & 1];
    const uint8_t* sb = sbuf[st & 1];
    // the stage's key operands: the lane's block of entry 16t + col, read once per tile
    uint4 b[NT];
    int bs[NT];
    // bit t: tile t holds a (head, key) pair of either query whose float32 sum may be inexact
    uint32_t slow = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int r = t * 16 + col;
      b[t] = *reinterpret_cast<const uint4*>(kb + r * IF_RS + g * 16);
      bs[t] = sb[r * KS + g];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int sk = code_spread(bs[t]);
      slow |= (__ballot(max(sq[0], sq[1]) + sk > FP4_EXACT_SPREAD) != 0 ? 1u : 0u) << t;
    }
    auto mm = [&](int u, f32x4 (&a)[HT]) {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) a[ht] = mfma_fp4(qa[u & 1][ht], qs[u & 1][ht], b[u >> 1], bs[u >> 1]);
    };
    // The stage's units; MAY_SLOW: some tile needs the block-wise sum (the wave's flags say
    // which).  Without it the loop is free of that branch, so the MFMAs of the next unit and
    // the epilogue of this one are scheduled together.
    auto run_stage = [&](auto may_slow) {
    constexpr bool MAY_SLOW = decltype(may_slow)::value;
    f32x4 acc[2][HT];
    // part[t][qq]: tile t of the current 64-entry run, query qq, the lane's 16 heads
    double part[4][2];
    mm(0, acc[0]);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (u + 1 < NU) mm(u + 1, acc[(u + 1) & 1]);
      const int qq = u & 1, t = (u >> 1) & 3;
      double p = 0.0;
      if (!MAY_SLOW || !((slow >> (u >> 1)) & 1u)) {
        // the head sum of head_sum_f64, in the same order
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int e = 0; e < 4; ++e) p = fma(W[qq][ht][e], (double)relu(acc[u & 1][ht][e]), p);
      } else {
        p = head_sum_f64_blocks<HT>(qa[qq], qs[qq], W[qq], b[u >> 1], bs[u >> 1], g);
      }
      part[t][qq] = p;
      if ((u & 7) != 7) continue;
      // a 64-entry run is complete: reduce-scatter over the lane groups as in k_indexer_tile,
      // so lane (col, g) ends with entry g * 16 + col of the run, summed over all 64 heads
      const bool hi2 = g >= 2, odd = g & 1;
      double r1[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const double keep = hi2 ? part[2 + j][q2] : part[j][q2];
          const double send = hi2 ? part[j][q2] : part[2 + j][q2];
          r1[j][q2] = keep + lane_xor32_d(send);
        }
      const int s = e_lo + st * IF_STAGE + (u >> 3) * 64 + g * 16 + col;
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const double keep = odd ? r1[1][q2] : r1[0][q2];
        const double send = odd ? r1[0][q2] : r1[1][q2];
        const double total = keep + lane_xor16_d(send);
        if (s < min(V[q2], e_hi)) scores[(size_t)(qt0 + 2 * wave + q2) * ld + s] = bf16_nearest_from_f64(total);
      }
    }
    };
    if (slow == 0u) run_stage(std::false_type{});
    else run_stage(std::true_type{});
    if (st + 1 < nst) lstore((st + 1) & 1, nv, ns);
    __syncthreads();
  }
}

// float32 indexer (fp32 formats): one thread per (query, entry).
__global__ __launch_bounds__(256) void k_indexer_f32(
    const float* __restrict__ qI, const float* __restrict__ wI, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int Q, const float* __restrict__ ki, RowMap rm,
    const int32_t* __restrict__ n_entries, int m, int nh, int cI, float* __restrict__ scores,
    int64_t ld) {
  const int q = blockIdx.y;
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= Q) return;
  const int seq = q_seq ? q_seq[q] : q;
  const int V = max(0, min(q_pos[q] / m, n_entries[seq]));
  if (s >= V) return;
  const float* k = ki + row_of(rm, seq, s) * cI;
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

// The tiled launch shape: nsplit workgroups per group of IT_Q queries (about one workgroup
// per CU overall), each scoring a chunk of the row (a multiple of the stage).
static void tile_shape(int32_t Q, int32_t cap, int stage, int* chunk, int* nchunk) {
  const int ntile = (Q + IT_Q - 1) / IT_Q;
  const int nsplit = std::max(1, (256 + ntile - 1) / ntile);
  int ch = (cap + nsplit - 1) / nsplit;
  ch = (ch + stage - 1) / stage * stage;
  *chunk = ch;
  *nchunk = (cap + ch - 1) / ch;
}

// Candidate-list capacity per segment: the final pass holds TOPK_FINAL_CAND candidates in all;
// each segment's list takes up to four times its even share (at least 1024).
static int cand_cs(int nseg) {
  return std::min(TOPK_FINAL_CAND, std::max(1024, 4 * TOPK_FINAL_CAND / nseg));
}

bool indexer_cand_applies(const csa_dims& d, int32_t Q) {
  return d.idx_fmt == CSA_FMT_E4M3 && d.n_hI == 64 && d.c_I == IX_CI && Q >= IT_Q;
}

size_t indexer_cand_bytes(const csa_dims& d, int32_t Q, int32_t cap) {
  if (!indexer_cand_applies(d, Q)) return 0;
  int chunk, nseg;
  tile_shape(Q, cap, IT_STAGE_CAND, &chunk, &nseg);
  const size_t n = (size_t)Q * nseg;
  const size_t list = ((n * cand_cs(nseg) * 4) + 255) / 256 * 256;
  return 2 * list + (n * 4 + 255) / 256 * 256 + ((size_t)Q * 4 + 255) / 256 * 256;
}

hipError_t launch_indexer_cand(const csa_dims& d, const csa_cache& c, const void* qI, const void* w,
                               const int32_t* q_seq, const int32_t* q_pos, int32_t Q, float* scores,
                               int64_t ld, void* ws, CandLists* cl, hipStream_t s) {
  if (!indexer_cand_applies(d, Q)) return hipErrorInvalidValue;
  int chunk, nseg;
  tile_shape(Q, c.cap, IT_STAGE_CAND, &chunk, &nseg);
  const int cs = cand_cs(nseg);
  const size_t n = (size_t)Q * nseg;
  const size_t list = ((n * cs * 4) + 255) / 256 * 256;
  char* p = static_cast<char*>(ws);
  cl->idx = reinterpret_cast<int32_t*>(p);
  cl->key = reinterpret_cast<uint32_t*>(p + list);
  cl->cnt = reinterpret_cast<int32_t*>(p + 2 * list);
  cl->vis = reinterpret_cast<int32_t*>(p + 2 * list + (n * 4 + 255) / 256 * 256);
  cl->nseg = nseg;
  cl->cs = cs;
  const dim3 grid((Q + IT_Q - 1) / IT_Q, nseg);
  hipLaunchKernelGGL((k_indexer_tile<true, IT_STAGE_CAND>), grid, dim3(512), 0, s, (const uint8_t*)qI, (const uint16_t*)w,
                     q_seq, q_pos, Q, (const uint8_t*)c.ki, row_map(d, c), c.n_entries, d.m, scores, ld,
                     chunk, *cl);
  return hipGetLastError();
}

hipError_t launch_indexer(const csa_dims& d, const csa_cache& c, const void* qI, const void* w,
                          const int32_t* q_seq, const int32_t* q_pos, int32_t Q, void* scores,
                          int64_t ld, bool tiled, hipStream_t s) {
  const bool fp4 = d.idx_fmt == CSA_FMT_MXFP4;
  const RowMap rm = row_map(d, c);
  if (tiled && (fp4 || d.idx_fmt == CSA_FMT_E4M3) && d.n_hI == 64 && Q >= IT_Q) {
    // every aligned group of IT_Q queries belongs to one sequence (the caller guarantees it)
    int chunk, nchunk;
    tile_shape(Q, c.cap, fp4 ? IF_STAGE : IT_STAGE, &chunk, &nchunk);
    dim3 grid((Q + IT_Q - 1) / IT_Q, nchunk);
    if (fp4)
      hipLaunchKernelGGL(k_indexer_tile_fp4, grid, dim3(512), 0, s, (const uint8_t*)qI,
                         (const uint16_t*)w, q_seq, q_pos, Q, (const uint8_t*)c.ki, rm,
                         c.n_entries, d.m, static_cast<uint16_t*>(scores), ld, chunk);
    else
      hipLaunchKernelGGL((k_indexer_tile<false, IT_STAGE>), grid, dim3(512), 0, s, (const uint8_t*)qI,
                         (const uint16_t*)w, q_seq, q_pos, Q, (const uint8_t*)c.ki, rm,
                         c.n_entries, d.m, static_cast<float*>(scores), ld, chunk, CandLists{});
    return hipGetLastError();
  }
  if (d.idx_fmt == CSA_FMT_F32) {
    dim3 grid((c.cap + 255) / 256, Q);
    hipLaunchKernelGGL(k_indexer_f32, grid, dim3(256), 0, s, (const float*)qI, (const float*)w,
                       q_seq, q_pos, Q, (const float*)c.ki, rm, c.n_entries, d.m, d.n_hI,
                       d.c_I, static_cast<float*>(scores), ld);
    return hipGetLastError();
  }
  // E4M3 keys (bf16 MFMA) or MXFP4 keys (block-scaled FP4 MFMA).  One query per group; entry chunks sized so that the grid is about
  // two workgroups (8 waves) per CU, each wave streaming a long run of tiles.
  const int target_wgs = 512;
  const int per_q = std::max(1, target_wgs / std::max(Q, 1));
  int chunk = (c.cap + per_q - 1) / per_q;
  chunk = std::max(256, (chunk + 255) / 256 * 256);
  // paged keys: a wave's tiles (64 entries apart, 4 prefetched past the end) must number at
  // most 64, one page id per lane
  if (rm.bt) chunk = std::min(chunk, 2048);
  const int nchunk = (c.cap + chunk - 1) / chunk;
  const IndexerArgs ia{(const uint8_t*)qI, (const uint16_t*)w, q_seq, q_pos, Q, (const uint8_t*)c.ki,
                       c.cap, c.n_entries, d.m, scores, ld, chunk, rm};
  dim3 grid(Q, nchunk);
#define IX_LAUNCH(NHV)                                                                          \
  if (fp4) hipLaunchKernelGGL((k_indexer_fp4<NHV, 1>), grid, dim3(256), 0, s, ia);                \
  else hipLaunchKernelGGL((k_indexer_bf16<NHV, 1>), grid, dim3(256), 0, s, ia)
  switch (d.n_hI) {
    case 64: IX_LAUNCH(64); break;
    case 32: IX_LAUNCH(32); break;
    case 16: IX_LAUNCH(16); break;
    default: return hipErrorInvalidValue;
  }
#undef IX_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
