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
// E4M3/bf16 rows: 64-row tiles are loaded straight into MFMA operand registers, widened
// exactly from E4M3 to bf16, contracted with the queries on bf16 MFMA (float32 accumulation)
// and written once to LDS, from where P.V reads them transposed.  A workgroup (4 waves) covers
// 16 heads of one query.  When there are too few such workgroups to fill the CUs, a query's
// rows are split over several workgroups, whose (max, sum, output) triples a second kernel
// merges.
#include <type_traits>

#include "csa_internal.h"
#include "fold.h"

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
  const uint8_t* kv;          // [B][cap][576], or a pool of pages (rm)
  const uint8_t* win;         // [B][win_cap][576]
  const int32_t* win_pos;     // [B][win_cap]
  const int32_t* n_entries;   // [B]
  int cap, win_cap, m, n_win;
  float scale_log2;           // softmax scale * log2(e)
  float eps;
  double log2_base;
  int splits, tiles_per_split;
  RowMap rm;                  // where a sequence's entries live
  uint16_t* out;              // [Q][n_h][512] bf16 (splits == 1)
  uint16_t* part_o;           // [Q][n_h][splits][512] bf16 (splits > 1)
  float* part_ml;             // [Q][n_h][splits][2]
  int n_att;                  // attention workgroups; with fold_on, the blocks past them fold
  int fold_on;                // a one-token step's fold shares the launch (dense, T = 1)
  FoldArgs fo;
};

// Sum of squares of 8 bf16 values packed in a uint4 (packed bf16 dot products with float32
// accumulation; the values stay packed, so the widened copies are not kept alive).
__device__ __forceinline__ float sumsq_bf16x8(const uint4& v) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf2 x = __builtin_bit_cast(bf2, w[e]);
    s = __builtin_amdgcn_fdot2_f32_bf16(x, x, s, false);
  }
  return s;
}

// Scale 8 bf16 query dims by inv * gamma (gamma dims in g0, g1) and repack them as bf16.
__device__ __forceinline__ uint4 norm_q8(const uint4& v, float inv, const float4& g0, const float4& g1) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = pack_bf16x2(bf16_bits_to_f32(w[e] & 0xffffu) * inv * gm[2 * e],
                       bf16_bits_to_f32(w[e] >> 16) * inv * gm[2 * e + 1]);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Rotate 8 bf16 RoPE dims (dim0 .. dim0+7, dim0 >= 448) to tau: pair j = (dim - 448) / 2
// turns by the angle whose cos/sin sit at cs[2j], cs[2j+1].
__device__ __forceinline__ uint4 rope_q8(const uint4& v, int dim0, const float* cs) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float y0 = bf16_bits_to_f32(w[e] & 0xffffu), y1 = bf16_bits_to_f32(w[e] >> 16);
    const int j = (dim0 + 2 * e - ANOPE) >> 1;
    const float c = cs[2 * j], sn = cs[2 * j + 1];
    o[e] = pack_bf16x2(y0 * c - y1 * sn, y0 * sn + y1 * c);
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

// One workgroup = 4 waves = 16 heads of one query over a range of
// 64-row tiles (all of the query's rows unless the plan splits them).
//   Q.K  wave w loads rows 16w .. 16w+15 of a tile straight into MFMA A-operand registers
//        (lane (row, g) holds a quarter of the row's dims), widens E4M3 to bf16 there and
//        contracts against the 16 heads' queries, also in registers: no LDS on this side;
//   P.V  the widened rows are also written to LDS as a bf16 row-major tile, and wave w
//        produces output dims 128w .. 128w+127 over all 64 rows: A = V^T through the
//        transposing LDS read, B = P^T from a head-major LDS copy of the probabilities.
// LDS rows are 1040 bytes apart (a 16-byte bank shift per row).  Tile row p sits in LDS row
// sigma(p) = 16(p / 16) + 8((p % 16) / 8) + 2(p % 4) + (p / 4) % 2, so the rows that one
// transposing read gathers (8g + 2x, x < 4; +1 for the second read) are 32 bytes apart in
// bank space, and MFMA K slot j of lane group g in P.V meets tile row 8g + j again: P^T is
// stored by tile row.  Both the row writes (16 consecutive tile rows, same chunk) and the
// transposing reads are then free of bank conflicts, and every LDS address is a per-lane
// base plus an immediate offset.
// A row is loaded as nine 64-byte pieces, the four lane groups g taking 16 bytes each, so
// every load instruction covers whole 64-byte segments.  The contraction over dims then
// pairs MFMA step ks, lane group g, slot j with
//   dim 64(ks / 2) + 16g + 8(ks % 2) + j   (ks < 14: E4M3 dims, 16 per 16-byte piece)
//   dim 448 + 32(ks - 14) + 8g + j         (ks = 14, 15: bf16 RoPE dims, 8 per piece)
// on both the key and the query side.  The softmax statistics of a tile are combined over
// the four waves through LDS, so every wave holds the same running max and sum.
constexpr int HS_ROWS = 64;                        // rows per tile
constexpr int HS_MAX_ROWS = 2048;                  // rows one workgroup covers
constexpr int HS_IPT = HS_MAX_ROWS / 256;          // index loads per lane
constexpr int HS_PLD = 72;                         // bf16 pitch of a head's probabilities
constexpr int HS_PITCH = AC * 2 + 16;              // LDS row pitch in bytes
constexpr int HS_DEPTH = 1;                        // tiles loaded ahead of the one in use
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int hs_sigma(int p) {
  return (p & ~15) + 8 * ((p >> 3) & 1) + 2 * (p & 3) + ((p >> 2) & 1);
}

// Row formats.  FMT 0: E4M3_BF16 rows as above.  FMT 1: MXFP4_BF16 rows (CSA2's FP4 main
// KV, 384 bytes): six 64-byte pieces, 0 and 1 the bf16 RoPE dims (lane group g of piece i:
// dims 448 + 32i + 8g ..), 2 .. 4 and the first half of 5 the E2M1 codes (lane group g of
// piece i: the 32 dims of block 4(i - 2) + g), the third quarter of 5 the 14 scale codes.
// Each code piece widens (exactly, by the hardware's scaled FP4 conversion) into four
// 8-dim MFMA slices; piece 5 feeds its four steps from lane groups 0 and 1 only (the others
// contribute zeros), so a row takes 18 MFMA steps instead of 16.
template <int FMT> struct RowFmt;
template <> struct RowFmt<0> { static constexpr int BYTES = 576, PIECES = 9, KSTEPS = 16; };
template <> struct RowFmt<1> { static constexpr int BYTES = 384, PIECES = 6, KSTEPS = 18; };

// First dim of MFMA step ks for lane group g (the dim pairings above).
template <int FMT>
__device__ __forceinline__ int hs_dim(int ks, int g) {
  if constexpr (FMT == 0) {
    return ks < 14 ? 64 * (ks >> 1) + 16 * g + 8 * (ks & 1) : ANOPE + 32 * (ks - 14) + 8 * g;
  } else {
    if (ks < 2) return ANOPE + 32 * ks + 8 * g;
    if (ks < 14) return 32 * (4 * ((ks - 2) >> 2) + g) + 8 * ((ks - 2) & 3);
    return g < 2 ? 32 * (12 + g) + 8 * (ks - 14) : 0;   // g >= 2: zero key operand
  }
}

__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

template <bool SPARSE, bool PAGED, int FMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_attend_hs(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t Ks[HS_ROWS * HS_PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t PsT[16 * HS_PLD];
  __shared__ float redm[4][16], reds[4][16];
  // entry rows of the workgroup's part: index-list entries, or with a paged cache the pool
  // rows they live in (-1: not a visible entry)
  constexpr int NRIDX = (SPARSE || PAGED) ? HS_MAX_ROWS : 1;
  __shared__ int ridx[NRIDX];
  __shared__ float rope_cs[AR];

  // A one-token step's fold in the same launch (dense attention only, so the sparse
  // instances do not carry its registers): its blocks run the fold kernel's code.
  if constexpr (!SPARSE) {
    if (a.fold_on && (int)blockIdx.x >= a.n_att) {
      const int f = (int)blockIdx.x - a.n_att, fx = fold_grid_x(a.fo);
      fold_block<4, true>(a.fo, f % fx, f / fx, &redm[0][0]);
      return;
    }
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int nhs = a.n_h / 16;
  // the head groups of one (query, split) are adjacent, so they share an XCD's L2
  const uint32_t L = xcd_logical_id(blockIdx.x, a.n_att);
  const int hgrp = L % nhs;
  const int rest = L / nhs;
  const int split = rest % a.splits;
  const int q = rest / a.splits;
  const int h = hgrp * 16 + col;       // this lane's head
  const int myrow = wave * 16 + col;   // this lane's row within a tile (Q.K side)
  const int r_lo = split * a.tiles_per_split * HS_ROWS;
  const int32_t* qidx = SPARSE ? a.idx + (size_t)q * a.k : nullptr;
  const int seq = a.q_seq ? a.q_seq[q] : q;
  const int tau = a.q_pos[q];

  // ---- first the loads that depend on no other load: the entry indices of this lane's rows
  // in the first two tiles, the rest of this wave's indices (lane l of batch i: tile
  // (64i + l) / 16, row (64i + l) % 16 of the wave's 16), the norm weights, the sink logit
  // and the 16 heads' query rows (16 KB, 64 contiguous bytes per thread).  Optional inputs
  // are read through a valid stand-in address and replaced afterwards, so that no load sits
  // in a branch.
  int s01[HS_DEPTH] = {};
  int rid[HS_IPT] = {};
  auto rid_row = [&](int i) { const int f = 64 * i + lane; return r_lo + (f >> 4) * HS_ROWS + wave * 16 + (f & 15); };
  if constexpr (SPARSE) {
#pragma unroll
    for (int t = 0; t < HS_DEPTH; ++t) s01[t] = qidx[min(r_lo + t * HS_ROWS + myrow, a.k - 1)];
#pragma unroll
    for (int i = 0; i < HS_IPT; ++i) rid[i] = qidx[min(rid_row(i), a.k - 1)];
  }
  const float* gsrc = (a.gamma_q ? a.gamma_q : reinterpret_cast<const float*>(a.q)) + 32 * (tid & 15);
  float4 gq[8];   // the norm weights of this thread's 32 query dims
#pragma unroll
  for (int k = 0; k < 8; ++k) gq[k] = *reinterpret_cast<const float4*>(gsrc + 4 * k);
  const float sraw = *(a.sink ? a.sink + h : reinterpret_cast<const float*>(a.q));
  const uint8_t* qblk = reinterpret_cast<const uint8_t*>(a.q + ((size_t)q * a.n_h + hgrp * 16) * AC);
  // (four named registers: an array here would be moved to LDS by the compiler)
  const uint4 qr0 = *reinterpret_cast<const uint4*>(qblk + 64 * tid);
  const uint4 qr1 = *reinterpret_cast<const uint4*>(qblk + 64 * tid + 16);
  const uint4 qr2 = *reinterpret_cast<const uint4*>(qblk + 64 * tid + 32);
  const uint4 qr3 = *reinterpret_cast<const uint4*>(qblk + 64 * tid + 48);
  // keep the issue order above and below (neither the optimiser nor the scheduler may move
  // memory operations across these fences, which wait for nothing)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  const int w0 = max(0, tau - a.n_win + 1);
  // entries visible at tau
  const int V = max(0, min(tau / a.m, a.n_entries[seq]));
  const int nsel = SPARSE ? a.k : V;
  const int nrows = nsel + (tau - w0 + 1);
  const int r_hi = min(nrows, r_lo + a.tiles_per_split * HS_ROWS);
  // With the fold in this launch the new token's window row may not be in the ring yet: the
  // workgroups whose part ends with it finalize it from the token's partial projections with
  // the fold's own code (so the same bytes as the fold stores), store it, and read it back
  // like any other row.
  if constexpr (!SPARSE) {
    if (a.fold_on && r_hi == nrows && r_lo < nrows) {   // uniform over the workgroup
      const int u = 2 * tid;
      float x0 = 0.f, x1 = 0.f;
      if (u < a.fo.c) {
        x0 = proj<true>(a.fo, seq, tau, tau, u);
        x1 = proj<true>(a.fo, seq, tau, tau, u + 1);
      }
      const int slot = tau % a.win_cap;
      finalize_store<4>(a.fo, x0, x1, tau, a.fo.win + ((size_t)seq * a.win_cap + slot) * a.fo.rowB, &reds[0][0]);
      if (tid == 0) a.fo.win_pos[(size_t)seq * a.win_cap + slot] = tau;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  }
  // paged: row numbers are pool rows (kv is the pool), looked up once per entry here, so
  // that the loop below reads them from LDS like an index list; entries past the visible
  // ones become -1, and only window rows then need the visibility test
  constexpr int ROWB = RowFmt<FMT>::BYTES, NPIECE = RowFmt<FMT>::PIECES, NKS = RowFmt<FMT>::KSTEPS;
  const uint8_t* kvseq = PAGED ? a.kv : a.kv + (size_t)seq * a.cap * ROWB;
  if constexpr (PAGED) {
    auto pool_row = [&](int e) {
      return e >= 0 && e < min(V, a.cap) ? page_of(a.rm, seq, e) * a.rm.epp + e % a.rm.epp : -1;
    };
#pragma unroll
    for (int t = 0; t < HS_DEPTH; ++t) s01[t] = pool_row(SPARSE ? s01[t] : r_lo + t * HS_ROWS + myrow);
#pragma unroll
    for (int i = 0; i < HS_IPT; ++i) rid[i] = pool_row(SPARSE ? rid[i] : rid_row(i));
  }
  const uint8_t* winseq = a.win + (size_t)seq * a.win_cap * ROWB;
  const int32_t* wpseq = a.win_pos + (size_t)seq * a.win_cap;

  // ---- row gather: lane (row, g) loads bytes 64i + 16g .. +15 of the row (i < 9; pieces
  // 0..6 hold E4M3 dims, 7 and 8 bf16 RoPE dims) and the position its window slot holds.
  // Rows past the part's end and entries that are not visible are not loaded at all: their
  // lanes keep the values of an earlier row (finite, or the zeros they start with), and the
  // softmax gives them weight 0.  Window rows always load (a slot holding another position
  // is a finite row too) and are masked by the position check.
  uint4 pre[HS_DEPTH][NPIECE];
#pragma unroll
  for (int t = 0; t < HS_DEPTH; ++t)
#pragma unroll
    for (int i = 0; i < NPIECE; ++i) pre[t][i] = make_uint4(0u, 0u, 0u, 0u);
  bool ldk[HS_DEPTH];   // whether this lane's row of the tile is loaded
  int chk[HS_DEPTH], wpv[HS_DEPTH], sv[HS_DEPTH];   // chk: 1 entry row, 0 masked, else window position + 2
  // source row of this lane for the tile at t0 (plus its window-slot position load and the
  // facts its validity is decided from)
  auto gather_src = [&](int t0, int s_in, auto bconst) {
    constexpr int b = decltype(bconst)::value;
    const int r = t0 + myrow;
    const bool in = r < r_hi, ent = r < nsel;
    const int s = (SPARSE || PAGED) ? s_in : r;
    const bool ok_a = in && ent && s >= 0 && (PAGED || (s < a.cap && s < V));
    const int slot = (ent ? 0 : w0 + (r - nsel)) % a.win_cap;
    const uint8_t* src = ent ? kvseq + (size_t)(ok_a ? s : 0) * ROWB
                             : (in ? winseq + (size_t)slot * ROWB : kvseq);
    wpv[b] = wpseq[slot];
    chk[b] = ent ? (ok_a ? 1 : 0) : (in ? w0 + (r - nsel) + 2 : 0);
    sv[b] = s;
    ldk[b] = ent ? ok_a : in;
    return src;
  };
  auto gather = [&](int t0, int s_in, auto bconst) {
    constexpr int b = decltype(bconst)::value;
    const uint8_t* src = gather_src(t0, s_in, bconst);
    if (ldk[b]) {
#pragma unroll
      for (int i = 0; i < NPIECE; ++i) pre[b][i] = *reinterpret_cast<const uint4*>(src + 64 * i + 16 * g);
    }
  };
  gather(r_lo, s01[0], std::integral_constant<int, 0>{});
  if constexpr (HS_DEPTH > 1) gather(r_lo + HS_ROWS, s01[HS_DEPTH - 1], std::integral_constant<int, HS_DEPTH - 1>{});
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // ---- LDS: the normalised query rows (RMSNorm over a head's 512 dims, whose 16 threads
  // hold 32 dims each, times the norm weights; in the tile buffer, pitch HS_PITCH), this
  // wave's entry indices and the RoPE table at tau
  {
    float ss = (sumsq_bf16x8(qr0) + sumsq_bf16x8(qr1)) + (sumsq_bf16x8(qr2) + sumsq_bf16x8(qr3));
    ss = __int_as_float(row_allreduce(__float_as_int(ss), OpAddF()));
    const float inv = 1.0f / sqrtf(ss / (float)AC + a.eps);
    if (!a.gamma_q) {
#pragma unroll
      for (int k = 0; k < 8; ++k) gq[k] = make_float4(1.f, 1.f, 1.f, 1.f);
    }
    uint8_t* qd = Ks + (tid >> 4) * HS_PITCH + 64 * (tid & 15);
    *reinterpret_cast<uint4*>(qd) = norm_q8(qr0, inv, gq[0], gq[1]);
    *reinterpret_cast<uint4*>(qd + 16) = norm_q8(qr1, inv, gq[2], gq[3]);
    *reinterpret_cast<uint4*>(qd + 32) = norm_q8(qr2, inv, gq[4], gq[5]);
    *reinterpret_cast<uint4*>(qd + 48) = norm_q8(qr3, inv, gq[6], gq[7]);
  }
  if constexpr (SPARSE || PAGED) {
#pragma unroll
    for (int i = 0; i < HS_IPT; ++i) ridx[min(rid_row(i) - r_lo, HS_MAX_ROWS - 1)] = rid[i];
  }
  if (tid < AR / 2) rope_cos_sin(tau, tid, AR, a.log2_base, rope_cs[2 * tid], rope_cs[2 * tid + 1]);
  lds_barrier();

  // ---- bf16 B operands of Q.K, with RoPE at tau on dims 448..511 (steps 14 and 15)
  bf16x8 Qop[NKS];
  {
    const uint8_t* qs = Ks + col * HS_PITCH;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int d0 = hs_dim<FMT>(ks, g);
      const uint4 v = *reinterpret_cast<const uint4*>(qs + 2 * d0);
      const bool rope = FMT == 0 ? ks >= 14 : ks < 2;
      Qop[ks] = __builtin_bit_cast(bf16x8, rope ? rope_q8(v, d0, rope_cs) : v);
    }
  }
  lds_barrier();   // the tile buffer is rewritten next

  const float sink2 = a.sink ? sraw * LOG2E : NEG_BIG;
  float m_run = sink2;
  float l_run = 0.f;
  f32x4 O[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) O[i] = f32x4{0, 0, 0, 0};

  auto tile = [&](int t0, auto bconst) {
    constexpr int b = decltype(bconst)::value;
    // the entry index of this lane's row in the tile after next, read before this tile's
    // LDS writes so that waiting for it does not wait for them
    const int tn = t0 + HS_DEPTH * HS_ROWS;
    const int s_next = (SPARSE || PAGED) ? ridx[min(max(tn + myrow - r_lo, 0), NRIDX - 1)] : 0;
    const bool ok = (chk[b] == 1 && (PAGED || sv[b] < V)) || (chk[b] >= 2 && wpv[b] == chk[b] - 2);
    const uint64_t okm = __ballot(ok);   // bit r of the low 16: row 16w + r is valid

    // ---- widen, write the V tile, and contract Q.K for this wave's 16 rows (four
    // independent accumulation chains, added at the end)
    f32x4 Sp[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
    uint8_t* const Kb = Ks;
    uint16_t* const Pb = PsT;
    uint8_t* wrow = Kb + hs_sigma(myrow) * HS_PITCH;
    if constexpr (FMT == 1) {
      // the row's scale codes, from its lane group 2 (piece 5): code piece i of lane group g
      // takes byte g of dword i - 2
      typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
      const int sl = ((lane & 15) + 32) << 2;
      const uint32_t scw[4] = {(uint32_t)__builtin_amdgcn_ds_bpermute(sl, (int)pre[b][5].x),
                               (uint32_t)__builtin_amdgcn_ds_bpermute(sl, (int)pre[b][5].y),
                               (uint32_t)__builtin_amdgcn_ds_bpermute(sl, (int)pre[b][5].z),
                               (uint32_t)__builtin_amdgcn_ds_bpermute(sl, (int)pre[b][5].w)};
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        uint4 v = pre[b][i];
        if (i < 2) {
          *reinterpret_cast<uint4*>(wrow + 16 * (56 + 4 * i + g)) = v;
          Sp[i & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), Qop[i], Sp[i & 3], 0, 0, 0);
        } else {
          const bool has = i < 5 || g < 2;   // piece 5: codes in lane groups 0, 1 only
          if (!has) v = make_uint4(0u, 0u, 0u, 0u);
          int code = (scw[i - 2] >> (8 * g)) & 0xff;
          if (!ok || !has) code = 127;       // masked rows: scale 1 on zero codes
          const float scale = __int_as_float(code ? code << 23 : 0x00400000);   // 2^(code - 127)
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
          const int blk = 4 * (i - 2) + g;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], scale, 0);
            const bf2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], scale, 1);
            const bf2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], scale, 2);
            const bf2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], scale, 3);
            const uint4 cw = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                        __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
            if (has) *reinterpret_cast<uint4*>(wrow + 64 * blk + 16 * j) = cw;
            const int ks = 2 + 4 * (i - 2) + j;
            Sp[ks & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cw), Qop[ks], Sp[ks & 3], 0, 0, 0);
          }
        }
      }
    } else {
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const uint4 v = pre[b][i];
      if (i < 7) {
        uint32_t x[8];
        e4m3x4_to_bf16x4(v.x, x[0], x[1]);
        e4m3x4_to_bf16x4(v.y, x[2], x[3]);
        e4m3x4_to_bf16x4(v.z, x[4], x[5]);
        e4m3x4_to_bf16x4(v.w, x[6], x[7]);
        const uint4 c0 = make_uint4(x[0], x[1], x[2], x[3]);
        const uint4 c1 = make_uint4(x[4], x[5], x[6], x[7]);
        *reinterpret_cast<uint4*>(wrow + 16 * (8 * i + 2 * g)) = c0;
        *reinterpret_cast<uint4*>(wrow + 16 * (8 * i + 2 * g + 1)) = c1;
        Sp[(2 * i) & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, c0), Qop[2 * i], Sp[(2 * i) & 3], 0, 0, 0);
        Sp[(2 * i + 1) & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, c1), Qop[2 * i + 1], Sp[(2 * i + 1) & 3], 0, 0, 0);
      } else {
        *reinterpret_cast<uint4*>(wrow + 16 * (56 + 4 * (i - 7) + g)) = v;
        Sp[(7 + i) & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), Qop[7 + i], Sp[(7 + i) & 3], 0, 0, 0);
      }
    }
    }
    f32x4 S = (Sp[0] + Sp[1]) + (Sp[2] + Sp[3]);
    // the tile after next goes into the registers just consumed, its loads in flight during
    // the softmax and P.V (one predicated block: per-load branches would split P.V's LDS
    // reads and MFMAs into separately scheduled pieces)
    gather(tn, s_next, bconst);

    // ---- online softmax: lane holds head col, rows 16w + 4g + e
    float mx = NEG_BIG;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool rv = (okm >> (4 * g + e)) & 1u;
      S[e] = rv ? S[e] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, S[e]);
    }
    mx = fmaxf(mx, lane_xor16(mx));
    mx = fmaxf(mx, lane_xor32(mx));
    if (g == 0) redm[wave][col] = mx;
    lds_barrier();
    const float m_tile = fmaxf(fmaxf(redm[0][col], redm[1][col]), fmaxf(redm[2][col], redm[3][col]));
    const float m_new = fmaxf(m_run, m_tile);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      S[e] = __builtin_amdgcn_exp2f(S[e] - m_new);
      ls += S[e];
    }
    // every wave holds the same running max, so each keeps the sum over its own rows and
    // the four are added once at the end
    l_run = l_run * alpha + ls;
    m_run = m_new;
    *reinterpret_cast<uint2*>(&Pb[col * HS_PLD + wave * 16 + 4 * g]) =
        make_uint2(pack_bf16x2(S[0], S[1]), pack_bf16x2(S[2], S[3]));
    lds_barrier();
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) O[i] *= alpha;
    }

    // ---- O^T += V^T . P^T over the 64 rows (two K chunks of 32) for this wave's 128 dims.
    // Transposing read: source lane j of a 16-lane group reads LDS row 32kc + 8g + 2(j >> 2)
    // (+1 for the second read), dims c0 + 4(j & 3) .. +3; lane i then holds dim c0 + i of
    // tile rows 32kc + 8g .. +3 (+4 .. +7).
    const uint8_t* vbase = Kb + (8 * g + 2 * (col >> 2)) * HS_PITCH + 2 * (wave * 128 + 4 * (col & 3));
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const bf16x8 Bp = *reinterpret_cast<const bf16x8*>(&Pb[col * HS_PLD + 32 * kc + 8 * g]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint8_t* va = vbase + 32 * kc * HS_PITCH + 32 * dt;
        const s16x4 lo = lds_read_tr16(va);
        const s16x4 hi = lds_read_tr16(va + HS_PITCH);
        const bf16x8 Av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Av, Bp, O[dt], 0, 0, 0);
      }
    }
    lds_barrier();   // the next tile rewrites the row and probability buffers
  };
  // with HS_DEPTH > 1 tiles go in groups whose last ones may lie past the end: fully masked,
  // they change nothing
  for (int t0 = r_lo; t0 < r_hi; t0 += HS_DEPTH * HS_ROWS) {
    tile(t0, std::integral_constant<int, 0>{});
    if constexpr (HS_DEPTH > 1) tile(t0 + HS_ROWS, std::integral_constant<int, HS_DEPTH - 1>{});
  }

  // the sum over all rows: lanes hold a wave's 16 rows of one tile position (4g + e), summed
  // over lane groups here and over waves through LDS
  l_run += lane_xor16(l_run);
  l_run += lane_xor32(l_run);
  if (g == 0) reds[wave][col] = l_run;
  lds_barrier();
  l_run = ((reds[0][col] + reds[1][col]) + reds[2][col]) + reds[3][col];

  // O[dt][e]: head h, dim 128w + 16dt + 4g + e
  if (a.splits == 1) {
    const float Lsum = l_run + (a.sink ? exp2f(sink2 - m_run) : 0.f);
    const float invL = Lsum > 0.f ? 1.0f / Lsum : 0.f;
    uint16_t* orow = a.out + ((size_t)q * a.n_h + h) * AC;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) store_out4(O[dt], invL, orow, wave * 128 + 16 * dt + 4 * g, rope_cs);
  } else {
    // unnormalised partial output, already rotated back (the rotation is linear, so it
    // commutes with the merge)
    const size_t pidx = ((size_t)q * a.n_h + h) * a.splits + split;
    uint16_t* po = a.part_o + pidx * AC;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) store_out4(O[dt], 1.0f, po, wave * 128 + 16 * dt + 4 * g, rope_cs);
    if (wave == 0 && g == 0) {
      a.part_ml[pidx * 2] = m_run;
      a.part_ml[pidx * 2 + 1] = l_run;
    }
  }
}

// Merge split partials (already rotated back): one 64-thread workgroup per (query, head), 8
// dims per lane.  Splits are taken NS at a time, every load of a chunk in flight at once (NS
// is the smallest of 4, 8, 16 that holds the plan's splits, else 16 and several chunks),
// merged with a running max.
constexpr int COMB_MAX = 256;  // most splits a plan uses

template <int NS>
__global__ __launch_bounds__(64) void k_attend_combine(AttendArgs a) {
  const int qh = blockIdx.x;
  const int h = qh % a.n_h;
  const int d = 8 * threadIdx.x;
  const float* ml = a.part_ml + (size_t)qh * a.splits * 2;
  const uint16_t* po = a.part_o + (size_t)qh * a.splits * AC + d;
  const float sink2 = a.sink ? a.sink[h] * LOG2E : NEG_BIG;
  float M = a.sink ? sink2 : NEG_BIG;
  float Lsum = a.sink ? 1.0f : 0.f;   // the sink's term exp2(sink2 - M) with M = sink2
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < a.splits; s0 += NS) {
    float2 mls[NS];
    uint4 ov[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int s = min(s0 + i, a.splits - 1);
      mls[i] = *reinterpret_cast<const float2*>(ml + 2 * s);
      ov[i] = *reinterpret_cast<const uint4*>(po + (size_t)s * AC);
    }
    float Mc = M;
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (s0 + i < a.splits) Mc = fmaxf(Mc, mls[i].x);
    const float r = exp2f(M - Mc);
    Lsum *= r;
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] *= r;
#pragma unroll
    for (int i = 0; i < NS; ++i) {   // past the last split: a repeat of it, weighted 0
      const float f = s0 + i < a.splits ? exp2f(mls[i].x - Mc) : 0.f;
      Lsum = fmaf(mls[i].y, f, Lsum);
      const uint32_t w[4] = {ov[i].x, ov[i].y, ov[i].z, ov[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[2 * j] = fmaf(bf16_bits_to_f32(w[j] & 0xffffu), f, y[2 * j]);
        y[2 * j + 1] = fmaf(bf16_bits_to_f32(w[j] >> 16), f, y[2 * j + 1]);
      }
    }
    M = Mc;
  }
  const float invL = Lsum > 0.f ? 1.0f / Lsum : 0.f;
  *reinterpret_cast<uint4*>(a.out + (size_t)qh * AC + d) =
      make_uint4(pack_bf16x2(y[0] * invL, y[1] * invL), pack_bf16x2(y[2] * invL, y[3] * invL),
                 pack_bf16x2(y[4] * invL, y[5] * invL), pack_bf16x2(y[6] * invL, y[7] * invL));
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
                                                   RowMap rm, int win_cap, int m, int n_win, int c,
                                                   int r, float scale, float eps, double log2_base,
                                                   float* __restrict__ out) {
  __shared__ float qs[1024];
  __shared__ float z[AF_MAXK];
  __shared__ const float* rows[AF_MAXK];
  const int qh = blockIdx.x;
  const int q = qh / n_h, h = qh % n_h, t = threadIdx.x;
  const int seq = q_seq ? q_seq[q] : q, tau = q_pos[q];
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
      if (s >= 0 && s < min(V, rm.cap)) p = kv + row_of(rm, seq, s) * c;
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

// Rows of a query are split over workgroups when there are too few (query, 16-head)
// workgroups to keep the CUs busy.  The plan minimises a cost in tile times: a CU runs up to
// two workgroups at once, which then finish about 1.2x faster than one after the other; each
// round of workgroups on a CU pays a prologue of about 1.5 tiles (index, query and first row
// loads); a split plan pays about 2.5 tiles for the merge pass.  A part holds at most
// HS_MAX_ROWS rows (their indices sit in LDS).
constexpr int HS_CUS = 256;

SplitPlan plan_splits(const csa_dims& d, int32_t Q, int32_t cap, bool dense) {
  const int64_t max_rows = (int64_t)(dense ? cap : d.top_k) + d.n_win;
  const int ntiles = (int)((max_rows + HS_ROWS - 1) / HS_ROWS);
  const int64_t blocks = (int64_t)Q * (d.n_h / 16);
  SplitPlan best{0, 0};
  double best_cost = 0.0;
  for (int s = 1; s <= std::min(ntiles, COMB_MAX); ++s) {
    const int tps = (ntiles + s - 1) / s;
    if (tps > HS_MAX_ROWS / HS_ROWS || (ntiles + tps - 1) / tps != s) continue;
    const int64_t per_cu = (blocks * s + HS_CUS - 1) / HS_CUS;
    const double rounds = (double)((per_cu + 1) / 2);
    const double cost = rounds * (tps * (per_cu > 1 ? 1.65 : 1.0) + 1.5) + (s > 1 ? 2.5 + 0.02 * s : 0.0);
    if (best.splits == 0 || cost < best_cost) {
      best = {s, tps};
      best_cost = cost;
    }
  }
  if (best.splits == 0) {   // more rows than COMB_MAX parts hold: callers reject such calls
    const int tps = HS_MAX_ROWS / HS_ROWS;
    best = {std::min(COMB_MAX, (ntiles + tps - 1) / tps), tps};
  }
  return best;
}

}  // namespace

int64_t attend_max_rows() { return (int64_t)COMB_MAX * HS_MAX_ROWS; }

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
                         void* ws, hipStream_t s, const FoldArgs* fold) {
  const float scale = d.scale > 0.f ? d.scale : 1.0f / sqrtf((float)d.c);
  if (d.kv_fmt == CSA_FMT_F32) {
    if (fold) return hipErrorInvalidValue;   // the fold rides only in the quantized kernel
    hipLaunchKernelGGL(k_attend_f32, dim3(Q * d.n_h), dim3(64), 0, s, (const float*)q, gamma_q,
                       sink, q_seq, q_pos, d.n_h, idx, d.top_k, (const float*)c.kv,
                       (const float*)c.win, c.win_pos, c.n_entries, row_map(d, c), c.win_cap, d.m,
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
  a.rm = row_map(d, c);
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
  a.n_att = Q * (d.n_h / 16) * p.splits;
  a.fold_on = fold ? 1 : 0;
  if (fold) {
    if (idx || fold->T != 1 || !fold->part || fold->keys_entry) return hipErrorInvalidValue;
    a.fo = *fold;
  }
  const dim3 grid(a.n_att + (fold ? fold_grid_x(*fold) * fold->B : 0));
#define ATT_LAUNCH(F)                                                                         \
  if (a.rm.bt) {                                                                              \
    if (idx) hipLaunchKernelGGL((k_attend_hs<true, true, F>), grid, dim3(256), 0, s, a);      \
    else hipLaunchKernelGGL((k_attend_hs<false, true, F>), grid, dim3(256), 0, s, a);         \
  } else {                                                                                    \
    if (idx) hipLaunchKernelGGL((k_attend_hs<true, false, F>), grid, dim3(256), 0, s, a);     \
    else hipLaunchKernelGGL((k_attend_hs<false, false, F>), grid, dim3(256), 0, s, a);        \
  }
  if (d.kv_fmt == CSA_FMT_MXFP4_BF16) {
    ATT_LAUNCH(1)
  } else {
    ATT_LAUNCH(0)
  }
#undef ATT_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const dim3 cgrid(Q * d.n_h);
  if (p.splits <= 4) hipLaunchKernelGGL(k_attend_combine<4>, cgrid, dim3(64), 0, s, a);
  else if (p.splits <= 8) hipLaunchKernelGGL(k_attend_combine<8>, cgrid, dim3(64), 0, s, a);
  else hipLaunchKernelGGL(k_attend_combine<16>, cgrid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
