// Per-query top-k selection for gfx950 (reading notes "DeepSeekV4技术报告阅读笔记" §2.3.2
// eq. 17: keep the entries whose index score is among the k largest).
//
// Keys are the scores mapped to order-preserving uint32 (-0 counts as +0); scores are
// finite.  The selection is exact: equal scores go to the lower index, and the output holds
// the chosen indices in increasing order, padded with -1.
//
// One workgroup of 1024 threads selects from up to 1024*E items held in registers, thread t
// holding the contiguous run [t*E, t*E + E), so thread order is index order:
//   1. a block min/max of the scores, then a 2048-bin histogram linear in the score over
//      [min, max]; the bin holding the k-th largest is found by one wave, and every item in
//      a higher bin is taken.  Linear bins spread the scores over many bins, so the bin
//      that is left (the "window") is small and the LDS atomics rarely collide;
//   2. inside the window, radix passes over the keys (offset by the window's smallest key,
//      11 bits at a time) narrow it until it is a single key value or is taken whole;
//   3. one packed block scan gives every taken item its output slot: all items above the
//      window, and the `need` lowest-index items of the window.
// Rows of up to 8192 scores take one workgroup and one launch.  Longer rows go through a
// threshold pass and a final pass:
//   filter  one workgroup per (query, 8192-score segment).  All segments of a query draw the
//           same sample (64 evenly spaced runs of 64 scores) and bin it linearly over its range; the
//           bin b holding the sample's r-th largest, r chosen so that about 3k scores of the
//           row are expected at or above it, is the threshold.  Binning is monotone in the
//           score, so the scores in bins >= b form an upper set of the row: when it holds at
//           least k scores it holds the top k (ties included).  Each segment writes its
//           passing scores in index order with their count;
//   final   one workgroup per query gathers the candidate lists (in index order) and selects
//           k exactly, holding 2, 4 or 8 candidates per thread as their number requires.
//           When the candidates are too few, too many, or a segment overflowed its list, it
//           selects exactly from the whole row instead, 8192 - k scores at a time against the
//           running top k held in LDS.
// Wave reductions and scans use DPP lane moves and readlane rather than LDS-routed permutes.
#include "csa_internal.h"
#include "step_project.h"
#include "fold.h"

namespace csa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_BINS = 2048;
constexpr int TK_SEG = 8192;     // scores per segment (E = 8)
constexpr int TK_NS = 4096;      // threshold sample (4 per thread)
constexpr int TK_FINAL = TOPK_FINAL_CAND;   // candidates the final pass holds (E = 8)
constexpr int TK_MAXSEG = 1024;  // segments per row
constexpr int TK_ROW_MAX = 65536; // rows up to this long: one workgroup per query, one launch
constexpr int TK_MAXK = 4096;

struct TopkShared {
  int hist[2][TK_BINS];
  int red_n[TK_WAVES];
  float red_lo[TK_WAVES], red_hi[TK_WAVES];
  uint32_t red_klo[TK_WAVES], red_khi[TK_WAVES];
  int scan[TK_WAVES];
  int sel_bin, sel_above;
};

__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

struct OpAdd { __device__ int operator()(int a, int b) const { return a + b; } };
struct OpMinU { __device__ int operator()(int a, int b) const { return (int)min((uint32_t)a, (uint32_t)b); } };
struct OpMaxU { __device__ int operator()(int a, int b) const { return (int)max((uint32_t)a, (uint32_t)b); } };
struct OpMinF { __device__ int operator()(int a, int b) const { return __float_as_int(fminf(__int_as_float(a), __int_as_float(b))); } };
struct OpMaxF { __device__ int operator()(int a, int b) const { return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b))); } };

__device__ __forceinline__ int wave_sum_i(int v) { return wave_allreduce(v, OpAdd()); }
__device__ __forceinline__ float wave_min_f(float v) { return __int_as_float(wave_allreduce(__float_as_int(v), OpMinF())); }
__device__ __forceinline__ float wave_max_f(float v) { return __int_as_float(wave_allreduce(__float_as_int(v), OpMaxF())); }
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) { return (uint32_t)wave_allreduce((int)v, OpMinU()); }
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) { return (uint32_t)wave_allreduce((int)v, OpMaxU()); }

// Cross-wave reductions of per-wave slots: lane j reads slot j & 15, then each row of 16
// lanes combines them.
__device__ __forceinline__ int slots_sum(const int* v) { return row_allreduce(v[threadIdx.x & 15], OpAdd()); }
__device__ __forceinline__ float slots_min(const float* v) {
  return __int_as_float(row_allreduce(__float_as_int(v[threadIdx.x & 15]), OpMinF()));
}
__device__ __forceinline__ float slots_max(const float* v) {
  return __int_as_float(row_allreduce(__float_as_int(v[threadIdx.x & 15]), OpMaxF()));
}
__device__ __forceinline__ uint32_t slots_min_u(const uint32_t* v) {
  return (uint32_t)row_allreduce((int)v[threadIdx.x & 15], OpMinU());
}
__device__ __forceinline__ uint32_t slots_max_u(const uint32_t* v) {
  return (uint32_t)row_allreduce((int)v[threadIdx.x & 15], OpMaxU());
}

// Wave 0: find the bin d with S(d) >= rem > S(d + 1), S(d) = number of items in bins >= d,
// and publish d and S(d + 1).  Requires 1 <= rem <= S(0).  Lane l first sums bins
// 32l .. 32l + 31 (read in a staggered order so the lanes spread over the LDS banks); a
// suffix scan over the lanes finds the lane whose range holds d, and 32 lanes then scan
// that range in parallel.
template <class SH>
__device__ void find_bin(const int* H, int rem, SH& sh) {
  const int lane = threadIdx.x & 63;
  int own = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) own += H[32 * lane + ((j + lane) & 31)];
  const int incl = wave_incl_scan(own);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  const int suf = total - incl + own;  // items in bins of lanes >= lane
  const int after = suf - own;         // items in bins of higher lanes
  const unsigned long long hit = __ballot(suf >= rem && after < rem);
  const int L = __ffsll(hit) - 1;  // exactly one lane
  const int base = __builtin_amdgcn_readlane(after, L);
  const int j = lane & 31;
  const int h = lane < 32 ? H[32 * L + j] : 0;
  const int pin = wave_incl_scan(h);   // lanes 0..31: bins 32L .. 32L + j
  const int s = __builtin_amdgcn_readlane(pin, 31) - pin + h;  // bins 32L + j .. 32L + 31
  if (lane < 32 && base + s >= rem && base + s - h < rem) {
    sh.sel_bin = 32 * L + j;
    sh.sel_above = base + s - h;
  }
}

// The items a thread holds: E keys with their indices.  A row segment's indices are the
// contiguous run first .. first + E - 1 (valid below V); a merge's come from the lists
// (valid when >= 0).
template <int E>
struct RunItems {
  uint32_t key[E];
  int first, V;
  __device__ int idx(int i) const { return first + i; }
  __device__ bool valid(int i) const { return first + i < V; }
};
template <int E>
struct ListItems {
  uint32_t key[E];
  int id[E];
  __device__ int idx(int i) const { return id[i]; }
  __device__ bool valid(int i) const { return id[i] >= 0; }
};

// Select the k largest valid items of the block (equal keys: lower index first) and write
// their indices in index order to out_idx (keys to out_key when non-null).  Returns the
// number written, min(k, number of valid items).
template <int E, class Items>
__device__ int select_topk(const Items& it, int k, TopkShared& sh, int* out_idx, uint32_t* out_key) {
  const uint32_t (&key)[E] = it.key;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // (a) valid count and score range; both histograms cleared
  int nv = 0;
  float fmn = INFINITY, fmx = -INFINITY;
#pragma unroll
  for (int i = 0; i < E; ++i)
    if (it.valid(i)) {
      ++nv;
      const float f = key_score(key[i]);
      fmn = fminf(fmn, f);
      fmx = fmaxf(fmx, f);
    }
  nv = wave_sum_i(nv);
  fmn = wave_min_f(fmn);
  fmx = wave_max_f(fmx);
  if (lane == 0) { sh.red_n[w] = nv; sh.red_lo[w] = fmn; sh.red_hi[w] = fmx; }
  for (int b = tid; b < TK_BINS; b += TK_THREADS) { sh.hist[0][b] = 0; sh.hist[1][b] = 0; }
  __syncthreads();
  const int nvalid = slots_sum(sh.red_n);
  fmn = slots_min(sh.red_lo);
  fmx = slots_max(sh.red_hi);
  const bool take_all = nvalid <= k;

  // (b) one pass over bins linear in the score; (c) radix passes inside the window.  Each
  // item's bin is computed once and kept packed, two 16-bit bins per register.
  const float range = fmx - fmn;
  const float scale = (range > 0.f && range < INFINITY) ? (float)TK_BINS / range : 0.f;
  constexpr int NB = (E + 1) / 2;
  uint32_t bins[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) bins[j] = 0u;
  auto bin_of = [&](int i) { return (int)((bins[i >> 1] >> (16 * (i & 1))) & 0xffffu); };
  int wbin = TK_BINS;             // window bin (TK_BINS: no window, every valid item taken)
  uint32_t lo = 0u, hi = ~0u;     // key range of the window inside its bin
  int need = 0;                   // items taken from the window, lowest index first
  if (!take_all) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int b = min(TK_BINS - 1, (int)((key_score(key[i]) - fmn) * scale));
      bins[i >> 1] |= (uint32_t)b << (16 * (i & 1));
      if (it.valid(i)) atomicAdd(&sh.hist[0][b], 1);
    }
    __syncthreads();
    if (w == 0) find_bin(sh.hist[0], k, sh);
    __syncthreads();
    wbin = sh.sel_bin;
    int rem = k - sh.sel_above;
    int nwin = sh.hist[0][wbin];
    uint32_t kmn = ~0u, kmx = 0u;
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (it.valid(i) && bin_of(i) == wbin) { kmn = min(kmn, key[i]); kmx = max(kmx, key[i]); }
    kmn = wave_min_u(kmn);
    kmx = wave_max_u(kmx);
    if (lane == 0) { sh.red_klo[w] = kmn; sh.red_khi[w] = kmx; }
    __syncthreads();
    lo = slots_min_u(sh.red_klo);
    hi = slots_max_u(sh.red_khi);
    // Histogram p uses hist[p & 1]; the other one is cleared while wave 0 searches, after
    // every thread has read what it needed from it.  At most 3 passes: each one takes 11
    // bits off the span of the window.
    int p = 1;
    while (lo != hi && rem != nwin) {  // uniform: every operand comes from LDS
      const int shift = max(0, 32 - __clz(hi - lo) - 11);
      int* H = sh.hist[p & 1];
#pragma unroll
      for (int i = 0; i < E; ++i)
        if (it.valid(i) && bin_of(i) == wbin && key[i] >= lo && key[i] <= hi)
          atomicAdd(&H[(key[i] - lo) >> shift], 1);
      __syncthreads();
      if (w == 0) {
        find_bin(H, rem, sh);
      } else {
        int* other = sh.hist[(p + 1) & 1];
        for (int b = tid - 64; b < TK_BINS; b += TK_THREADS - 64) other[b] = 0;
      }
      __syncthreads();
      const int d = sh.sel_bin;
      rem -= sh.sel_above;
      nwin = H[d];
      const uint32_t nlo = lo + ((uint32_t)d << shift);
      hi = min(hi, nlo + ((1u << shift) - 1u));
      lo = nlo;
      ++p;
    }
    need = rem;
  }

  // (d) output slots: above-window items, then the window's lowest-index `need` items
  auto klass = [&](int i) {  // 2: above the window, 1: in the window, 0: not taken
    if (!it.valid(i)) return 0;
    if (take_all) return 2;
    const int b = bin_of(i);
    if (b > wbin || (b == wbin && key[i] > hi)) return 2;
    return (b == wbin && key[i] >= lo) ? 1 : 0;
  };
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int c = klass(i);
    gt += c == 2 ? 1 : 0;
    eq += c == 1 ? 1 : 0;
  }
  // one exclusive block scan of (gt << 16 | eq); block totals stay below 65536
  const int own = (gt << 16) | eq;
  const int x = wave_incl_scan(own);
  if (lane == 63) sh.scan[w] = x;
  __syncthreads();
  // waves ahead of this one
  const int before = row_allreduce((tid & 15) < w ? sh.scan[tid & 15] : 0, OpAdd());
  const int ex = x - own + before;
  int gt_before = ex >> 16, eq_before = ex & 0xffff;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int c = klass(i);
    if (c == 2) {
      const int pos = gt_before + min(eq_before, need);
      out_idx[pos] = it.idx(i);
      if (out_key) out_key[pos] = key[i];
      ++gt_before;
    } else if (c == 1) {
      if (eq_before < need) {
        const int pos = gt_before + eq_before;
        out_idx[pos] = it.idx(i);
        if (out_key) out_key[pos] = key[i];
      }
      ++eq_before;
    }
  }
  return take_all ? nvalid : k;
}

__device__ __forceinline__ int visible(const int32_t* q_seq, const int32_t* q_pos,
                                       const int32_t* n_entries, int m, int q) {
  return max(0, min(q_pos[q] / m, n_entries[q_seq ? q_seq[q] : q]));
}

// A query's row of scores: float32, or (BF) bfloat16 widened exactly to float32.
template <bool BF>
struct ScoreRow {
  const void* p;
  __device__ __forceinline__ float operator[](int e) const {
    if constexpr (BF) return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[e] << 16);
    else return static_cast<const float*>(p)[e];
  }
};
template <bool BF>
__device__ __forceinline__ ScoreRow<BF> score_row(const void* scores, int64_t ld, int q) {
  if constexpr (BF) return {static_cast<const uint16_t*>(scores) + (size_t)q * ld};
  else return {static_cast<const float*>(scores) + (size_t)q * ld};
}

// Level 0: blockIdx.x = query, blockIdx.y = segment of 1024*E scores.
// direct != 0: the segment is the whole row; write the final selection to idx_out [Q][k].
// Otherwise write the segment's candidates to cand_idx/cand_key [Q][nseg][k] (-1 padded).
template <int E, bool BF>
__global__ __launch_bounds__(TK_THREADS) void k_topk_segment(
    const void* __restrict__ scores, int64_t ld, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_entries, int m, int k,
    int direct, int32_t* __restrict__ idx_out, int32_t* __restrict__ cand_idx,
    uint32_t* __restrict__ cand_key) {
  __shared__ TopkShared sh;
  const int q = blockIdx.x, seg = blockIdx.y, nseg = gridDim.y;
  const int V = visible(q_seq, q_pos, n_entries, m, q);
  const int base = seg * TK_THREADS * E;
  int32_t* oidx;
  uint32_t* okey = nullptr;
  if (direct) {
    oidx = idx_out + (size_t)q * k;
  } else {
    oidx = cand_idx + ((size_t)q * nseg + seg) * k;
    okey = cand_key + ((size_t)q * nseg + seg) * k;
  }
  RunItems<E> it;
  it.first = base + threadIdx.x * E;
  it.V = V;
  const int first = it.first;
  const ScoreRow<BF> row = score_row<BF>(scores, ld, q);
  bool loaded = false;
  if constexpr (E % 4 == 0 && !BF) {
    if (first + E <= V && ((ld & 3) == 0)) {
#pragma unroll
      for (int i = 0; i < E; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(row.p) + first + i);
        it.key[i] = score_key(v.x);
        it.key[i + 1] = score_key(v.y);
        it.key[i + 2] = score_key(v.z);
        it.key[i + 3] = score_key(v.w);
      }
      loaded = true;
    }
  }
  if (!loaded) {
    // every load issued (a position past V reads the row's last visible score, or its first),
    // then masked: per-element branches would make each load wait for the one before
    float v[E];
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = row[max(0, min(first + i, V - 1))];
#pragma unroll
    for (int i = 0; i < E; ++i) it.key[i] = first + i < V ? score_key(v[i]) : 0u;
  }
  const int n = select_topk<E>(it, k, sh, oidx, okey);
  for (int i = n + threadIdx.x; i < k; i += TK_THREADS) {
    oidx[i] = -1;
    if (okey) okey[i] = 0u;
  }
}

// Raw float bits u pass iff u - lo <= span (unsigned): exactly the scores whose key is at
// least score_key(t) (-0 equal to +0, NaNs beyond the infinities on their sign's side).
__device__ __forceinline__ void pass_interval(float t, uint32_t& lo, uint32_t& span) {
  uint32_t b = __float_as_uint(t);
  if (b == 0x80000000u) b = 0u;
  if (b != 0u && (b & 0x80000000u) == 0u) {   // t > 0: the positive floats from t up, +NaN
    lo = b;
    span = 0x7fffffffu - b;
  } else {                                     // t <= 0: everything from +NaN down to t
    lo = 0u;
    span = b == 0u ? 0x80000000u : b;
  }
}

// Threshold pass: one workgroup per (query, segment of TK_SEG scores).  Writes the segment's
// scores with keys at or above the threshold key (all valid scores when the row has at most
// TK_FINAL) to cand_idx/cand_key [Q][nseg][cs] in index order, and their count (which may
// exceed cs) to cand_cnt [Q][nseg].
struct FilterArgs {
  const void* scores;     // float32, or bfloat16 (BF)
  int64_t ld;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const int32_t* n_entries;
  int m, k, cs, nseg;
  int spw;                // segments per workgroup (consecutive; one sample and threshold)
  int32_t* cand_idx;
  uint32_t* cand_key;
  int32_t* cand_cnt;
  int32_t* vis;           // [Q] the visible count each query was filtered with
};

// Every workgroup of a row draws the same sample, 64 evenly spaced runs of 64 scores, and
// takes as threshold the lower edge of the histogram bin (2048 bins between the sample's
// extremes) above which about 3k of the row's V scores are expected (at most 3/4 of the final
// pass's TK_FINAL).  Segment layout: wave w reads the run at 512 w, lane l element i at
// 64 i + l (each load one contiguous 256-byte read, a wave's (i, l) order is index order);
// the passing scores are compacted with wave ballots and lane counts below the lane.  Reads
// of a segment start at min(c0, L - TK_SEG), L = max(V, TK_SEG) <= the row stride (these
// rows are longer than TK_SEG), so every read stays in the row; elements outside [c0, V) are
// masked.  A workgroup filters segments seg0 .. seg0 + n - 1 of the row against one threshold
// (the sample is the same for every segment of a row), the next segment's loads in flight
// while one is compacted.
template <bool BF>
__device__ __forceinline__ void topk_filter_body(const FilterArgs& fa, int q, int seg0, int n, TopkShared& sh) {
  const int k = fa.k, cs = fa.cs, nseg = fa.nseg;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int V = visible(fa.q_seq, fa.q_pos, fa.n_entries, fa.m, q);
  const ScoreRow<BF> row = score_row<BF>(fa.scores, fa.ld, q);
  const bool take_all = V <= TK_FINAL;
  const int L = max(V, TK_SEG);
  // the sample first, then the segment, so their latencies overlap
  const int bs = ((int)((int64_t)(tid >> 4) * (L - 64) / 63) & ~3) + 4 * (tid & 15);
  float smp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) smp[i] = row[bs + i];
  const int nlast = min(seg0 + n, nseg) - 1;
  auto seg_base = [&](int seg) { return min(seg * TK_SEG, L - TK_SEG) + 512 * w; };
  float sv[8];
  {
    const int a0 = seg_base(seg0);
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = row[a0 + 64 * i + lane];
  }
  uint32_t lo = 0u, span = 0xffffffffu;   // every score passes
  if (!take_all) {   // uniform
#pragma unroll
    for (int i = 0; i < 4; ++i) smp[i] = key_score(score_key(smp[i]));
    float mn = fminf(fminf(smp[0], smp[1]), fminf(smp[2], smp[3]));
    float mx = fmaxf(fmaxf(smp[0], smp[1]), fmaxf(smp[2], smp[3]));
    mn = wave_min_f(mn);
    mx = wave_max_f(mx);
    if (lane == 0) { sh.red_lo[w] = mn; sh.red_hi[w] = mx; }
    for (int b = tid; b < TK_BINS; b += TK_THREADS) sh.hist[0][b] = 0;
    __syncthreads();
    const float fmn = slots_min(sh.red_lo);
    const float range = slots_max(sh.red_hi) - fmn;
    const float scale = (range > 0.f && range < INFINITY) ? (float)TK_BINS / range : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) atomicAdd(&sh.hist[0][min(TK_BINS - 1, (int)((smp[i] - fmn) * scale))], 1);
    __syncthreads();
    const int target = min(3 * k, TK_FINAL * 3 / 4);
    const int r = (int)min((int64_t)TK_NS, ((int64_t)target * TK_NS + V - 1) / V);
    if (w == 0) find_bin(sh.hist[0], r, sh);
    __syncthreads();
    if (scale > 0.f) pass_interval(fmn + (float)sh.sel_bin / scale, lo, span);
  }
  for (int seg = seg0; seg <= nlast; ++seg) {
    const int c0 = seg * TK_SEG;
    const int a0 = seg_base(seg);
    const int vlo = max(0, c0 - a0), vspan = max(0, min(512, V - a0) - vlo);   // uniform
    bool p[8];
    uint64_t bal[8];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __float_as_uint(sv[i]) - lo <= span && (uint32_t)(64 * i + lane - vlo) < (uint32_t)vspan;
      bal[i] = __ballot(p[i]);
      cnt += __popcll(bal[i]);
    }
    // the passing scores' keys are taken now, so that the next segment can be loaded into sv
    uint32_t kv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kv[i] = score_key(sv[i]);
    if (seg < nlast) {
      const int a1 = seg_base(seg + 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = row[a1 + 64 * i + lane];
    }
    if (lane == 0) sh.scan[w] = cnt;
    __syncthreads();
    const int sw = sh.scan[lane & 15];
    const int before = __builtin_amdgcn_readfirstlane(row_allreduce((lane & 15) < w ? sw : 0, OpAdd()));
    const int total = row_allreduce(sw, OpAdd());   // every lane of the row takes part
    __syncthreads();   // sh.scan is rewritten by the next segment
    int32_t* ci = fa.cand_idx + ((size_t)q * nseg + seg) * cs;
    uint32_t* ck = fa.cand_key + ((size_t)q * nseg + seg) * cs;
    uint32_t base = (uint32_t)before;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (p[i]) {
        const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[i] >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)bal[i], base));
        if (pos < cs) {
          ci[pos] = a0 + 64 * i + lane;
          ck[pos] = kv[i];
        }
      }
      base += (uint32_t)__popcll(bal[i]);
    }
    if (tid == 0) fa.cand_cnt[(size_t)q * nseg + seg] = total;
    if (tid == 0 && seg == 0) fa.vis[q] = V;
  }
}

template <bool BF>
__global__ __launch_bounds__(TK_THREADS) void k_topk_filter(FilterArgs fa) {
  __shared__ TopkShared sh;
  topk_filter_body<BF>(fa, blockIdx.x, blockIdx.y * fa.spw, fa.spw, sh);
}

// The threshold pass and a one-token projection in one launch (they are independent), so the
// projection's weight stream runs beside the filter.  Blocks [0, Q * nseg) filter and then run
// tpb projection units (waves 0 .. tpb - 1, one unit each: units ncar * upb + tpb * b + wave);
// in the rest (the carriers) waves 0 .. upb - 1 run one unit each.  The launch fills the 256
// CUs once, and upb and tpb are chosen so that both kinds of workgroup finish together: each
// CU then streams its share of the weights.
template <bool BF>
__global__ __launch_bounds__(TK_THREADS) void k_topk_filter_project(FilterArgs fa, int Q, ProjectStepArgs pa,
                                                                     int units, int upb, int tpb, int ncar) {
  __shared__ TopkShared sh;
  const int nf = Q * fa.nseg;
  const int b = blockIdx.x, wave = threadIdx.x >> 6;
  if (b < nf) {
    topk_filter_body<BF>(fa, b % Q, b / Q, 1, sh);
    const int u = ncar * upb + tpb * b + wave;
    if (wave < tpb && u < units) project_unit<2>(pa, u);
  } else if (wave < upb) {
    const int u = upb * (b - nf) + wave;
    if (u < units) project_unit<2>(pa, u);
  }
}

// Projection units per workgroup of the combined launch (0: the launch cannot carry them).
int carry_units_per_block(int nf, int units) {
  if (nf >= 256) return 0;
  const int upb = (units + (256 - nf) - 1) / (256 - nf);
  return upb <= TK_WAVES ? upb : 0;
}

// The split of the units between the 256 - nf carriers (upb each) and the nf threshold
// workgroups (tpb each, after their filter).  One CU streams some 25 GB/s, and a threshold
// workgroup's filter takes about 4 us, so a threshold workgroup finishes with the carriers
// when it runs r = 100 KB / (bytes per unit) fewer units (a unit's weights are 2 tiles x 16
// columns x K / PU_SLICES bf16 = 4 K bytes): upb is the smallest count with nf max(0, upb - r)
// + (256 - nf) upb >= units, and tpb the fewest the threshold workgroups then need.
void carry_split(int nf, int units, int K, int* upb, int* tpb) {
  const int ncar = 256 - nf;
  const int r = (int)((25000 + K / 2) / K);
  for (int u = 1; u <= TK_WAVES; ++u) {
    const int t = std::min(TK_WAVES, std::max(0, u - r));
    if ((int64_t)nf * t + (int64_t)ncar * u >= units) {
      *upb = u;
      const int64_t rest = std::max<int64_t>(0, units - (int64_t)ncar * u);
      *tpb = (int)((rest + nf - 1) / nf);
      return;
    }
  }
  *upb = carry_units_per_block(nf, units);
  *tpb = 0;
}

struct FinalShared {
  TopkShared sh;
  int segoff[TK_MAXSEG + 1];
  int r_idx[TK_MAXK];
  uint32_t r_key[TK_MAXK];
};

// The candidates (N <= TK_THREADS * E, in index order) into E items per thread; select k.
template <int E>
__device__ __forceinline__ int final_fast(int q, int nseg, int cs, int N, int k, const int32_t* __restrict__ cand_idx,
                          const uint32_t* __restrict__ cand_key, FinalShared& fs, int32_t* out) {
  const int tid = threadIdx.x;
  ListItems<E> it;
  const int p0 = tid * E;
  int sg = 0;   // segment of p0: the last with segoff <= p0
  for (int step = TK_MAXSEG; step >= 1; step >>= 1)
    if (sg + step <= nseg && fs.segoff[sg + step] <= p0) sg += step;
  // the list positions of the thread's items first, then every load at once (a position
  // past N reads the query's first list slot and is masked): loads in branches would each
  // wait for the one before
  size_t at[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int p = p0 + i;
    while (sg < nseg && fs.segoff[sg + 1] <= p) ++sg;
    const int sc = min(sg, nseg - 1);
    at[i] = p < N ? ((size_t)q * nseg + sc) * cs + (p - fs.segoff[sc]) : (size_t)q * nseg * cs;
  }
  int32_t ci[E];
  uint32_t ck[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    ci[i] = cand_idx[at[i]];
    ck[i] = cand_key[at[i]];
  }
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const bool ok = p0 + i < N;
    it.id[i] = ok ? ci[i] : -1;
    it.key[i] = ok ? ck[i] : 0u;
  }
  return select_topk<E>(it, k, fs.sh, out, nullptr);
}

// Final pass: blockIdx.x = query.  Selects k from the candidate lists, or from the whole row
// when they cannot be trusted (see the file comment), and writes idx_out [Q][k].
struct FinalArgs {
  const void* scores;     // float32, or bfloat16 (BF)
  int64_t ld;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const int32_t* n_entries;
  int m, k, nseg, cs;
  const int32_t* cand_idx;
  const uint32_t* cand_key;
  const int32_t* cand_cnt;
  const int32_t* vis;     // [Q] visible counts from the threshold pass (entry counts may have
                          // moved since, when a fold shares the launch)
  int32_t* idx_out;
};

template <bool BF>
__device__ __forceinline__ void topk_final_body(const FinalArgs& fa, int q, FinalShared& fs) {
  const int64_t ld = fa.ld;
  const int32_t* __restrict__ q_seq = fa.q_seq;
  const int32_t* __restrict__ q_pos = fa.q_pos;
  const int32_t* __restrict__ n_entries = fa.n_entries;
  const int m = fa.m, k = fa.k, nseg = fa.nseg, cs = fa.cs;
  const int32_t* __restrict__ cand_idx = fa.cand_idx;
  const uint32_t* __restrict__ cand_key = fa.cand_key;
  const int32_t* __restrict__ cand_cnt = fa.cand_cnt;
  int32_t* __restrict__ idx_out = fa.idx_out;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int V = fa.vis[q];
  (void)q_seq;
  (void)q_pos;
  (void)n_entries;
  (void)m;
  int32_t* out = idx_out + (size_t)q * k;
  // segment offsets (one segment per thread, nseg <= TK_MAXSEG = TK_THREADS)
  const int c = tid < nseg ? cand_cnt[(size_t)q * nseg + tid] : 0;
  const int x = wave_incl_scan(c);
  if (lane == 63) fs.sh.scan[w] = x;
  const bool over = __syncthreads_or(c > cs) != 0;
  const int sw = fs.sh.scan[tid & 15];
  const int before = row_allreduce((tid & 15) < w ? sw : 0, OpAdd());
  const int N = row_allreduce(sw, OpAdd());
  if (tid < nseg) fs.segoff[tid] = before + x - c;
  if (tid == 0) fs.segoff[nseg] = N;
  __syncthreads();
  int n;
  if (!over && N >= min(k, V) && N <= TK_FINAL) {   // uniform
    if (N <= 2 * TK_THREADS) n = final_fast<2>(q, nseg, cs, N, k, cand_idx, cand_key, fs, out);
    else if (N <= 4 * TK_THREADS) n = final_fast<4>(q, nseg, cs, N, k, cand_idx, cand_key, fs, out);
    else n = final_fast<8>(q, nseg, cs, N, k, cand_idx, cand_key, fs, out);
  } else {
    // exact selection over the whole row: the running top k (in index order, in LDS) plus
    // the next TK_FINAL - k scores, once per chunk
    const ScoreRow<BF> row = score_row<BF>(fa.scores, ld, q);
    const int ch = TK_FINAL - k;
    int nr = 0;
    for (int c0 = 0; c0 < V; c0 += ch) {
      ListItems<8> it;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int p = tid * 8 + i;
        if (p < nr) {
          it.id[i] = fs.r_idx[p];
          it.key[i] = fs.r_key[p];
        } else {
          const int e = c0 + (p - nr);
          const bool ok = p - nr < ch && e < V;
          it.id[i] = ok ? e : -1;
          it.key[i] = ok ? score_key(row[e]) : 0u;
        }
      }
      __syncthreads();   // the running list is read before it is rewritten
      nr = select_topk<8>(it, k, fs.sh, fs.r_idx, fs.r_key);
      __syncthreads();
    }
    for (int i = tid; i < nr; i += TK_THREADS) out[i] = fs.r_idx[i];
    n = nr;
  }
  for (int i = n + tid; i < k; i += TK_THREADS) out[i] = -1;
}

template <bool BF>
__global__ __launch_bounds__(TK_THREADS) void k_topk_final(FinalArgs fa) {
  __shared__ FinalShared fs;
  topk_final_body<BF>(fa, blockIdx.x, fs);
}

// The final pass and a one-token fold in one launch (independent: blocks [0, Q) select, the
// rest fold with 1024-thread blocks, whose columns past c hold zeros).
// EK: the fold projects CSA2 index keys from the entries (LDS for the entry row and key).
template <bool BF, bool EK>
__global__ __launch_bounds__(TK_THREADS) void k_topk_final_fold(FinalArgs fa, int Q, FoldArgs fo, int fx) {
  __shared__ FinalShared fs;
  __shared__ float red[TK_WAVES];
  __shared__ float ybuf[EK ? 512 : 1], kbuf[EK ? 512 : 1];
  __shared__ float pnew[FOLD_PNEW];
  const int b = blockIdx.x;
  if (b < Q) topk_final_body<BF>(fa, b, fs);
  else fold_block<TK_WAVES, true>(fo, (b - Q) % fx, (b - Q) / fx, red, EK ? ybuf : nullptr, EK ? kbuf : nullptr, pnew);
}

// ----------------------------------------------------------------------- one-launch rows
// Rows of up to TK_ROW_MAX scores: one workgroup per query draws a sample of the row, takes a
// threshold from it (as the filter pass does), streams the row in TK_SEG-score chunks keeping
// the scores at or above the threshold in LDS (in index order), and selects k from them; the
// same whole-row fallback covers the cases the threshold cannot.
//
// Chunk layout: wave w holds the run of 512 scores at 512 w, lane l element i at 64 i + l, so
// each load instruction is one contiguous 256-byte read and a wave's (i, l) order is index
// order.  A wave's passing scores are compacted with ballots: one compare per score, the
// write position from the ballot's lane count below the lane.
struct RowShared {
  TopkShared sh;
  int c_idx[TK_FINAL + 1];        // +1: the spare slot writes past TK_FINAL land in
  uint32_t c_key[TK_FINAL + 1];   // raw score bits in the filter phase, keys in the fallback
};

struct RowArgs {
  const void* scores;     // float32, or bfloat16 (BF)
  int64_t ld;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const int32_t* n_entries;
  int m, k;
  int32_t* idx_out;
};

template <int E>
__device__ __forceinline__ int select_lds(RowShared& rs, int N, int k, int32_t* out) {
  ListItems<E> it;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int p = threadIdx.x * E + i;
    it.id[i] = p < N ? rs.c_idx[p] : -1;
    it.key[i] = p < N ? score_key(__uint_as_float(rs.c_key[p])) : 0u;
  }
  return select_topk<E>(it, k, rs.sh, out, nullptr);
}

// One chunk of the row (scores v, wave w's run starting at a0 = s + 512 w) into the LDS
// candidate list at N.  Element e = a0 + 64 i + lane counts when c0 <= e < V (FULL: all do).
template <bool FULL>
__device__ __forceinline__ void row_chunk(const float (&v)[8], int a0, int c0, int V, uint32_t lo,
                                          uint32_t span, int& N, RowShared& rs, int w, int lane) {
  bool p[8];
  uint64_t bal[8];
  int cnt = 0;
  const int vlo = max(0, c0 - a0), vspan = max(0, min(512, V - a0) - vlo);   // uniform
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = __float_as_uint(v[i]) - lo <= span;
    if constexpr (!FULL) p[i] = p[i] && (uint32_t)(64 * i + lane - vlo) < (uint32_t)vspan;
    bal[i] = __ballot(p[i]);
    cnt += __popcll(bal[i]);
  }
  if (lane == 0) rs.sh.scan[w] = cnt;
  __syncthreads();
  const int sw = rs.sh.scan[lane & 15];
  const int before = __builtin_amdgcn_readfirstlane(row_allreduce((lane & 15) < w ? sw : 0, OpAdd()));
  const int total = __builtin_amdgcn_readfirstlane(row_allreduce(sw, OpAdd()));
  uint32_t base = (uint32_t)(N + before);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (p[i]) {
      const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[i] >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal[i], base));
      const int slot = min(pos, TK_FINAL);   // past TK_FINAL: the count overflows, the fallback runs
      rs.c_idx[slot] = a0 + 64 * i + lane;
      rs.c_key[slot] = __float_as_uint(v[i]);
    }
    base += (uint32_t)__popcll(bal[i]);
  }
  N += total;
  __syncthreads();   // sh.scan is rewritten by the next chunk
}

template <bool BF>
__device__ __forceinline__ void topk_row_body(const RowArgs& ra, int q, RowShared& rs) {
  TopkShared& sh = rs.sh;
  const int k = ra.k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int V = visible(ra.q_seq, ra.q_pos, ra.n_entries, ra.m, q);
  const ScoreRow<BF> row = score_row<BF>(ra.scores, ra.ld, q);
  int32_t* out = ra.idx_out + (size_t)q * k;
  const bool take_all = V <= TK_FINAL;
  // Reads of chunk c0 start at min(c0, L - TK_SEG), L = max(V, TK_SEG) <= the row stride (the
  // rows here are longer than TK_SEG), so every read stays in the row; the last chunk's run is
  // moved back to end at V and its elements below c0 are masked.
  const int L = max(V, TK_SEG);
  // the sample first (64 evenly spaced runs of 64; rows of at most TK_FINAL take every score
  // and ignore it), then RG chunks at once, so the latencies overlap
  const int bs = ((int)((int64_t)(tid >> 4) * (L - 64) / 63) & ~3) + 4 * (tid & 15);
  float smp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) smp[i] = row[bs + i];
  constexpr int RG = 4;
  float sv[RG][8];
  auto load_group = [&](int g0) {
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const int e0 = min(g0 + j * TK_SEG, L - TK_SEG) + 512 * w + lane;
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[j][i] = row[e0 + 64 * i];
    }
  };
  load_group(0);
  // the threshold: scores at or above t pass (lo = 0, span = ~0: every score)
  uint32_t lo = 0u, span = 0xffffffffu;
  if (!take_all) {   // uniform
#pragma unroll
    for (int i = 0; i < 4; ++i) smp[i] = key_score(score_key(smp[i]));
    float mn = fminf(fminf(smp[0], smp[1]), fminf(smp[2], smp[3]));
    float mx = fmaxf(fmaxf(smp[0], smp[1]), fmaxf(smp[2], smp[3]));
    mn = wave_min_f(mn);
    mx = wave_max_f(mx);
    if (lane == 0) { sh.red_lo[w] = mn; sh.red_hi[w] = mx; }
    for (int b = tid; b < TK_BINS; b += TK_THREADS) sh.hist[0][b] = 0;
    __syncthreads();
    const float fmn = slots_min(sh.red_lo);
    const float range = slots_max(sh.red_hi) - fmn;
    const float scale = (range > 0.f && range < INFINITY) ? (float)TK_BINS / range : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) atomicAdd(&sh.hist[0][min(TK_BINS - 1, (int)((smp[i] - fmn) * scale))], 1);
    __syncthreads();
    // samples at or above the threshold: about 3k (at most 3/4 of TK_FINAL) of the row's V
    // scores are then expected to pass
    const int target = min(3 * k, TK_FINAL * 3 / 4);
    const int r = (int)min((int64_t)TK_NS, ((int64_t)target * TK_NS + V - 1) / V);
    if (w == 0) find_bin(sh.hist[0], r, sh);
    __syncthreads();
    if (scale > 0.f) pass_interval(fmn + (float)sh.sel_bin / scale, lo, span);
  }
  // the row, chunk by chunk: passing scores go to LDS in index order
  int N = 0;   // uniform
  for (int g0 = 0; g0 < V; g0 += RG * TK_SEG) {
    if (g0 > 0) load_group(g0);
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const int c0 = g0 + j * TK_SEG;
      if (c0 >= V) break;   // uniform
      const int s = min(c0, L - TK_SEG);
      if (s == c0 && c0 + TK_SEG <= V) row_chunk<true>(sv[j], s + 512 * w, c0, V, lo, span, N, rs, w, lane);
      else row_chunk<false>(sv[j], s + 512 * w, c0, V, lo, span, N, rs, w, lane);
    }
  }
  int n;
  if (N >= min(k, V) && N <= TK_FINAL) {   // uniform
    if (N <= 2 * TK_THREADS) n = select_lds<2>(rs, N, k, out);
    else if (N <= 4 * TK_THREADS) n = select_lds<4>(rs, N, k, out);
    else n = select_lds<8>(rs, N, k, out);
  } else {
    // exact selection over the whole row: the running top k (in index order, in LDS) plus
    // the next TK_FINAL - k scores, once per chunk
    const int ch = TK_FINAL - k;
    int nr = 0;
    for (int c0 = 0; c0 < V; c0 += ch) {
      ListItems<8> it;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int p = tid * 8 + i;
        if (p < nr) {
          it.id[i] = rs.c_idx[p];
          it.key[i] = rs.c_key[p];
        } else {
          const int e = c0 + (p - nr);
          const bool ok = p - nr < ch && e < V;
          it.id[i] = ok ? e : -1;
          it.key[i] = ok ? score_key(row[e]) : 0u;
        }
      }
      __syncthreads();   // the running list is read before it is rewritten
      nr = select_topk<8>(it, k, sh, rs.c_idx, rs.c_key);
      __syncthreads();
    }
    for (int i = tid; i < nr; i += TK_THREADS) out[i] = rs.c_idx[i];
    n = nr;
  }
  for (int i = n + tid; i < k; i += TK_THREADS) out[i] = -1;
}

template <bool BF>
__global__ __launch_bounds__(TK_THREADS) void k_topk_row(RowArgs ra) {
  __shared__ RowShared rs;
  topk_row_body<BF>(ra, blockIdx.x, rs);
}

int items_E(int n) {
  int E = 1;
  while (E * TK_THREADS < n) E *= 2;
  return E;
}

int filter_cap(int k) { return std::min(TK_SEG, std::max(1024, 4 * k)); }

}  // namespace

int32_t topk_max_visible(const csa_dims& d) {
  if (d.top_k <= 0 || d.top_k > TK_MAXK) return 0;
  return TK_SEG * TK_MAXSEG;
}

size_t topk_workspace_bytes(const csa_dims& d, int32_t Q, int32_t cap) {
  return cap <= TK_ROW_MAX ? 0 : topk_filter_workspace_bytes(d, Q, cap);
}

size_t topk_filter_workspace_bytes(const csa_dims& d, int32_t Q, int32_t cap) {
  if (cap <= TK_SEG) return 0;
  const size_t nseg = (size_t)(cap + TK_SEG - 1) / TK_SEG;
  const size_t cs = (size_t)filter_cap(d.top_k);
  return (size_t)Q * nseg * (cs * (sizeof(int32_t) + sizeof(uint32_t)) + sizeof(int32_t)) +
         (size_t)Q * sizeof(int32_t);
}

bool topk_can_carry(const csa_cache& c) { return c.cap > TK_SEG; }

// Only while the threshold and projection workgroups (1024 threads, one per CU) all fit on
// the 256 CUs at once: beyond that the carried step only lengthens the pass.
bool topk_can_carry_step(const csa_cache& c, int32_t Q, int32_t step_units) {
  if (!topk_can_carry(c)) return false;
  const int64_t nf = (int64_t)Q * ((c.cap + TK_SEG - 1) / TK_SEG);
  return nf < 256 && carry_units_per_block((int)nf, step_units) > 0;
}

template <bool BF>
hipError_t launch_topk_t(const csa_dims& d, const csa_cache& c, const int32_t* q_seq,
                         const int32_t* q_pos, int32_t Q, const void* scores, int64_t ld,
                         int32_t* idx, void* ws, hipStream_t s, const ProjectStepArgs* step,
                         const FoldArgs* fold) {
  const int k = d.top_k;
  if (c.cap <= TK_SEG) {
    if (step || fold) return hipErrorInvalidValue;   // the carrying passes exist only for long rows
#define TK_DIRECT(EE)                                                                          \
  hipLaunchKernelGGL((k_topk_segment<EE, BF>), dim3(Q, 1), dim3(TK_THREADS), 0, s, scores, ld, q_seq, \
                     q_pos, c.n_entries, d.m, k, 1, idx, nullptr, nullptr)
    switch (items_E(c.cap)) {
      case 1: TK_DIRECT(1); break;
      case 2: TK_DIRECT(2); break;
      case 4: TK_DIRECT(4); break;
      default: TK_DIRECT(8); break;
    }
#undef TK_DIRECT
    return hipGetLastError();
  }
  if (c.cap <= TK_ROW_MAX && !step && !fold) {
    const RowArgs ra{scores, ld, q_seq, q_pos, c.n_entries, d.m, k, idx};
    hipLaunchKernelGGL(k_topk_row<BF>, dim3(Q), dim3(TK_THREADS), 0, s, ra);
    return hipGetLastError();
  }
  const int nseg = (c.cap + TK_SEG - 1) / TK_SEG;
  const int cs = filter_cap(k);
  int32_t* ci = (int32_t*)ws;
  uint32_t* ck = (uint32_t*)(ci + (size_t)Q * nseg * cs);
  int32_t* cc = (int32_t*)(ck + (size_t)Q * nseg * cs);
  int32_t* fvis = cc + (size_t)Q * nseg;   // the counts the threshold pass filtered with
  // segments per threshold workgroup: one while that still leaves a few workgroups per CU
  // (decode), four on long prefill batches (the sample and its histogram are then taken once
  // per four segments)
  const int spw = (int64_t)Q * nseg >= 16 * 256 ? 4 : 1;
  const FilterArgs fa{scores, ld, q_seq, q_pos, c.n_entries, d.m, k, cs, nseg, spw, ci, ck, cc, fvis};
  if (step) {
    const int units = project_units(step->NP, step->M, 2);
    if (carry_units_per_block(Q * nseg, units) == 0) return hipErrorInvalidValue;
    int upb, tpb;
    carry_split(Q * nseg, units, step->K, &upb, &tpb);
    // carriers needed once the threshold workgroups have taken their share
    const int ncar = (int)std::min<int64_t>(256 - Q * nseg, ((int64_t)units + upb - 1) / upb);
    hipLaunchKernelGGL(k_topk_filter_project<BF>, dim3(Q * nseg + ncar), dim3(TK_THREADS), 0, s,
                       fa, Q, *step, units, upb, tpb, ncar);
  } else {
    hipLaunchKernelGGL(k_topk_filter<BF>, dim3(Q, (nseg + spw - 1) / spw), dim3(TK_THREADS), 0, s, fa);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const FinalArgs fin{scores, ld, q_seq, q_pos, c.n_entries, d.m, k, nseg, cs, ci, ck, cc, fvis, idx};
  if (fold) {
    if (!fold->part) return hipErrorInvalidValue;   // the carried fold is a one-token step's
    const int fx = fold_grid_x(*fold);
    if (fold->keys_entry)
      hipLaunchKernelGGL((k_topk_final_fold<BF, true>), dim3(Q + fx * c.B), dim3(TK_THREADS), 0, s, fin, Q, *fold, fx);
    else
      hipLaunchKernelGGL((k_topk_final_fold<BF, false>), dim3(Q + fx * c.B), dim3(TK_THREADS), 0, s, fin, Q, *fold, fx);
  } else {
    hipLaunchKernelGGL(k_topk_final<BF>, dim3(Q), dim3(TK_THREADS), 0, s, fin);
  }
  return hipGetLastError();
}

hipError_t launch_topk_final_lists(const csa_dims& d, const csa_cache& c, int32_t Q,
                                   const float* scores, int64_t ld, const CandLists& cl,
                                   int32_t* idx, hipStream_t s) {
  if (cl.nseg < 1 || cl.nseg > TK_MAXSEG || d.top_k > TK_MAXK) return hipErrorInvalidValue;
  const FinalArgs fin{scores, ld, nullptr, nullptr, c.n_entries, d.m, d.top_k, cl.nseg, cl.cs,
                      cl.idx, cl.key, cl.cnt, cl.vis, idx};
  hipLaunchKernelGGL(k_topk_final<false>, dim3(Q), dim3(TK_THREADS), 0, s, fin);
  return hipGetLastError();
}

hipError_t launch_topk(const csa_dims& d, const csa_cache& c, const int32_t* q_seq,
                       const int32_t* q_pos, int32_t Q, const void* scores, int64_t ld,
                       int32_t* idx, void* ws, hipStream_t s, const ProjectStepArgs* step,
                       const FoldArgs* fold) {
  // the MXFP4 indexer path scores in bfloat16
  if (d.idx_fmt == CSA_FMT_MXFP4) return launch_topk_t<true>(d, c, q_seq, q_pos, Q, scores, ld, idx, ws, s, step, fold);
  return launch_topk_t<false>(d, c, q_seq, q_pos, Q, scores, ld, idx, ws, s, step, fold);
}

}  // namespace csa
