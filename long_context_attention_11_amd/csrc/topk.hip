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
// Rows of up to 8192 scores take one workgroup and one launch.  Longer rows are cut into
// 8192-score segments; each keeps its own top k (a superset of its share of the answer
// under the same total order), and a merge level selects from the candidate lists, which
// stay in index order.
#include "csa_internal.h"

namespace csa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_BINS = 2048;
constexpr int TK_SEG = 8192;     // scores per segment (E = 8)
constexpr int TK_MERGE = 8192;   // candidates one merge workgroup takes (E <= 8)

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

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_min_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// Cross-wave reductions of per-wave slots: lane j reads slot j & 15, then 16 lanes combine.
__device__ __forceinline__ int slots_sum(const int* v) {
  int x = v[threadIdx.x & 15];
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ float slots_min(const float* v) {
  float x = v[threadIdx.x & 15];
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x = fminf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float slots_max(const float* v) {
  float x = v[threadIdx.x & 15];
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ uint32_t slots_min_u(const uint32_t* v) {
  uint32_t x = v[threadIdx.x & 15];
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x = min(x, (uint32_t)__shfl_xor((int)x, o, 64));
  return x;
}
__device__ __forceinline__ uint32_t slots_max_u(const uint32_t* v) {
  uint32_t x = v[threadIdx.x & 15];
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o, 64));
  return x;
}

// Wave 0: find the bin d with S(d) >= rem > S(d + 1), S(d) = number of items in bins >= d,
// and publish d and S(d + 1).  Requires 1 <= rem <= S(0).  Lane l first sums bins
// 32l .. 32l + 31 (read in a staggered order so the lanes spread over the LDS banks); a
// suffix scan over the lanes finds the lane whose range holds d, and 32 lanes then scan
// that range in parallel.
__device__ void find_bin(const int* H, int rem, TopkShared& sh) {
  const int lane = threadIdx.x & 63;
  int own = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) own += H[32 * lane + ((j + lane) & 31)];
  int suf = own;  // inclusive suffix sum over lanes >= lane
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_down(suf, o, 64);
    if (lane + o < 64) suf += y;
  }
  const int after = suf - own;  // items in bins of higher lanes
  const unsigned long long hit = __ballot(suf >= rem && after < rem);
  const int L = __ffsll(hit) - 1;  // exactly one lane
  const int base = __shfl(after, L, 64);
  const int j = lane & 31;
  const int h = H[32 * L + j];
  int s = h;  // items in bins 32L + j .. 32L + 31
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    const int y = __shfl_down(s, o, 64);
    if (j + o < 32) s += y;
  }
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
  int x = (gt << 16) | eq;
  const int own = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.scan[w] = x;
  __syncthreads();
  int before = (threadIdx.x & 15) < w ? sh.scan[threadIdx.x & 15] : 0;  // waves ahead of this one
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) before += __shfl_xor(before, o, 64);
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
  return max(0, min(q_pos[q] / m, n_entries[q_seq[q]]));
}

// Level 0: blockIdx.x = query, blockIdx.y = segment of 1024*E scores.
// direct != 0: the segment is the whole row; write the final selection to idx_out [Q][k].
// Otherwise write the segment's candidates to cand_idx/cand_key [Q][nseg][k] (-1 padded).
template <int E>
__global__ __launch_bounds__(TK_THREADS) void k_topk_segment(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ q_seq,
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
  const float* row = scores + (size_t)q * ld;
  bool loaded = false;
  if constexpr (E % 4 == 0) {
    if (first + E <= V && ((ld & 3) == 0)) {
#pragma unroll
      for (int i = 0; i < E; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(row + first + i);
        it.key[i] = score_key(v.x);
        it.key[i + 1] = score_key(v.y);
        it.key[i + 2] = score_key(v.z);
        it.key[i + 3] = score_key(v.w);
      }
      loaded = true;
    }
  }
  if (!loaded) {
#pragma unroll
    for (int i = 0; i < E; ++i) it.key[i] = first + i < V ? score_key(row[first + i]) : 0u;
  }
  const int n = select_topk<E>(it, k, sh, oidx, okey);
  for (int i = n + threadIdx.x; i < k; i += TK_THREADS) {
    oidx[i] = -1;
    if (okey) okey[i] = 0u;
  }
}

// Merge level: blockIdx.x = query, blockIdx.y = group of G consecutive candidate lists
// (of nlist per query, k each, in index order).  direct != 0: one group covers every list;
// write the final selection.  Otherwise write one list of k per group.
template <int E>
__global__ __launch_bounds__(TK_THREADS) void k_topk_merge(
    const int32_t* __restrict__ in_idx, const uint32_t* __restrict__ in_key, int nlist, int G,
    int k, int direct, int32_t* __restrict__ idx_out, int32_t* __restrict__ out_idx,
    uint32_t* __restrict__ out_key) {
  __shared__ TopkShared sh;
  const int q = blockIdx.x, grp = blockIdx.y, ngrp = gridDim.y;
  const int l0 = grp * G, l1 = min(nlist, l0 + G);
  const int n = (l1 - l0) * k;
  const int32_t* ci = in_idx + ((size_t)q * nlist + l0) * k;
  const uint32_t* ck = in_key + ((size_t)q * nlist + l0) * k;
  ListItems<E> it;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int p = threadIdx.x * E + i;
    it.id[i] = p < n ? ci[p] : -1;
    it.key[i] = it.id[i] >= 0 ? ck[p] : 0u;
  }
  int32_t* oidx;
  uint32_t* okey = nullptr;
  if (direct) {
    oidx = idx_out + (size_t)q * k;
  } else {
    oidx = out_idx + ((size_t)q * ngrp + grp) * k;
    okey = out_key + ((size_t)q * ngrp + grp) * k;
  }
  const int cnt = select_topk<E>(it, k, sh, oidx, okey);
  for (int i = cnt + threadIdx.x; i < k; i += TK_THREADS) {
    oidx[i] = -1;
    if (okey) okey[i] = 0u;
  }
}

int items_E(int n) {
  int E = 1;
  while (E * TK_THREADS < n) E *= 2;
  return E;
}

// One selection tree: segments of TK_SEG scores, then merges of up to TK_MERGE candidates.
struct TopkPlan {
  int nseg;        // level-0 segments (0: the whole row in one direct workgroup)
  int seg_E;
  int levels;      // merge levels after level 0
};

TopkPlan plan_topk(int k, int cap) {
  TopkPlan p{0, items_E(cap), 0};
  if (cap <= TK_SEG) return p;
  p.nseg = (cap + TK_SEG - 1) / TK_SEG;
  p.seg_E = TK_SEG / TK_THREADS;
  int lists = p.nseg;
  const int G = std::max(2, TK_MERGE / k);
  while (true) {
    ++p.levels;
    if ((long)lists * k <= TK_MERGE) break;
    lists = (lists + G - 1) / G;
  }
  return p;
}

#define TK_SEG_LAUNCH(EE, grid, direct, out_idx, cidx, ckey)                                     \
  hipLaunchKernelGGL((k_topk_segment<EE>), grid, dim3(TK_THREADS), 0, s, scores, ld, q_seq, q_pos, \
                     c.n_entries, d.m, k, direct, out_idx, cidx, ckey)
#define TK_MERGE_LAUNCH(EE, grid, group)                                                          \
  hipLaunchKernelGGL((k_topk_merge<EE>), grid, dim3(TK_THREADS), 0, s, in_i, in_k, lists, group, k, \
                     direct, idx, out_i, out_k)

}  // namespace

int32_t topk_max_visible(const csa_dims& d) {
  if (d.top_k <= 0 || 2 * d.top_k > TK_MERGE) return 0;
  return INT32_MAX / 2;
}

size_t topk_workspace_bytes(const csa_dims& d, int32_t Q, int32_t cap) {
  const TopkPlan p = plan_topk(d.top_k, cap);
  if (p.nseg == 0) return 0;
  // two ping-pong candidate buffers, the first sized for level 0
  const int G = std::max(2, TK_MERGE / d.top_k);
  const size_t lists1 = (size_t)(p.nseg + G - 1) / G;
  const size_t per = (size_t)Q * d.top_k * (sizeof(int32_t) + sizeof(uint32_t));
  return per * ((size_t)p.nseg + lists1);
}

hipError_t launch_topk(const csa_dims& d, const csa_cache& c, const int32_t* q_seq,
                       const int32_t* q_pos, int32_t Q, const float* scores, int64_t ld,
                       int32_t* idx, void* ws, hipStream_t s) {
  const int k = d.top_k;
  const TopkPlan p = plan_topk(k, c.cap);
  if (p.nseg == 0) {
    switch (p.seg_E) {
      case 1: TK_SEG_LAUNCH(1, dim3(Q, 1), 1, idx, nullptr, nullptr); break;
      case 2: TK_SEG_LAUNCH(2, dim3(Q, 1), 1, idx, nullptr, nullptr); break;
      case 4: TK_SEG_LAUNCH(4, dim3(Q, 1), 1, idx, nullptr, nullptr); break;
      default: TK_SEG_LAUNCH(8, dim3(Q, 1), 1, idx, nullptr, nullptr); break;
    }
    return hipGetLastError();
  }
  const int G = std::max(2, TK_MERGE / k);
  const size_t lists1 = (size_t)(p.nseg + G - 1) / G;
  int32_t* bufA_i = (int32_t*)ws;
  uint32_t* bufA_k = (uint32_t*)(bufA_i + (size_t)Q * p.nseg * k);
  int32_t* bufB_i = (int32_t*)(bufA_k + (size_t)Q * p.nseg * k);
  uint32_t* bufB_k = (uint32_t*)(bufB_i + (size_t)Q * lists1 * k);
  TK_SEG_LAUNCH(8, dim3(Q, p.nseg), 0, idx, bufA_i, bufA_k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int lists = p.nseg;
  const int32_t* in_i = bufA_i;
  const uint32_t* in_k = bufA_k;
  bool in_A = true;
  for (int lev = 0; lev < p.levels; ++lev) {
    const int direct = (long)lists * k <= TK_MERGE ? 1 : 0;
    const int groups = direct ? 1 : (lists + G - 1) / G;
    const int per_group = direct ? lists : G;
    int32_t* out_i = in_A ? bufB_i : bufA_i;
    uint32_t* out_k = in_A ? bufB_k : bufA_k;
    switch (items_E(per_group * k)) {
      case 1: TK_MERGE_LAUNCH(1, dim3(Q, groups), per_group); break;
      case 2: TK_MERGE_LAUNCH(2, dim3(Q, groups), per_group); break;
      case 4: TK_MERGE_LAUNCH(4, dim3(Q, groups), per_group); break;
      default: TK_MERGE_LAUNCH(8, dim3(Q, groups), per_group); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess || direct) return e;
    lists = groups;
    in_i = out_i;
    in_k = out_k;
    in_A = !in_A;
  }
  return hipGetLastError();
}

}  // namespace csa
