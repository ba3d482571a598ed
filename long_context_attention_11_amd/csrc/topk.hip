// Per-query top-k selection for gfx950 (reading notes "DeepSeekV4技术报告阅读笔记" §2.3.2
// eq. 17: keep the entries whose index score is among the k largest).
//
// Keys are the scores mapped to order-preserving uint32 (-0 counts as +0).  The selection is
// exact: the k-th largest key T is found by a radix select (digits of 11, 11 and 10 bits,
// LDS histograms), every key > T is taken, and of the keys == T the lowest indices fill the
// remaining slots.  Output indices are in increasing order, padded with -1.
//
// One workgroup of 1024 threads holds up to 1024*E items in registers, thread t holding a
// contiguous run, so thread order is index order and in-order compaction is one block scan.
// Rows longer than 4096 are cut into segments of 4096; each segment keeps its own top-k (a
// superset of its share of the global top-k under the same total order).  Merge levels then
// take groups of candidate lists (up to 16384 candidates per workgroup) down to one list.
// Every list stays in index order, so the final one is the answer, already sorted.
#include "csa_internal.h"

namespace csa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_DIRECT_MAX = 4096;  // rows up to this length: one workgroup, one launch
constexpr int TK_SEG0 = 4096;        // scores per level-0 segment (E = 4)
constexpr int TK_MERGE = 16384;      // candidates one merge workgroup takes (E <= 16)

struct TopkShared {
  int hist[2048];
  int scan[32];
  int sel_digit;
  int sel_gt;
};

// Exclusive scan of one int per thread across the 1024-thread block; returns the exclusive
// prefix and writes the total to *total.
__device__ int block_excl_scan(int v, int* scan, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) scan[w] = x;
  __syncthreads();
  if (w == 0) {
    int s = lane < 16 ? scan[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    if (lane < 16) scan[16 + lane] = s;
  }
  __syncthreads();
  const int before = w > 0 ? scan[16 + w - 1] : 0;
  *total = scan[16 + 15];
  return before + x - v;
}

// Select the top k of the valid items held by the block; write them in index order to
// out_idx[0..) (and out_key if non-null); return the count written (min(k, valid)).
template <int E>
__device__ int block_select(const uint32_t (&key)[E], const int (&idx)[E], const bool (&valid)[E],
                            int k, TopkShared& sh, int* out_idx, uint32_t* out_key) {
  int nv_local = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) nv_local += valid[i] ? 1 : 0;
  int nvalid;
  (void)block_excl_scan(nv_local, sh.scan, &nvalid);

  uint32_t T = 0u;
  int need = 0;
  const bool take_all = nvalid <= k;
  if (!take_all) {
    uint32_t prefix = 0u, pmask = 0u;
    int remaining = k;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const int sh_ = shifts[p], nb = 1 << widths[p];
      const uint32_t dmask = (uint32_t)nb - 1u;
      for (int b = threadIdx.x; b < 2048; b += TK_THREADS) sh.hist[b] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < E; ++i)
        if (valid[i] && (key[i] & pmask) == prefix) atomicAdd(&sh.hist[(key[i] >> sh_) & dmask], 1);
      __syncthreads();
      // suffix counts: S(d) = #items with digit >= d.  Thread t owns digits 2t, 2t+1.
      const int d0 = 2 * threadIdx.x;
      int h0 = d0 < nb ? sh.hist[d0] : 0, h1 = d0 + 1 < nb ? sh.hist[d0 + 1] : 0;
      int tot;
      int ex = block_excl_scan(h0 + h1, sh.scan, &tot);
      const int S0 = tot - ex;  // digits >= d0
      const int S1 = S0 - h0;   // digits >= d0 + 1
      const int S2 = S1 - h1;   // digits >= d0 + 2
      if (d0 < nb) {
        if (S0 >= remaining && S1 < remaining) { sh.sel_digit = d0; sh.sel_gt = S1; }
        if (d0 + 1 < nb && S1 >= remaining && S2 < remaining) { sh.sel_digit = d0 + 1; sh.sel_gt = S2; }
      }
      __syncthreads();
      const int dsel = sh.sel_digit;
      remaining -= sh.sel_gt;
      prefix |= (uint32_t)dsel << sh_;
      pmask |= dmask << sh_;
      __syncthreads();
    }
    T = prefix;
    need = remaining;  // how many items equal to T are taken (lowest indices first)
  }
  int eq_local = 0;
  if (!take_all) {
#pragma unroll
    for (int i = 0; i < E; ++i) eq_local += (valid[i] && key[i] == T) ? 1 : 0;
  }
  int eq_total;
  int eq_before = block_excl_scan(eq_local, sh.scan, &eq_total);
  bool sel[E];
  int nsel = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    bool s;
    if (take_all) {
      s = valid[i];
    } else if (valid[i] && key[i] > T) {
      s = true;
    } else if (valid[i] && key[i] == T) {
      s = eq_before < need;
      ++eq_before;
    } else {
      s = false;
    }
    sel[i] = s;
    nsel += s ? 1 : 0;
  }
  int total;
  int pos = block_excl_scan(nsel, sh.scan, &total);
#pragma unroll
  for (int i = 0; i < E; ++i) {
    if (sel[i]) {
      out_idx[pos] = idx[i];
      if (out_key) out_key[pos] = key[i];
      ++pos;
    }
  }
  return total;
}

__device__ __forceinline__ int visible(const int32_t* q_seq, const int32_t* q_pos,
                                       const int32_t* n_entries, int m, int q) {
  return max(0, min(q_pos[q] / m, n_entries[q_seq[q]]));
}

// Level 0: blockIdx.x = query, blockIdx.y = segment of E*1024 scores.
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
  uint32_t key[E];
  int idx[E];
  bool valid[E];
  const int first = base + threadIdx.x * E;
  const float* row = scores + (size_t)q * ld;
  bool loaded = false;
  if constexpr (E % 4 == 0) {
    if (first + E <= V && ((ld & 3) == 0)) {
#pragma unroll
      for (int i = 0; i < E; i += 4) {
        float4 v = *reinterpret_cast<const float4*>(row + first + i);
        key[i] = score_key(v.x);
        key[i + 1] = score_key(v.y);
        key[i + 2] = score_key(v.z);
        key[i + 3] = score_key(v.w);
      }
#pragma unroll
      for (int i = 0; i < E; ++i) { idx[i] = first + i; valid[i] = true; }
      loaded = true;
    }
  }
  if (!loaded) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      idx[i] = first + i;
      valid[i] = idx[i] < V;
      key[i] = valid[i] ? score_key(row[idx[i]]) : 0u;
    }
  }
  const int n = block_select<E>(key, idx, valid, k, sh, oidx, okey);
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
  uint32_t key[E];
  int idx[E];
  bool valid[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int p = threadIdx.x * E + i;
    idx[i] = p < n ? ci[p] : -1;
    valid[i] = idx[i] >= 0;
    key[i] = valid[i] ? ck[p] : 0u;
  }
  int32_t* oidx;
  uint32_t* okey = nullptr;
  if (direct) {
    oidx = idx_out + (size_t)q * k;
  } else {
    oidx = out_idx + ((size_t)q * ngrp + grp) * k;
    okey = out_key + ((size_t)q * ngrp + grp) * k;
  }
  const int cnt = block_select<E>(key, idx, valid, k, sh, oidx, okey);
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

// One selection tree: segments of TK_SEG0 scores, then merges of up to TK_MERGE candidates.
struct TopkPlan {
  int nseg;        // level-0 segments (0: one direct segment)
  int seg_E;
  int levels;      // merge levels after level 0
};

TopkPlan plan_topk(int k, int cap) {
  TopkPlan p{0, items_E(cap), 0};
  if (cap <= TK_DIRECT_MAX) return p;
  p.nseg = (cap + TK_SEG0 - 1) / TK_SEG0;
  p.seg_E = TK_SEG0 / TK_THREADS;
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
  if (d.top_k <= 0 || d.top_k > TK_MERGE) return 0;
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
      default: TK_SEG_LAUNCH(4, dim3(Q, 1), 1, idx, nullptr, nullptr); break;
    }
    return hipGetLastError();
  }
  const int G = std::max(2, TK_MERGE / k);
  const size_t lists1 = (size_t)(p.nseg + G - 1) / G;
  int32_t* bufA_i = (int32_t*)ws;
  uint32_t* bufA_k = (uint32_t*)(bufA_i + (size_t)Q * p.nseg * k);
  int32_t* bufB_i = (int32_t*)(bufA_k + (size_t)Q * p.nseg * k);
  uint32_t* bufB_k = (uint32_t*)(bufB_i + (size_t)Q * lists1 * k);
  TK_SEG_LAUNCH(4, dim3(Q, p.nseg), 0, idx, bufA_i, bufA_k);
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
      case 8: TK_MERGE_LAUNCH(8, dim3(Q, groups), per_group); break;
      default: TK_MERGE_LAUNCH(16, dim3(Q, groups), per_group); break;
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
