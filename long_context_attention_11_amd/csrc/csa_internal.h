// Internal declarations of the CSA library: device helpers shared by the kernels and the
// host-side launch functions the C ABI calls.  Built for gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "../../include/csa.h"

namespace csa {

struct ProjectStepArgs;
struct FoldArgs;

// ----------------------------------------------------------------------------- formats

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (read once; not kept in the caches).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float32 -> bfloat16 bits, round to nearest even; NaN -> quiet NaN with the input's sign.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t qnan = ((u >> 16) & 0x8000u) | 0x7fc0u;
  return ((u & 0x7fffffffu) > 0x7f800000u) ? qnan : rounded;  // select, no branch
}

// Two float32 -> packed bfloat16 pair (low half = a), round to nearest even, by the gfx950
// packed conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// float32 -> OCP E4M3 (e4m3fn) code: nearest, ties to even, saturating at +-448; NaN -> 0x7f.
// Written from the format's definition: 4 exponent bits (bias 7), 3 mantissa bits,
// subnormals in units of 2^-9, no infinities.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(f);
  if (!(a == a)) return 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {                         // below 2^-6: subnormal grid of 2^-9
    float q = __builtin_rintf(a * 512.0f);     // exact scaling, round half to even
    return sign | (uint32_t)q;                 // q == 8 is the smallest normal, code 0x08
  }
  uint32_t ua = __float_as_uint(a);
  int ef = (int)(ua >> 23) - 127 + 7;          // biased E4M3 exponent, 1..15
  uint32_t mant = ua & 0x7fffffu;
  uint32_t keep = mant >> 20, rest = mant & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) { keep = 0u; ++ef; }
  uint32_t code = ((uint32_t)ef << 3) | keep;
  if (code > 0x7eu) code = 0x7eu;
  return sign | code;
}

// Four E4M3 codes (one dword) -> four bfloat16 (two dwords).  Exact: every E4M3 value is a
// bfloat16 value.  Uses the gfx950 scaled conversion with scale 1.
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t src, uint32_t& lo, uint32_t& hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)src, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)src, 1.0f, true);
  lo = __builtin_bit_cast(uint32_t, a);
  hi = __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  uint32_t lo, hi;
  e4m3x4_to_bf16x4(code & 0xffu, lo, hi);
  return bf16_bits_to_f32(lo & 0xffffu);
}

// FP4 E2M1 code of x (already divided by its block scale): nearest of 0, 0.5, 1, 1.5, 2, 3, 4,
// 6 with ties to the even code, saturating at 6; the sign is kept (code 8 is -0).
__device__ __forceinline__ uint32_t e2m1_code(float x) {
  const float a = fabsf(x);
  const uint32_t mag = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                       (a >= 3.5f) + (a > 5.0f);
  return (signbit(x) ? 8u : 0u) | mag;
}

// Order-preserving map of a float score to uint32 (larger score -> larger key); -0 -> +0.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ----------------------------------------------------------------------------- cache rows

// Where a cache's entries live: cap rows per sequence in one run, or pages of epp entries
// found through a per-sequence block table (bt[seq * max_blocks + j] = pool page of the
// sequence's entries j epp .. j epp + epp - 1).
struct RowMap {
  const int32_t* bt;   // null: contiguous
  int32_t max_blocks, epp, n_pages, cap;
};

// Pool page of entry i of sequence seq (paged maps only), clamped to the pool.
__device__ __forceinline__ int page_of(const RowMap& rm, int seq, int i) {
  const int p = rm.bt[(int64_t)seq * rm.max_blocks + min(i / rm.epp, rm.max_blocks - 1)];
  return min(max(p, 0), rm.n_pages - 1);
}
// Row of entry i of sequence seq in its tensor (row-major rows of one width).
__device__ __forceinline__ int64_t row_of(const RowMap& rm, int seq, int i) {
  if (!rm.bt) return (int64_t)seq * rm.cap + i;
  return (int64_t)page_of(rm, seq, i) * rm.epp + i % rm.epp;
}
// MXFP4 keys are stored in groups: a group of n rows holds n rows of element bytes, then n
// rows of scale codes; a group is a sequence (n = cap) or a page (n = epp).  Byte offsets of
// entry i's element bytes and scale codes (rows of ce and cs bytes).
__device__ __forceinline__ void mx_offsets(const RowMap& rm, int seq, int i, int ce, int cs,
                                           int64_t& codes, int64_t& scales) {
  int64_t g0;
  int n, r;
  if (!rm.bt) {
    g0 = (int64_t)seq * rm.cap;
    n = rm.cap;
    r = i;
  } else {
    g0 = (int64_t)page_of(rm, seq, i) * rm.epp;
    n = rm.epp;
    r = i % rm.epp;
  }
  codes = g0 * (ce + cs) + (int64_t)r * ce;
  scales = g0 * (ce + cs) + (int64_t)n * ce + (int64_t)r * cs;
}

// ----------------------------------------------------------------------------- wave helpers

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations complete, then all
// waves meet.  Unlike __syncthreads() it does not wait for the wave's outstanding global
// loads, so loads prefetched into registers stay in flight across it (the compiler still
// waits for each one before its registers are used).  Use only where the barrier orders LDS
// accesses and no global memory written by one wave is read by another.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Map a hardware workgroup id to a logical one so that logical ids [k*n/8, (k+1)*n/8) run on
// XCD k (workgroups are dealt to the 8 XCDs round-robin).  Neighbouring logical tiles then
// share an L2.  Identity when n is not a multiple of 8.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t hw, uint32_t n) {
  if (n % 8u) return hw;
  return (hw % 8u) * (n / 8u) + hw / 8u;
}

// ---- wave primitives on DPP (row-local lane moves, a few cycles each) and readlane, so
// that reductions and scans avoid chains of LDS-routed lane permutes.  Every lane of the
// wave must be active.
template <int CTRL>
__device__ __forceinline__ int dpp_(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_QUAD_1032 = 0xB1, DPP_QUAD_2301 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
constexpr int DPP_SHR1 = 0x111, DPP_SHR2 = 0x112, DPP_SHR4 = 0x114, DPP_SHR8 = 0x118;

// Combine over the 16 lanes of each row; every lane of the row gets the result.
template <class F>
__device__ __forceinline__ int row_allreduce(int x, F op) {
  x = op(x, dpp_<DPP_QUAD_1032>(x));
  x = op(x, dpp_<DPP_QUAD_2301>(x));
  x = op(x, dpp_<DPP_HALF_MIRROR>(x));
  return op(x, dpp_<DPP_MIRROR>(x));
}
template <class F>
__device__ __forceinline__ int wave_allreduce(int x, F op) {
  x = row_allreduce(x, op);
  return op(op(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
            op(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_<DPP_SHR1>(x);
  x += dpp_<DPP_SHR2>(x);
  x += dpp_<DPP_SHR4>(x);
  x += dpp_<DPP_SHR8>(x);
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

struct OpAddF {
  __device__ int operator()(int a, int b) const { return __float_as_int(__int_as_float(a) + __int_as_float(b)); }
};

// Value of lane l ^ 32 (resp. l ^ 16), through the gfx950 lane-half swaps rather than an
// LDS-routed permute.  Every lane of the wave must be active.
__device__ __forceinline__ float lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}

// RoPE cos/sin of the angle pos * theta_j, theta_j = base^(-2j/rope_dim).  The product is
// formed in float64 (a float32 product is ~0.06 rad off at pos ~ 1e6), reduced to [-pi, pi]
// with a two-constant Cody-Waite step in float64, and only the reduced angle goes through
// float32 sincos.  log2_base = log2(base), computed on the host.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, int pair, int rope_dim,
                                             double log2_base, float& c, float& s) {
  const double theta = exp2(-2.0 * (double)pair / (double)rope_dim * log2_base);
  const double ang = (double)pos * theta;
  const double k = rint(ang * 0.15915494309189535);            // 1 / (2 pi)
  double red = fma(-k, 6.283185307179586, ang);                 // 2 pi, high part
  red = fma(-k, 2.4492935982947064e-16, red);                   // 2 pi - high part
  sincosf((float)red, &s, &c);
}

// ----------------------------------------------------------------------------- host side

struct Status {
  int code = CSA_OK;
  std::string msg;
};

void set_error(const std::string& msg);

// Kernel launchers (defined in the .hip files).  Each returns a hipError_t of its launch.
hipError_t launch_project(const csa_dims& d, const csa_weights& w, const void* H, int32_t M,
                          int32_t ksplit, float* P, hipStream_t s);
// One-token steps (T = 1, bf16, d % 1024 == 0): the projection writes partial sums over
// slices of K to part (project_part_bytes); the fold (P = null, the same part) adds them and
// also stores the new token's row into the state ring.
bool project_step_ok(const csa_dims& d, int32_t T);
size_t project_part_bytes(const csa_dims& d, int32_t B);
int32_t project_step_units(const csa_dims& d, int32_t B);   // wave-sized units
hipError_t launch_project_step(const csa_dims& d, const csa_weights& w, const csa_cache& c,
                               const void* H, float* part, hipStream_t s);
hipError_t launch_fold(const csa_dims& d, const csa_weights& w, const csa_cache& c,
                       int32_t T, const int32_t* pos0, const float* P, int32_t ksplit,
                       hipStream_t s, const float* part = nullptr);
hipError_t launch_state_update(const csa_dims& d, const csa_cache& c, int32_t T,
                               const int32_t* pos0, const float* P, int32_t ksplit,
                               hipStream_t s);
// `tiled`: every aligned group of 16 queries (0-15, 16-31, ...) belongs to one sequence, so
// the prefill-shaped kernel may share key tiles between them.
// Scores are float32, or bfloat16 with the MXFP4 indexer path.
hipError_t launch_indexer(const csa_dims& d, const csa_cache& c, const void* qI, const void* w,
                          const int32_t* q_seq, const int32_t* q_pos, int32_t Q, void* scores,
                          int64_t ld_scores, bool tiled, hipStream_t s);
// Candidates the final top-k selection holds: a query whose candidate lists total more (or
// fewer than k) is selected from its whole score row instead.
constexpr int TOPK_FINAL_CAND = 8192;

// A query's candidate lists, one per segment of its row (entries at or above one threshold,
// in index order), as the final top-k selection reads them.
struct CandLists {
  int32_t* idx;   // [Q][nseg][cs] entry indices
  uint32_t* key;  // [Q][nseg][cs] their order-preserving score keys
  int32_t* cnt;   // [Q][nseg] entries that passed (more than cs: the list overflowed)
  int32_t* vis;   // [Q] the visible count each query was scored with
  int nseg, cs;
};
// The prefill indexer that thresholds its own scores (tiled, E4M3 keys, 64 heads): every
// visible score goes to `scores` (row stride ld) as with launch_indexer, and the entries at or
// above a per-query threshold to candidate lists in ws (indexer_cand_bytes), described in
// *cl; the final selection then needs no threshold pass.
bool indexer_cand_applies(const csa_dims& d, int32_t Q);
size_t indexer_cand_bytes(const csa_dims& d, int32_t Q, int32_t cap);
hipError_t launch_indexer_cand(const csa_dims& d, const csa_cache& c, const void* qI, const void* w,
                               const int32_t* q_seq, const int32_t* q_pos, int32_t Q, float* scores,
                               int64_t ld_scores, void* ws, CandLists* cl, hipStream_t s);
// The final top-k selection from such lists (float32 scores).
hipError_t launch_topk_final_lists(const csa_dims& d, const csa_cache& c, int32_t Q,
                                   const float* scores, int64_t ld_scores, const CandLists& cl,
                                   int32_t* idx, hipStream_t s);
// Rows longer than one top-k segment (topk_can_carry) can take the threshold + final passes,
// whose launches carry other work: with step non-null (only where topk_can_carry_step allows
// it) the threshold pass also runs that one-token projection step, and with fold non-null the
// final pass runs that fold (of the same cache).  Those passes need
// topk_filter_workspace_bytes of workspace; without step and fold, rows of up to 65536
// entries are selected in one launch with none (topk_workspace_bytes).
bool topk_can_carry(const csa_cache& c);
bool topk_can_carry_step(const csa_cache& c, int32_t Q, int32_t step_units);
hipError_t launch_topk(const csa_dims& d, const csa_cache& c, const int32_t* q_seq,
                       const int32_t* q_pos, int32_t Q, const void* scores, int64_t ld_scores,
                       int32_t* idx, void* ws, hipStream_t s,
                       const struct ProjectStepArgs* step = nullptr,
                       const struct FoldArgs* fold = nullptr);
// fold: with dense attention of one-token HCA steps, the step's fold runs as extra
// workgroups of the attention launch (its partial projections already computed).
hipError_t launch_attend(const csa_dims& d, const csa_cache& c, const void* q,
                         const float* gamma_q, const float* sink, const int32_t* q_seq,
                         const int32_t* q_pos, int32_t Q, const int32_t* idx, void* out,
                         void* ws, hipStream_t s, const FoldArgs* fold = nullptr);
hipError_t launch_reduce_partials(const float* P, int32_t ksplit, int64_t n, float* out,
                                  hipStream_t s);
hipError_t launch_query_meta(int32_t B, int32_t T, const int32_t* pos0, int32_t* q_seq,
                             int32_t* q_pos, hipStream_t s);

// Layer kinds: CSA (dual), HCA (single path, dense) and CSA2 (single path with an indexer
// whose keys are projected from the main entry).
inline bool has_indexer(const csa_dims& d) { return d.top_k > 0; }
inline bool keys_from_entry(const csa_dims& d) { return !d.dual && d.top_k > 0; }

// The row map of a cache (host).
inline RowMap row_map(const csa_dims& d, const csa_cache& c) {
  RowMap rm;
  rm.bt = c.block_table;
  rm.max_blocks = c.block_table ? c.max_blocks : 0;
  rm.epp = c.block_table ? c.page_tokens / d.m : 0;
  rm.n_pages = c.block_table ? c.n_pages : 0;
  rm.cap = c.cap;
  return rm;
}

// Planning helpers shared by the API and the launchers (pure host arithmetic).
int32_t project_ksplit(const csa_dims& d, int32_t M);
size_t topk_workspace_bytes(const csa_dims& d, int32_t Q, int32_t cap);
size_t topk_filter_workspace_bytes(const csa_dims& d, int32_t Q, int32_t cap);
int32_t topk_max_visible(const csa_dims& d);
// which: 0 = sparse attention (idx given), 1 = dense (idx = NULL), 2 = the larger of both.
size_t attend_workspace_bytes(const csa_dims& d, int32_t Q, int32_t cap, int which);
int64_t attend_max_rows();  // keys per query the quantized attention path handles
int32_t state_width(const csa_dims& d);
int32_t state_rows(const csa_dims& d);
size_t row_bytes(const csa_dims& d);

// proj.hip: the query-side and grouped output projections, and the large-input GEMM the
// compression projection uses
bool project_gemm_ok(int32_t M);
hipError_t launch_project_gemm(const uint16_t* H, const uint16_t* wkv, const uint16_t* widx, int nkv, int M,
                               int NP, int K, int ksplit, float* P, hipStream_t s);
size_t query_project_ws_bytes(const csa_dims& d, int32_t d_c, int32_t T);
size_t output_project_ws_bytes(const csa_dims& d, int32_t g, int32_t d_g, int32_t T);
hipError_t launch_query_project(const csa_dims& d, const csa_proj_weights& w, const void* h, int32_t T,
                                void* q, void* qI, void* wI, void* ws, hipStream_t s);
hipError_t launch_output_project(const csa_dims& d, const csa_proj_weights& w, const void* o, int32_t T,
                                 void* out, void* ws, hipStream_t s);

}  // namespace csa
