// C ABI of the CSA library: argument checks, workspace planning and kernel dispatch.
// Every check runs on the host before anything is enqueued; nothing here allocates device
// memory or synchronises the stream.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "csa_internal.h"
#include "step_project.h"
#include "fold.h"

namespace csa {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

namespace {

int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_weights(const csa_dims& d, const csa_weights* w) {
  if (!w || !w->w_kv) return fail(CSA_ERR_INVALID_ARGUMENT, "weights: w_kv is required");
  if (d.dual && (!w->bias || !w->w_idx || !w->bias_idx))
    return fail(CSA_ERR_INVALID_ARGUMENT, "CSA weights: bias, w_idx and bias_idx are required");
  if (!d.dual && !has_indexer(d) && !w->bias)
    return fail(CSA_ERR_INVALID_ARGUMENT, "HCA weights: bias is required");
  if (keys_from_entry(d) && !w->w_idx)
    return fail(CSA_ERR_INVALID_ARGUMENT, "CSA2 weights: w_idx (the index-key projection) is required");
  return CSA_OK;
}

// Checks the dims on their own.  Returns CSA_OK or an error (message set).
int check_dims(const csa_dims* d) {
  if (!d) return fail(CSA_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (d->d < 1 || d->c < 2 || d->n_h < 1 || d->m < 1 || d->n_win < 1)
    return fail(CSA_ERR_INVALID_ARGUMENT, "d, c, n_h, m and n_win must be positive (c >= 2)");
  if (d->rope_dim < 0 || d->rope_dim > d->c || (d->rope_dim & 1) || (d->c & 1))
    return fail(CSA_ERR_INVALID_ARGUMENT, "rope_dim must be even and <= c, c even");
  // a query at tau sees the entries of complete blocks only, so the window must reach back
  // over the open block's tokens (m * floor(tau / m) .. tau), for CSA and HCA alike
  if (d->n_win < d->m)
    return fail(CSA_ERR_INVALID_ARGUMENT, "n_win must be >= m so the window covers the open block");
  if (d->dual != 0 && d->dual != 1) return fail(CSA_ERR_INVALID_ARGUMENT, "dual must be 0 or 1");
  if (d->top_k < 0) return fail(CSA_ERR_INVALID_ARGUMENT, "top_k must be >= 0");
  if (d->dual && d->top_k < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "CSA needs top_k >= 1");
  const bool idx = has_indexer(*d);
  if (idx && (d->c_I < 2 || (d->c_I & 1) || d->n_hI < 1))
    return fail(CSA_ERR_INVALID_ARGUMENT, "an indexer needs c_I >= 2 (even) and n_hI >= 1");
  if (keys_from_entry(*d) && d->c_I > 512)
    return fail(CSA_ERR_UNSUPPORTED, "CSA2 index keys are built for c_I <= 512");
  if (!(d->rope_base > 0.f) || !(d->rms_eps >= 0.f))
    return fail(CSA_ERR_INVALID_ARGUMENT, "rope_base must be > 0 and rms_eps >= 0");
  if (d->c > 512) return fail(CSA_ERR_UNSUPPORTED, "c > 512 is not built");
  const bool f32 = d->act_fmt == CSA_FMT_F32 && d->kv_fmt == CSA_FMT_F32 &&
                   (!idx || d->idx_fmt == CSA_FMT_F32);
  const bool q = d->act_fmt == CSA_FMT_BF16 &&
                 (d->kv_fmt == CSA_FMT_E4M3_BF16 || d->kv_fmt == CSA_FMT_MXFP4_BF16) &&
                 (!idx || d->idx_fmt == CSA_FMT_E4M3 || d->idx_fmt == CSA_FMT_MXFP4);
  if (!f32 && !q)
    return fail(CSA_ERR_UNSUPPORTED,
                "supported formats: all F32, or act BF16 + kv E4M3_BF16 or MXFP4_BF16 + idx E4M3 or MXFP4");
  if (q) {
    if (d->c != 512 || d->rope_dim != 64)
      return fail(CSA_ERR_UNSUPPORTED, "quantized KV rows are built for c = 512, rope_dim = 64");
    if (d->n_h % 16) return fail(CSA_ERR_UNSUPPORTED, "n_h must be a multiple of 16");
    if (idx && (d->c_I != 128 || (d->n_hI != 16 && d->n_hI != 32 && d->n_hI != 64)))
      return fail(CSA_ERR_UNSUPPORTED, "the quantized indexer is built for c_I = 128, n_hI in {16, 32, 64}");
    if (d->d % 64) return fail(CSA_ERR_UNSUPPORTED, "bf16 projection needs d % 64 == 0");
  }
  return CSA_OK;
}

int check_cache(const csa_dims* d, const csa_cache* c, bool need_state) {
  if (!c) return fail(CSA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (c->B < 1 || c->cap < 1 || c->win_cap < 1)
    return fail(CSA_ERR_INVALID_ARGUMENT, "cache B, cap and win_cap must be positive");
  if (c->win_cap < d->n_win) return fail(CSA_ERR_INVALID_ARGUMENT, "win_cap must be >= n_win");
  if (!c->kv || !c->n_entries || !c->win || !c->win_pos)
    return fail(CSA_ERR_INVALID_ARGUMENT, "cache kv, n_entries, win and win_pos must be set");
  if (has_indexer(*d) && !c->ki) return fail(CSA_ERR_INVALID_ARGUMENT, "a cache with an indexer needs ki");
  if (need_state && !c->state) return fail(CSA_ERR_INVALID_ARGUMENT, "cache state is NULL");
  const size_t rb = row_bytes(*d);
  if ((size_t)c->cap * rb > (size_t)1 << 40)
    return fail(CSA_ERR_INVALID_ARGUMENT, "cache capacity overflows");
  if (c->block_table) {
    if (c->page_tokens < d->m || c->page_tokens % d->m)
      return fail(CSA_ERR_INVALID_ARGUMENT, "page_tokens must be a positive multiple of m");
    if (c->max_blocks < 1 || c->n_pages < 1)
      return fail(CSA_ERR_INVALID_ARGUMENT, "a paged cache needs max_blocks >= 1 and n_pages >= 1");
    const int64_t epp = c->page_tokens / d->m;
    if ((int64_t)c->cap > (int64_t)c->max_blocks * epp)
      return fail(CSA_ERR_INVALID_ARGUMENT, "cap exceeds max_blocks * page_tokens / m");
    if ((size_t)c->n_pages * (size_t)epp * rb > (size_t)1 << 40)
      return fail(CSA_ERR_INVALID_ARGUMENT, "page pool size overflows");
    // the quantized decode indexer scores 16-entry tiles that must not straddle a page
    if (has_indexer(*d) && d->idx_fmt != CSA_FMT_F32 && epp % 16)
      return fail(CSA_ERR_UNSUPPORTED, "a paged CSA cache with quantized keys needs page_tokens / m % 16 == 0");
  }
  return CSA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(CSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

struct Layout {
  size_t off[8] = {0};
  size_t total = 0;
  size_t add(int i, size_t bytes) {
    off[i] = total;
    total = align_up(total + bytes, 256);
    return off[i];
  }
};

// split-K partials [ks][M][P] and, when ks > 1, their sum [M][P]
size_t compress_ws(const csa_dims& d, int32_t B, int32_t T) {
  if (project_step_ok(d, T)) return project_part_bytes(d, B);
  const int32_t M = B * T;
  const int32_t ks = project_ksplit(d, M);
  return (size_t)(ks + (ks > 1 ? 1 : 0)) * M * state_width(d) * sizeof(float);
}

// scores [q][cap] + top-k candidates for `Qc` queries (through the top-k passes, or lists the
// prefill indexer fills itself)
size_t index_ws(const csa_dims& d, int32_t Qc, int32_t cap) {
  return align_up((size_t)Qc * cap * sizeof(float), 256) +
         std::max(topk_workspace_bytes(d, Qc, cap), indexer_cand_bytes(d, Qc, cap));
}

// The same through the threshold + final passes, whose launches carry a one-token step.
size_t index_ws_carry(const csa_dims& d, int32_t Qc, int32_t cap) {
  return align_up((size_t)Qc * cap * sizeof(float), 256) + topk_filter_workspace_bytes(d, Qc, cap);
}

}  // namespace
}  // namespace csa

using namespace csa;

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case CSA_ERR_UNSUPPORTED: return "unsupported";
    case CSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case CSA_ERR_HIP: return "hip error";
    default: return "unknown status";
  }
}

const char* csa_last_error(void) { return g_last_error.c_str(); }

size_t csa_row_bytes(const csa_dims* dims) {
  if (check_dims(dims) != CSA_OK) return 0;
  return row_bytes(*dims);
}

int32_t csa_state_width(const csa_dims* dims) {
  if (check_dims(dims) != CSA_OK) return 0;
  return state_width(*dims);
}

int32_t csa_state_rows(const csa_dims* dims) {
  if (check_dims(dims) != CSA_OK) return 0;
  return state_rows(*dims);
}

int csa_workspace_size(const csa_dims* dims, int32_t op, int32_t B, int32_t T, int32_t Q,
                       int32_t cap, int32_t q_chunk, size_t* bytes) {
  g_last_error.clear();
  int st = check_dims(dims);
  if (st) return st;
  if (!bytes) return fail(CSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  const csa_dims& d = *dims;
  switch (op) {
    case CSA_OP_COMPRESS:
      if (B < 1 || T < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "B and T must be positive");
      *bytes = compress_ws(d, B, T);
      return CSA_OK;
    case CSA_OP_INDEX_TOPK:
      if (!has_indexer(d)) return fail(CSA_ERR_INVALID_ARGUMENT, "HCA has no indexer");
      if (Q < 1 || cap < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "Q and cap must be positive");
      *bytes = index_ws(d, Q, cap);
      return CSA_OK;
    case CSA_OP_ATTEND:
      if (Q < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "Q must be positive");
      *bytes = attend_workspace_bytes(d, Q, std::max(cap, 1), 2);
      return CSA_OK;
    case CSA_OP_FORWARD: {
      if (B < 1 || T < 1 || cap < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "B, T, cap must be positive");
      const int32_t Qn = B * T;
      const int32_t Qc = (q_chunk > 0 && q_chunk < Qn) ? q_chunk : Qn;
      Layout L;
      L.add(0, 2 * sizeof(int32_t) * (size_t)Qn);                 // q_seq, q_pos
      L.add(1, has_indexer(d) ? sizeof(int32_t) * (size_t)Qn * d.top_k : 0);  // idx
      size_t phase = compress_ws(d, B, T);
      if (has_indexer(d)) phase = std::max(phase, index_ws(d, Qc, cap));
      if (has_indexer(d) && T == 1)
        phase = std::max(phase, align_up(index_ws_carry(d, Qn, cap), 256) + project_part_bytes(d, B));
      // forward attends a layer with an indexer sparsely
      phase = std::max(phase, attend_workspace_bytes(d, Qn, cap, has_indexer(d) ? 0 : 1));
      // one-token HCA steps keep the projection partials through the attention launch
      if (!has_indexer(d) && T == 1 && d.kv_fmt != CSA_FMT_F32)
        phase = std::max(phase, align_up(attend_workspace_bytes(d, Qn, cap, 1), 256) + compress_ws(d, B, T));
      L.add(2, phase);
      *bytes = L.total;
      return CSA_OK;
    }
    default:
      return fail(CSA_ERR_INVALID_ARGUMENT, "unknown op");
  }
}

int csa_compress(const csa_dims* dims, const csa_weights* w, const csa_cache* cache,
                 const void* H, int32_t T, const int32_t* pos0, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  g_last_error.clear();
  int st = check_dims(dims);
  if (st) return st;
  const csa_dims& d = *dims;
  if ((st = check_cache(dims, cache, true))) return st;
  if ((st = check_weights(d, w))) return st;
  if (!H || !pos0) return fail(CSA_ERR_INVALID_ARGUMENT, "H and pos0 must be set");
  if (T < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "T must be >= 1");
  const int32_t M = cache->B * T;
  const size_t need = compress_ws(d, cache->B, T);
  if (need && (!ws || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE_TOO_SMALL, "compress needs " + std::to_string(need) + " bytes of workspace");
  if (project_step_ok(d, T)) {
    // one new token per sequence: partial projections, then the fold adds them up (and
    // stores the token's row in the state ring)
    float* part = (float*)ws;
    hipError_t e = launch_project_step(d, *w, *cache, H, part, stream);
    if (e != hipSuccess) return hip_fail(e, "projection launch");
    e = launch_fold(d, *w, *cache, T, pos0, nullptr, 1, stream, part);
    if (e != hipSuccess) return hip_fail(e, "fold launch");
    return CSA_OK;
  }
  const int32_t ks = project_ksplit(d, M);
  float* P = (float*)ws;
  hipError_t e = launch_project(d, *w, H, M, ks, P, stream);
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  if (ks > 1) {
    const int64_t n = (int64_t)M * state_width(d);
    float* Psum = P + (size_t)ks * n;
    e = launch_reduce_partials(P, ks, n, Psum, stream);
    if (e != hipSuccess) return hip_fail(e, "split-K reduce launch");
    P = Psum;
  }
  e = launch_fold(d, *w, *cache, T, pos0, P, 1, stream);
  if (e != hipSuccess) return hip_fail(e, "fold launch");
  e = launch_state_update(d, *cache, T, pos0, P, 1, stream);
  if (e != hipSuccess) return hip_fail(e, "state launch");
  return CSA_OK;
}

static int index_topk_impl(const csa_dims& d, const csa_cache& c, const void* qI, const void* w,
                           const int32_t* q_seq, const int32_t* q_pos, int32_t Q, int32_t* idx_out,
                           void* scores_out, void* ws, size_t ws_bytes, bool tiled,
                           hipStream_t stream, const ProjectStepArgs* step = nullptr,
                           const FoldArgs* fold = nullptr) {
  const size_t sc_bytes = scores_out ? 0 : align_up((size_t)Q * c.cap * sizeof(float), 256);
  const size_t need = sc_bytes + ((step || fold) ? topk_filter_workspace_bytes(d, Q, c.cap)
                                                   : topk_workspace_bytes(d, Q, c.cap));
  if (need && (!ws || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE_TOO_SMALL, "index_topk needs " + std::to_string(need) + " bytes of workspace");
  void* scores = scores_out ? scores_out : ws;
  void* tws = (char*)ws + sc_bytes;
  if (tiled && !step && !fold && indexer_cand_applies(d, Q)) {
    // the prefill indexer thresholds its own scores; the final selection reads its lists
    if (!ws || sc_bytes + indexer_cand_bytes(d, Q, c.cap) > ws_bytes)
      return fail(CSA_ERR_WORKSPACE_TOO_SMALL, "index_topk needs " + std::to_string(sc_bytes + indexer_cand_bytes(d, Q, c.cap)) +
                                                   " bytes of workspace");
    CandLists cl;
    hipError_t e = launch_indexer_cand(d, c, qI, w, q_seq, q_pos, Q, (float*)scores, c.cap, tws, &cl, stream);
    if (e != hipSuccess) return hip_fail(e, "indexer launch");
    e = launch_topk_final_lists(d, c, Q, (const float*)scores, c.cap, cl, idx_out, stream);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
    return CSA_OK;
  }
  hipError_t e = launch_indexer(d, c, qI, w, q_seq, q_pos, Q, scores, c.cap, tiled, stream);
  if (e != hipSuccess) return hip_fail(e, "indexer launch");
  e = launch_topk(d, c, q_seq, q_pos, Q, scores, c.cap, idx_out, tws, stream, step, fold);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return CSA_OK;
}

static int index_topk_entry(const csa_dims* dims, const csa_cache* cache, const void* qI, const void* w,
                            const int32_t* q_seq, const int32_t* q_pos, int32_t Q, int32_t* idx_out,
                            void* scores_out, void* ws, size_t ws_bytes, bool grouped, hipStream_t stream) {
  g_last_error.clear();
  int st = check_dims(dims);
  if (st) return st;
  const csa_dims& d = *dims;
  if (!has_indexer(d)) return fail(CSA_ERR_INVALID_ARGUMENT, "HCA (top_k = 0) has no indexer");
  if ((st = check_cache(dims, cache, false))) return st;
  if (!qI || !w || !q_seq || !q_pos || !idx_out)
    return fail(CSA_ERR_INVALID_ARGUMENT, "qI, w, q_seq, q_pos and idx_out must be set");
  if (Q < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "Q must be >= 1");
  if (cache->cap > topk_max_visible(d))
    return fail(CSA_ERR_UNSUPPORTED, "cap exceeds the entries the top-k kernels handle for this top_k (" +
                                         std::to_string(topk_max_visible(d)) + ")");
  return index_topk_impl(d, *cache, qI, w, q_seq, q_pos, Q, idx_out, scores_out, ws, ws_bytes,
                         grouped, stream);
}

int csa_index_topk(const csa_dims* dims, const csa_cache* cache, const void* qI, const void* w,
                   const int32_t* q_seq, const int32_t* q_pos, int32_t Q, int32_t* idx_out,
                   void* scores_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return index_topk_entry(dims, cache, qI, w, q_seq, q_pos, Q, idx_out, scores_out, ws, ws_bytes, false, stream);
}

int csa_index_topk_grouped(const csa_dims* dims, const csa_cache* cache, const void* qI, const void* w,
                           const int32_t* q_seq, const int32_t* q_pos, int32_t Q, int32_t* idx_out,
                           void* scores_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return index_topk_entry(dims, cache, qI, w, q_seq, q_pos, Q, idx_out, scores_out, ws, ws_bytes, true, stream);
}

int csa_index_scores(const csa_dims* dims, const csa_cache* cache, const void* qI, const void* w,
                     const int32_t* q_seq, const int32_t* q_pos, int32_t Q, void* scores,
                     int64_t ld, hipStream_t stream) {
  g_last_error.clear();
  int st = check_dims(dims);
  if (st) return st;
  if (!has_indexer(*dims)) return fail(CSA_ERR_INVALID_ARGUMENT, "HCA (top_k = 0) has no indexer");
  if ((st = check_cache(dims, cache, false))) return st;
  if (!qI || !w || !q_seq || !q_pos || !scores)
    return fail(CSA_ERR_INVALID_ARGUMENT, "qI, w, q_seq, q_pos and scores must be set");
  if (Q < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "Q must be >= 1");
  if (ld < cache->cap) return fail(CSA_ERR_INVALID_ARGUMENT, "ld must be >= cap");
  hipError_t e = launch_indexer(*dims, *cache, qI, w, q_seq, q_pos, Q, scores, ld, false, stream);
  if (e != hipSuccess) return hip_fail(e, "indexer launch");
  return CSA_OK;
}

int csa_index_scores_grouped(const csa_dims* dims, const csa_cache* cache, const void* qI, const void* w,
                             const int32_t* q_seq, const int32_t* q_pos, int32_t Q, void* scores,
                             int64_t ld, hipStream_t stream) {
  g_last_error.clear();
  int st = check_dims(dims);
  if (st) return st;
  if (!has_indexer(*dims)) return fail(CSA_ERR_INVALID_ARGUMENT, "HCA (top_k = 0) has no indexer");
  if ((st = check_cache(dims, cache, false))) return st;
  if (!qI || !w || !q_seq || !q_pos || !scores)
    return fail(CSA_ERR_INVALID_ARGUMENT, "qI, w, q_seq, q_pos and scores must be set");
  if (Q < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "Q must be >= 1");
  if (ld < cache->cap) return fail(CSA_ERR_INVALID_ARGUMENT, "ld must be >= cap");
  hipError_t e = launch_indexer(*dims, *cache, qI, w, q_seq, q_pos, Q, scores, ld, true, stream);
  if (e != hipSuccess) return hip_fail(e, "indexer launch");
  return CSA_OK;
}

size_t csa_topk_workspace_size(const csa_dims* dims, int32_t Q, int32_t cap) {
  if (check_dims(dims) != CSA_OK || Q < 1 || cap < 1) return 0;
  return topk_workspace_bytes(*dims, Q, cap);
}

int csa_topk(const csa_dims* dims, const csa_cache* cache, const int32_t* q_seq,
             const int32_t* q_pos, int32_t Q, const void* scores, int64_t ld, int32_t* idx_out,
             void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  int st = check_dims(dims);
  if (st) return st;
  if (!has_indexer(*dims)) return fail(CSA_ERR_INVALID_ARGUMENT, "HCA (top_k = 0) has no top-k");
  if ((st = check_cache(dims, cache, false))) return st;
  if (!q_seq || !q_pos || !scores || !idx_out)
    return fail(CSA_ERR_INVALID_ARGUMENT, "q_seq, q_pos, scores and idx_out must be set");
  if (Q < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "Q must be >= 1");
  if (ld < cache->cap) return fail(CSA_ERR_INVALID_ARGUMENT, "ld must be >= cap");
  if (cache->cap > topk_max_visible(*dims))
    return fail(CSA_ERR_UNSUPPORTED, "cap exceeds the entries the top-k kernels handle for this top_k");
  const size_t need = topk_workspace_bytes(*dims, Q, cache->cap);
  if (need && (!ws || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE_TOO_SMALL, "top-k needs " + std::to_string(need) + " bytes of workspace");
  hipError_t e = launch_topk(*dims, *cache, q_seq, q_pos, Q, scores, ld, idx_out, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return CSA_OK;
}

static int attend_checks(const csa_dims& d, const csa_cache& c, bool sparse) {
  if (d.kv_fmt == CSA_FMT_F32) {
    const long rows = (long)(sparse ? d.top_k : c.cap) + d.n_win;
    if (rows > 4096) return fail(CSA_ERR_UNSUPPORTED, "fp32 attention handles at most 4096 keys per query");
    if (d.c > 1024) return fail(CSA_ERR_UNSUPPORTED, "fp32 attention handles c <= 1024");
  } else {
    const int64_t rows = (int64_t)(sparse ? d.top_k : c.cap) + d.n_win;
    if (rows > attend_max_rows())
      return fail(CSA_ERR_UNSUPPORTED, "attention handles at most " + std::to_string(attend_max_rows()) + " keys per query");
  }
  return CSA_OK;
}

int csa_attend(const csa_dims* dims, const csa_cache* cache, const void* q, const float* gamma_q,
               const float* sink, const int32_t* q_seq, const int32_t* q_pos, int32_t Q,
               const int32_t* idx, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  int st = check_dims(dims);
  if (st) return st;
  const csa_dims& d = *dims;
  if ((st = check_cache(dims, cache, false))) return st;
  if (!q || !q_seq || !q_pos || !out) return fail(CSA_ERR_INVALID_ARGUMENT, "q, q_seq, q_pos and out must be set");
  if (Q < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "Q must be >= 1");
  if ((st = attend_checks(d, *cache, idx != nullptr))) return st;
  const size_t need = attend_workspace_bytes(d, Q, cache->cap, idx ? 0 : 1);
  if (need && (!ws || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE_TOO_SMALL, "attend needs " + std::to_string(need) + " bytes of workspace");
  hipError_t e = launch_attend(d, *cache, q, gamma_q, sink, q_seq, q_pos, Q, idx, out, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "attend launch");
  return CSA_OK;
}

// The host-side checks of a forward call, and the least workspace it can run in (*min_ws).
static int forward_checks(const csa_dims* dims, const csa_weights* w, const csa_cache* cache,
                          const void* H, int32_t T, const int32_t* pos0, const void* q, const void* qI,
                          const void* wI, void* out, int32_t* idx_out, size_t* min_ws) {
  int st = check_dims(dims);
  if (st) return st;
  const csa_dims& d = *dims;
  if ((st = check_cache(dims, cache, true))) return st;
  if ((st = check_weights(d, w))) return st;
  if (!H || !pos0 || !q || !out) return fail(CSA_ERR_INVALID_ARGUMENT, "H, pos0, q and out must be set");
  if (has_indexer(d) && (!qI || !wI)) return fail(CSA_ERR_INVALID_ARGUMENT, "a forward with an indexer needs qI and wI");
  if (T < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "T must be >= 1");
  if (cache->win_cap < T + d.n_win - 1)
    return fail(CSA_ERR_INVALID_ARGUMENT, "win_cap must be >= T + n_win - 1 for the chunk's queries");
  if (has_indexer(d) && cache->cap > topk_max_visible(d))
    return fail(CSA_ERR_UNSUPPORTED, "cap exceeds the entries the top-k kernels handle for this top_k");
  if ((st = attend_checks(d, *cache, has_indexer(d)))) return st;
  const int32_t Qn = cache->B * T;
  Layout L;
  L.add(0, 2 * sizeof(int32_t) * (size_t)Qn);
  L.add(1, (has_indexer(d) && !idx_out) ? sizeof(int32_t) * (size_t)Qn * d.top_k : 0);
  size_t min_phase = std::max(compress_ws(d, cache->B, T),
                              attend_workspace_bytes(d, Qn, cache->cap, has_indexer(d) ? 0 : 1));
  if (has_indexer(d)) min_phase = std::max(min_phase, index_ws(d, 1, cache->cap));
  *min_ws = L.total + min_phase;
  return CSA_OK;
}

int csa_forward(const csa_dims* dims, const csa_weights* w, const csa_cache* cache, const void* H,
                int32_t T, const int32_t* pos0, const void* q, const void* qI, const void* wI,
                const float* gamma_q, const float* sink, void* out, int32_t* idx_out, void* ws,
                size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  size_t min_ws = 0;
  int st = forward_checks(dims, w, cache, H, T, pos0, q, qI, wI, out, idx_out, &min_ws);
  if (st) return st;
  const csa_dims& d = *dims;
  if (!ws || ws_bytes < min_ws)
    return fail(CSA_ERR_WORKSPACE_TOO_SMALL, "forward needs at least " + std::to_string(min_ws) + " bytes of workspace");
  const int32_t Qn = cache->B * T;
  // fixed part of the workspace, then the largest query chunk the rest allows
  Layout L;
  L.add(0, 2 * sizeof(int32_t) * (size_t)Qn);
  L.add(1, (has_indexer(d) && !idx_out) ? sizeof(int32_t) * (size_t)Qn * d.top_k : 0);
  const size_t fixed = L.total;
  int32_t* q_seq = (int32_t*)((char*)ws + L.off[0]);
  int32_t* q_pos = q_seq + Qn;
  int32_t* idx = idx_out ? idx_out : (int32_t*)((char*)ws + L.off[1]);
  void* phase_ws = (char*)ws + fixed;
  const size_t phase_bytes = ws_bytes - fixed;

  // One new token per sequence (decode) with rows longer than a top-k segment: the query at
  // tau sees floor(tau / m) entries, all completed by earlier tokens, so the entry this call
  // may complete is not among them and the compression can move after scoring.  Its
  // projection step then rides in the top-k threshold launch (independent work on the CUs
  // that pass leaves idle) when both fit on the CUs at once, else runs first, and its fold
  // rides in the final selection's launch.  With a cache whose entry count trails the
  // positions, this order scores the entries present before the call.
  // With T = 1, query i is token pos0[i] of sequence i, so the kernels take the sequence as
  // the query index (null q_seq) and pos0 as q_pos.
  const size_t ix_bytes = align_up(index_ws_carry(d, Qn, cache->cap), 256);
  if (has_indexer(d) && project_step_ok(d, T) && topk_can_carry(*cache) &&
      ix_bytes + project_part_bytes(d, cache->B) <= phase_bytes) {
    float* part = (float*)((char*)phase_ws + ix_bytes);
    const ProjectStepArgs pa = project_step_args(d, *w, *cache, H, part);
    const bool carry = topk_can_carry_step(*cache, Qn, project_step_units(d, cache->B));
    if (!carry) {   // too many workgroups to share the threshold launch: project first
      hipError_t e = launch_project_step(d, *w, *cache, H, part, stream);
      if (e != hipSuccess) return hip_fail(e, "projection launch");
    }
    const FoldArgs fo = fold_args(d, *w, *cache, T, pos0, nullptr, part);
    st = index_topk_impl(d, *cache, qI, wI, nullptr, pos0, Qn, idx, nullptr, phase_ws, phase_bytes,
                         false, stream, carry ? &pa : nullptr, &fo);
    if (st) return st;
    hipError_t e = launch_attend(d, *cache, q, gamma_q, sink, nullptr, pos0, Qn, idx, out, phase_ws, stream);
    if (e != hipSuccess) return hip_fail(e, "attend launch");
    return CSA_OK;
  }

  // One new token per sequence of an HCA layer: projection, then attention with the fold as
  // extra workgroups of its launch (the attention workgroups that need the new token's
  // window row finalize it themselves), then the merge: one launch fewer than compressing
  // first.  The query at tau sees floor(tau / m) entries, none of them the one this step may
  // complete, and the fold's other stores (state ring, entry, count) are not read by it.
  if (!has_indexer(d) && project_step_ok(d, T) && d.kv_fmt != CSA_FMT_F32) {
    const size_t att_bytes = align_up(attend_workspace_bytes(d, Qn, cache->cap, 1), 256);
    if (att_bytes + project_part_bytes(d, cache->B) <= phase_bytes) {
      float* part = (float*)((char*)phase_ws + att_bytes);
      hipError_t e = launch_project_step(d, *w, *cache, H, part, stream);
      if (e != hipSuccess) return hip_fail(e, "projection launch");
      const FoldArgs fo = fold_args(d, *w, *cache, T, pos0, nullptr, part);
      e = launch_attend(d, *cache, q, gamma_q, sink, nullptr, pos0, Qn, nullptr, out, phase_ws, stream, &fo);
      if (e != hipSuccess) return hip_fail(e, "attend launch");
      return CSA_OK;
    }
  }

  st = csa_compress(dims, w, cache, H, T, pos0, phase_ws, phase_bytes, stream);
  if (st) return st;
  // largest query chunk whose scores and candidates fit
  int32_t Qc = Qn;
  if (has_indexer(d)) {
    while (Qc > 1 && index_ws(d, Qc, cache->cap) > phase_bytes) Qc = (Qc + 1) / 2;
    // Query q is token q % T of sequence q / T.  With T and the chunk a multiple of 16, every
    // aligned group of 16 queries of a chunk is one sequence and the indexer can tile them.
    if (Qc >= 16) Qc -= Qc % 16;
  }
  // T = 1 in one chunk: the query index is the sequence and pos0 the positions (null q_seq)
  const bool ident = T == 1 && Qc == Qn;
  const int32_t* qs_ = ident ? nullptr : q_seq;
  const int32_t* qp_ = ident ? pos0 : q_pos;
  hipError_t e;
  if (!ident) {
    e = launch_query_meta(cache->B, T, pos0, q_seq, q_pos, stream);
    if (e != hipSuccess) return hip_fail(e, "query metadata launch");
  }
  if (has_indexer(d)) {
    const bool tiled = T % 16 == 0 && Qc % 16 == 0;
    const size_t qI_row = d.idx_fmt == CSA_FMT_MXFP4 ? (size_t)d.n_hI * (d.c_I / 2 + d.c_I / 32)
                                                      : (size_t)d.n_hI * d.c_I * (d.idx_fmt == CSA_FMT_F32 ? 4 : 1);
    const size_t w_row = (size_t)d.n_hI * (d.act_fmt == CSA_FMT_F32 ? 4 : 2);
    for (int32_t q0 = 0; q0 < Qn; q0 += Qc) {
      const int32_t n = std::min(Qc, Qn - q0);
      st = index_topk_impl(d, *cache, (const char*)qI + q0 * qI_row, (const char*)wI + q0 * w_row,
                           qs_ ? qs_ + q0 : nullptr, qp_ + q0, n, idx + (size_t)q0 * d.top_k, nullptr,
                           phase_ws, phase_bytes, tiled, stream);
      if (st) return st;
    }
  }
  e = launch_attend(d, *cache, q, gamma_q, sink, qs_, qp_, Qn, has_indexer(d) ? idx : nullptr, out,
                    phase_ws, stream);
  if (e != hipSuccess) return hip_fail(e, "attend launch");
  return CSA_OK;
}

// ------------------------------------------------------------------ forward without allocation

}  // extern "C"

// Scratch of csa_forward_noalloc: a file-scope device array, one copy per GPU, held from the
// library's load until the process ends.  In host code `scratch` names a host-side stand-in,
// not a device address; the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace csa {
namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES];   // device address of `scratch` per device, once looked up

// The current device's copy of `scratch` (looked up on the first call on that device, with
// that device current, and kept).
int device_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return fail(CSA_ERR_UNSUPPORTED, "device index beyond the scratch table (" + std::to_string(dev) + ")");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return CSA_OK;
}

}  // namespace
}  // namespace csa

extern "C" {

size_t csa_noalloc_scratch_bytes(void) { return CSA_NOALLOC_SCRATCH_BYTES; }

int csa_forward_noalloc(const csa_dims* dims, const csa_weights* w, const csa_cache* cache,
                        const void* H, int32_t T, const int32_t* pos0, const void* q, const void* qI,
                        const void* wI, const float* gamma_q, const float* sink, void* out,
                        int32_t* idx_out, hipStream_t stream) {
  g_last_error.clear();
  size_t min_ws = 0;
  int st = forward_checks(dims, w, cache, H, T, pos0, q, qI, wI, out, idx_out, &min_ws);
  if (st) return st;
  if (min_ws > CSA_NOALLOC_SCRATCH_BYTES)
    return fail(CSA_ERR_WORKSPACE_TOO_SMALL,
                "csa_forward_noalloc: this call needs at least " + std::to_string(min_ws) +
                    " bytes of scratch, more than the static " + std::to_string((size_t)CSA_NOALLOC_SCRATCH_BYTES) +
                    "; call csa_forward with a workspace instead");
  void* ws = nullptr;
  if ((st = device_scratch(&ws))) return st;
  st = csa_forward(dims, w, cache, H, T, pos0, q, qI, wI, gamma_q, sink, out, idx_out, ws,
                   CSA_NOALLOC_SCRATCH_BYTES, stream);
  return st;
}

// ------------------------------------------------------------------ projections around the path

static int check_proj(const csa_dims* dims, const csa_proj_weights* pw, int32_t T) {
  int st = check_dims(dims);
  if (st) return st;
  if (!pw) return fail(CSA_ERR_INVALID_ARGUMENT, "projection weights are NULL");
  if (T < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "T must be >= 1");
  if (dims->act_fmt != CSA_FMT_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "the projections are built for act BF16");
  if (pw->d_c < 64 || pw->d_c % 64) return fail(CSA_ERR_UNSUPPORTED, "d_c must be a positive multiple of 64");
  if (pw->g < 1 || dims->n_h % pw->g || (dims->n_h * dims->c / pw->g) % 64)
    return fail(CSA_ERR_UNSUPPORTED, "g must divide n_h with c n_h / g a multiple of 64");
  if (pw->d_g < 64 || pw->d_g % 64) return fail(CSA_ERR_UNSUPPORTED, "d_g must be a positive multiple of 64");
  return CSA_OK;
}

size_t csa_query_project_workspace_size(const csa_dims* dims, const csa_proj_weights* pw, int32_t T) {
  if (check_proj(dims, pw, T) != CSA_OK) return 0;
  return csa::query_project_ws_bytes(*dims, pw->d_c, T);
}

int csa_query_project(const csa_dims* dims, const csa_proj_weights* pw, const void* h, int32_t T, void* q,
                      void* qI, void* w, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  int st = check_proj(dims, pw, T);
  if (st) return st;
  if (!h || !q || !pw->w_dq || !pw->w_uq)
    return fail(CSA_ERR_INVALID_ARGUMENT, "h, q, w_dq and w_uq must be set");
  if (has_indexer(*dims) && (!qI || !w || !pw->w_iuq || !pw->w_w))
    return fail(CSA_ERR_INVALID_ARGUMENT, "CSA needs qI, w, w_iuq and w_w");
  const size_t need = csa::query_project_ws_bytes(*dims, pw->d_c, T);
  if (!ws || ws_bytes < need)
    return fail(CSA_ERR_WORKSPACE_TOO_SMALL, "query projection needs " + std::to_string(need) + " bytes of workspace");
  hipError_t e = csa::launch_query_project(*dims, *pw, h, T, q, qI, w, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "query projection launch");
  return CSA_OK;
}

size_t csa_output_project_workspace_size(const csa_dims* dims, const csa_proj_weights* pw, int32_t T) {
  if (check_proj(dims, pw, T) != CSA_OK) return 0;
  return csa::output_project_ws_bytes(*dims, pw->g, pw->d_g, T);
}

int csa_output_project(const csa_dims* dims, const csa_proj_weights* pw, const void* o, int32_t T, void* out,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  int st = check_proj(dims, pw, T);
  if (st) return st;
  if (!o || !out || !pw->w_og || !pw->w_o)
    return fail(CSA_ERR_INVALID_ARGUMENT, "o, out, w_og and w_o must be set");
  const size_t need = csa::output_project_ws_bytes(*dims, pw->g, pw->d_g, T);
  if (!ws || ws_bytes < need)
    return fail(CSA_ERR_WORKSPACE_TOO_SMALL, "output projection needs " + std::to_string(need) + " bytes of workspace");
  hipError_t e = csa::launch_output_project(*dims, *pw, o, T, out, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "output projection launch");
  return CSA_OK;
}

}  // extern "C"
