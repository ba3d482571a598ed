/*
 * csa.h — C ABI of the compressed sparse attention library for AMD Instinct MI355X (gfx950).
 *
 * The library computes one attention layer of the kind the DeepSeek-V4 pages describe:
 *   1. overlapping dual-window KV compression: every m tokens fold into one entry, the
 *      softmax taken per column over 2m weighted projections with a learned positional bias
 *      (reading notes "DeepSeekV4技术报告阅读笔记", zouxinn.github.io, §2.3.1 eqs. 9-12;
 *      PaperTrace "02 · DeepSeek-V4: 压缩注意力撑起 1M 上下文" §2.1), or the single-path,
 *      non-overlapping variant with m' tokens per entry (reading notes §2.4.1 eqs. 20-23),
 *      which with m = 4, no bias and an indexer is the CSA2 layer (PaperTrace §6.4,
 *      V4.1-Flash paragraph);
 *   2. lightning-indexer scores I_{t,s} = sum_h w_{t,h} ReLU(q^I_{t,h} . K^I_s)
 *      (reading notes §2.3.2 eq. 16);
 *   3. per-query top-k over the visible entries (reading notes eq. 17);
 *   4. shared-KV multi-query attention over the selected entries plus a window of the
 *      n_win most recent uncompressed tokens, with a per-head sink logit in the softmax
 *      denominator, RMSNorm on query and KV heads, RoPE on the last rope_dim dims and the
 *      output de-rotated by the query position (reading notes eq. 19, §2.5.1-2.5.4 eq. 27;
 *      PaperTrace §2.4).
 *
 * Conventions that hold for every entry point:
 *   - Every pointer argument that names a tensor is a DEVICE pointer owned by the caller.
 *     The library allocates no device memory and keeps no state between calls; scratch space
 *     is the caller's `ws` buffer, sized with csa_workspace_size().
 *   - Work is enqueued on `stream` and the call returns without waiting for it.  A fault
 *     inside a kernel surfaces at the caller's next synchronisation.
 *   - Positions are 0-based token indices and live in device memory, so they cannot be
 *     checked on the host: they are clamped, not validated (visible entries of a query at
 *     position tau are min(tau / m, n_entries[seq])).
 *   - All argument checks run on the host before anything is enqueued.  On error nothing
 *     is enqueued, the return value is a csa_status and csa_last_error() holds a message.
 *   - Tensors are dense, row-major, with the shapes given in brackets.
 *   - Calls that share a cache, workspace or output buffer and overlap in time (different
 *     streams without ordering) race.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 2

typedef enum csa_status {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive or inconsistent sizes */
  CSA_ERR_UNSUPPORTED = 2,      /* a size/format combination the library has no kernel for */
  CSA_ERR_WORKSPACE_TOO_SMALL = 3,
  CSA_ERR_HIP = 4               /* a HIP launch failed; csa_last_error() has the HIP text */
} csa_status;

typedef enum csa_format {
  CSA_FMT_F32 = 0,        /* float32 */
  CSA_FMT_BF16 = 1,       /* bfloat16 */
  CSA_FMT_E4M3 = 2,       /* OCP FP8 E4M3 (e4m3fn), unit scale */
  CSA_FMT_E4M3_BF16 = 3,  /* KV rows: c - rope_dim E4M3 bytes, then rope_dim bfloat16 */
  CSA_FMT_MXFP4 = 4,      /* OCP MX FP4: blocks of 32 E2M1 elements sharing one E8M0 scale */
  CSA_FMT_MXFP4_BF16 = 5  /* KV rows (CSA2's FP4 main KV): rope_dim bfloat16, then the other
                             dims as MXFP4 element bytes, then their scale codes, zero-padded */
} csa_format;

/* Operation selector for csa_workspace_size(). */
typedef enum csa_op {
  CSA_OP_COMPRESS = 0,
  CSA_OP_INDEX_TOPK = 1,
  CSA_OP_ATTEND = 2,
  CSA_OP_FORWARD = 3
} csa_op;

/*
 * Layer shape and formats.
 *   d         hidden size of h_t.
 *   c         width of a KV entry and of each query head (reading notes eq. 19: o in R^c).
 *   rope_dim  trailing dims under RoPE (the pages use 64); even, <= c.
 *   n_h       query heads; n_hI, c_I indexer heads and width (reading notes §2.3.2).
 *   m         tokens per entry: m for CSA (pages: 4), m' for HCA (pages: 128).
 *   dual      1 = CSA (a|b overlapping fold, indexer, top-k); 0 = single path: HCA with
 *             top_k = 0 (dense), CSA2 with top_k > 0 (PaperTrace §6.4, V4.1-Flash paragraph:
 *             no overlapping windows and no in-block bias; the index keys are projected from
 *             the main entry, K^I = RMSNorm(entry) . W^IK, before RoPE and storage).
 *   top_k     entries kept per query (pages: 512 Flash, 1024 Pro); 0 = dense (HCA).
 *   n_win     sliding-window length (pages: 128); the window of a query at tau covers
 *             positions max(0, tau - n_win + 1) .. tau, the query's own token included.
 *             n_win >= m is required (INVALID_ARGUMENT otherwise), for CSA and HCA alike: a
 *             query sees only complete entries, so the window must cover the open block.
 *   scale     softmax scale on q.k; <= 0 selects 1/sqrt(c).
 *   rope_base RoPE base (10000); pair j of the RoPE dims turns by pos * base^(-2j/rope_dim).
 *   rms_eps   RMSNorm epsilon (1e-6).
 *   act_fmt   F32 or BF16: hidden states, projection weights, queries q, indexer weights w,
 *             and the attention output.
 *   kv_fmt    F32 (c floats per row), E4M3_BF16 (c - rope_dim + 2 * rope_dim bytes per row:
 *             RoPE dims kept in BF16, the rest in FP8, as the explainer's key-numbers table and
 *             PaperTrace §2.5 state) or MXFP4_BF16 (CSA2's FP4 main KV, PaperTrace §6.4: the
 *             FP8 dims become MXFP4 under the MX rule below, the RoPE dims stay BF16; for
 *             c = 512, rope_dim = 64 a 384-byte row: 128 bytes of BF16 RoPE dims, 224 bytes
 *             of E2M1 codes for dims 0..447 (dim 2i in the low nibble), 14 scale codes, 18
 *             zero bytes, so that a row fills three 128-byte lines).
 *   idx_fmt   F32, E4M3 or MXFP4: indexer keys K^I and indexer queries q^I.  MXFP4 is the
 *             pages' later FP4 indexer path (PaperTrace §3.3: 1x32 sub-blocks with their own
 *             scales) in the OCP MX v1.0 format: per block of 32 dims one E8M0
 *             scale code (2^(code - 127)) and 32 E2M1 codes, two per byte (dim 2i in the low
 *             nibble).  Per sequence, ki holds cap rows of c_I / 2 element bytes, then cap
 *             rows of c_I / 32 scale codes; per query, q^I holds n_hI rows of c_I / 2 element
 *             bytes, then n_hI rows of c_I / 32 scale codes.  Keys are encoded by the MX rule:
 *             scale 2^(floor(log2 max|v|) - 2) (1 for an all-zero block), elements rounded to
 *             nearest, ties to even, saturating at +-6.
 */
typedef struct csa_dims {
  int32_t d, c, rope_dim, n_h, c_I, n_hI, m;
  int32_t dual;
  int32_t top_k;
  int32_t n_win;
  float scale;
  float rope_base;
  float rms_eps;
  int32_t act_fmt;
  int32_t kv_fmt;
  int32_t idx_fmt;
} csa_dims;

/*
 * Compression weights, stored transposed (row u of a [width][d] matrix is column u of the
 * pages' W in R^{d x width}), in act_fmt.
 *   CSA: w_kv  [4][c][d]   = W^{aKV}, W^{bKV}, W^{aZ}, W^{bZ}       (reading notes eqs. 9-10)
 *        w_idx [4][c_I][d] = the same four for the indexer keys   (K^IComp: the deep dive,
 *                            §3.2, compresses the keys the same way at a smaller width)
 *        bias     [2][m][c]   = B^a, B^b (float32)                 (eq. 11)
 *        bias_idx [2][m][c_I] = the indexer's B^a, B^b (float32)
 *   HCA: w_kv  [2][c][d]   = W^{KV}, W^{Z}                          (eqs. 20-21)
 *        w_idx = NULL, bias [m][c] = B (float32) (eq. 22), bias_idx = NULL
 *   CSA2 (dual = 0, top_k > 0): w_kv [2][c][d] = W^{KV}, W^{Z}; bias = NULL (no in-block
 *        bias; a bias, if given, is added as for HCA); w_idx [c_I][c] = W^IK transposed, the
 *        projection of the normalised entry onto the index key; bias_idx = NULL.
 *   gamma_kv [c] float32 RMSNorm weight of the KV head, or NULL for ones.
 */
typedef struct csa_weights {
  const void* w_kv;
  const void* w_idx;
  const float* bias;
  const float* bias_idx;
  const float* gamma_kv;
} csa_weights;

/*
 * Per-sequence cache, all caller-owned device memory.
 *   B        number of sequences.
 *   cap      entry capacity per sequence; entries past it are not stored.  With a block
 *            table, the logical capacity: at most max_blocks * page_tokens / m.
 *   win_cap  window ring rows per sequence, >= n_win.  Token j's raw row sits in slot
 *            j % win_cap.  A compress call of T tokens needs win_cap >= T + n_win - 1 for
 *            the chunk's own queries to find their window rows.
 *   kv       [B][cap][row_bytes]   finalized entries (RMSNorm, RoPE at position m*i).
 *   ki       [B][cap][c_I]         indexer keys in idx_fmt (CSA and CSA2; NULL for HCA).
 *   n_entries[B] int32             complete entries; written by csa_compress.
 *   win      [B][win_cap][row_bytes] raw window rows: the a-path row C^a_j (HCA, CSA2:
 *                                  C_j), finalized at position j, in kv_fmt.
 *   win_pos  [B][win_cap] int32    position held by each ring slot, -1 when empty; the
 *                                  caller fills it with -1 before a sequence's first call.
 *   state    [B][S][P] float32     projections of the last S tokens (S = 2m for CSA, m for
 *                                  HCA and CSA2; P = 4c + 4c_I for CSA, 2c for HCA and
 *                                  CSA2), slot j % S, so
 *                                  that a block split across calls still folds.
 * Successive csa_compress calls on a sequence must cover consecutive positions.
 *
 * Paged layout (PaperTrace "02 · DeepSeek-V4: 压缩注意力撑起 1M 上下文" §3.3, KV-cache
 * paragraph: compressed entries are kept in blocks of lcm(m, m') = 128 raw tokens, and each
 * request holds one fixed-size state block for the window KV and the uncompressed tail).
 * With block_table set, kv and ki are pools of n_pages pages instead of per-sequence runs:
 *   page_tokens  raw tokens per page (128 = lcm(4, 128) serves CSA and HCA layers with one
 *                table); a multiple of m, so a page holds E = page_tokens / m entries.
 *   block_table  [B][max_blocks] int32 device array: logical page j of sequence b (its
 *                entries j E .. j E + E - 1) is pool page block_table[b][j].  Page ids are not
 *                validated (they live in device memory); they are clamped to [0, n_pages).
 *   kv           [n_pages][E][row_bytes]; entry i of sequence b at page
 *                block_table[b][i / E], row i % E.
 *   ki           E4M3 / F32: [n_pages][E][c_I]; MXFP4: per page E rows of c_I / 2 element
 *                bytes, then E rows of c_I / 32 scale codes.
 *   win, win_pos, state, n_entries stay per sequence: they are the request's state block.
 * The table is read, never written: the caller maps pages before a call writes into them.
 * With block_table NULL (max_blocks, page_tokens and n_pages ignored) the layout is the
 * contiguous one above.
 */
typedef struct csa_cache {
  int32_t B;
  int32_t cap;
  int32_t win_cap;
  void* kv;
  void* ki;
  int32_t* n_entries;
  void* win;
  int32_t* win_pos;
  float* state;
  const int32_t* block_table;
  int32_t max_blocks;
  int32_t page_tokens;
  int32_t n_pages;
} csa_cache;

/* Version of this header the library was built from (CSA_ABI_VERSION). */
int csa_abi_version(void);

/* Static text for a csa_status value. */
const char* csa_status_string(int status);

/* Message of the last failed call on this host thread ("" if none).  Thread-local. */
const char* csa_last_error(void);

/* Bytes of one stored KV row for these dims (4c, or c - rope_dim + 2 rope_dim); 0 if the
 * dims are invalid. */
size_t csa_row_bytes(const csa_dims* dims);

/* Floats per token held in csa_cache.state (P above) and state rows per sequence (S). */
int32_t csa_state_width(const csa_dims* dims);
int32_t csa_state_rows(const csa_dims* dims);

/*
 * Workspace bytes for one call of `op`:
 *   COMPRESS   B sequences x T tokens.
 *   INDEX_TOPK Q queries against entry capacity cap.
 *   ATTEND     Q queries against entry capacity cap; enough for a sparse (idx given) or a
 *              dense (idx = NULL) call.
 *   FORWARD    B x T new tokens, queries = those tokens, entry capacity cap.  With
 *              q_chunk > 0 the indexer works on q_chunk queries at a time and the score
 *              buffer shrinks accordingly; 0 means all B*T at once.
 * Returns CSA_OK and writes *bytes, or an error for invalid dims.
 */
int csa_workspace_size(const csa_dims* dims, int32_t op, int32_t B, int32_t T, int32_t Q,
                       int32_t cap, int32_t q_chunk, size_t* bytes);

/*
 * Compress T new tokens of each of cache->B sequences (reading notes eqs. 9-12 / 20-23).
 *   H     [B][T][d] hidden states in act_fmt; token t of sequence b sits at position
 *         pos0[b] + t.
 *   pos0  [B] int32 device array: position of each sequence's first new token.
 * Writes: the raw window row of every new token (ring slot, win_pos); every entry whose
 * block completes inside the chunk (kv, ki; entry i of a CSA layer folds the a-rows of
 * tokens m i .. m i + m - 1 and the b-rows of tokens m(i-1) .. m i - 1, entry 0 a-rows only);
 * n_entries[b] = min(cap, (pos0[b] + T) / m); and the projection state.
 * Entries are RMS-normalised with gamma_kv and rotated to position m*i; indexer keys are
 * stored as folded (no norm, no rotation).
 * Errors: INVALID_ARGUMENT (null pointer, T < 1, win_cap < n_win), UNSUPPORTED,
 * WORKSPACE_TOO_SMALL, HIP_ERROR.
 */
int csa_compress(const csa_dims* dims, const csa_weights* w, const csa_cache* cache,
                 const void* H, int32_t T, const int32_t* pos0, void* ws, size_t ws_bytes,
                 hipStream_t stream);

/*
 * Indexer scores and top-k selection for Q queries (reading notes eqs. 16-17), CSA only.
 *   qI      [Q][n_hI][c_I] indexer queries in idx_fmt.
 *   w       [Q][n_hI] indexer head weights in act_fmt.
 *   q_seq   [Q] int32 sequence of each query; q_pos [Q] int32 its position tau.
 *   idx_out [Q][top_k] int32: the selected entry indices in increasing order, -1 padded.
 *           A query sees V = min(tau / m, n_entries[seq]) entries (its own block is
 *           excluded); if V <= top_k all V are taken; equal scores go to the lower index.
 *   scores_out  NULL, or [Q][cap] receiving the scores of the visible entries (entries
 *           s >= V are left untouched): float32, or with idx_fmt MXFP4 bfloat16, the pages'
 *           BF16 index scores of the FP4 path (PaperTrace §3.3), each the exact score
 *           rounded to nearest even.
 * Errors: INVALID_ARGUMENT (null pointer, Q < 1, top_k = 0), UNSUPPORTED
 * (V could exceed what the selection kernels handle for this top_k), WORKSPACE_TOO_SMALL,
 * HIP_ERROR.
 */
int csa_index_topk(const csa_dims* dims, const csa_cache* cache, const void* qI,
                   const void* w, const int32_t* q_seq, const int32_t* q_pos, int32_t Q,
                   int32_t* idx_out, void* scores_out, void* ws, size_t ws_bytes,
                   hipStream_t stream);

/*
 * csa_index_topk for queries laid out as a prefill chunk's are (every aligned group of 16
 * queries belongs to one sequence, as for csa_index_scores_grouped; the caller guarantees
 * it).  The selection is csa_index_topk's, index for index.  With E4M3 keys and 64 indexer
 * heads the indexer shares key tiles among a group's queries and also takes each query's
 * threshold itself: from a sample of the group's scores it keeps, per query, every score at
 * or above the sample's r-th largest (r set for about 3072 of the row), and the selection
 * runs on those lists (an upper set of the row, so they hold the top k whenever they number
 * at least k; otherwise, or when they overflow, on the whole row).  This is the indexer and
 * selection csa_forward runs on a chunk of such queries.  ws: as csa_index_topk
 * (csa_workspace_size(INDEX_TOPK) covers both).
 * Errors: as csa_index_topk.
 */
int csa_index_topk_grouped(const csa_dims* dims, const csa_cache* cache, const void* qI,
                           const void* w, const int32_t* q_seq, const int32_t* q_pos, int32_t Q,
                           int32_t* idx_out, void* scores_out, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * The indexer on its own (reading notes eq. 16): scores[q][s] for s < V of each query, in
 * float32 (bfloat16 with idx_fmt MXFP4, as in csa_index_topk), row stride ld (>= the largest V; cache->cap always works).  Entries s >= V are
 * left untouched.  csa_index_topk = csa_index_scores + csa_topk.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, HIP_ERROR.
 */
int csa_index_scores(const csa_dims* dims, const csa_cache* cache, const void* qI,
                     const void* w, const int32_t* q_seq, const int32_t* q_pos, int32_t Q,
                     void* scores, int64_t ld, hipStream_t stream);

/*
 * csa_index_scores for queries laid out as a prefill chunk's are (query b*T + t is token t of
 * sequence b, T a multiple of 16): every aligned group of 16 queries (0-15, 16-31, ...)
 * belongs to one sequence, which the caller guarantees (it cannot be checked on the host).
 * The scores are those of csa_index_scores, bit for bit; the kernel shares each key tile
 * among a group's 16 queries (the indexer csa_forward runs on a chunk of such queries).
 * Errors: as csa_index_scores.
 */
int csa_index_scores_grouped(const csa_dims* dims, const csa_cache* cache, const void* qI,
                             const void* w, const int32_t* q_seq, const int32_t* q_pos, int32_t Q,
                             void* scores, int64_t ld, hipStream_t stream);

/*
 * The top-k selection on its own (reading notes eq. 17) over scores [Q][ld] as written by
 * csa_index_scores (float32, or bfloat16 with idx_fmt MXFP4): idx_out[Q][top_k] as in csa_index_topk.  ws as csa_workspace_size(
 * INDEX_TOPK) minus the score buffer: csa_topk_workspace_size(), which is 0 for caches of
 * up to 65536 entries (one workgroup selects each query's row) and ws may then be NULL.
 */
int csa_topk(const csa_dims* dims, const csa_cache* cache, const int32_t* q_seq,
             const int32_t* q_pos, int32_t Q, const void* scores, int64_t ld,
             int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes of csa_topk for Q queries against entry capacity cap. */
size_t csa_topk_workspace_size(const csa_dims* dims, int32_t Q, int32_t cap);

/*
 * Shared-KV MQA for Q queries (reading notes eqs. 19/26, 27; §2.5.1-2.5.2).
 *   q       [Q][n_h][c] query heads in act_fmt (before RMSNorm and RoPE).
 *   gamma_q [c] float32 RMSNorm weight shared by the query heads, or NULL for ones.
 *   sink    [n_h] float32 sink logits z'_h, or NULL for no sink.
 *   idx     [Q][top_k] int32 entry indices (-1 = unused slot), or NULL to attend densely to
 *           every visible entry (HCA).
 *   out     [Q][n_h][c] in act_fmt: for each head, sum_j s_j key_j over the selected entries
 *           and the window rows in one softmax with the sink in the denominator, the last
 *           rope_dim dims rotated by -tau.  Keys are shared by all heads (K = V).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP_ERROR.
 */
int csa_attend(const csa_dims* dims, const csa_cache* cache, const void* q,
               const float* gamma_q, const float* sink, const int32_t* q_seq,
               const int32_t* q_pos, int32_t Q, const int32_t* idx, void* out, void* ws,
               size_t ws_bytes, hipStream_t stream);

/*
 * The whole path for a chunk of T new tokens per sequence: csa_compress, then (CSA, CSA2)
 * csa_index_topk and csa_attend with the new tokens as queries (query b*T + t sits at
 * position pos0[b] + t), or (HCA) dense csa_attend.  A CSA2 layer that reuses an earlier
 * layer's KV and top-k (PaperTrace §6.4) runs no forward of its own: it calls csa_attend on
 * that layer's cache with that layer's idx_out and its own queries.
 *   q, qI, w  per-query inputs as in csa_index_topk / csa_attend, Q = B*T.
 *   idx_out   [Q][top_k] int32 receiving the selection, or NULL (CSA: then it lives in ws).
 * The indexer works on q_chunk queries at a time, the largest that fits ws_bytes.
 * With T = 1 a query at tau sees floor(tau / m) entries, none of which the call's own
 * compression writes, so for CSA the library may score and select before compressing (the
 * one-token projection then shares a launch with the top-k threshold pass).  For a cache whose
 * n_entries keeps pace with the positions the result is the same either way; when it trails
 * them, T = 1 calls score the entries present before the call.
 */
int csa_forward(const csa_dims* dims, const csa_weights* w, const csa_cache* cache,
                const void* H, int32_t T, const int32_t* pos0, const void* q, const void* qI,
                const void* wI, const float* gamma_q, const float* sink, void* out,
                int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa_forward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Arguments and results are those of
 * csa_forward; the workspace is a static device array of CSA_NOALLOC_SCRATCH_BYTES inside the
 * library (one per GPU, held from the first call on that GPU until the process ends), so the
 * call allocates nothing.  The device current at the call is the one used; `stream` must
 * belong to it.  Calls that overlap in time on one GPU share that array and race; calls in
 * stream order do not (nothing in the array has to survive from one call to the next, and
 * nothing in it has to start zeroed).
 * Errors: as csa_forward; WORKSPACE_TOO_SMALL (before any HIP call) when the call needs more
 * workspace than the array holds (csa_workspace_size with op FORWARD tells; decode steps of one
 * token per sequence need a few MiB, prefill chunks of some thousand tokens fit, longer chunks
 * need csa_forward); HIP_ERROR when the array's device address cannot be looked up.
 */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int csa_forward_noalloc(const csa_dims* dims, const csa_weights* w, const csa_cache* cache,
                        const void* H, int32_t T, const int32_t* pos0, const void* q, const void* qI,
                        const void* wI, const float* gamma_q, const float* sink, void* out,
                        int32_t* idx_out, hipStream_t stream);

/* Size of csa_forward_noalloc's static scratch (CSA_NOALLOC_SCRATCH_BYTES). */
size_t csa_noalloc_scratch_bytes(void);

/*
 * The projections around the attention core: the low-rank query path before it (reading
 * notes "DeepSeekV4技术报告阅读笔记" §2.3.2 eqs. 13-15 and §2.3.3 eq. 18: one latent
 * c^Q = h W^DQ of width d_c feeds both the attention queries q = c^Q W^UQ and the indexer
 * queries q^I = c^Q W^IUQ; the indexer head weights are w = h W^w) and the grouped output
 * projection after it (§2.3.3, "Grouped Output Projection"; deep dive "DeepSeek-V4 架构设计深度
 * 解析" stage three: the n_h heads form g consecutive groups, group i's c n_h / g values are
 * projected to d_g by its own map, and the g d_g concatenated values are projected to d;
 * g = 16 (Pro) or 8 (Flash), d_g = 1024; PaperTrace §1: d_c = 1536 from the 1536 x 128 x 512
 * query up-projection, §2.2: g and d_g).
 * Every matrix W in R^{a x b} is stored transposed, bf16 [b][a] (one row per output column,
 * the a inputs contiguous).  The weights are the caller's; the library only reads them.
 */
typedef struct csa_proj_weights {
  const void* w_dq;   /* [d_c][d] bf16: W^DQ */
  const void* w_uq;   /* [n_h * c][d_c] bf16: W^UQ */
  const void* w_iuq;  /* [n_hI * c_I][d_c] bf16: W^IUQ (CSA, CSA2; not read when top_k = 0) */
  const void* w_w;    /* [n_hI][d] bf16: W^w (CSA, CSA2; not read when top_k = 0) */
  const void* w_og;   /* [g][d_g][n_h * c / g] bf16: group i's map at w_og + i d_g (n_h c / g) */
  const void* w_o;    /* [d][g * d_g] bf16: the map of the concatenated groups to d */
  int32_t d_c;        /* latent width, a multiple of 64 */
  int32_t g;          /* output groups: divides n_h, with c n_h / g a multiple of 64 */
  int32_t d_g;        /* width of a group's projection, a multiple of 64 */
} csa_proj_weights;

/*
 * Bytes of workspace csa_query_project needs for T tokens (0 on invalid arguments).
 */
size_t csa_query_project_workspace_size(const csa_dims* dims, const csa_proj_weights* pw,
                                        int32_t T);

/*
 * The query side for T tokens, formats act BF16 (with kv E4M3_BF16):
 *   h   [T][d] bf16 hidden states (device).
 *   q   [T][n_h][c] bf16 out: the attention queries, as csa_attend reads them.
 *   qI  [T] rows out in the indexer's format (idx_fmt E4M3: [n_hI][c_I] codes; MXFP4: n_hI
 *       rows of c_I / 2 element bytes then n_hI rows of c_I / 32 scale codes, the encoding
 *       of the keys), as csa_index_topk reads them.  NULL when top_k = 0 (HCA).
 *   w   [T][n_hI] bf16 out: the indexer head weights.  NULL when top_k = 0 (HCA).
 * c^Q is held in bf16 between the two products; accumulation is float32.  ws (device,
 * csa_query_project_workspace_size bytes) holds c^Q and split-K partial sums.
 * Errors: INVALID_ARGUMENT (null pointer, T < 1), UNSUPPORTED (formats or widths outside the
 * above), WORKSPACE_TOO_SMALL, HIP_ERROR.
 */
int csa_query_project(const csa_dims* dims, const csa_proj_weights* pw, const void* h,
                      int32_t T, void* q, void* qI, void* w, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * Bytes of workspace csa_output_project needs for T tokens (0 on invalid arguments).
 */
size_t csa_output_project_workspace_size(const csa_dims* dims, const csa_proj_weights* pw,
                                         int32_t T);

/*
 * The grouped output projection for T tokens:
 *   o    [T][n_h][c] bf16 attention output (device; csa_attend's out).
 *   out  [T][d] bf16 out.
 * The g d_g concatenated group outputs are held in bf16 before the last product;
 * accumulation is float32.  ws as csa_output_project_workspace_size.
 * Errors: as csa_query_project.
 */
int csa_output_project(const csa_dims* dims, const csa_proj_weights* pw, const void* o,
                       int32_t T, void* out, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
