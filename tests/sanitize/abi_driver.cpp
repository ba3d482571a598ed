// Host-side driver for the sanitizer build of libcsa: calls every entry point of csa.h on
// argument-error paths and the pure host planners (sizes, workspace plans), with no GPU.
// Built with AddressSanitizer and UndefinedBehaviorSanitizer on the host code; any report
// fails the run.  Fake device pointers are never dereferenced: every call below fails its
// host checks before anything is enqueued.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "csa.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::printf("FAILED line %d: %s (%s)\n", __LINE__, #cond, csa_last_error()); \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

static csa_dims flash(int dual, int top_k, int kv_fmt, int idx_fmt) {
  csa_dims d;
  std::memset(&d, 0, sizeof d);
  d.d = 4096; d.c = 512; d.rope_dim = 64; d.n_h = 64; d.c_I = 128; d.n_hI = 64; d.m = 4;
  d.dual = dual; d.top_k = top_k; d.n_win = 128; d.scale = 0.f; d.rope_base = 10000.f;
  d.rms_eps = 1e-6f; d.act_fmt = CSA_FMT_BF16; d.kv_fmt = kv_fmt; d.idx_fmt = idx_fmt;
  return d;
}

int main() {
  void* fake = reinterpret_cast<void*>(0x1000);
  EXPECT(csa_abi_version() == CSA_ABI_VERSION);
  for (int st = 0; st < 6; ++st) EXPECT(csa_status_string(st) != nullptr);

  const csa_dims layers[] = {flash(1, 512, CSA_FMT_E4M3_BF16, CSA_FMT_E4M3),
                             flash(1, 512, CSA_FMT_E4M3_BF16, CSA_FMT_MXFP4),
                             flash(0, 0, CSA_FMT_E4M3_BF16, CSA_FMT_E4M3),
                             flash(0, 512, CSA_FMT_MXFP4_BF16, CSA_FMT_E4M3)};
  for (const csa_dims& d : layers) {
    EXPECT(csa_row_bytes(&d) > 0);
    EXPECT(csa_state_width(&d) > 0);
    EXPECT(csa_state_rows(&d) > 0);
    size_t b = 0;
    for (int op = 0; op < 4; ++op) {
      const int st = csa_workspace_size(&d, op, 16, 1, 16, 32768, 0, &b);
      EXPECT(st == CSA_OK || (op == CSA_OP_INDEX_TOPK && d.top_k == 0));
    }
    EXPECT(csa_workspace_size(&d, CSA_OP_FORWARD, 1, 32768, 0, 270336, 4096, &b) == CSA_OK);
    EXPECT(csa_workspace_size(&d, 99, 1, 1, 1, 1, 0, &b) == CSA_ERR_INVALID_ARGUMENT);
    EXPECT(csa_workspace_size(&d, CSA_OP_COMPRESS, 1, 1, 1, 1, 0, nullptr) == CSA_ERR_INVALID_ARGUMENT);
    // rows longer than one selection workgroup's share need candidate lists
    EXPECT(csa_topk_workspace_size(&d, 4, 262144) > 0 || d.top_k == 0);
  }
  // invalid dims: every check path
  csa_dims bad = layers[0];
  bad.c = 63;
  EXPECT(csa_row_bytes(&bad) == 0);
  bad = layers[0]; bad.rope_dim = 70;
  EXPECT(csa_state_width(&bad) == 0);
  bad = layers[0]; bad.n_win = 2;
  size_t b = 0;
  EXPECT(csa_workspace_size(&bad, CSA_OP_COMPRESS, 1, 1, 1, 1, 0, &b) == CSA_ERR_INVALID_ARGUMENT);
  bad = layers[0]; bad.c = 256;
  EXPECT(csa_workspace_size(&bad, CSA_OP_COMPRESS, 1, 1, 1, 1, 0, &b) == CSA_ERR_UNSUPPORTED);
  EXPECT(csa_row_bytes(nullptr) == 0);

  // caches: contiguous and paged, with argument errors
  csa_cache c;
  std::memset(&c, 0, sizeof c);
  c.B = 2; c.cap = 64; c.win_cap = 128;
  c.kv = fake; c.ki = fake; c.n_entries = (int32_t*)fake; c.win = fake; c.win_pos = (int32_t*)fake;
  c.state = (float*)fake;
  csa_weights w;
  std::memset(&w, 0, sizeof w);
  w.w_kv = fake; w.w_idx = fake; w.bias = (const float*)fake; w.bias_idx = (const float*)fake;
  const csa_dims& d2 = layers[0];
  EXPECT(csa_compress(&d2, &w, &c, fake, 0, (const int32_t*)fake, fake, 1 << 30, nullptr) == CSA_ERR_INVALID_ARGUMENT);
  EXPECT(csa_compress(&d2, &w, &c, fake, 4, (const int32_t*)fake, fake, 16, nullptr) == CSA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(csa_compress(&d2, nullptr, &c, fake, 4, (const int32_t*)fake, fake, 1 << 30, nullptr) == CSA_ERR_INVALID_ARGUMENT);
  EXPECT(csa_index_topk(&d2, &c, fake, fake, (const int32_t*)fake, (const int32_t*)fake, 0, (int32_t*)fake, nullptr,
                        fake, 1 << 30, nullptr) == CSA_ERR_INVALID_ARGUMENT);
  EXPECT(csa_index_topk_grouped(&d2, &c, fake, fake, (const int32_t*)fake, (const int32_t*)fake, 0, (int32_t*)fake,
                                nullptr, fake, 1 << 30, nullptr) == CSA_ERR_INVALID_ARGUMENT);
  EXPECT(csa_index_topk_grouped(&d2, &c, fake, fake, (const int32_t*)fake, (const int32_t*)fake, 16, (int32_t*)fake,
                                nullptr, fake, 16, nullptr) == CSA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(csa_index_scores(&d2, &c, fake, fake, (const int32_t*)fake, (const int32_t*)fake, 1, fake, 8, nullptr) ==
         CSA_ERR_INVALID_ARGUMENT);
  EXPECT(csa_index_scores_grouped(&d2, &c, fake, fake, (const int32_t*)fake, (const int32_t*)fake, 1, fake, 8,
                                  nullptr) == CSA_ERR_INVALID_ARGUMENT);
  EXPECT(csa_topk(&d2, &c, (const int32_t*)fake, (const int32_t*)fake, 1, fake, 8, (int32_t*)fake, fake, 1 << 30,
                  nullptr) == CSA_ERR_INVALID_ARGUMENT);
  EXPECT(csa_attend(&d2, &c, fake, nullptr, nullptr, (const int32_t*)fake, (const int32_t*)fake, 0, (const int32_t*)fake,
                    fake, fake, 1 << 30, nullptr) == CSA_ERR_INVALID_ARGUMENT);
  EXPECT(csa_forward(&d2, &w, &c, fake, 64, (const int32_t*)fake, fake, fake, fake, nullptr, nullptr, fake, nullptr,
                     fake, 1 << 30, nullptr) == CSA_ERR_INVALID_ARGUMENT);
  csa_cache big = c;
  big.B = 1; big.cap = 270336; big.win_cap = 32768 + 128;
  EXPECT(csa_forward_noalloc(&d2, &w, &big, fake, 32768, (const int32_t*)fake, fake, fake, fake, nullptr, nullptr,
                             fake, (int32_t*)fake, nullptr) == CSA_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(csa_noalloc_scratch_bytes() == CSA_NOALLOC_SCRATCH_BYTES);
  // paged caches
  csa_cache pg = c;
  pg.block_table = (const int32_t*)fake; pg.max_blocks = 4; pg.page_tokens = 102; pg.n_pages = 8;
  EXPECT(csa_attend(&d2, &pg, fake, nullptr, nullptr, (const int32_t*)fake, (const int32_t*)fake, 1, (const int32_t*)fake,
                    fake, fake, 1 << 30, nullptr) == CSA_ERR_INVALID_ARGUMENT);   // not a multiple of m
  pg.page_tokens = 8;
  EXPECT(csa_attend(&d2, &pg, fake, nullptr, nullptr, (const int32_t*)fake, (const int32_t*)fake, 1, (const int32_t*)fake,
                    fake, fake, 1 << 30, nullptr) == CSA_ERR_INVALID_ARGUMENT);   // cap beyond the table
  // CSA2 weights without the key projection
  csa_weights w2 = w;
  w2.w_idx = nullptr;
  EXPECT(csa_compress(&layers[3], &w2, &c, fake, 4, (const int32_t*)fake, fake, 1 << 30, nullptr) ==
         CSA_ERR_INVALID_ARGUMENT);
  // projections
  csa_proj_weights pw;
  std::memset(&pw, 0, sizeof pw);
  pw.w_dq = fake; pw.w_uq = fake; pw.w_iuq = fake; pw.w_w = fake; pw.w_og = fake; pw.w_o = fake;
  pw.d_c = 1536; pw.g = 8; pw.d_g = 1024;
  EXPECT(csa_query_project_workspace_size(&d2, &pw, 16) > 0);
  EXPECT(csa_output_project_workspace_size(&d2, &pw, 16) > 0);
  EXPECT(csa_query_project(&d2, &pw, fake, 0, fake, fake, fake, fake, 1 << 30, nullptr) == CSA_ERR_INVALID_ARGUMENT);
  EXPECT(csa_output_project(&d2, &pw, fake, 0, fake, fake, 1 << 30, nullptr) == CSA_ERR_INVALID_ARGUMENT);
  std::printf("sanitizer driver: %d failures\n", failures);
  return failures ? 1 : 0;
}
