// Host-side checks of libfdllm's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point is called with arguments it
// must reject (NULL descriptors and pointers, out-of-range scalars,
// misaligned pointers, short workspaces, extreme sizes) and must return the
// documented FDLLM_ERR_* code with a message, before any launch.  The
// workspace and packed-size queries run over valid geometries up to the
// largest sizes the header allows, so the planners' size arithmetic runs
// under the overflow checks too.  No GPU is needed: nothing here reaches a
// kernel launch.  Exit status 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <limits>

#include "fdllm.h"

static int g_failures = 0;
static int g_checks = 0;

static void expect(fdllm_status got, fdllm_status want, const char* what) {
  ++g_checks;
  const char* msg = fdllm_last_error();
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d (%s), want %d; last error: %s\n", what, (int)got,
            fdllm_status_string(got), (int)want, msg ? msg : "(null)");
    ++g_failures;
  } else if (want != FDLLM_OK && (!msg || !msg[0])) {
    fprintf(stderr, "FAIL %s: rejected without a message\n", what);
    ++g_failures;
  }
}

static void expect_zero(size_t got, const char* what) {
  ++g_checks;
  if (got != 0) {
    fprintf(stderr, "FAIL %s: %zu, want 0\n", what, got);
    ++g_failures;
  }
}

// Stand-ins for device buffers: never dereferenced on a rejection path.
// Slot n is 1 TiB past slot n - 1, so no two of them overlap whatever the
// tensor sizes the geometry implies; an offset below 256 misaligns one.
static void* P(size_t off = 0) { return (void*)((uintptr_t)(1 + off / 256) << 40 | (off % 256)); }

static fdllm_seq_desc dream_seq() {
  fdllm_seq_desc s;
  memset(&s, 0, sizeof(s));
  s.batch = 8;
  s.max_seq_len = 2048;
  s.gen_len = 1024;
  s.block_size = 32;
  s.prompt_len = 1024;
  s.block_idx = 3;
  return s;
}

static fdllm_attn_desc dream_attn() {
  fdllm_attn_desc a;
  a.n_q_heads = 28;
  a.n_kv_heads = 4;
  a.head_dim = 128;
  a.dtype = FDLLM_BF16;
  a.scale = 0.f;
  return a;
}

static fdllm_status attn_call(const fdllm_seq_desc* s, const fdllm_attn_desc* a, int32_t mode, int32_t rows,
                              const void* q, const void* kn, const void* vn, const void* kc, const void* vc,
                              void* out, void* ws, size_t ws_bytes) {
  return fdllm_block_attn(s, a, mode, rows, q, kn, vn, kc, vc, out, ws, ws_bytes, nullptr);
}

static void attention() {
  fdllm_seq_desc s = dream_seq();
  fdllm_attn_desc a = dream_attn();
  const int D = FDLLM_CACHE_DUAL;
  void *q = P(0), *kn = P(256), *vn = P(512), *kc = P(768), *vc = P(1024), *out = P(1280);
  expect(attn_call(nullptr, &a, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn NULL seq");
  expect(attn_call(&s, nullptr, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn NULL desc");
  expect(attn_call(&s, &a, 7, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn mode");
  expect(attn_call(&s, &a, D, 31, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn fresh_rows");
  expect(attn_call(&s, &a, D, 32, nullptr, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn NULL q");
  expect(attn_call(&s, &a, D, 32, q, kn, vn, nullptr, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG,
         "attn NULL cache (dual)");
  expect(attn_call(&s, &a, D, 32, P(8), kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn misaligned q");
  expect(attn_call(&s, &a, D, 32, q, kn, vn, kc, vc, (void*)q, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn out aliases q");
  fdllm_attn_desc b = a;
  b.head_dim = 96;
  expect(attn_call(&s, &b, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_UNSUPPORTED, "attn head_dim 96");
  b = a;
  b.n_q_heads = 30;
  expect(attn_call(&s, &b, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn Hq % Hkv");
  b = a;
  b.scale = -1.f;
  expect(attn_call(&s, &b, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn negative scale");
  b.scale = std::numeric_limits<float>::quiet_NaN();
  expect(attn_call(&s, &b, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn NaN scale");
  b = a;
  b.dtype = 9;
  expect(attn_call(&s, &b, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn dtype");
  b = a;
  b.n_kv_heads = 0;
  expect(attn_call(&s, &b, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn Hkv 0");
  // geometry
  fdllm_seq_desc t = s;
  t.batch = 0;
  expect(attn_call(&t, &a, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn batch 0");
  t = s;
  t.gen_len = 1000;
  expect(attn_call(&t, &a, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn G % B");
  t = s;
  t.block_idx = 32;
  expect(attn_call(&t, &a, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn block_idx");
  t = s;
  t.prompt_len = std::numeric_limits<int32_t>::max();
  expect(attn_call(&t, &a, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn P + G overflow");
  t = s;
  t.max_seq_len = 2047;
  expect(attn_call(&t, &a, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG, "attn L > Lcap");
  t = s;
  t.prompt_lens = (const int32_t*)P(2048);
  t.max_prompt_len = -1;
  expect(attn_call(&t, &a, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_INVALID_ARG,
         "attn max_prompt_len -1");
  // workspace: a geometry with split partials, called without a workspace
  t = s;
  t.batch = 1;
  const size_t need = fdllm_block_attn_workspace(&t, &a, D, 32);
  if (need > 0) {
    expect(attn_call(&t, &a, D, 32, q, kn, vn, kc, vc, out, nullptr, 0), FDLLM_ERR_WORKSPACE, "attn no workspace");
    expect(attn_call(&t, &a, D, 32, q, kn, vn, kc, vc, out, P(16), need - 16), FDLLM_ERR_WORKSPACE,
           "attn short workspace");
    expect(attn_call(&t, &a, D, 32, q, kn, vn, kc, vc, out, P(8), need), FDLLM_ERR_INVALID_ARG,
           "attn misaligned workspace");
  }
  expect_zero(fdllm_block_attn_workspace(nullptr, &a, D, 32), "attn workspace NULL seq");
  expect_zero(fdllm_block_attn_workspace(&s, &a, 5, 32), "attn workspace bad mode");
  // the planners over many valid geometries (sizes only; largest first)
  const int32_t modes[3] = {FDLLM_CACHE_NONE, FDLLM_CACHE_PREFIX, FDLLM_CACHE_DUAL};
  const int32_t batches[4] = {1, 7, 64, 4096};
  const int32_t gens[3] = {32, 256, 1024};
  const int32_t prompts[3] = {0, 37, 8192};
  const int32_t dims[2] = {64, 128};
  for (int32_t m : modes)
    for (int32_t bb : batches)
      for (int32_t G : gens)
        for (int32_t Pp : prompts)
          for (int32_t d : dims)
            for (int32_t dt = 0; dt < 2; ++dt) {
              fdllm_seq_desc u = s;
              u.batch = bb;
              u.gen_len = G;
              u.prompt_len = Pp;
              u.block_idx = 0;
              u.max_seq_len = Pp + G;
              fdllm_attn_desc v = a;
              v.head_dim = d;
              v.dtype = dt;
              const int32_t rows = m == FDLLM_CACHE_DUAL ? 32 : m == FDLLM_CACHE_PREFIX ? G : Pp + G;
              (void)fdllm_block_attn_workspace(&u, &v, m, rows);
            }
}

static void unmask() {
  fdllm_seq_desc s = dream_seq();
  int32_t* tok = (int32_t*)P(0);
  uint8_t* mask = (uint8_t*)P(256);
  int32_t* nd = (int32_t*)P(512);
  const void* lg = P(1024);
  const int32_t V = 126464;
  const int64_t ss = (int64_t)32 * V, rs = V;
  expect(fdllm_unmask_threshold(nullptr, V, FDLLM_BF16, lg, ss, rs, 0.9f, 0, tok, mask, nd, nullptr, nullptr, nullptr,
                                nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "unmask NULL seq");
  expect(fdllm_unmask_threshold(&s, 0, FDLLM_BF16, lg, ss, rs, 0.9f, 0, tok, mask, nd, nullptr, nullptr, nullptr,
                                nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "unmask vocab 0");
  expect(fdllm_unmask_threshold(&s, V, 5, lg, ss, rs, 0.9f, 0, tok, mask, nd, nullptr, nullptr, nullptr, nullptr,
                                nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "unmask dtype");
  expect(fdllm_unmask_threshold(&s, V, FDLLM_BF16, nullptr, ss, rs, 0.9f, 0, tok, mask, nd, nullptr, nullptr,
                                nullptr, nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "unmask NULL logits");
  expect(fdllm_unmask_threshold(&s, V, FDLLM_BF16, lg, ss, rs, std::numeric_limits<float>::quiet_NaN(), 0, tok, mask,
                                nd, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "unmask NaN threshold");
  expect(fdllm_unmask_threshold(&s, V, FDLLM_BF16, lg, ss, rs, 0.9f, 0x80, tok, mask, nd, nullptr, nullptr, nullptr,
                                nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "unmask unknown flag");
  expect(fdllm_unmask_threshold(&s, V, FDLLM_BF16, lg, ss, rs, 0.9f, FDLLM_UNMASK_ADVANCE_BLOCK, tok, mask, nd,
                                nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "unmask advance without block_idxs");
  expect(fdllm_unmask_threshold(&s, V, FDLLM_BF16, lg, ss, V - 1, 0.9f, 0, tok, mask, nd, nullptr, nullptr, nullptr,
                                nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "unmask row_stride < vocab");
  expect(fdllm_unmask_threshold(&s, V, FDLLM_BF16, lg, rs, rs, 0.9f, 0, tok, mask, nd, nullptr, nullptr, nullptr,
                                nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "unmask seq_stride overlap");
  const size_t need = fdllm_unmask_workspace(&s, V, FDLLM_BF16);
  if (need > 0)
    expect(fdllm_unmask_threshold(&s, V, FDLLM_BF16, lg, ss, rs, 0.9f, 0, tok, mask, nd, nullptr, nullptr, nullptr,
                                  nullptr, P(0), need - 1, nullptr),
           FDLLM_ERR_WORKSPACE, "unmask short workspace");
  expect(fdllm_unmask_topk(&s, V, FDLLM_BF16, lg, ss, rs, 0, 0, tok, mask, nd, nullptr, nullptr, nullptr, nullptr,
                           nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "topk k 0");
  expect(fdllm_unmask_topk(&s, V, FDLLM_BF16, lg, ss, rs, -5, 0, tok, mask, nd, nullptr, nullptr, nullptr, nullptr,
                           nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "topk k negative");
  expect(fdllm_unmask_topk(&s, V, FDLLM_BF16, lg, ss, rs, 33, 0, tok, mask, nd, nullptr, nullptr, nullptr, nullptr,
                           nullptr, 0, nullptr),
         FDLLM_ERR_WORKSPACE, "topk k > block is valid; no workspace");
  expect(fdllm_unmask_threshold_static(nullptr, V, FDLLM_BF16, lg, ss, rs, 0.9f, 0, tok, mask, nd, nullptr, nullptr,
                                       nullptr, nullptr, nullptr),
         FDLLM_ERR_INVALID_ARG, "static NULL seq");
  fdllm_seq_desc big = s;
  big.batch = 8192;
  expect(fdllm_unmask_threshold_static(&big, V, FDLLM_BF16, lg, ss, rs, 0.9f, 0, tok, mask, nd, nullptr, nullptr,
                                       nullptr, nullptr, nullptr),
         FDLLM_ERR_UNSUPPORTED, "static batch above its limit");
  fdllm_seq_desc t = s;
  t.block_size = 2048;
  t.gen_len = 2048;
  t.max_seq_len = 4096;
  t.block_idx = 0;
  expect_zero(fdllm_unmask_workspace(&t, V, FDLLM_BF16), "unmask workspace block_size 2048");
  expect_zero(fdllm_unmask_workspace(&s, 1 << 29, FDLLM_BF16), "unmask workspace vocab 2^29");
  for (int32_t bb : {1, 64, 65535})
    for (int32_t v : {1, 1000, 126464, 1 << 28}) {
      fdllm_seq_desc u = s;
      u.batch = bb;
      (void)fdllm_unmask_workspace(&u, v, FDLLM_BF16);
      (void)fdllm_unmask_workspace(&u, v, FDLLM_F32);
    }
}

static void lmhead() {
  fdllm_seq_desc s = dream_seq();
  const int32_t V = 152064, H = 3584;
  expect_zero(fdllm_lmhead_packed_bytes(0, H), "packed bytes vocab 0");
  expect_zero(fdllm_lmhead_packed_bytes(V, 12), "packed bytes hidden 12");
  expect_zero(fdllm_lmhead_packed_bytes(V, (1 << 20) + 8), "packed bytes hidden 2^20 + 8");
  for (int32_t v : {1, 255, 256, 152064, 1 << 28})
    for (int32_t h : {8, 4096, 1 << 20}) (void)fdllm_lmhead_packed_bytes(v, h);
  const size_t pb = fdllm_lmhead_packed_bytes(V, H);
  expect(fdllm_lmhead_pack(V, H, P(0), P(256), pb - 1, nullptr), FDLLM_ERR_INVALID_ARG, "pack short output");
  expect(fdllm_lmhead_pack(V, H, nullptr, P(256), pb, nullptr), FDLLM_ERR_INVALID_ARG, "pack NULL w");
  expect(fdllm_lmhead_pack(V, 12, P(0), P(256), pb, nullptr), FDLLM_ERR_UNSUPPORTED, "pack hidden 12");
  int32_t* tok = (int32_t*)P(0);
  uint8_t* mask = (uint8_t*)P(256);
  int32_t* nd = (int32_t*)P(512);
  const int64_t ss = (int64_t)32 * H, rs = H;
  expect(fdllm_lmhead_unmask_threshold(&s, V, H, P(8), ss, rs, P(1024), 0.9f, 0, tok, mask, nd, nullptr, nullptr,
                                       nullptr, nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "lmhead misaligned x");
  expect(fdllm_lmhead_unmask_threshold(&s, V, H, P(0), ss, rs - 8, P(1024), 0.9f, 0, tok, mask, nd, nullptr, nullptr,
                                       nullptr, nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "lmhead row_stride < hidden");
  expect(fdllm_lmhead_unmask_threshold(&s, V, H, P(0), ss, rs + 4, P(1024), 0.9f, 0, tok, mask, nd, nullptr, nullptr,
                                       nullptr, nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "lmhead row_stride not a multiple of 8");
  expect(fdllm_lmhead_unmask_threshold(&s, V, H, P(0), ss, rs, nullptr, 0.9f, 0, tok, mask, nd, nullptr, nullptr,
                                       nullptr, nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "lmhead NULL weights");
  expect(fdllm_lmhead_unmask_topk(&s, V, H, P(0), ss, rs, P(1024), 0, 0, tok, mask, nd, nullptr, nullptr, nullptr,
                                  nullptr, nullptr, 0, nullptr),
         FDLLM_ERR_INVALID_ARG, "lmhead topk k 0");
  const size_t need = fdllm_lmhead_unmask_workspace(&s, V, H);
  if (need > 0)
    expect(fdllm_lmhead_unmask_threshold(&s, V, H, P(0), ss, rs, P(1024), 0.9f, 0, tok, mask, nd, nullptr, nullptr,
                                         nullptr, nullptr, P(0), need - 1, nullptr),
           FDLLM_ERR_WORKSPACE, "lmhead short workspace");
  for (int32_t bb : {1, 32, 4096})
    for (int32_t v : {1, 152064}) {
      fdllm_seq_desc u = s;
      u.batch = bb;
      (void)fdllm_lmhead_unmask_workspace(&u, v, 4096);
    }
}

static void refresh_and_settings() {
  fdllm_seq_desc s = dream_seq();
  fdllm_attn_desc a = dream_attn();
  expect(fdllm_kv_refresh(nullptr, &a, FDLLM_CACHE_DUAL, P(0), P(256), P(512), P(768), nullptr, nullptr, nullptr),
         FDLLM_ERR_INVALID_ARG, "refresh NULL seq");
  expect(fdllm_kv_refresh(&s, &a, 4, P(0), P(256), P(512), P(768), nullptr, nullptr, nullptr), FDLLM_ERR_INVALID_ARG,
         "refresh mode");
  expect(fdllm_kv_refresh(&s, &a, FDLLM_CACHE_DUAL, nullptr, P(256), P(512), P(768), nullptr, nullptr, nullptr),
         FDLLM_ERR_INVALID_ARG, "refresh NULL source");
  expect(fdllm_kv_refresh(&s, &a, FDLLM_CACHE_DUAL, P(0), P(256), P(512), P(768), (const int32_t*)P(1024), nullptr,
                          nullptr),
         FDLLM_ERR_INVALID_ARG, "refresh seq_ids without n_seq");
  {
    const void* ks[2] = {P(0), P(256)};
    const void* vs[2] = {P(512), P(768)};
    void* kc[2] = {P(1024), P(1280)};
    void* vc[2] = {P(1536), P(1792)};
    void* kc_alias[2] = {P(1024), P(256)};
    expect(fdllm_kv_refresh_layers(&s, &a, FDLLM_CACHE_DUAL, 0, ks, vs, kc, vc, nullptr, nullptr, nullptr),
           FDLLM_ERR_INVALID_ARG, "refresh_layers no layer");
    expect(fdllm_kv_refresh_layers(&s, &a, FDLLM_CACHE_DUAL, 65, ks, vs, kc, vc, nullptr, nullptr, nullptr),
           FDLLM_ERR_INVALID_ARG, "refresh_layers too many layers");
    expect(fdllm_kv_refresh_layers(&s, &a, FDLLM_CACHE_DUAL, 2, nullptr, vs, kc, vc, nullptr, nullptr, nullptr),
           FDLLM_ERR_INVALID_ARG, "refresh_layers NULL array");
    expect(fdllm_kv_refresh_layers(&s, &a, FDLLM_CACHE_DUAL, 2, ks, vs, kc_alias, vc, nullptr, nullptr, nullptr),
           FDLLM_ERR_INVALID_ARG, "refresh_layers cache on a source");
    expect(fdllm_kv_refresh_layers(&s, &a, FDLLM_CACHE_NONE, 2, ks, vs, kc, vc, nullptr, nullptr, nullptr), FDLLM_OK,
           "refresh_layers none");
  }
  expect(fdllm_workspace_init(nullptr, 256, nullptr), FDLLM_ERR_INVALID_ARG, "workspace_init NULL");
  expect(fdllm_workspace_init(P(8), 256, nullptr), FDLLM_ERR_INVALID_ARG, "workspace_init misaligned");
  expect(fdllm_set_tuning(3, 0, 0), FDLLM_ERR_INVALID_ARG, "tuning qt 3");
  expect(fdllm_set_tuning(0, -1, 0), FDLLM_ERR_INVALID_ARG, "tuning negative target");
  expect(fdllm_set_tuning(0, 0, 65537), FDLLM_ERR_INVALID_ARG, "tuning target too large");
  expect(fdllm_set_tuning(16, 65536, 1), FDLLM_OK, "tuning in range");
  expect(fdllm_set_tuning(0, 0, 0), FDLLM_OK, "tuning reset");
  expect(fdllm_set_debug(2), FDLLM_ERR_INVALID_ARG, "debug 2");
  expect(fdllm_set_lmhead_tuning(3), FDLLM_ERR_INVALID_ARG, "lmhead tuning 3");
  for (int32_t st : {-1, 0, 1, 2, 3, 4, 5, 1 << 30}) {
    const char* m = fdllm_status_string(st);
    ++g_checks;
    if (!m || !m[0]) {
      fprintf(stderr, "FAIL status_string(%d) empty\n", st);
      ++g_failures;
    }
  }
  ++g_checks;
  if (fdllm_version() != FDLLM_VERSION) {
    fprintf(stderr, "FAIL version\n");
    ++g_failures;
  }
}

int main() {
  attention();
  unmask();
  lmhead();
  refresh_and_settings();
  printf("%d checks, %d failures\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
