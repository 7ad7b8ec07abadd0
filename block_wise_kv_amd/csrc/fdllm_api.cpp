// Host side of the libfdllm C ABI: argument validation, workspace sizing,
// grid planning and kernel dispatch.  No call allocates, synchronises or
// touches the HIP runtime before its arguments have been validated.
#include <limits.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "fdllm.h"
#include "fdllm_internal.h"

using namespace fdllm;

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_timing_start = nullptr;
thread_local hipEvent_t g_timing_stop = nullptr;

fdllm_status fail(fdllm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

fdllm_status ok() {
  g_err.clear();
  return FDLLM_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Debug checks of device-resident arrays: FDLLM_DEBUG=1 in the environment
// (read once) or fdllm_set_debug (process-wide, read atomically).
std::atomic<int> g_debug{-1};
bool debug_on() {
  int v = g_debug.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = getenv("FDLLM_DEBUG");
    int expected = -1;
    g_debug.compare_exchange_strong(expected, (e && atoi(e) != 0) ? 1 : 0, std::memory_order_relaxed);
    v = g_debug.load(std::memory_order_relaxed);
  }
  return v == 1;
}

// In debug mode, validate the device arrays a call is about to use (a
// kernel, then a synchronisation of `stream`); FDLLM_OK otherwise.
fdllm_status debug_validate(const SeqArgs& sa, int max_P, const int32_t* seq_ids, const int32_t* n_seq,
                            void* stream) {
  if (!debug_on() || (!sa.plens && !sa.bidx && !seq_ids && !n_seq)) return FDLLM_OK;
  int key = INT_MAX;
  hipError_t e = run_validate(sa, max_P, seq_ids, n_seq, (hipStream_t)stream, &key);
  if (e != hipSuccess) return fail(FDLLM_ERR_LAUNCH, "debug validation failed: %s", hipGetErrorString(e));
  if (key == INT_MAX) return FDLLM_OK;
  const int idx = key / 8, code = key % 8;
  switch (code) {
    case VALIDATE_PROMPT:
      return fail(FDLLM_ERR_INVALID_ARG, "prompt_lens[%d] outside [0, max_prompt_len %d]", idx, max_P);
    case VALIDATE_BLOCK:
      return fail(FDLLM_ERR_INVALID_ARG, "block_idxs[%d] outside [0, %d)", idx, sa.G / sa.B);
    case VALIDATE_NSEQ:
      return fail(FDLLM_ERR_INVALID_ARG, "n_seq outside [0, batch %d]", sa.b);
    default:
      return fail(FDLLM_ERR_INVALID_ARG, "seq_ids[%d] outside [0, batch %d)", idx, sa.b);
  }
}

// Validate the sequence descriptor; fills `sa` and the host bounds.
fdllm_status check_seq(const fdllm_seq_desc* s, SeqArgs& sa, int& max_P) {
  if (!s) return fail(FDLLM_ERR_INVALID_ARG, "seq descriptor is NULL");
  if (s->batch < 1) return fail(FDLLM_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", s->batch);
  if (s->gen_len < 1) return fail(FDLLM_ERR_INVALID_ARG, "gen_len must be >= 1 (got %d)", s->gen_len);
  if (s->block_size < 1) return fail(FDLLM_ERR_INVALID_ARG, "block_size must be >= 1 (got %d)", s->block_size);
  if (s->gen_len % s->block_size != 0)
    return fail(FDLLM_ERR_INVALID_ARG, "gen_len %% block_size != 0 (%d %% %d)", s->gen_len, s->block_size);
  if (s->max_seq_len < 1) return fail(FDLLM_ERR_INVALID_ARG, "max_seq_len must be >= 1");
  if (s->prompt_lens) {
    if (s->max_prompt_len < 0) return fail(FDLLM_ERR_INVALID_ARG, "max_prompt_len must be >= 0");
    max_P = s->max_prompt_len;
  } else {
    if (s->prompt_len < 0) return fail(FDLLM_ERR_INVALID_ARG, "prompt_len must be >= 0");
    max_P = s->prompt_len;
  }
  if ((int64_t)max_P + s->gen_len > s->max_seq_len)
    return fail(FDLLM_ERR_INVALID_ARG, "prompt + gen_len (%lld) exceeds max_seq_len (%d)",
                (long long)max_P + s->gen_len, s->max_seq_len);
  const int nblocks = s->gen_len / s->block_size;
  if (!s->block_idxs && (s->block_idx < 0 || s->block_idx >= nblocks))
    return fail(FDLLM_ERR_INVALID_ARG, "block_idx %d outside [0, %d)", s->block_idx, nblocks);
  sa.b = s->batch;
  sa.Lcap = s->max_seq_len;
  sa.G = s->gen_len;
  sa.B = s->block_size;
  sa.P = s->prompt_len;
  sa.k = s->block_idx;
  sa.plens = s->prompt_lens;
  sa.bidx = s->block_idxs;
  return FDLLM_OK;
}

fdllm_status check_attn_desc(const fdllm_attn_desc* d, bool need_q) {
  if (!d) return fail(FDLLM_ERR_INVALID_ARG, "attn descriptor is NULL");
  if (d->n_kv_heads < 1) return fail(FDLLM_ERR_INVALID_ARG, "n_kv_heads must be >= 1");
  if (need_q) {
    if (d->n_q_heads < 1) return fail(FDLLM_ERR_INVALID_ARG, "n_q_heads must be >= 1");
    if (d->n_q_heads % d->n_kv_heads != 0)
      return fail(FDLLM_ERR_INVALID_ARG, "n_q_heads %% n_kv_heads != 0 (%d, %d)", d->n_q_heads, d->n_kv_heads);
    if (!(d->scale >= 0.f) || isinf(d->scale))
      return fail(FDLLM_ERR_INVALID_ARG, "scale must be finite and >= 0 (0 = 1/sqrt(d))");
  }
  if (d->dtype != FDLLM_BF16 && d->dtype != FDLLM_F32)
    return fail(FDLLM_ERR_INVALID_ARG, "dtype %d is not a fdllm_dtype", d->dtype);
  if (d->head_dim < 1) return fail(FDLLM_ERR_INVALID_ARG, "head_dim must be >= 1");
  return FDLLM_OK;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

int fresh_len_uniform(int mode, int P, int G, int B, int k) {
  if (mode == FDLLM_CACHE_NONE) return P + G;
  if (mode == FDLLM_CACHE_PREFIX) return G - k * B;
  return B;
}

struct AttnSetup {
  SeqArgs sa;
  int max_P;
  int nq_max;               // query rows of this call (the bound when ragged)
  int nq_bound;             // query rows of the geometry at any block index
  int L_max;
  AttnPlan plan;
  size_t counter_bytes;     // counter region at the start of the workspace
  size_t ws_call;           // bytes this call uses (0: no workspace)
  size_t ws_geometry;       // bytes that serve every block index (the query's answer)
};

fdllm_status setup_attn(const fdllm_seq_desc* seq, const fdllm_attn_desc* ad, int32_t mode, int32_t fresh_rows,
                        AttnSetup& su) {
  fdllm_status st = check_seq(seq, su.sa, su.max_P);
  if (st) return st;
  st = check_attn_desc(ad, true);
  if (st) return st;
  if (mode < FDLLM_CACHE_NONE || mode > FDLLM_CACHE_DUAL)
    return fail(FDLLM_ERR_INVALID_ARG, "mode %d is not a fdllm_cache_mode", mode);
  if (ad->head_dim != 64 && ad->head_dim != 128)
    return fail(FDLLM_ERR_UNSUPPORTED, "attention supports head_dim 64 or 128 (got %d)", ad->head_dim);
  const bool ragged = seq->prompt_lens || seq->block_idxs;
  int need;
  if (!ragged) {
    need = fresh_len_uniform(mode, seq->prompt_len, seq->gen_len, seq->block_size, seq->block_idx);
  } else {
    need = mode == FDLLM_CACHE_DUAL ? seq->block_size
         : mode == FDLLM_CACHE_PREFIX ? seq->gen_len : su.max_P + seq->gen_len;
  }
  if (fresh_rows < need)
    return fail(FDLLM_ERR_INVALID_ARG, "fresh_rows %d < %d rows needed by this mode/geometry", fresh_rows, need);
  su.nq_max = need;
  su.nq_bound = mode == FDLLM_CACHE_DUAL ? seq->block_size
              : mode == FDLLM_CACHE_PREFIX ? seq->gen_len : su.max_P + seq->gen_len;
  su.L_max = su.max_P + seq->gen_len;
  const int64_t q_elems = (int64_t)seq->batch * fresh_rows * ad->n_q_heads * ad->head_dim;
  const int64_t c_elems = (int64_t)seq->batch * ad->n_kv_heads * seq->max_seq_len * ad->head_dim;
  if (q_elems >= ((int64_t)1 << 40) || c_elems >= ((int64_t)1 << 40))
    return fail(FDLLM_ERR_INVALID_ARG, "tensor too large");
  if ((int64_t)seq->batch * ad->n_q_heads * ((need + 31) / 32) * ((su.L_max + 127) / 128) >= ((int64_t)1 << 31))
    return fail(FDLLM_ERR_INVALID_ARG, "grid too large");
  const bool ragged_lens = seq->prompt_lens != nullptr;
  su.plan = plan_block_attn(ad->dtype, seq->batch, ad->n_q_heads, ad->n_kv_heads, ad->head_dim, need, su.L_max,
                            ragged_lens);
  su.counter_bytes = attn_counter_bytes(seq->batch, ad->n_q_heads, su.nq_bound);
  su.ws_call = su.plan.part_bytes > 0 ? su.counter_bytes + su.plan.part_bytes : 0;
  su.ws_geometry = attn_workspace_bytes(ad->dtype, seq->batch, ad->n_q_heads, ad->n_kv_heads, ad->head_dim,
                                        su.nq_bound, su.L_max, ragged_lens);
  return FDLLM_OK;
}

struct UnmaskSetup {
  SeqArgs sa;
  int max_P;
  int chunk, nchunk;
  size_t ws;
};

fdllm_status setup_unmask(const fdllm_seq_desc* seq, int32_t vocab, int32_t dtype, UnmaskSetup& su) {
  fdllm_status st = check_seq(seq, su.sa, su.max_P);
  if (st) return st;
  if (vocab < 1) return fail(FDLLM_ERR_INVALID_ARG, "vocab must be >= 1");
  if (dtype != FDLLM_BF16 && dtype != FDLLM_F32) return fail(FDLLM_ERR_INVALID_ARG, "logits dtype %d invalid", dtype);
  if (seq->block_size > 1024) return fail(FDLLM_ERR_UNSUPPORTED, "block_size > 1024");
  if (seq->batch > 65535) return fail(FDLLM_ERR_UNSUPPORTED, "batch > 65535");
  if (vocab > (1 << 28)) return fail(FDLLM_ERR_UNSUPPORTED, "vocab > 2^28");
  const UnmaskPlan up = plan_unmask(dtype, vocab, seq->batch * seq->block_size);
  su.chunk = up.chunk;
  su.nchunk = up.nchunk;
  if ((int64_t)su.nchunk * seq->block_size >= ((int64_t)1 << 31) - 1)
    return fail(FDLLM_ERR_INVALID_ARG, "vocab too large");
  su.ws = unmask_workspace_bytes(seq->batch, seq->block_size, su.nchunk);
  return FDLLM_OK;
}

struct LmheadSetup {
  SeqArgs sa;
  int max_P;
  LmheadPlan plan;
  size_t ws;
};

fdllm_status check_lmhead_dims(int32_t vocab, int32_t hidden) {
  if (vocab < 1) return fail(FDLLM_ERR_INVALID_ARG, "vocab must be >= 1");
  if (vocab > (1 << 28)) return fail(FDLLM_ERR_UNSUPPORTED, "vocab > 2^28");
  if (hidden < 8 || hidden % 8 != 0)
    return fail(FDLLM_ERR_UNSUPPORTED, "hidden must be a positive multiple of 8 (got %d)", hidden);
  if (hidden > (1 << 20)) return fail(FDLLM_ERR_UNSUPPORTED, "hidden > 2^20");
  return FDLLM_OK;
}

fdllm_status setup_lmhead(const fdllm_seq_desc* seq, int32_t vocab, int32_t hidden, LmheadSetup& su) {
  fdllm_status st = check_seq(seq, su.sa, su.max_P);
  if (st) return st;
  st = check_lmhead_dims(vocab, hidden);
  if (st) return st;
  if (seq->block_size > 1024) return fail(FDLLM_ERR_UNSUPPORTED, "block_size > 1024");
  if (seq->batch > 65535) return fail(FDLLM_ERR_UNSUPPORTED, "batch > 65535");
  const int64_t M = (int64_t)seq->batch * seq->block_size;
  if (M >= ((int64_t)1 << 24)) return fail(FDLLM_ERR_UNSUPPORTED, "batch * block_size >= 2^24");
  su.plan = plan_lmhead((int)M, vocab);
  if ((int64_t)su.plan.grid >= ((int64_t)1 << 31)) return fail(FDLLM_ERR_INVALID_ARG, "grid too large");
  su.ws = unmask_workspace_bytes(seq->batch, seq->block_size, su.plan.n_vwg);
  return FDLLM_OK;
}

// The threshold rule (topk == 0) and the fixed-step rule (topk > 0) on the
// logits of the fused vocabulary projection.
fdllm_status run_lmhead_unmask(const fdllm_seq_desc* seq, int32_t vocab, int32_t hidden, const void* x,
                               int64_t seq_stride, int64_t row_stride, const void* w_packed, float threshold,
                               int32_t topk, uint32_t flags, int32_t* tokens, uint8_t* mask, int32_t* n_decoded,
                               int32_t* decoded_pos, double* conf, int32_t* done_seqs, int32_t* n_done,
                               void* workspace, size_t workspace_bytes, void* stream) {
  LmheadSetup su;
  fdllm_status st = setup_lmhead(seq, vocab, hidden, su);
  if (st) return st;
  if (!x || !w_packed || !tokens || !mask || !n_decoded)
    return fail(FDLLM_ERR_INVALID_ARG, "x, w_packed, tokens, mask and n_decoded must be non-NULL");
  if (flags & ~FDLLM_UNMASK_ADVANCE_BLOCK) return fail(FDLLM_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((flags & FDLLM_UNMASK_ADVANCE_BLOCK) && !seq->block_idxs)
    return fail(FDLLM_ERR_INVALID_ARG, "FDLLM_UNMASK_ADVANCE_BLOCK needs a device block_idxs array");
  if (!aligned16(x) || !aligned16(w_packed))
    return fail(FDLLM_ERR_INVALID_ARG, "x and w_packed must be 16-byte aligned");
  if (row_stride % 8 != 0 || seq_stride % 8 != 0)
    return fail(FDLLM_ERR_INVALID_ARG, "x strides must be multiples of 8 elements (16 bytes)");
  if (row_stride < hidden) return fail(FDLLM_ERR_INVALID_ARG, "row_stride %lld < hidden %d", (long long)row_stride, hidden);
  if (seq->batch > 1 && seq_stride < (int64_t)(seq->block_size - 1) * row_stride + hidden)
    return fail(FDLLM_ERR_INVALID_ARG, "seq_stride %lld overlaps the rows of the previous sequence",
                (long long)seq_stride);
  if (!workspace || workspace_bytes < su.ws)
    return fail(FDLLM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", su.ws,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(FDLLM_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  st = debug_validate(su.sa, su.max_P, nullptr, nullptr, stream);
  if (st) return st;
  const LmheadPlan& p = su.plan;
  UnmaskArgs ua{};
  ua.sq = su.sa;
  ua.V = vocab;
  ua.tau = threshold;
  ua.topk = topk;
  ua.flags = flags;
  ua.tokens = tokens;
  ua.mask = mask;
  ua.n_decoded = n_decoded;
  ua.decoded_pos = decoded_pos;
  ua.conf = conf;
  ua.done_seqs = done_seqs;
  ua.n_done = n_done;
  ua.nchunk = p.n_vwg;  // partials per row ([row][n_vwg] here)
  unmask_bind_workspace(ua, workspace);
  LmheadArgs la{};
  la.M = seq->batch * seq->block_size;
  la.B = seq->block_size;
  la.H = hidden;
  la.Hp = (hidden + kLmheadHpad - 1) / kLmheadHpad * kLmheadHpad;
  la.V = vocab;
  la.nvt = (vocab + 31) / 32;
  la.n_vwg = p.n_vwg;
  la.tiles_per_wg = p.tiles_per_wg;
  la.n_rg = p.n_rg;
  la.n_items = p.n_items;
  la.per_xcd = p.per_xcd;
  la.seq_stride = seq_stride;
  la.row_stride = row_stride;
  la.x = (const uint16_t*)x;
  la.wp = (const uint4*)w_packed;
  la.part = ua.part;
  const LaunchEvents ev = take_launch_events();
  hipError_t e = launch_lmhead(la, p, (hipStream_t)stream, ev.start);
  if (e != hipSuccess) return fail(FDLLM_ERR_LAUNCH, "lmhead launch failed: %s", hipGetErrorString(e));
  e = launch_lmhead_finalize(ua, ua.part, p.n_vwg, (hipStream_t)stream, ev.stop);
  if (e != hipSuccess) return fail(FDLLM_ERR_LAUNCH, "lmhead finalize launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

namespace fdllm {
LaunchEvents take_launch_events() {
  LaunchEvents e{g_timing_start, g_timing_stop};
  g_timing_start = g_timing_stop = nullptr;
  return e;
}
}  // namespace fdllm

extern "C" {

fdllm_status fdllm_set_tuning(int32_t attn_qt, int32_t attn_wgs, int32_t unmask_wgs) {
  if (attn_qt != 0 && attn_qt != 1 && attn_qt != 2 && attn_qt != 4 && attn_qt != 8 && attn_qt != 16)
    return fail(FDLLM_ERR_INVALID_ARG, "attn_qt must be 0, 1, 2, 4, 8 or 16 (got %d)", attn_qt);
  if (attn_wgs < 0 || unmask_wgs < 0 || attn_wgs > 65536 || unmask_wgs > 65536)
    return fail(FDLLM_ERR_INVALID_ARG, "workgroup targets must be in [0, 65536]");
  set_attn_tuning(attn_qt, attn_wgs);
  set_unmask_tuning(unmask_wgs);
  return ok();
}

fdllm_status fdllm_set_debug(int32_t on) {
  if (on != 0 && on != 1) return fail(FDLLM_ERR_INVALID_ARG, "on must be 0 or 1 (got %d)", on);
  g_debug.store(on, std::memory_order_relaxed);
  return ok();
}

fdllm_status fdllm_set_timing_events(void* start_event, void* stop_event) {
  g_timing_start = (hipEvent_t)start_event;
  g_timing_stop = (hipEvent_t)stop_event;
  return ok();
}

size_t fdllm_block_attn_workspace(const fdllm_seq_desc* seq, const fdllm_attn_desc* attn, int32_t mode,
                                  int32_t fresh_rows) {
  AttnSetup su;
  if (setup_attn(seq, attn, mode, fresh_rows, su)) return 0;
  ok();
  return su.ws_geometry;
}

fdllm_status fdllm_block_attn(const fdllm_seq_desc* seq, const fdllm_attn_desc* attn, int32_t mode,
                              int32_t fresh_rows, const void* q, const void* k_new, const void* v_new,
                              const void* k_cache, const void* v_cache, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  AttnSetup su;
  fdllm_status st = setup_attn(seq, attn, mode, fresh_rows, su);
  if (st) return st;
  if (!q || !k_new || !v_new || !out) return fail(FDLLM_ERR_INVALID_ARG, "q, k_new, v_new and out must be non-NULL");
  if (mode != FDLLM_CACHE_NONE && (!k_cache || !v_cache))
    return fail(FDLLM_ERR_INVALID_ARG, "k_cache and v_cache are required in PREFIX and DUAL modes");
  const void* ptrs[] = {q, k_new, v_new, out, k_cache, v_cache};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(FDLLM_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const size_t es = attn->dtype == FDLLM_BF16 ? 2 : 4;
  const size_t qb = (size_t)seq->batch * fresh_rows * attn->n_q_heads * attn->head_dim * es;
  const size_t kvb = (size_t)seq->batch * fresh_rows * attn->n_kv_heads * attn->head_dim * es;
  const size_t cb = (size_t)seq->batch * attn->n_kv_heads * seq->max_seq_len * attn->head_dim * es;
  if (ranges_overlap(out, qb, q, qb) || ranges_overlap(out, qb, k_new, kvb) || ranges_overlap(out, qb, v_new, kvb) ||
      (mode != FDLLM_CACHE_NONE && (ranges_overlap(out, qb, k_cache, cb) || ranges_overlap(out, qb, v_cache, cb))))
    return fail(FDLLM_ERR_INVALID_ARG, "out must not alias an input");
  if (su.ws_call > 0) {
    if (!workspace || workspace_bytes < su.ws_call)
      return fail(FDLLM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", su.ws_call,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(FDLLM_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  st = debug_validate(su.sa, su.max_P, nullptr, nullptr, stream);
  if (st) return st;
  AttnArgs a{};
  a.sq = su.sa;
  a.mode = mode;
  a.fresh_rows = fresh_rows;
  a.Hq = attn->n_q_heads;
  a.Hkv = attn->n_kv_heads;
  a.g = a.Hq / a.Hkv;
  a.scale = attn->scale > 0.f ? attn->scale : 1.0f / sqrtf((float)attn->head_dim);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.q = q;
  a.kn = k_new;
  a.vn = v_new;
  a.kc = k_cache;
  a.vc = v_cache;
  a.out = out;
  attn_bind_workspace(a, su.plan, workspace, su.counter_bytes);
  hipError_t e = launch_block_attn(a, su.plan, attn->dtype, attn->head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FDLLM_ERR_LAUNCH, "block_attn launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t fdllm_unmask_workspace(const fdllm_seq_desc* seq, int32_t vocab, int32_t logits_dtype) {
  UnmaskSetup su;
  if (setup_unmask(seq, vocab, logits_dtype, su)) return 0;
  ok();
  return su.ws;
}

}  // extern "C"

// ---- scratch of the allocation-free threshold unmask
// (fdllm_unmask_threshold_static).  One array per device, held until the
// process ends: the arrival counters first, at offsets that do not depend
// on the batch (the finished-sequence counter at 0, the per-sequence done
// flags at 256, the per-sequence arrival counters, one per 128-byte line,
// at 64 KB: counters that must read zero never overlap a word another call
// left non-zero), then the vocabulary-chunk partials.  The kernels reset every counter they
// use, so after one clear per device the array stays ready for the next
// call.  Calls that overlap on one device share it and race.
namespace {
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
constexpr size_t kStaticCounterBytes = (size_t)576 << 10;
constexpr int kStaticMaxBatch = 4096;
constexpr size_t kStaticDoneFlagOffset = 256;
constexpr size_t kStaticSeqCntOffset = (size_t)64 << 10;
static_assert(kStaticDoneFlagOffset + 8 * (size_t)kStaticMaxBatch <= kStaticSeqCntOffset, "counter layout");
static_assert(kStaticSeqCntOffset + 4 * (size_t)kSeqCntStride * kStaticMaxBatch <= kStaticCounterBytes,
              "counter layout");
constexpr int kMaxDevices = 64;
}  // namespace

__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` on each device (null: not set up)

// Bind the unmask arguments to this device's copy of `scratch`.  The first
// call on a device looks up the array's device address (the host-side name
// is only a stand-in) and clears its counter region with a fill kernel on
// `stream`, ordered before this call's kernel.
fdllm_status bind_static_scratch(UnmaskArgs& a, void* stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FDLLM_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FDLLM_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(FDLLM_ERR_LAUNCH, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      e = launch_fill_zero(p, kStaticCounterBytes, (hipStream_t)stream);
      if (e != hipSuccess) return fail(FDLLM_ERR_LAUNCH, "scratch clear failed: %s", hipGetErrorString(e));
      g_scratch_ptr[dev] = p;
    }
    base = g_scratch_ptr[dev];
  }
  char* w = (char*)base;
  a.glob = (uint64_t*)w;
  a.seq_cnt = (uint32_t*)(w + kStaticSeqCntOffset);
  a.done_flag = (int32_t*)(w + kStaticDoneFlagOffset);
  a.part = (UnmaskPartial*)(w + kStaticCounterBytes);
  return FDLLM_OK;
}
}  // namespace

namespace {
// The threshold rule (topk == 0) and the fixed-step rule (topk > 0) share
// the vocabulary pass and differ only in the selection of the finalisation.
fdllm_status run_unmask(const fdllm_seq_desc* seq, int32_t vocab, int32_t logits_dtype, const void* logits,
                        int64_t seq_stride, int64_t row_stride, float threshold, int32_t topk, uint32_t flags,
                        int32_t* tokens, uint8_t* mask, int32_t* n_decoded, int32_t* decoded_pos, double* conf,
                        int32_t* done_seqs, int32_t* n_done, void* workspace, size_t workspace_bytes,
                        void* stream, bool use_static = false) {
  UnmaskSetup su;
  fdllm_status st = setup_unmask(seq, vocab, logits_dtype, su);
  if (st) return st;
  if (!logits || !tokens || !mask || !n_decoded)
    return fail(FDLLM_ERR_INVALID_ARG, "logits, tokens, mask and n_decoded must be non-NULL");
  if (flags & ~FDLLM_UNMASK_ADVANCE_BLOCK) return fail(FDLLM_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((flags & FDLLM_UNMASK_ADVANCE_BLOCK) && !seq->block_idxs)
    return fail(FDLLM_ERR_INVALID_ARG, "FDLLM_UNMASK_ADVANCE_BLOCK needs a device block_idxs array");
  if (row_stride < vocab) return fail(FDLLM_ERR_INVALID_ARG, "row_stride %lld < vocab %d", (long long)row_stride, vocab);
  if (seq->batch > 1 && seq_stride < (int64_t)(seq->block_size - 1) * row_stride + vocab)
    return fail(FDLLM_ERR_INVALID_ARG, "seq_stride %lld overlaps the rows of the previous sequence",
                (long long)seq_stride);
  if (use_static) {
    const size_t part = (size_t)seq->batch * seq->block_size * su.nchunk * sizeof(UnmaskPartial);
    if (seq->batch > kStaticMaxBatch)
      return fail(FDLLM_ERR_UNSUPPORTED, "batch %d exceeds the static scratch's limit of %d sequences", seq->batch,
                  kStaticMaxBatch);
    if (part > kStaticScratchBytes - kStaticCounterBytes)
      return fail(FDLLM_ERR_UNSUPPORTED,
                  "batch x block_size x vocab chunks needs %zu bytes of partials; the static scratch holds %zu",
                  part, kStaticScratchBytes - kStaticCounterBytes);
  } else {
    if (!workspace || workspace_bytes < su.ws)
      return fail(FDLLM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", su.ws,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(FDLLM_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  st = debug_validate(su.sa, su.max_P, nullptr, nullptr, stream);
  if (st) return st;
  const size_t es = logits_dtype == FDLLM_BF16 ? 2 : 4;
  const bool vec = aligned16(logits) && ((size_t)row_stride * es) % 16 == 0 && ((size_t)seq_stride * es) % 16 == 0;
  UnmaskArgs a{};
  a.sq = su.sa;
  a.V = vocab;
  a.seq_stride = seq_stride;
  a.row_stride = row_stride;
  a.logits = logits;
  a.vec = vec ? 1 : 0;
  a.tau = threshold;
  a.topk = topk;
  a.flags = flags;
  a.tokens = tokens;
  a.mask = mask;
  a.n_decoded = n_decoded;
  a.decoded_pos = decoded_pos;
  a.conf = conf;
  a.done_seqs = done_seqs;
  a.n_done = n_done;
  a.nchunk = su.nchunk;
  a.chunk = su.chunk;
  if (use_static) {
    st = bind_static_scratch(a, stream);
    if (st) return st;
  } else {
    unmask_bind_workspace(a, workspace);
  }
  hipError_t e = launch_unmask(a, logits_dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FDLLM_ERR_LAUNCH, "unmask launch failed: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace

static_assert(kMaxRefreshLayers == FDLLM_MAX_REFRESH_LAYERS, "refresh layer limit");

namespace {
// fdllm_kv_refresh (one layer, `layers` false) and fdllm_kv_refresh_layers:
// the same checks, then one launch over n_layers layers (host arrays of
// per-layer device pointers).
fdllm_status run_refresh(const fdllm_seq_desc* seq, const fdllm_attn_desc* attn, int32_t mode, int32_t n_layers,
                         const void* const* k_src, const void* const* v_src, void* const* k_cache,
                         void* const* v_cache, const int32_t* seq_ids, const int32_t* n_seq, void* stream,
                         bool layers) {
  SeqArgs sa;
  int max_P;
  fdllm_status st = check_seq(seq, sa, max_P);
  if (st) return st;
  st = check_attn_desc(attn, false);
  if (st) return st;
  if (mode < FDLLM_CACHE_NONE || mode > FDLLM_CACHE_DUAL)
    return fail(FDLLM_ERR_INVALID_ARG, "mode %d is not a fdllm_cache_mode", mode);
  if (seq_ids && !n_seq) return fail(FDLLM_ERR_INVALID_ARG, "seq_ids needs the device count n_seq");
  if (layers && (n_layers < 1 || n_layers > kMaxRefreshLayers))
    return fail(FDLLM_ERR_INVALID_ARG, "n_layers %d outside [1, %d]", n_layers, kMaxRefreshLayers);
  if (layers && (!k_src || !v_src || !k_cache || !v_cache))
    return fail(FDLLM_ERR_INVALID_ARG, "the per-layer pointer arrays must be non-NULL");
  if (mode == FDLLM_CACHE_NONE) return ok();  // nothing is cached
  for (int l = 0; l < n_layers; ++l) {
    if (!k_src[l] || !v_src[l] || !k_cache[l] || !v_cache[l])
      return layers ? fail(FDLLM_ERR_INVALID_ARG, "layer %d: k_src, v_src, k_cache and v_cache must be non-NULL", l)
                    : fail(FDLLM_ERR_INVALID_ARG, "k_src, v_src, k_cache and v_cache must be non-NULL");
    const void* ptrs[] = {k_src[l], v_src[l], k_cache[l], v_cache[l]};
    for (const void* p : ptrs)
      if (!aligned16(p)) return fail(FDLLM_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  }
  const size_t es = attn->dtype == FDLLM_BF16 ? 2 : 4;
  const size_t row_bytes = (size_t)attn->head_dim * es;
  if (row_bytes % 16 != 0) return fail(FDLLM_ERR_UNSUPPORTED, "head_dim * element size must be a multiple of 16");
  size_t vpr = row_bytes / 16;
  int shift = 0;
  while ((1u << shift) < vpr) ++shift;
  if ((1u << shift) != vpr) return fail(FDLLM_ERR_UNSUPPORTED, "head_dim * element size / 16 must be a power of two");
  if ((((int64_t)seq->max_seq_len * attn->n_kv_heads) << shift) >= ((int64_t)1 << 31))
    return fail(FDLLM_ERR_INVALID_ARG, "per-sequence cache too large");
  const size_t cb = (size_t)seq->batch * attn->n_kv_heads * seq->max_seq_len * row_bytes;
  // no cache may overlap another cache or any source (of any layer): the
  // result would depend on the order of the stores
  const void* dst[2 * kMaxRefreshLayers];
  const void* src[2 * kMaxRefreshLayers];
  for (int l = 0; l < n_layers; ++l) {
    dst[2 * l] = k_cache[l];
    dst[2 * l + 1] = v_cache[l];
    src[2 * l] = k_src[l];
    src[2 * l + 1] = v_src[l];
  }
  bool alias = false;
  for (int x = 0; x < 2 * n_layers && !alias; ++x) {
    for (int y = 0; y < 2 * n_layers && !alias; ++y) alias = ranges_overlap(dst[x], cb, src[y], cb);
    for (int y = x + 1; y < 2 * n_layers && !alias; ++y) alias = ranges_overlap(dst[x], cb, dst[y], cb);
  }
  if (alias) return fail(FDLLM_ERR_INVALID_ARG, "caches must not alias the sources or each other");
  st = debug_validate(sa, max_P, seq_ids, n_seq, stream);
  if (st) return st;
  RefreshArgs a{};
  a.sq = sa;
  a.mode = mode;
  a.Hkv = attn->n_kv_heads;
  a.row_vec_shift = shift;
  a.hkv_div = make_fastdiv((uint32_t)attn->n_kv_heads);
  a.seq_ids = seq_ids;
  a.n_seq = n_seq;
  const int max_rows = max_P + seq->gen_len;
  hipError_t e;
  if (!layers) {
    a.k_src = (const uint4*)k_src[0];
    a.v_src = (const uint4*)v_src[0];
    a.k_cache = (uint4*)k_cache[0];
    a.v_cache = (uint4*)v_cache[0];
    e = launch_kv_refresh(a, max_rows, (hipStream_t)stream);
  } else {
    RefreshLayerPtrs p{};
    for (int l = 0; l < n_layers; ++l) {
      p.k_src[l] = (const uint4*)k_src[l];
      p.v_src[l] = (const uint4*)v_src[l];
      p.k_cache[l] = (uint4*)k_cache[l];
      p.v_cache[l] = (uint4*)v_cache[l];
    }
    e = launch_kv_refresh_layers(a, p, n_layers, max_rows, (hipStream_t)stream);
  }
  if (e != hipSuccess) return fail(FDLLM_ERR_LAUNCH, "kv_refresh launch failed: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace

extern "C" {

fdllm_status fdllm_unmask_threshold(const fdllm_seq_desc* seq, int32_t vocab, int32_t logits_dtype,
                                    const void* logits, int64_t seq_stride, int64_t row_stride, float threshold,
                                    uint32_t flags, int32_t* tokens, uint8_t* mask, int32_t* n_decoded,
                                    int32_t* decoded_pos, double* conf, int32_t* done_seqs, int32_t* n_done,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (isnan(threshold)) return fail(FDLLM_ERR_INVALID_ARG, "threshold is NaN");
  return run_unmask(seq, vocab, logits_dtype, logits, seq_stride, row_stride, threshold, 0, flags, tokens, mask,
                    n_decoded, decoded_pos, conf, done_seqs, n_done, workspace, workspace_bytes, stream);
}

fdllm_status fdllm_unmask_threshold_static(const fdllm_seq_desc* seq, int32_t vocab, int32_t logits_dtype,
                                           const void* logits, int64_t seq_stride, int64_t row_stride,
                                           float threshold, uint32_t flags, int32_t* tokens, uint8_t* mask,
                                           int32_t* n_decoded, int32_t* decoded_pos, double* conf,
                                           int32_t* done_seqs, int32_t* n_done, void* stream) {
  if (isnan(threshold)) return fail(FDLLM_ERR_INVALID_ARG, "threshold is NaN");
  return run_unmask(seq, vocab, logits_dtype, logits, seq_stride, row_stride, threshold, 0, flags, tokens, mask,
                    n_decoded, decoded_pos, conf, done_seqs, n_done, nullptr, 0, stream, true);
}

fdllm_status fdllm_unmask_topk(const fdllm_seq_desc* seq, int32_t vocab, int32_t logits_dtype, const void* logits,
                               int64_t seq_stride, int64_t row_stride, int32_t k, uint32_t flags, int32_t* tokens,
                               uint8_t* mask, int32_t* n_decoded, int32_t* decoded_pos, double* conf,
                               int32_t* done_seqs, int32_t* n_done, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (k < 1) return fail(FDLLM_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
  return run_unmask(seq, vocab, logits_dtype, logits, seq_stride, row_stride, 0.f, k, flags, tokens, mask,
                    n_decoded, decoded_pos, conf, done_seqs, n_done, workspace, workspace_bytes, stream);
}

size_t fdllm_lmhead_packed_bytes(int32_t vocab, int32_t hidden) {
  if (check_lmhead_dims(vocab, hidden)) return 0;
  ok();
  return lmhead_packed_bytes(vocab, hidden);
}

fdllm_status fdllm_lmhead_pack(int32_t vocab, int32_t hidden, const void* w, void* w_packed, size_t w_packed_bytes,
                               void* stream) {
  fdllm_status st = check_lmhead_dims(vocab, hidden);
  if (st) return st;
  if (!w || !w_packed) return fail(FDLLM_ERR_INVALID_ARG, "w and w_packed must be non-NULL");
  if (!aligned16(w) || !aligned16(w_packed)) return fail(FDLLM_ERR_INVALID_ARG, "w and w_packed must be 16-byte aligned");
  const size_t need = lmhead_packed_bytes(vocab, hidden);
  if (w_packed_bytes < need)
    return fail(FDLLM_ERR_INVALID_ARG, "w_packed needs %zu bytes (got %zu)", need, w_packed_bytes);
  if (ranges_overlap(w, (size_t)vocab * hidden * 2, w_packed, need))
    return fail(FDLLM_ERR_INVALID_ARG, "w_packed must not alias w");
  hipError_t e = launch_lmhead_pack(w, w_packed, vocab, hidden, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FDLLM_ERR_LAUNCH, "lmhead pack launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t fdllm_lmhead_unmask_workspace(const fdllm_seq_desc* seq, int32_t vocab, int32_t hidden) {
  LmheadSetup su;
  if (setup_lmhead(seq, vocab, hidden, su)) return 0;
  ok();
  return su.ws;
}

fdllm_status fdllm_lmhead_unmask_threshold(const fdllm_seq_desc* seq, int32_t vocab, int32_t hidden, const void* x,
                                           int64_t seq_stride, int64_t row_stride, const void* w_packed,
                                           float threshold, uint32_t flags, int32_t* tokens, uint8_t* mask,
                                           int32_t* n_decoded, int32_t* decoded_pos, double* conf,
                                           int32_t* done_seqs, int32_t* n_done, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (isnan(threshold)) return fail(FDLLM_ERR_INVALID_ARG, "threshold is NaN");
  return run_lmhead_unmask(seq, vocab, hidden, x, seq_stride, row_stride, w_packed, threshold, 0, flags, tokens,
                           mask, n_decoded, decoded_pos, conf, done_seqs, n_done, workspace, workspace_bytes, stream);
}

fdllm_status fdllm_lmhead_unmask_topk(const fdllm_seq_desc* seq, int32_t vocab, int32_t hidden, const void* x,
                                      int64_t seq_stride, int64_t row_stride, const void* w_packed, int32_t k,
                                      uint32_t flags, int32_t* tokens, uint8_t* mask, int32_t* n_decoded,
                                      int32_t* decoded_pos, double* conf, int32_t* done_seqs, int32_t* n_done,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (k < 1) return fail(FDLLM_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
  return run_lmhead_unmask(seq, vocab, hidden, x, seq_stride, row_stride, w_packed, 0.f, k, flags, tokens, mask,
                           n_decoded, decoded_pos, conf, done_seqs, n_done, workspace, workspace_bytes, stream);
}

fdllm_status fdllm_set_lmhead_tuning(int32_t vt) {
  if (vt < 0 || vt > 2) return fail(FDLLM_ERR_INVALID_ARG, "vt must be 0, 1 or 2 (got %d)", vt);
  set_lmhead_tuning(vt);
  return ok();
}

fdllm_status fdllm_kv_refresh(const fdllm_seq_desc* seq, const fdllm_attn_desc* attn, int32_t mode,
                              const void* k_src, const void* v_src, void* k_cache, void* v_cache,
                              const int32_t* seq_ids, const int32_t* n_seq, void* stream) {
  const void* ks = k_src;
  const void* vs = v_src;
  void* kc = k_cache;
  void* vc = v_cache;
  return run_refresh(seq, attn, mode, 1, &ks, &vs, &kc, &vc, seq_ids, n_seq, stream, false);
}

fdllm_status fdllm_kv_refresh_layers(const fdllm_seq_desc* seq, const fdllm_attn_desc* attn, int32_t mode,
                                     int32_t n_layers, const void* const* k_src, const void* const* v_src,
                                     void* const* k_cache, void* const* v_cache, const int32_t* seq_ids,
                                     const int32_t* n_seq, void* stream) {
  return run_refresh(seq, attn, mode, n_layers, k_src, v_src, k_cache, v_cache, seq_ids, n_seq, stream, true);
}

fdllm_status fdllm_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (bytes == 0) return ok();
  if (!workspace) return fail(FDLLM_ERR_INVALID_ARG, "workspace is NULL");
  if (bytes % 4 != 0 || !aligned16(workspace))
    return fail(FDLLM_ERR_INVALID_ARG, "workspace must be 16-byte aligned and a multiple of 4 bytes");
  hipError_t e = launch_fill_zero(workspace, bytes, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FDLLM_ERR_LAUNCH, "fill launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* fdllm_status_string(int32_t status) {
  switch (status) {
    case FDLLM_OK: return "FDLLM_OK";
    case FDLLM_ERR_INVALID_ARG: return "FDLLM_ERR_INVALID_ARG";
    case FDLLM_ERR_UNSUPPORTED: return "FDLLM_ERR_UNSUPPORTED";
    case FDLLM_ERR_WORKSPACE: return "FDLLM_ERR_WORKSPACE";
    case FDLLM_ERR_LAUNCH: return "FDLLM_ERR_LAUNCH";
    default: return "FDLLM_ERR_UNKNOWN";
  }
}

const char* fdllm_last_error(void) { return g_err.c_str(); }

int32_t fdllm_version(void) { return FDLLM_VERSION; }

}  // extern "C"
