/*
 * fdllm.h -- C ABI of libfdllm, the per-step hot path of Fast-dLLM
 * block-wise masked-diffusion decoding on AMD Instinct MI355X (gfx950).
 *
 * Sources for what each call computes:
 *   [ABS]    Fast-dLLM: Training-free Acceleration of Diffusion LLM by
 *            Enabling KV Cache and Parallel Decoding, paper summary page
 *            (arXiv 2505.22618v3), "Abstract" and method notes.
 *   [NEWS]   aibase news article on Fast-dLLM, "Innovations in the Fast-dLLM
 *            Framework" items 1-2, "The Challenges and Opportunities".
 *   [README] Fast-dLLM project README mirror, "Key techniques" items 1-2 and
 *            "Usage" (flags --gen_length, --block_size, --use_cache,
 *            --if_cache_position, --threshold).
 *   [REV]    ICLR reviews of Fast-dLLM, review 4 (refresh after each block).
 *
 * Conventions (all calls):
 *   - Pointers are DEVICE pointers unless marked "host".  Descriptors are
 *     host structs read during the call only.
 *   - The caller owns every buffer.  The library never allocates device
 *     memory and never synchronises; every call is asynchronous and ordered
 *     on `stream` (a hipStream_t passed as void*, NULL = default stream).
 *   - Host-side scalars and pointers are validated before any launch; on
 *     failure nothing is launched, an FDLLM_ERR_* code is returned and
 *     fdllm_last_error() describes it.  Device-resident per-sequence arrays
 *     (prompt_lens, block_idxs, seq_ids, n_seq) are trusted, except in
 *     debug mode (fdllm_set_debug, or FDLLM_DEBUG=1 in the environment):
 *     then a validation kernel checks them and the call synchronises the
 *     stream to read its verdict before launching anything else.
 *   - No exception or abort crosses the ABI.  Thread-safe: calls keep no
 *     state between them except per-host-thread settings (the last error,
 *     the timing hook, the planner overrides) and the debug-mode switch;
 *     debug-mode calls from several threads take turns on a host lock.
 *   - Workspaces hold self-resetting counters: zero a workspace once with
 *     fdllm_workspace_init after allocating it; every call leaves its
 *     counters at zero again.  The counters sit at the start of the
 *     workspace, at a place fixed by the geometry (batch, heads, mode and
 *     the row bounds below), never by the block index or the planner's
 *     choice, so one workspace serves every block index of a decode loop.
 *     A workspace belongs to one geometry at a time: a call of another
 *     geometry may overwrite the counter area of the first with partial
 *     results, so re-zero it when switching.  Two calls that share a
 *     workspace must not run concurrently (same stream, or ordered
 *     streams).
 *
 * Notation: batch b; sequence i has prompt length P_i, shared gen length G,
 * L_i = P_i + G; block size B (G % B == 0); block index k_i in [0, G/B);
 * block k covers positions [P_i + k*B, P_i + (k+1)*B).  Hq query heads,
 * Hkv key/value heads (Hq % Hkv == 0, query head h reads KV head
 * h / (Hq/Hkv)), head dim d.  Lcap = row capacity of tokens, mask and caches.
 */
#ifndef FDLLM_H
#define FDLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FDLLM_VERSION 100 /* 1.0.0 */

typedef enum {
  FDLLM_OK = 0,
  FDLLM_ERR_INVALID_ARG = 1, /* a scalar, pointer or size is invalid */
  FDLLM_ERR_UNSUPPORTED = 2, /* valid, but not implemented (dtype, head_dim, alignment) */
  FDLLM_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace query */
  FDLLM_ERR_LAUNCH = 4       /* the HIP runtime rejected a kernel launch */
} fdllm_status;

/* Which K/V rows are recomputed ("fresh") this step; all others are read
 * from the cache.  [NEWS] item 1, [README] item 1 and its Usage flags:
 *   NONE   (no cache)                       fresh rows [0, L_i)
 *   PREFIX (--use_cache)                    fresh rows [P_i + k_i*B, L_i)
 *   DUAL   (--use_cache --if_cache_position) fresh rows [P_i + k_i*B, P_i + (k_i+1)*B)
 * The fresh rows are also the query rows: nq_i = a1 - a0. */
typedef enum { FDLLM_CACHE_NONE = 0, FDLLM_CACHE_PREFIX = 1, FDLLM_CACHE_DUAL = 2 } fdllm_cache_mode;

typedef enum { FDLLM_BF16 = 0, FDLLM_F32 = 1 } fdllm_dtype;

/* Per-batch sequence geometry (host struct). */
typedef struct {
  int32_t batch;            /* b >= 1 */
  int32_t max_seq_len;      /* Lcap >= every L_i */
  int32_t gen_len;          /* G >= 1, G % block_size == 0 */
  int32_t block_size;       /* B >= 1 */
  int32_t prompt_len;       /* uniform P, used when prompt_lens == NULL */
  int32_t block_idx;        /* uniform k, used when block_idxs == NULL; 0 <= k < G/B */
  const int32_t* prompt_lens; /* device [b] or NULL (then every P_i = prompt_len) */
  int32_t* block_idxs;      /* device [b] or NULL (then every k_i = block_idx);
                               fdllm_unmask_threshold may advance it */
  int32_t max_prompt_len;   /* host upper bound of prompt_lens (used only when
                               prompt_lens != NULL, for grid sizing);
                               max_prompt_len + G <= Lcap */
} fdllm_seq_desc;

/* Attention geometry (host struct). */
typedef struct {
  int32_t n_q_heads;   /* Hq >= 1 */
  int32_t n_kv_heads;  /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;    /* d: 64 or 128 (bf16 d = 128 runs on the matrix cores,
                          bf16 d = 64 and f32 on the vector ALUs) */
  int32_t dtype;       /* fdllm_dtype of q, k, v, caches and out */
  float scale;         /* softmax scale; 0 selects 1/sqrt(d) */
} fdllm_attn_desc;

/* ------------------------------------------------------------------ */
/* (a) block attention                                                 */
/* ------------------------------------------------------------------ */

/* Bytes of workspace fdllm_block_attn needs for this geometry at any block
 * index (0 when no block index splits the key range across workgroups):
 * the result does not depend on seq->block_idx or on fresh_rows beyond
 * their validation, so it can be queried once for a whole decode loop.
 * Calls check the bytes they use against workspace_bytes
 * (FDLLM_ERR_WORKSPACE when short).  Returns 0 on invalid input. */
size_t fdllm_block_attn_workspace(const fdllm_seq_desc* seq, const fdllm_attn_desc* attn,
                                  int32_t mode, int32_t fresh_rows);

/* Bidirectional attention of the fresh rows of each sequence over the key
 * rows [0, L_i), with K/V row j taken from k_new/v_new when a0 <= j < a1
 * and from the cache otherwise ([README] item 1, [NEWS] "Challenges": no
 * causal mask).  out[r] = sum_j softmax_j(scale * q[r].K_j) V_j.
 *
 *   q       [b][fresh_rows][Hq][d]   row r holds position a0 + r
 *   k_new   [b][fresh_rows][Hkv][d]  fresh K rows, same row convention
 *   v_new   [b][fresh_rows][Hkv][d]
 *   k_cache [b][Hkv][Lcap][d]        head-major cache; NULL allowed in NONE
 *   v_cache [b][Hkv][Lcap][d]
 *   out     [b][fresh_rows][Hq][d]   same dtype as the inputs; rows >= nq_i
 *                                    are not written; must not alias inputs
 * fresh_rows: row capacity per sequence of the fresh tensors; must be
 * >= nq_i for every sequence (checked on the host for uniform batches; for
 * ragged batches it must be >= B (DUAL), G (PREFIX), max_prompt_len + G
 * (NONE)).  All tensors contiguous; base pointers 16-byte aligned. */
fdllm_status fdllm_block_attn(const fdllm_seq_desc* seq, const fdllm_attn_desc* attn,
                              int32_t mode, int32_t fresh_rows,
                              const void* q, const void* k_new, const void* v_new,
                              const void* k_cache, const void* v_cache, void* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ */
/* (b) confidence-aware parallel unmasking                            */
/* ------------------------------------------------------------------ */

#define FDLLM_UNMASK_ADVANCE_BLOCK 1u /* k_i += 1 when block i is done and k_i + 1 < G/B
                                         (needs seq->block_idxs != NULL) */

/* Workspace bytes of fdllm_unmask_threshold / _topk (0 on invalid input).
 * Its counters (at the start, placed by the batch size alone) are shared
 * with the fused LM-head calls of the same batch. */
size_t fdllm_unmask_workspace(const fdllm_seq_desc* seq, int32_t vocab, int32_t logits_dtype);

/* One decoding step of the threshold rule ([README] item 2, [NEWS] item 2,
 * [ABS]).  For every masked position of the current block (row t <->
 * position P_i + k_i*B + t):
 *   m_t = max_v logit, Z_t = sum_v exp(logit - m_t), conf_t = 1 / Z_t,
 *   tok_t = lowest v with logit == m_t.
 * Selected set S_i = { t masked : conf_t > threshold } (strict, compared in
 * float64); if S_i is empty and some row is masked, S_i = { the masked row
 * with the largest conf_t, lowest t on a tie }.  For t in S_i:
 * tokens[pos] = tok_t, mask[pos] = 0.  Decoded tokens are never re-masked.
 *
 *   logits     [b][B][vocab] addressed as logits + i*seq_stride + t*row_stride
 *              (strides in elements); rows of unmasked positions are not read.
 *              bf16 or f32; every logit must be finite.
 *   tokens     int32 [b][Lcap] in/out;  mask uint8 [b][Lcap] in/out (1 = masked)
 *   n_decoded  int32 [b] out: |S_i|
 *   decoded_pos int32 [b][B] out or NULL: S_i ascending, padded with -1
 *   conf       double [b][B] out or NULL: conf_t for masked rows, NaN otherwise
 *   done_seqs  int32 [b] out or NULL: ascending ids of sequences whose block
 *              has no masked position left after this step
 *   n_done     int32 [1] out or NULL: number of entries in done_seqs
 * threshold: any finite float (>= 1 always falls back to one token; <= 0
 * decodes every masked row); NaN is rejected.
 * Vector path: logits, seq_stride and row_stride 16-byte aligned (in bytes);
 * otherwise a scalar path is used. */
fdllm_status fdllm_unmask_threshold(const fdllm_seq_desc* seq, int32_t vocab, int32_t logits_dtype,
                                    const void* logits, int64_t seq_stride, int64_t row_stride,
                                    float threshold, uint32_t flags,
                                    int32_t* tokens, uint8_t* mask, int32_t* n_decoded,
                                    int32_t* decoded_pos, double* conf,
                                    int32_t* done_seqs, int32_t* n_done,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* fdllm_unmask_threshold without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, rule, outputs and
 * kernels as fdllm_unmask_threshold minus workspace / workspace_bytes: the
 * arrival counters and vocabulary-chunk partials live in a static scratch
 * array of the library (8 MiB per device, held until the process ends; the
 * first call on a device finds its address and clears its counters with a
 * fill kernel on `stream`).  Limits: batch <= 4096 and batch x block_size x
 * vocabulary chunks x 16 bytes <= 8 MiB - 576 KiB (a call beyond them returns
 * FDLLM_ERR_UNSUPPORTED and launches nothing).  Every call on a device
 * shares that device's scratch: calls that overlap in time on one device
 * (different streams without ordering, or several host threads) race and
 * must not be issued; the first call on a device must be ordered before
 * calls on other streams.  Allocates nothing, synchronises nothing. */
fdllm_status fdllm_unmask_threshold_static(const fdllm_seq_desc* seq, int32_t vocab, int32_t logits_dtype,
                                           const void* logits, int64_t seq_stride, int64_t row_stride,
                                           float threshold, uint32_t flags,
                                           int32_t* tokens, uint8_t* mask, int32_t* n_decoded,
                                           int32_t* decoded_pos, double* conf,
                                           int32_t* done_seqs, int32_t* n_done, void* stream);

/* One step of fixed-step decoding ([README] "Usage": a fixed number of
 * sampling steps, so a fixed number of tokens per step -- the decoding the
 * evaluation table's "LLaDA" and "+cache" columns use).  Same vocabulary
 * pass, confidence and token as fdllm_unmask_threshold; the selected set is
 * the min(k, m_i) masked rows of the current block with the largest conf_t,
 * the lower t first among equal conf_t (compared in float64).  Outputs,
 * flags, strides, workspace (fdllm_unmask_workspace) and alignment as in
 * fdllm_unmask_threshold; done_seqs / n_done list the sequences whose block
 * has no masked row left.  k >= 1, else FDLLM_ERR_INVALID_ARG; for a
 * schedule of `steps` steps over gen_len tokens in blocks of B, k =
 * B / (steps / (gen_len / B)). */
fdllm_status fdllm_unmask_topk(const fdllm_seq_desc* seq, int32_t vocab, int32_t logits_dtype,
                               const void* logits, int64_t seq_stride, int64_t row_stride,
                               int32_t k, uint32_t flags,
                               int32_t* tokens, uint8_t* mask, int32_t* n_decoded,
                               int32_t* decoded_pos, double* conf,
                               int32_t* done_seqs, int32_t* n_done,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ */
/* (b') the vocabulary projection fused with the confidence pass      */
/* ------------------------------------------------------------------ */

/* The logits whose softmax maximum is the confidence and whose argmax is
 * the token ([README] "Key techniques" item 2) come from projecting each
 * block row's final hidden state onto the vocabulary:
 *   logits[i][t][v] = sum_k x[i][t][k] * w[v][k]   (no bias),
 * computed in fp32 from bf16 x and w on the matrix cores and reduced in
 * registers; the logits are never written to memory.  The steps below then
 * equal fdllm_unmask_threshold / fdllm_unmask_topk applied to those fp32
 * logits (conf_t = 1 / sum_v exp(logit_v - max), tok_t = lowest argmax).
 *
 * w is first rearranged once into the kernel's layout: 1 KB fragments, one
 * per (32 vocabulary rows, 16 hidden dims), each holding what a wave feeds
 * one 32x32x16 matrix instruction; the hidden dimension is zero-padded to a
 * multiple of 512 and the vocabulary to a multiple of 32.
 *
 * Sizes: 1 <= vocab <= 2^28; hidden a positive multiple of 8, <= 2^20. */

/* Bytes of the packed weight for (vocab, hidden); 0 on invalid sizes. */
size_t fdllm_lmhead_packed_bytes(int32_t vocab, int32_t hidden);

/* Pack w (bf16 [vocab][hidden], row-major, contiguous) into w_packed
 * (w_packed_bytes >= fdllm_lmhead_packed_bytes).  Both 16-byte aligned, not
 * overlapping.  One kernel on `stream`; bit-exact rearrangement. */
fdllm_status fdllm_lmhead_pack(int32_t vocab, int32_t hidden, const void* w, void* w_packed,
                               size_t w_packed_bytes, void* stream);

/* Workspace bytes of fdllm_lmhead_unmask_threshold / _topk (0 on invalid
 * input).  Zero it once with fdllm_workspace_init; its counters reset
 * themselves. */
size_t fdllm_lmhead_unmask_workspace(const fdllm_seq_desc* seq, int32_t vocab, int32_t hidden);

/* One threshold-rule step (as fdllm_unmask_threshold) on the logits of
 * the hidden states x:
 *   x        bf16 [b][B][hidden] addressed as x + i*seq_stride + t*row_stride
 *            (strides in elements, multiples of 8; row_stride >= hidden;
 *            16-byte aligned).  Every row of the block is projected; rows of
 *            unmasked positions are computed and discarded.
 *   w_packed the output of fdllm_lmhead_pack for the same vocab and hidden.
 * threshold, flags, tokens, mask, n_decoded, decoded_pos, conf, done_seqs,
 * n_done: as in fdllm_unmask_threshold.  Two kernels on `stream` (the
 * projection, then a per-sequence finalisation); a timing-event pair armed
 * with fdllm_set_timing_events brackets both. */
fdllm_status fdllm_lmhead_unmask_threshold(const fdllm_seq_desc* seq, int32_t vocab, int32_t hidden,
                                           const void* x, int64_t seq_stride, int64_t row_stride,
                                           const void* w_packed, float threshold, uint32_t flags,
                                           int32_t* tokens, uint8_t* mask, int32_t* n_decoded,
                                           int32_t* decoded_pos, double* conf,
                                           int32_t* done_seqs, int32_t* n_done,
                                           void* workspace, size_t workspace_bytes, void* stream);

/* One fixed-step step (as fdllm_unmask_topk, k >= 1) on the logits of the
 * hidden states x; arguments as in fdllm_lmhead_unmask_threshold. */
fdllm_status fdllm_lmhead_unmask_topk(const fdllm_seq_desc* seq, int32_t vocab, int32_t hidden,
                                      const void* x, int64_t seq_stride, int64_t row_stride,
                                      const void* w_packed, int32_t k, uint32_t flags,
                                      int32_t* tokens, uint8_t* mask, int32_t* n_decoded,
                                      int32_t* decoded_pos, double* conf,
                                      int32_t* done_seqs, int32_t* n_done,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ */
/* (c) KV-cache refresh at a block boundary                           */
/* ------------------------------------------------------------------ */

/* Copy the K/V of a full forward into the caches ([REV] review 4, [NEWS]
 * item 1): cache[i][h][j][:] = src[i][j][h][:] for j < L_i (DUAL),
 * j < P_i + k_i*B (PREFIX, with the block index of the block about to be
 * decoded), nothing (NONE).  Other rows are untouched.  Bit-exact copy.
 *
 *   k_src, v_src     [b][Lcap][Hkv][d] token-major
 *   k_cache, v_cache [b][Hkv][Lcap][d] head-major
 *   seq_ids  int32 device list of sequences to refresh, or NULL for all b
 *   n_seq    int32 device [1]: entries of seq_ids (required with seq_ids),
 *            e.g. the done_seqs / n_done outputs of fdllm_unmask_threshold.
 * Uses attn->n_kv_heads, head_dim and dtype; n_q_heads and scale are ignored.
 * Pointers 16-byte aligned. */
fdllm_status fdllm_kv_refresh(const fdllm_seq_desc* seq, const fdllm_attn_desc* attn, int32_t mode,
                              const void* k_src, const void* v_src, void* k_cache, void* v_cache,
                              const int32_t* seq_ids, const int32_t* n_seq, void* stream);

/* The refresh of several layers at one block boundary ([REV] review 4: the
 * K/V of every layer are recomputed once a block is decoded) in one kernel
 * launch: for l < n_layers, layer l's caches k_cache[l] / v_cache[l] get
 * exactly what fdllm_kv_refresh(seq, attn, mode, k_src[l], v_src[l],
 * k_cache[l], v_cache[l], seq_ids, n_seq, stream) writes.  The per-layer
 * calls of a small refresh (a few finished sequences) each last about a
 * launch and one memory round trip; one launch for all layers streams them
 * at the full rate.
 *   n_layers 1..FDLLM_MAX_REFRESH_LAYERS
 *   k_src, v_src, k_cache, v_cache  HOST arrays of n_layers DEVICE pointers
 *            (the caller keeps them; read during the call only), each laid
 *            out as in fdllm_kv_refresh, 16-byte aligned.
 * No cache may overlap another layer's cache or any layer's source
 * (FDLLM_ERR_INVALID_ARG); sources may be shared.  Other arguments and
 * errors as in fdllm_kv_refresh. */
#define FDLLM_MAX_REFRESH_LAYERS 64
fdllm_status fdllm_kv_refresh_layers(const fdllm_seq_desc* seq, const fdllm_attn_desc* attn, int32_t mode,
                                     int32_t n_layers, const void* const* k_src, const void* const* v_src,
                                     void* const* k_cache, void* const* v_cache, const int32_t* seq_ids,
                                     const int32_t* n_seq, void* stream);

/* ------------------------------------------------------------------ */
/* utilities                                                           */
/* ------------------------------------------------------------------ */

/* Zero a workspace (a fill kernel on `stream`; no memset node, so it can be
 * captured in a graph).  bytes must be a multiple of 4. */
fdllm_status fdllm_workspace_init(void* workspace, size_t bytes, void* stream);

/* Debug mode (process-wide; initial value from the environment variable
 * FDLLM_DEBUG): 1 = before its kernels, every call that reads device-
 * resident per-sequence arrays checks them on the device -- 0 <=
 * prompt_lens[i] <= max_prompt_len, 0 <= block_idxs[i] < gen_len /
 * block_size, 0 <= *n_seq <= batch, 0 <= seq_ids[j] < batch for j < *n_seq
 * -- then synchronises `stream` and returns FDLLM_ERR_INVALID_ARG (naming
 * the first bad entry) without launching anything when one fails.  Not for
 * use under stream capture; concurrent debug-mode calls from several host
 * threads take turns (a host lock spans each check).
 * 0 = the arrays are trusted (default).  FDLLM_ERR_INVALID_ARG for other
 * values. */
fdllm_status fdllm_set_debug(int32_t on);

/* Measurement hook for profilers and benchmarks: the next kernel launched by
 * an fdllm_* call on this host thread records start_event when it begins and
 * stop_event when it ends (hipExtLaunchKernel), so hipEventElapsedTime gives
 * the kernel's own duration.  Both are hipEvent_t (as void*) created by the
 * caller; either may be NULL.  The hook is consumed by that one launch;
 * (NULL, NULL) disarms it.  Not for use under stream capture. */
fdllm_status fdllm_set_timing_events(void* start_event, void* stop_event);

/* Launch-planner overrides, for tuning and for tests that exercise every
 * kernel variant on one input.  0 keeps the automatic choice (which the
 * environment variables FDLLM_ATTN_QT, FDLLM_ATTN_TARGET_WGS and
 * FDLLM_UNMASK_TARGET_WGS, read once per process, also override).
 *   attn_qt     1: split-key attention kernel (one query tile per
 *               workgroup, bf16); 2 or 4: LDS-ring kernel with that many
 *               query tiles of one KV head per workgroup; 8: 8-wave LDS ring
 *               with one query tile per wave (8 per workgroup), key-chunk
 *               partials merged by a second kernel in the same call; 16:
 *               the 8-wave ring run over the whole batch's K/V tile stream,
 *               cut into equal ranges, one persistent workgroup per CU, the
 *               pieces of cut (sequence, KV head) segments merged by a
 *               second kernel (one query tile per head and at most 8 heads
 *               per KV head; other geometries take 8).
 *   attn_wgs    workgroups the attention key split aims for (0..65536).
 *   unmask_wgs  workgroups the unmask vocab split aims for (0..65536).
 * Per host thread: they apply to the calls and workspace queries made on
 * the calling thread only.  The workspace sizes reported afterwards follow
 * the new plan: query them again and re-zero a workspace sized under the
 * old setting before reusing it (calls check the size they need).
 * FDLLM_ERR_INVALID_ARG for an attn_qt outside {0, 1, 2, 4, 8, 16} or a target
 * outside [0, 65536]. */
fdllm_status fdllm_set_tuning(int32_t attn_qt, int32_t attn_wgs, int32_t unmask_wgs);

/* Planner override of the fused vocabulary projection: vocabulary tiles of
 * 32 rows per wave (1 or 2; 0 = automatic, which the environment variable
 * FDLLM_LMHEAD_VT also overrides).  Calls with more than 64 rows (batch x
 * block size) always use 1.  Per host thread, like fdllm_set_tuning; query
 * fdllm_lmhead_unmask_workspace again afterwards.  FDLLM_ERR_INVALID_ARG
 * outside {0, 1, 2}. */
fdllm_status fdllm_set_lmhead_tuning(int32_t vt);

const char* fdllm_status_string(int32_t status);
const char* fdllm_last_error(void);
int32_t fdllm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FDLLM_H */
