// Internal declarations shared by the host API and the kernel translation
// units of libfdllm.  Not installed; the public ABI is include/fdllm.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fdllm {

// Division by a run-time invariant divisor with one multiply-high and a
// shift (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994).  Valid for 0 <= n < 2^31 and 1 <= d < 2^31.
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.s = s;
  // m = floor(2^32 * (2^s - d) / d) + 1
  f.m = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  uint32_t t = __umulhi(n, f.m);
  return (t + n) >> f.s;
}

// Sequence geometry resolved for the device.
struct SeqArgs {
  int b, Lcap, G, B;
  int P, k;                 // uniform values when the pointers are null
  const int32_t* plens;     // [b] or null
  int32_t* bidx;            // [b] or null
};

__device__ __forceinline__ int seq_prompt(const SeqArgs& s, int i) { return s.plens ? s.plens[i] : s.P; }
__device__ __forceinline__ int seq_block(const SeqArgs& s, int i) { return s.bidx ? s.bidx[i] : s.k; }

enum { MODE_NONE = 0, MODE_PREFIX = 1, MODE_DUAL = 2 };

// ------------------------------------------------------------------ refresh
struct RefreshArgs {
  SeqArgs sq;
  int mode;
  int Hkv;
  int row_vec_shift;        // log2(16-byte vectors per (row, head))
  FastDiv hkv_div;
  const uint4* k_src;
  const uint4* v_src;
  uint4* k_cache;
  uint4* v_cache;
  const int32_t* seq_ids;   // null = all
  const int32_t* n_seq;
};
hipError_t launch_kv_refresh(const RefreshArgs& a, int max_rows, hipStream_t st);
// The refresh of several layers in one launch: layer l (grid z) moves
// k_src[l] / v_src[l] into k_cache[l] / v_cache[l] with RefreshArgs' geometry.
constexpr int kMaxRefreshLayers = 64;
struct RefreshLayerPtrs {
  const uint4* k_src[kMaxRefreshLayers];
  const uint4* v_src[kMaxRefreshLayers];
  uint4* k_cache[kMaxRefreshLayers];
  uint4* v_cache[kMaxRefreshLayers];
};
hipError_t launch_kv_refresh_layers(const RefreshArgs& a, const RefreshLayerPtrs& p, int n_layers, int max_rows,
                                    hipStream_t st);

// ------------------------------------------------------------------ unmask
struct UnmaskPartial {      // per (sequence, row, vocab chunk)
  float m;                  // max logit of the chunk
  int32_t idx;              // lowest vocab id attaining m in the chunk
  double z;                 // sum over the chunk of exp(logit - m)
};

// The per-sequence arrival counters sit one to a 128-byte line: atomics on
// one line serialise, and with the counters packed 32 to a line the
// arrivals of a 64-sequence batch split two ways took 88 us instead of 82.
constexpr int kSeqCntStride = 32;

struct UnmaskArgs {
  SeqArgs sq;
  int V;
  int64_t seq_stride, row_stride;  // elements
  const void* logits;
  int vec;                  // 1: 16-byte vector loads (aligned rows)
  float tau;
  int topk;                 // > 0: fixed-step rule (the topk most confident masked rows); 0: threshold rule
  uint32_t flags;
  int32_t* tokens;
  uint8_t* mask;
  int32_t* n_decoded;
  int32_t* decoded_pos;
  double* conf;
  int32_t* done_seqs;
  int32_t* n_done;
  UnmaskPartial* part;      // [b][nchunk][B] chunk partials (a chunk's rows adjacent)
  uint64_t* glob;           // [2] finished-sequence counter (and done bits)
  int32_t* done_flag;       // [b] x 8 bytes
  uint32_t* seq_cnt;        // [b] x kSeqCntStride words: one arrival counter per 128-byte line
  int nchunk;               // vocab chunks per row (one workgroup each)
  int chunk;                // vocab entries per chunk (multiple of the vector width)
};
struct UnmaskPlan {
  int nchunk, chunk;
};
UnmaskPlan plan_unmask(int dtype, int V, int rows);
void set_unmask_tuning(int wgs);
size_t unmask_workspace_bytes(int b, int B, int nchunk);
void unmask_bind_workspace(UnmaskArgs& a, void* workspace);
hipError_t launch_unmask(const UnmaskArgs& a, int dtype, hipStream_t st);

// ------------------------------------------------------------------ LM head
// The vocabulary projection fused with the confidence pass (lmhead.hip) and
// the per-sequence finalisation of its partials (unmask.hip).
constexpr int kLmheadHpad = 512;  // packed hidden size is a multiple of this

struct LmheadArgs {
  int M;                    // rows = b * B (row r = i * B + t)
  int B;
  int H, Hp;                // hidden size; padded to a multiple of kLmheadHpad
  int V, nvt;               // vocabulary; 32-row tiles
  int n_vwg;                // vocabulary workgroups = partials per row
  int tiles_per_wg;         // vocabulary tiles per workgroup
  int n_rg;                 // row groups (32 * RT rows each)
  int n_items;              // n_vwg * n_rg
  int per_xcd;              // work items per XCD slice of the grid
  int64_t seq_stride, row_stride;  // hidden-state strides in elements
  const uint16_t* x;        // bf16 hidden states
  const uint4* wp;          // packed weight
  UnmaskPartial* part;      // [M][n_vwg]
};
struct LmheadPlan {
  int rt, vt;               // row tiles per workgroup, vocabulary tiles per wave
  int n_vwg, n_rg, tiles_per_wg, n_items, per_xcd, grid;
};
LmheadPlan plan_lmhead(int M, int V);
void set_lmhead_tuning(int vt);
size_t lmhead_packed_bytes(int V, int H);
hipError_t launch_lmhead_pack(const void* w, void* wp, int V, int H, hipStream_t st);
hipError_t launch_lmhead(const LmheadArgs& a, const LmheadPlan& p, hipStream_t st, hipEvent_t ev_start);
hipError_t launch_lmhead_finalize(const UnmaskArgs& a, const UnmaskPartial* part, int n_vwg, hipStream_t st,
                                  hipEvent_t ev_stop);

// ------------------------------------------------------------------ attention
struct AttnArgs {
  SeqArgs sq;
  int mode;
  int fresh_rows;
  int Hq, Hkv, g;
  float scale;              // softmax scale
  float scale_log2;         // scale * log2(e)
  const void* q;
  const void* kn;
  const void* vn;
  const void* kc;
  const void* vc;
  void* out;
  float* part;              // split-key partials [b][Hq][n_qt][n_split] (null when n_split == 1)
  uint32_t* cnt;            // arrival counters of the in-kernel merges (start of the workspace)
  int n_qt;                 // query tiles per (sequence, query head)
  int n_grp;                // query-tile groups per (sequence, KV head)
  int n_split;              // key chunks per group
  int kchunk;               // keys per chunk
  int n_items;
  int per_xcd;              // work items per XCD slice of the grid
};

struct AttnPlan {
  int qt_per_wg;            // query tiles sharing each K/V tile in a workgroup (1, 2 or 4)
  int n_qt, n_grp, n_split, kchunk, n_items, per_xcd, grid;
  size_t part_bytes;        // split partials (after the counters); 0: one key chunk, no workspace
};
AttnPlan plan_block_attn(int dtype, int b, int Hq, int Hkv, int d, int nq_max, int L_max, bool ragged);
void set_attn_tuning(int qt, int wgs);
size_t attn_counter_bytes(int b, int Hq, int nq_bound);
size_t attn_workspace_bytes(int dtype, int b, int Hq, int Hkv, int d, int nq_bound, int L_max, bool ragged);
void attn_bind_workspace(AttnArgs& a, const AttnPlan& p, void* workspace, size_t counter_bytes);
hipError_t launch_block_attn(const AttnArgs& a, const AttnPlan& p, int dtype, int d, hipStream_t st);

// ------------------------------------------------------------------ misc
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

// Debug-mode check of the device-resident per-sequence arrays (validate.hip):
// key_out receives index * 8 + code of the first problem, or INT_MAX.
enum { VALIDATE_PROMPT = 1, VALIDATE_BLOCK = 2, VALIDATE_NSEQ = 3, VALIDATE_SEQID = 4 };
hipError_t run_validate(const SeqArgs& sq, int max_P, const int32_t* seq_ids, const int32_t* n_seq, hipStream_t st,
                        int* key_out);

// Measurement hook (fdllm_set_timing_events): returns the armed start/stop
// events of the calling host thread (null when not armed) and disarms it.
struct LaunchEvents {
  hipEvent_t start, stop;
};
LaunchEvents take_launch_events();

// Launch `kernel` on `st`.  With a start and/or stop event, the launch
// records them at the kernel's start / end (hipExtLaunchKernel).  A call that
// runs several kernels passes the start event to the first and the stop
// event to the last.
template <typename... Args>
hipError_t launch_kernel(void (*kernel)(Args...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t st,
                         hipEvent_t ev_start, hipEvent_t ev_stop, Args... args) {
  if (ev_start || ev_stop) {
    void* argv[] = {(void*)&args...};
    return hipExtLaunchKernel((const void*)kernel, grid, block, argv, shmem, st, ev_start, ev_stop, 0);
  }
  hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
  return hipGetLastError();
}

}  // namespace fdllm
