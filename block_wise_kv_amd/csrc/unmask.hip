// Confidence-aware parallel unmasking: one decoding step of the threshold rule.
//
// Fast-dLLM (project README "Key techniques" item 2; aibase news
// "Innovations" item 2; paper abstract): in each step every still-masked
// position of the current block whose confidence exceeds the threshold is
// decoded, the others stay masked.  Confidence is the largest softmax
// probability of the position and the decoded token its argmax (lowest id
// on a tie); when no position passes, the single most confident one is
// decoded so that every step makes progress.
//
// One launch, three levels:
//   1. workgroup (c, t, i) reads vocab chunk c (16384 bf16 or 8192 f32
//      logits) of block row t of sequence i once from HBM: every thread
//      issues all of its 16-byte loads at once; per thread (max, lowest
//      argmax, sum of exp(l - max)) with one exp per logit summed pairwise in
//      fp32; threads merge in fp64.  Rows are split into as many chunks as
//      needed and the hardware overlaps the workgroups of a CU;
//   2. if a row is split into several chunks, the last chunk workgroup to
//      arrive merges the row (fp64);
//   3. the last row to arrive for sequence i applies the threshold and the
//      fallback, commits tokens and mask, and writes the per-sequence
//      outputs; the last sequence writes the ascending done list.
// Partial results are published with agent-scope write-through stores
// followed by a wait for their completion and a relaxed counter atomic, and
// read back with agent-scope loads, so no L2 write-back or invalidate is
// needed.  Counters are reset by their last user (the workspace stays zeroed).
#include <float.h>
#include <limits.h>

#include "fdllm_device.h"
#include "fdllm_internal.h"

namespace fdllm {

constexpr int kUT = 256;           // threads per workgroup
constexpr int kUWaves = kUT / 64;
constexpr int kU = 8;              // 16-byte vectors per thread per iteration
constexpr int kMaxBlockSize = 1024;
constexpr int kMaxDoneList = 1024;   // done flags read per pass

__device__ __forceinline__ void put_partial(UnmaskPartial* p, float m, int idx, double z) {
  const uint64_t w0 = (uint64_t)__float_as_uint(m) | ((uint64_t)(uint32_t)idx << 32);
  st_coherent((uint64_t*)p, w0);
  st_coherent((uint64_t*)p + 1, (uint64_t)__double_as_longlong(z));
}
__device__ __forceinline__ void get_partial(const UnmaskPartial* p, float& m, int& idx, double& z) {
  const uint64_t w0 = ld_coherent((const uint64_t*)p);
  const uint64_t w1 = ld_coherent((const uint64_t*)p + 1);
  m = __uint_as_float((uint32_t)w0);
  idx = (int)(uint32_t)(w0 >> 32);
  z = __longlong_as_double((long long)w1);
}

// ---- logits vectors
template <bool BF16>
struct Vec;
template <>
struct Vec<true> {  // 8 bf16
  static constexpr int W = 8;
  __device__ static void unpack(const uint4& w, float* x) {
    x[0] = bf16lo(w.x); x[1] = bf16hi(w.x);
    x[2] = bf16lo(w.y); x[3] = bf16hi(w.y);
    x[4] = bf16lo(w.z); x[5] = bf16hi(w.z);
    x[6] = bf16lo(w.w); x[7] = bf16hi(w.w);
  }
  __device__ static float scalar(const void* row, int e) { return bf16_bits_to_f32(((const uint16_t*)row)[e]); }
};
template <>
struct Vec<false> {  // 4 f32
  static constexpr int W = 4;
  __device__ static void unpack(const uint4& w, float* x) {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
  __device__ static float scalar(const void* row, int e) { return ((const float*)row)[e]; }
};

// Pairwise sum of n floats in place (result in x[0]).
template <int N>
__device__ __forceinline__ float pairwise_sum(float* x) {
  constexpr int P = (N <= 1) ? 1 : (N <= 2) ? 2 : (N <= 4) ? 4 : (N <= 8) ? 8 : (N <= 16) ? 16
                  : (N <= 32) ? 32 : (N <= 64) ? 64 : 128;
#pragma unroll
  for (int w = P / 2; w >= 1; w /= 2) {
#pragma unroll
    for (int j = 0; j < w; ++j)
      if (j + w < N) x[j] += x[j + w];
  }
  return x[0];
}

// Running per-thread reduction state.
struct RowAcc {
  float m;
  int idx;
  double z;
};

// Fold one iteration's values (indices idx_of(k), ascending in k) into acc.
template <int N>
__device__ __forceinline__ void fold(RowAcc& acc, float* x, int base_index, int stride_vec, int W) {
  float lm = -INFINITY;
#pragma unroll
  for (int k = 0; k < N; ++k) lm = fmaxf(lm, x[k]);
  const float m_new = fmaxf(acc.m, lm);
  if (m_new == -INFINITY) return;
  if (lm > acc.m) {
    // the new maximum lies in this iteration: its first occurrence
    int found = INT_MAX;
#pragma unroll
    for (int k = N - 1; k >= 0; --k)
      if (x[k] == lm) found = base_index + (k / W) * stride_vec * W + (k % W);
    acc.idx = found;
  }
  // x - m_new is exact for bf16 / f32 logits of similar magnitude, so the
  // maximum contributes exactly 1 and only the small terms carry rounding
#pragma unroll
  for (int k = 0; k < N; ++k) x[k] = exp2_fast((x[k] - m_new) * kLog2e);
  const float s = pairwise_sum<N>(x);
  const double scale = (acc.m == -INFINITY) ? 0.0 : (double)exp2_fast((acc.m - m_new) * kLog2e);
  acc.z = acc.z * scale + (double)s;
  acc.m = m_new;
}

// Workgroup merge of per-thread states: (max, lowest index at the max, sum rescaled to the max).
__device__ RowAcc block_merge(const RowAcc& a) {
  __shared__ float s_m[kUWaves];
  __shared__ int s_i[kUWaves];
  __shared__ double s_z[kUWaves];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  float M = wave_max(a.m);
  if (lane == 0) s_m[wid] = M;
  __syncthreads();
  M = s_m[0];
#pragma unroll
  for (int w = 1; w < kUWaves; ++w) M = fmaxf(M, s_m[w]);
  int idx = (a.m == M) ? a.idx : INT_MAX;
  // the thread holding the maximum is rescaled by exactly 1
  double z = (a.m == -INFINITY) ? 0.0 : a.z * (double)exp2_fast((a.m - M) * kLog2e);
  idx = wave_min_i(idx);
  z = wave_sum_d(z);
  __syncthreads();
  if (lane == 0) {
    s_i[wid] = idx;
    s_z[wid] = z;
  }
  __syncthreads();
  RowAcc r;
  r.m = M;
  r.idx = s_i[0];
  r.z = s_z[0];
#pragma unroll
  for (int w = 1; w < kUWaves; ++w) {
    r.idx = min(r.idx, s_i[w]);
    r.z += s_z[w];
  }
  return r;
}

// Lexicographic max of (conf, -t): the highest confidence, lowest row on a tie.
__device__ __forceinline__ void best_of(double& c, int& t, double c2, int t2) {
  if (c2 > c || (c2 == c && t2 < t)) {
    c = c2;
    t = t2;
  }
}

// Per-sequence finalisation, run by the last row workgroup of sequence i.
// Rows are handled 256 at a time, one per thread; counts, the fallback
// argmax and the ranks of selected rows come from workgroup reductions.
__device__ void unmask_finalize(const UnmaskArgs& a, int i, int start) {
  __shared__ int s_cnt[kUWaves][2];
  __shared__ double s_bc[kUWaves];
  __shared__ int s_bt[kUWaves];
  __shared__ int s_rank[kUWaves];
  __shared__ int s_done, s_count;
  const int B = a.sq.B;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int32_t* trow = a.tokens + (size_t)i * a.sq.Lcap + start;
  uint8_t* mrow = a.mask + (size_t)i * a.sq.Lcap + start;
  const UnmaskPartial* rows = a.part + (size_t)a.sq.b * B * a.nchunk + (size_t)i * B;  // row results
  const double tau = (double)a.tau;
  const int np = (B + kUT - 1) / kUT;  // passes of 256 rows (B <= 1024)

  // pass 1: per-row confidence, counts and the most confident masked row
  double conf[kMaxBlockSize / kUT];
  int tok[kMaxBlockSize / kUT];
  bool msk[kMaxBlockSize / kUT];
  int n_masked = 0, n_pass = 0;
  double bc = -1.0;
  int bt = INT_MAX;
#pragma unroll
  for (int p = 0; p < kMaxBlockSize / kUT; ++p) {
    const int t = p * kUT + tid;
    msk[p] = false;
    conf[p] = 0.0;
    tok[p] = 0;
    if (p < np && t < B && mrow[t]) {
      float m;
      double z;
      get_partial(rows + t, m, tok[p], z);
      msk[p] = true;
      conf[p] = 1.0 / z;
      best_of(bc, bt, conf[p], t);
    }
    n_masked += msk[p];
    n_pass += msk[p] && conf[p] > tau;
  }
  // workgroup reductions
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    n_masked += __shfl_xor(n_masked, o, 64);
    n_pass += __shfl_xor(n_pass, o, 64);
    best_of(bc, bt, __shfl_xor(bc, o, 64), __shfl_xor(bt, o, 64));
  }
  if (lane == 0) {
    s_cnt[wid][0] = n_masked;
    s_cnt[wid][1] = n_pass;
    s_bc[wid] = bc;
    s_bt[wid] = bt;
  }
  __syncthreads();
  n_masked = 0;
  n_pass = 0;
  bc = -1.0;
  bt = INT_MAX;
#pragma unroll
  for (int w = 0; w < kUWaves; ++w) {
    n_masked += s_cnt[w][0];
    n_pass += s_cnt[w][1];
    best_of(bc, bt, s_bc[w], s_bt[w]);
  }
  const bool fallback = (n_pass == 0 && n_masked > 0);

  // pass 2: commit selected rows in ascending order
  int base = 0;
#pragma unroll
  for (int p = 0; p < kMaxBlockSize / kUT; ++p) {
    if (p >= np) break;
    const int t = p * kUT + tid;
    const bool sel = msk[p] && (fallback ? (t == bt) : (conf[p] > tau));
    const uint64_t bal = __ballot(sel);
    const int below = __popcll(bal & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) s_rank[wid] = __popcll(bal);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wid; ++w) off += s_rank[w];
    int tot = base;
    for (int w = 0; w < kUWaves; ++w) tot += s_rank[w];
    if (t < B) {
      if (sel) {
        trow[t] = tok[p];
        mrow[t] = 0;
        if (a.decoded_pos) a.decoded_pos[(size_t)i * B + off + below] = t;
      }
      if (a.conf) a.conf[(size_t)i * B + t] = msk[p] ? conf[p] : __longlong_as_double(0x7ff8000000000000ll);
    }
    base = tot;
  }
  const int n_sel = base;
  if (a.decoded_pos)
    for (int t = n_sel + tid; t < B; t += kUT) a.decoded_pos[(size_t)i * B + t] = -1;
  if (tid == 0) {
    a.n_decoded[i] = n_sel;
    const int done = (n_masked == n_sel) ? 1 : 0;
    if ((a.flags & 1u) && done && a.sq.bidx) {
      const int k = a.sq.bidx[i];
      if (k + 1 < a.sq.G / a.sq.B) a.sq.bidx[i] = k + 1;
    }
    a.seq_cnt[i] = 0u;
    s_done = done;
    s_count = 0;
  }
  if (!(a.done_seqs || a.n_done)) return;
  // the last sequence to finish writes the ascending list of finished ones
  __syncthreads();
  if (tid == 0) st_coherent((uint64_t*)(a.done_flag + 2 * i), (uint64_t)s_done);
  __shared__ int s_last;
  if (!block_arrive(a.glob_cnt, (unsigned)a.sq.b, &s_last)) return;
  for (int q = 0; q < a.sq.b; q += kUT) {
    const int s = q + tid;
    const bool fl = s < a.sq.b && ld_coherent((const uint64_t*)(a.done_flag + 2 * s)) != 0;
    const uint64_t bal = __ballot(fl);
    const int below = __popcll(bal & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) s_rank[wid] = __popcll(bal);
    __syncthreads();
    int off = s_count;
    for (int w = 0; w < wid; ++w) off += s_rank[w];
    if (fl && a.done_seqs) a.done_seqs[off + below] = s;
    __syncthreads();
    if (tid == 0)
      for (int w = 0; w < kUWaves; ++w) s_count += s_rank[w];
  }
  __syncthreads();
  if (tid == 0) {
    if (a.n_done) *a.n_done = s_count;
    *a.glob_cnt = 0u;
  }
}

template <bool BF16>
__global__ __launch_bounds__(kUT) void unmask_kernel(UnmaskArgs a) {
  using VT = Vec<BF16>;
  constexpr int W = VT::W;
  constexpr int N = kU * W;  // values per thread per iteration
  const int c = blockIdx.x, t = blockIdx.y, i = blockIdx.z;
  const int tid = threadIdx.x;
  const int B = a.sq.B;
  const int start = seq_prompt(a.sq, i) + seq_block(a.sq, i) * B;
  const bool masked = a.mask[(size_t)i * a.sq.Lcap + start + t] != 0;

  __shared__ int s_flag;
  UnmaskPartial* chunk_parts = a.part + ((size_t)i * B + t) * a.nchunk;
  UnmaskPartial* row_result = a.part + (size_t)a.sq.b * B * a.nchunk + (size_t)i * B + t;

  if (masked) {
    const size_t esz = BF16 ? 2 : 4;
    const char* row = (const char*)a.logits + ((size_t)i * a.seq_stride + (size_t)t * a.row_stride) * esz;
    const int e0 = c * a.chunk;                      // first vocab id of the chunk
    const int e1 = min(a.V, e0 + a.chunk);
    RowAcc acc{-INFINITY, INT_MAX, 0.0};
    // one chunk = at most kU vectors per thread: every load is issued at once
    if (a.vec) {
      const uint4* rv = (const uint4*)(row + (size_t)e0 * esz);
      const int nfull = (e1 - e0) / W;               // full vectors in the chunk
      if (nfull > 0) {
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) v[u] = rv[min(u * kUT + tid, nfull - 1)];
        float x[N];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          VT::unpack(v[u], x + u * W);
          const bool ok = u * kUT + tid < nfull;
#pragma unroll
          for (int e = 0; e < W; ++e) x[u * W + e] = ok ? x[u * W + e] : -INFINITY;
        }
        fold<N>(acc, x, e0 + tid * W, kUT, W);
      }
      // vocab entries past the last full vector of the chunk (fewer than W)
      if (tid == 0) {
        for (int e = e0 + nfull * W; e < e1; ++e) {
          float x1[1] = {VT::scalar(row, e)};
          fold<1>(acc, x1, e, 1, 1);
        }
      }
    } else {
      // unaligned rows: one logit per load
      float x[N];
#pragma unroll
      for (int k = 0; k < N; ++k) {
        const int e = e0 + k * kUT + tid;
        x[k] = (e < e1) ? VT::scalar(row, e) : -INFINITY;
      }
      fold<N>(acc, x, e0 + tid, kUT, 1);
    }
    const RowAcc r = block_merge(acc);
    if (tid == 0) put_partial(a.nchunk > 1 ? chunk_parts + c : row_result, r.m, r.idx, r.z);
  }

  // level 2: merge the row's chunks (only when the row is split); every
  // chunk partial is read at once (one per thread), then merged in fp64
  if (a.nchunk > 1) {
    if (!block_arrive(&a.row_cnt[(size_t)i * B + t], (unsigned)a.nchunk, &s_flag)) return;
    if (masked) {
      // one chunk per thread (nchunk <= 256): all partials read at once
      float m = -INFINITY;
      int idx = INT_MAX;
      double z = 0.0;
      if (tid < a.nchunk) get_partial(chunk_parts + tid, m, idx, z);
      RowAcc r{m, idx, z};
      r = block_merge(r);
      if (tid == 0) put_partial(row_result, r.m, r.idx, r.z);
    }
    if (tid == 0) a.row_cnt[(size_t)i * B + t] = 0u;
  }

  // level 3: the last row of the sequence finalises it
  if (!block_arrive(&a.seq_cnt[i], (unsigned)B, &s_flag)) return;
  unmask_finalize(a, i, start);
}

UnmaskPlan plan_unmask(int dtype, int V, int rows) {
  (void)rows;
  UnmaskPlan p{};
  const int W = dtype == 0 ? 8 : 4;
  p.chunk = kU * kUT * W;                        // one workgroup: kU vectors per thread
  p.nchunk = (V + p.chunk - 1) / p.chunk;
  return p;
}

size_t unmask_workspace_bytes(int b, int B, int nchunk) {
  size_t bytes = (size_t)b * B * nchunk * sizeof(UnmaskPartial);  // chunk partials
  bytes += (size_t)b * B * sizeof(UnmaskPartial);                 // row results
  bytes += (size_t)b * B * 4;                                     // row counters
  bytes += (size_t)b * 4;                                         // sequence counters
  bytes += 16;                                                    // global counter
  bytes += (size_t)b * 8;                                         // done flags
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_unmask(const UnmaskArgs& a, int dtype, hipStream_t st) {
  dim3 grid((unsigned)a.nchunk, (unsigned)a.sq.B, (unsigned)a.sq.b);
  dim3 block(kUT);
  const LaunchEvents ev = take_launch_events();
  return dtype == 0 ? launch_kernel(unmask_kernel<true>, grid, block, 0, st, ev.start, ev.stop, a)
                    : launch_kernel(unmask_kernel<false>, grid, block, 0, st, ev.start, ev.stop, a);
}

}  // namespace fdllm
