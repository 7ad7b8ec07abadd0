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
// One launch, two levels:
//   1. workgroup (c, t, i) reads vocab chunk c of block row t of sequence i
//      once from HBM, in iterations of 8 x 16-byte loads per thread; two
//      register buffers alternate so the next iteration's loads are in
//      flight while the current one is reduced.  Per thread it keeps the
//      running max, the iteration where that max first appeared, and the
//      sum of exp(l - max): one fma and one exp per logit, the exps of an
//      iteration summed pairwise in fp32 and accumulated in fp64.  The
//      lowest argmax is located after the chunk, only by the threads whose
//      max equals the chunk max (one reload of one iteration).
//   2. the last workgroup of sequence i to arrive merges every chunk of every
//      row (fp64), applies the threshold and the fallback with workgroup
//      reductions, commits tokens and mask, and writes the per-sequence
//      outputs; the last sequence writes the ascending done list.
// Partials are published with agent-scope write-through stores, a wait for
// their completion and a relaxed counter atomic, and read back with
// agent-scope loads: no L2 write-back or invalidate.  Counters are reset by
// their last user, so the workspace stays zeroed across calls.
#include <float.h>
#include <limits.h>
#include <stdlib.h>

#include <type_traits>

#include "fdllm_device.h"
#include "fdllm_internal.h"

namespace fdllm {

constexpr int kUT = 256;           // threads per workgroup
constexpr int kUWaves = kUT / 64;
constexpr int kU = 8;              // 16-byte vectors per thread per iteration
constexpr int kMaxBlockSize = 1024;
constexpr int kMaxChunks = 16;     // vocab chunks per row

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

// Pairwise sum of N floats in place (result in x[0]).
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

// Running per-thread state: max m, the iteration where m first appeared
// (-1: none, -2: in the scalar tail, whose index is idx), and
// z = sum over seen logits of exp(l - m).
struct RowAcc {
  float m;
  int it;
  int idx;
  double z;
};

// Fold n logits x[0..n) (one iteration) into acc.  The exps use the fp32
// reference r = round(m*log2 e): exp2(fma(x, log2 e, -r)) = exp(x - m) * 2^d
// with d = m*log2 e - r computed exactly by one more fma, so the iteration
// sum is corrected by 2^-d and the maximum contributes (to within an ulp)
// exactly 1.
template <int N>
__device__ __forceinline__ void fold(RowAcc& acc, float* x, int it) {
  float lm = -INFINITY;
#pragma unroll
  for (int k = 0; k < N; ++k) lm = fmaxf(lm, x[k]);
  if (lm > acc.m) acc.it = it;
  const float m_new = fmaxf(acc.m, lm);
  if (m_new == -INFINITY) return;
  const float r = m_new * kLog2e;
  const float d = fmaf(m_new, kLog2e, -r);
#pragma unroll
  for (int k = 0; k < N; ++k) x[k] = exp2_fast(fmaf(x[k], kLog2e, -r));
  const double s = (double)pairwise_sum<N>(x) * (double)exp2_fast(-d);
  const double scale = (acc.m == -INFINITY) ? 0.0 : (double)exp2_fast((acc.m - m_new) * kLog2e);
  acc.z = acc.z * scale + s;
  acc.m = m_new;
}

// Workgroup reductions.
__device__ float block_max(float v, float* s_f) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) s_f[wid] = v;
  __syncthreads();
  float r = s_f[0];
#pragma unroll
  for (int w = 1; w < kUWaves; ++w) r = fmaxf(r, s_f[w]);
  return r;
}
__device__ void block_sum_min(double z, int idx, double* s_d, int* s_i, double& z_out, int& idx_out) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  z = wave_sum_d(z);
  idx = wave_min_i(idx);
  __syncthreads();
  if (lane == 0) {
    s_d[wid] = z;
    s_i[wid] = idx;
  }
  __syncthreads();
  z_out = s_d[0];
  idx_out = s_i[0];
#pragma unroll
  for (int w = 1; w < kUWaves; ++w) {
    z_out += s_d[w];
    idx_out = min(idx_out, s_i[w]);
  }
}

// Lexicographic max of (conf, -t): the highest confidence, lowest row on a tie.
__device__ __forceinline__ void best_of(double& c, int& t, double c2, int t2) {
  if (c2 > c || (c2 == c && t2 < t)) {
    c = c2;
    t = t2;
  }
}

// Per-sequence finalisation by the last workgroup of sequence i.  Rows are
// handled 256 at a time, one per thread; every chunk partial of a row is
// loaded at once; counts, the fallback argmax and the ranks of selected rows
// come from workgroup reductions and ballots.
__device__ void unmask_finalize(const UnmaskArgs& a, int i, int start) {
  __shared__ int s_cnt[kUWaves][2];
  __shared__ double s_bc[kUWaves];
  __shared__ int s_bt[kUWaves];
  __shared__ int s_rank[kUWaves];
  __shared__ int s_done, s_count, s_last;
  const int B = a.sq.B;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int32_t* trow = a.tokens + (size_t)i * a.sq.Lcap + start;
  uint8_t* mrow = a.mask + (size_t)i * a.sq.Lcap + start;
  const double tau = (double)a.tau;
  const int np = (B + kUT - 1) / kUT;  // passes of 256 rows (B <= 1024)
  constexpr int kP = kMaxBlockSize / kUT;

  // pass 1: per-row confidence, counts and the most confident masked row
  double conf[kP];
  int tok[kP];
  bool msk[kP];
  int n_masked = 0, n_pass = 0;
  double bc = -1.0;
  int bt = INT_MAX;
#pragma unroll
  for (int p = 0; p < kP; ++p) {
    const int t = p * kUT + tid;
    msk[p] = false;
    conf[p] = 0.0;
    tok[p] = 0;
    if (p < np && t < B && mrow[t]) {
      const UnmaskPartial* pp = a.part + ((size_t)i * B + t) * a.nchunk;
      float mc[kMaxChunks];
      int ic[kMaxChunks];
      double zc[kMaxChunks];
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) get_partial(pp + min(c, a.nchunk - 1), mc[c], ic[c], zc[c]);
      float M = -INFINITY;
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) M = fmaxf(M, mc[c]);
      double Z = 0.0;
      int tk = INT_MAX;
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) {
        if (c < a.nchunk) {
          // the chunk holding the maximum is rescaled by exactly 1
          Z += zc[c] * (double)exp2_fast((mc[c] - M) * kLog2e);
          if (mc[c] == M) tk = min(tk, ic[c]);
        }
      }
      msk[p] = true;
      conf[p] = 1.0 / Z;
      tok[p] = tk;
      best_of(bc, bt, conf[p], t);
    }
    n_masked += msk[p];
    n_pass += msk[p] && conf[p] > tau;
  }
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
  for (int p = 0; p < kP; ++p) {
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
  constexpr int N = kU * W;            // logits per thread per iteration
  constexpr int kIterVec = kU * kUT;   // vectors per workgroup iteration
  const int c = blockIdx.x, t = blockIdx.y, i = blockIdx.z;
  const int tid = threadIdx.x;
  const int B = a.sq.B;
  const int start = seq_prompt(a.sq, i) + seq_block(a.sq, i) * B;
  const bool masked = a.mask[(size_t)i * a.sq.Lcap + start + t] != 0;

  __shared__ float s_f[kUWaves];
  __shared__ double s_d[kUWaves];
  __shared__ int s_i[kUWaves];
  __shared__ int s_flag;

  if (masked) {
    const size_t esz = BF16 ? 2 : 4;
    const char* row = (const char*)a.logits + ((size_t)i * a.seq_stride + (size_t)t * a.row_stride) * esz;
    const int e0 = c * a.chunk;                      // first vocab id of the chunk
    const int e1 = min(a.V, e0 + a.chunk);
    RowAcc acc{-INFINITY, -1, INT_MAX, 0.0};
    int nfull = 0;                                   // full vectors (vector path)
    const uint4* rv = (const uint4*)(row + (size_t)e0 * esz);
    if (a.vec) {
      nfull = (e1 - e0) / W;
      const int n_it = (nfull + kIterVec - 1) / kIterVec;
      // Loads are unconditional (past the chunk they re-read its last vector,
      // which stays in cache), so the loads in flight are the same on every
      // path and reducing one buffer never waits for the other.
      uint4 va[kU], vb[kU];
      auto load = [&](uint4 (&buf)[kU], int it) {
#pragma unroll
        for (int u = 0; u < kU; ++u) buf[u] = rv[min(it * kIterVec + u * kUT + tid, nfull - 1)];
      };
      auto reduce = [&](const uint4 (&buf)[kU], int it) {
        float x[N];
#pragma unroll
        for (int u = 0; u < kU; ++u) VT::unpack(buf[u], x + u * W);
        if ((it + 1) * kIterVec > nfull) {  // the chunk's last, partial iteration
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const bool ok = it * kIterVec + u * kUT + tid < nfull;
#pragma unroll
            for (int e = 0; e < W; ++e) x[u * W + e] = ok ? x[u * W + e] : -INFINITY;
          }
        }
        fold<N>(acc, x, it);
      };
      if (n_it > 0) {
        load(va, 0);
        for (int it = 0; it < n_it; it += 2) {
          load(vb, it + 1);
          reduce(va, it);
          load(va, it + 2);
          if (it + 1 < n_it) reduce(vb, it + 1);
        }
      }
      // vocab entries past the last full vector of the chunk (fewer than W)
      if (tid == 0) {
        for (int e = e0 + nfull * W; e < e1; ++e) {
          float x1[1] = {VT::scalar(row, e)};
          const float before = acc.m;
          fold<1>(acc, x1, -2);
          if (acc.m > before) acc.idx = e;
        }
      }
    } else {
      // unaligned rows: one logit per load, same iteration blocking
      for (int it = 0, base = e0; base < e1; ++it, base += N * kUT) {
        float x[N];
#pragma unroll
        for (int k = 0; k < N; ++k) {
          const int e = base + k * kUT + tid;
          x[k] = (e < e1) ? VT::scalar(row, e) : -INFINITY;
        }
        fold<N>(acc, x, it);
      }
    }
    // chunk max, then its lowest index: only threads holding the chunk max
    // look at the iteration where they first saw it
    const float M = block_max(acc.m, s_f);
    int idx = INT_MAX;
    if (acc.m == M && M != -INFINITY) {
      if (acc.it == -2) {
        idx = acc.idx;
      } else if (a.vec) {
        for (int u = 0; u < kU && idx == INT_MAX; ++u) {
          const int vi = acc.it * kIterVec + u * kUT + tid;
          if (vi < nfull) {
            float x[W];
            VT::unpack(rv[vi], x);
            for (int e = 0; e < W; ++e)
              if (x[e] == M) {
                idx = e0 + vi * W + e;
                break;
              }
          }
        }
      } else {
        const int base = e0 + acc.it * N * kUT;
        for (int k = 0; k < N && idx == INT_MAX; ++k) {
          const int e = base + k * kUT + tid;
          if (e < e1 && VT::scalar(row, e) == M) idx = e;
        }
      }
    }
    const double zt = (acc.m == -INFINITY) ? 0.0 : acc.z * (double)exp2_fast((acc.m - M) * kLog2e);
    double Z;
    int I;
    block_sum_min(zt, idx, s_d, s_i, Z, I);
    if (tid == 0) put_partial(a.part + ((size_t)i * B + t) * a.nchunk + c, M, I, Z);
  }

  // the last of the sequence's B x nchunk workgroups finalises it
  if (!block_arrive(&a.seq_cnt[i], (unsigned)(B * a.nchunk), &s_flag)) return;
  unmask_finalize(a, i, start);
}

// Workgroups the vocab split aims for (the environment variable
// FDLLM_UNMASK_TARGET_WGS overrides the default for tuning).
static long unmask_target_workgroups() {
  static long v = [] {
    const char* e = getenv("FDLLM_UNMASK_TARGET_WGS");
    long t = e ? atol(e) : 512;
    return t > 0 ? t : 512;
  }();
  return v;
}

UnmaskPlan plan_unmask(int dtype, int V, int rows) {
  UnmaskPlan p{};
  const int W = dtype == 0 ? 8 : 4;
  const int iter_elems = kU * kUT * W;           // one workgroup iteration
  // split rows so that about the target number of workgroups covers the
  // batch (at most one chunk per iteration and at most 16 chunks per row)
  const long target = unmask_target_workgroups();
  const int want = (int)((target + rows - 1) / rows);
  const int by_iter = (V + iter_elems - 1) / iter_elems;
  int nchunk = want < by_iter ? want : by_iter;
  if (nchunk > kMaxChunks) nchunk = kMaxChunks;
  if (nchunk < 1) nchunk = 1;
  int chunk = (V + nchunk - 1) / nchunk;
  chunk = (chunk + W - 1) / W * W;               // chunk starts stay 16-byte aligned
  p.nchunk = (V + chunk - 1) / chunk;
  p.chunk = chunk;
  return p;
}

size_t unmask_workspace_bytes(int b, int B, int nchunk) {
  size_t bytes = (size_t)b * B * nchunk * sizeof(UnmaskPartial);  // chunk partials
  bytes += (size_t)b * 8;                                         // done flags
  bytes += (size_t)b * 4;                                         // sequence counters
  bytes += 16;                                                    // global counter
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
