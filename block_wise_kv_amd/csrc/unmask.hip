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
// One launch.  Workgroup (c, t, i) reads vocab chunk c of block row t of
// sequence i once from HBM (16-byte loads, values kept in registers), and
// reduces it to (max, lowest argmax, sum of exp(l - max)); the sum is
// accumulated per thread in fp32 and combined across threads and chunks in
// fp64.  The last workgroup to arrive for sequence i (device-scope counter)
// merges the chunk partials of every masked row, applies the threshold and
// the fallback, commits tokens and mask, and writes the per-sequence
// outputs.  The last sequence to finish writes the ascending done list.
// Counters are reset by their last user, so the workspace stays zeroed.
#include <float.h>
#include <limits.h>

#include "fdllm_device.h"
#include "fdllm_internal.h"

namespace fdllm {

constexpr int kUnmaskThreads = 256;
constexpr int kMaxBlockSize = 1024;

template <bool BF16, bool VEC>
struct LogitLoad;

// bf16, 16-byte vectors: 8 logits per load
template <>
struct LogitLoad<true, true> {
  static constexpr int W = 8;
  __device__ static void load(const void* row, int V, int e0, float* x) {
    const uint16_t* r = (const uint16_t*)row;
    if (e0 + 8 <= V) {
      const uint4 w = *(const uint4*)(r + e0);
      x[0] = bf16lo(w.x); x[1] = bf16hi(w.x);
      x[2] = bf16lo(w.y); x[3] = bf16hi(w.y);
      x[4] = bf16lo(w.z); x[5] = bf16hi(w.z);
      x[6] = bf16lo(w.w); x[7] = bf16hi(w.w);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (e0 + e < V) ? bf16_bits_to_f32(r[e0 + e]) : -INFINITY;
    }
  }
};
// f32, 16-byte vectors: 4 logits per load
template <>
struct LogitLoad<false, true> {
  static constexpr int W = 4;
  __device__ static void load(const void* row, int V, int e0, float* x) {
    const float* r = (const float*)row;
    if (e0 + 4 <= V) {
      const float4 w = *(const float4*)(r + e0);
      x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (e0 + e < V) ? r[e0 + e] : -INFINITY;
    }
  }
};
// unaligned rows: one logit per load
template <>
struct LogitLoad<true, false> {
  static constexpr int W = 1;
  __device__ static void load(const void* row, int V, int e0, float* x) {
    x[0] = (e0 < V) ? bf16_bits_to_f32(((const uint16_t*)row)[e0]) : -INFINITY;
  }
};
template <>
struct LogitLoad<false, false> {
  static constexpr int W = 1;
  __device__ static void load(const void* row, int V, int e0, float* x) {
    x[0] = (e0 < V) ? ((const float*)row)[e0] : -INFINITY;
  }
};

// Per-sequence finalisation, run by the last workgroup of sequence i.
__device__ void unmask_finalize(const UnmaskArgs& a, int i, int start) {
  __shared__ double s_conf[kMaxBlockSize];
  __shared__ int s_tok[kMaxBlockSize];
  __shared__ unsigned char s_msk[kMaxBlockSize];
  const int B = a.sq.B;
  const int tid = threadIdx.x;
  int32_t* trow = a.tokens + (size_t)i * a.sq.Lcap + start;
  uint8_t* mrow = a.mask + (size_t)i * a.sq.Lcap + start;

  for (int t = tid; t < B; t += kUnmaskThreads) {
    const unsigned char m = mrow[t];
    s_msk[t] = m;
    double conf = 0.0;
    int tok = 0;
    if (m) {
      const UnmaskPartial* pp = a.part + ((size_t)i * B + t) * a.nchunk;
      float M = -INFINITY;
      for (int c = 0; c < a.nchunk; ++c) M = fmaxf(M, pp[c].m);
      double Z = 0.0;
      tok = INT_MAX;
      for (int c = 0; c < a.nchunk; ++c) {
        const float mc = pp[c].m;
        Z += pp[c].z * exp((double)mc - (double)M);
        if (mc == M && tok == INT_MAX) tok = pp[c].idx;
      }
      conf = 1.0 / Z;
    }
    s_conf[t] = conf;
    s_tok[t] = tok;
  }
  __syncthreads();
  if (tid == 0) {
    const double tau = (double)a.tau;
    int nm = 0, nsel = 0, best = -1;
    for (int t = 0; t < B; ++t) {
      if (!s_msk[t]) continue;
      ++nm;
      if (s_conf[t] > tau) ++nsel;
      if (best < 0 || s_conf[t] > s_conf[best]) best = t;
    }
    const bool fallback = (nsel == 0 && nm > 0);
    int w = 0;
    for (int t = 0; t < B; ++t) {
      const bool sel = s_msk[t] && (fallback ? (t == best) : (s_conf[t] > tau));
      if (sel) {
        trow[t] = s_tok[t];
        mrow[t] = 0;
        if (a.decoded_pos) a.decoded_pos[(size_t)i * B + w] = t;
        ++w;
      }
      if (a.conf) a.conf[(size_t)i * B + t] = s_msk[t] ? s_conf[t] : __longlong_as_double(0x7ff8000000000000ll);
    }
    if (a.decoded_pos)
      for (int t = w; t < B; ++t) a.decoded_pos[(size_t)i * B + t] = -1;
    a.n_decoded[i] = w;
    const int done = (nm == w) ? 1 : 0;
    if ((a.flags & 1u) && done && a.sq.bidx) {
      const int k = a.sq.bidx[i];
      if (k + 1 < a.sq.G / a.sq.B) a.sq.bidx[i] = k + 1;
    }
    a.done_flag[i] = done;
    a.seq_cnt[i] = 0u;
    if (a.done_seqs || a.n_done) {
      __threadfence();
      const unsigned old = atomicAdd(a.glob_cnt, 1u);
      if (old == (unsigned)a.sq.b - 1u) {
        __threadfence();
        int n = 0;
        for (int s = 0; s < a.sq.b; ++s) {
          if (__atomic_load_n(&a.done_flag[s], __ATOMIC_RELAXED)) {
            if (a.done_seqs) a.done_seqs[n] = s;
            ++n;
          }
        }
        if (a.n_done) *a.n_done = n;
        *a.glob_cnt = 0u;
      }
    }
  }
}

template <bool BF16, int E, bool VEC>
__global__ __launch_bounds__(kUnmaskThreads) void unmask_kernel(UnmaskArgs a) {
  using LD = LogitLoad<BF16, VEC>;
  constexpr int W = LD::W;
  constexpr int NV = E / W;  // loads per thread
  const int c = blockIdx.x, t = blockIdx.y, i = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int B = a.sq.B;
  const int start = seq_prompt(a.sq, i) + seq_block(a.sq, i) * B;
  const bool masked = a.mask[(size_t)i * a.sq.Lcap + start + t] != 0;

  __shared__ float s_m[4];
  __shared__ int s_i[4];
  __shared__ double s_z[4];
  __shared__ int s_last;

  if (masked) {
    const size_t esz = BF16 ? 2 : 4;
    const char* row = (const char*)a.logits + ((size_t)i * a.seq_stride + (size_t)t * a.row_stride) * esz;
    const int e_begin = c * a.chunk;
    float x[E];
#pragma unroll
    for (int it = 0; it < NV; ++it) LD::load(row, a.V, e_begin + (it * kUnmaskThreads + tid) * W, x + it * W);
    // chunk max
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) mt = fmaxf(mt, x[e]);
    float M = wave_max(mt);
    if (lane == 0) s_m[wid] = M;
    __syncthreads();
    M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    // lowest index attaining the max
    int idx = INT_MAX;
    if (mt == M) {
#pragma unroll
      for (int it = 0; it < NV; ++it) {
#pragma unroll
        for (int e = 0; e < W; ++e) {
          if (idx == INT_MAX && x[it * W + e] == M) idx = e_begin + (it * kUnmaskThreads + tid) * W + e;
        }
      }
    }
    idx = wave_min_i(idx);
    // sum of exp(l - M): one exp per logit
    float zt = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) zt += exp2_fast((x[e] - M) * kLog2e);
    double z = wave_sum_d((double)zt);
    if (lane == 0) {
      s_i[wid] = idx;
      s_z[wid] = z;
    }
    __syncthreads();
    if (tid == 0) {
      UnmaskPartial p;
      p.m = M;
      p.idx = min(min(s_i[0], s_i[1]), min(s_i[2], s_i[3]));
      p.z = (s_z[0] + s_z[1]) + (s_z[2] + s_z[3]);
      a.part[((size_t)i * B + t) * a.nchunk + c] = p;
    }
  }
  if (tid == 0) {
    __threadfence();
    const unsigned old = atomicAdd(&a.seq_cnt[i], 1u);
    s_last = (old == (unsigned)(B * a.nchunk) - 1u);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  unmask_finalize(a, i, start);
}

int unmask_chunk_elems(int dtype, int V, int rows) {
  (void)V;
  (void)rows;
  return dtype == 0 ? 32 * kUnmaskThreads : 16 * kUnmaskThreads;
}

size_t unmask_workspace_bytes(int b, int B, int nchunk) {
  size_t bytes = (size_t)b * B * nchunk * sizeof(UnmaskPartial);
  bytes += (size_t)b * 4;   // seq counters
  bytes += 16;              // global counter (padded)
  bytes += (size_t)b * 4;   // done flags
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_unmask(const UnmaskArgs& a, int dtype, bool vec, hipStream_t st) {
  dim3 grid((unsigned)a.nchunk, (unsigned)a.sq.B, (unsigned)a.sq.b);
  dim3 block(kUnmaskThreads);
  if (dtype == 0) {
    if (vec) hipLaunchKernelGGL((unmask_kernel<true, 32, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((unmask_kernel<true, 32, false>), grid, block, 0, st, a);
  } else {
    if (vec) hipLaunchKernelGGL((unmask_kernel<false, 16, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((unmask_kernel<false, 16, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace fdllm
