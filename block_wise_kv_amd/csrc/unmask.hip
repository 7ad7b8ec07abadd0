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
//      flight while the current one is reduced.  The first two iterations
//      are requested before the row's mask byte is known, so the mask read
//      adds no latency (an unmasked row discards them).  Per thread it keeps
//      the running max, the iteration and load slot where that max first
//      appeared, and the sum of exp(l - max): one fma and one exp per logit,
//      the exps of an iteration summed pairwise in fp32 and accumulated in
//      fp64.  After the chunk every thread re-reads its one slot (in flight
//      during the workgroup max) and the threads holding the chunk max give
//      its lowest index.
//   2. the last workgroup of sequence i to arrive merges every chunk of every
//      row (fp64), applies the threshold and the fallback with workgroup
//      reductions, commits tokens and mask, and writes the per-sequence
//      outputs; the last sequence writes the ascending done list.  For up to
//      48 sequences the finished flags ride in the same 64-bit atomic as the
//      arrival count, so the last sequence reads them from its own atomic.
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
constexpr int kBitsSeqs = 48;      // done list carried in one 64-bit atomic up to this batch

// A partial (m, idx, z) is one 16-byte write-through store / load.
__device__ __forceinline__ void put_partial(UnmaskPartial* p, float m, int idx, double z) {
  const uint64_t zb = (uint64_t)__double_as_longlong(z);
  st_coherent_b128(make_rsrc(p), 0,
                   make_float4(m, __int_as_float(idx), __uint_as_float((uint32_t)zb),
                               __uint_as_float((uint32_t)(zb >> 32))));
}
// `r` addresses the sequence's partials (a workgroup-uniform base), `off`
// is this partial's byte offset from it.
__device__ __forceinline__ void get_partial(__amdgpu_buffer_rsrc_t r, int off, float& m, int& idx, double& z) {
  const float4 w = ld_coherent_b128(r, off);
  m = w.x;
  idx = __float_as_int(w.y);
  z = __longlong_as_double((long long)((uint64_t)__float_as_uint(w.z) | ((uint64_t)__float_as_uint(w.w) << 32)));
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

// Running per-thread state: max m, the iteration it and load slot u where m
// first appeared (it = -1: none, -2: in the scalar tail, whose index is
// idx), and z = sum over seen logits of exp(l - m).
struct RowAcc {
  float m;
  int it;
  int u;
  int idx;
  double z;
};

// Fold one iteration, x[0..N) in S slots of N/S logits (one slot per load,
// in ascending vocab order), into acc.  The exps use the fp32 reference
// r = round(m*log2 e): exp2(fma(x, log2 e, -r)) = exp(x - m) * 2^d with
// d = m*log2 e - r computed exactly by one more fma, so the iteration sum is
// corrected by 2^-d and the maximum contributes (to within an ulp) exactly 1.
template <int N, int S>
__device__ __forceinline__ void fold(RowAcc& acc, float* x, int it) {
  constexpr int E = N / S;
  float sm[S];
#pragma unroll
  for (int q = 0; q < S; ++q) {
    sm[q] = x[q * E];
#pragma unroll
    for (int k = 1; k < E; ++k) sm[q] = fmaxf(sm[q], x[q * E + k]);
  }
  float lm = sm[0];
#pragma unroll
  for (int q = 1; q < S; ++q) lm = fmaxf(lm, sm[q]);
  int us = 0;
#pragma unroll
  for (int q = S - 1; q > 0; --q) us = (sm[q] == lm) ? q : us;
  if (lm > acc.m) {
    acc.it = it;
    acc.u = us;
  }
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
  lds_sync();
  if (lane == 0) s_f[wid] = v;
  lds_sync();
  float r = s_f[0];
#pragma unroll
  for (int w = 1; w < kUWaves; ++w) r = fmaxf(r, s_f[w]);
  return r;
}
__device__ void block_sum_min(double z, int idx, double* s_d, int* s_i, double& z_out, int& idx_out) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  z = wave_sum_d(z);
  idx = wave_min_i(idx);
  lds_sync();
  if (lane == 0) {
    s_d[wid] = z;
    s_i[wid] = idx;
  }
  lds_sync();
  z_out = s_d[0];
  idx_out = s_i[0];
#pragma unroll
  for (int w = 1; w < kUWaves; ++w) {
    z_out += s_d[w];
    idx_out = min(idx_out, s_i[w]);
  }
}

// Row t's merge over the vocabulary pass's chunk partials of one sequence:
// Z = sum of exp(logit - max) over the row, tk = its lowest argmax.  Every
// chunk partial is loaded at once (the count is a compile-time bound), and
// the chunk holding the maximum is rescaled by exactly 1.
struct ChunkMerge {
  __amdgpu_buffer_rsrc_t r;  // the sequence's partials [nchunk][B]
  int nchunk, B;
  __device__ __forceinline__ void operator()(int t, double& Z, int& tk) const {
    float mc[kMaxChunks];
    int ic[kMaxChunks];
    double zc[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      get_partial(r, (min(c, nchunk - 1) * B + t) * (int)sizeof(UnmaskPartial), mc[c], ic[c], zc[c]);
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) M = fmaxf(M, mc[c]);
    Z = 0.0;
    tk = INT_MAX;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      if (c < nchunk) {
        Z += zc[c] * (double)exp2_fast((mc[c] - M) * kLog2e);
        if (mc[c] == M) tk = min(tk, ic[c]);
      }
    }
  }
};

// Lexicographic max of (conf, -t): the highest confidence, lowest row on a tie.
__device__ __forceinline__ void best_of(double& c, int& t, double c2, int t2) {
  if (c2 > c || (c2 == c && t2 < t)) {
    c = c2;
    t = t2;
  }
}
// (c, t) <- the better of this lane's and lane ^ O's (best_of is symmetric)
template <int O>
__device__ __forceinline__ void best_of_lanes(double& c, int& t) {
  double c1, c2;
  int t1, t2;
  lane_pair<O>(c, c1, c2);
  lane_pair<O>(t, t1, t2);
  c = c1;
  t = t1;
  best_of(c, t, c2, t2);
}
__device__ __forceinline__ void best_of_wave(double& c, int& t) {
  best_of_lanes<32>(c, t);
  best_of_lanes<16>(c, t);
  best_of_lanes<8>(c, t);
  best_of_lanes<4>(c, t);
  best_of_lanes<2>(c, t);
  best_of_lanes<1>(c, t);
}

// Per-sequence finalisation by the last workgroup of sequence i.  Rows are
// handled 256 at a time, one per thread; a row's mask byte and every chunk
// partial are loaded together (the merge runs on every row and the mask
// selects); counts, the fallback argmax and the ranks of selected rows come
// from workgroup reductions and ballots.
// Blocks of up to 64 rows: one wave finalises (one row per lane, counts and
// ranks from ballots, no workgroup barrier); the finished-sequence atomic is
// issued as soon as the row count is known, so its round trip overlaps the
// commit stores.
template <class RowMerge>
__device__ void unmask_finalize_wave(const UnmaskArgs& a, int i, int start, const RowMerge& merge) {
  const int B = a.sq.B;
  const int t = threadIdx.x;  // lane of wave 0
  int32_t* trow = a.tokens + (size_t)i * a.sq.Lcap + start;
  uint8_t* mrow = a.mask + (size_t)i * a.sq.Lcap + start;
  const double tau = (double)a.tau;
  bool mk = false;
  double conf = 0.0;
  int tok = 0;
  if (t < B) {
    mk = mrow[t] != 0;
    double Z;
    int tk;
    merge(t, Z, tk);
    conf = mk ? 1.0 / Z : 0.0;
    tok = tk;
  }
  const uint64_t bal_m = __ballot(mk);
  const uint64_t bal_p = __ballot(mk && conf > tau);
  const int n_masked = __popcll(bal_m);
  double bc = mk ? conf : -1.0;
  int bt = mk ? t : INT_MAX;
  best_of_wave(bc, bt);
  const bool fallback = bal_p == 0 && n_masked > 0;
  uint64_t bal_s = fallback ? (bt < 64 ? (1ull << bt) : 0ull) : bal_p;
  if (a.topk > 0) {
    // fixed-step rule: the masked rows ranked by confidence (the lower
    // offset first among equal ones); row t is selected when fewer than k
    // masked rows outrank it.  k = 1 is the single best row found above and
    // k >= n_masked takes every masked row; otherwise each lane counts the
    // rows that outrank it, reading their confidences with readlane.
    if (a.topk == 1) {
      bal_s = (n_masked > 0 && bt < 64) ? (1ull << bt) : 0ull;
    } else if (a.topk >= n_masked) {
      bal_s = bal_m;
    } else {
      // every lane's confidence through LDS (wave-private, in order), read
      // back two rows per broadcast load
      __shared__ __attribute__((aligned(16))) double s_wconf[64];
      s_wconf[t] = conf;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // branch-free count over a fixed 32 or 64 rows (rows past B are not
      // in bal_m), 8 rows per group of loads
      auto count = [&](auto nrows) __attribute__((always_inline)) {
        int r = 0;
#pragma unroll
        for (int j0 = 0; j0 < decltype(nrows)::value; j0 += 8) {
          double2 c2[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) c2[q] = *(const double2*)&s_wconf[j0 + 2 * q];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int j = j0 + q;
            const double cj = (q & 1) ? c2[q >> 1].y : c2[q >> 1].x;
            const int above = (int)(cj > conf) | ((int)(cj == conf) & (int)(j < t));
            r += above & (int)((bal_m >> j) & 1ull);
          }
        }
        return r;
      };
      const int rank = B <= 32 ? count(std::integral_constant<int, 32>{}) : count(std::integral_constant<int, 64>{});
      bal_s = __ballot(mk && rank < a.topk);
    }
  }
  const int n_sel = __popcll(bal_s);
  const int done = (n_masked == n_sel) ? 1 : 0;
  const bool want_list = a.done_seqs || a.n_done;
  const int b = a.sq.b;
  uint64_t old = 0, add = 0;
  if (want_list && t == 0) {
    // count in the top 16 bits, finished flags below: adding distinct bits
    // is an or, so the last arriver holds every flag
    add = (1ull << 48) | ((uint64_t)done << i);
    old = __hip_atomic_fetch_add(a.glob, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const bool sel = (bal_s >> t) & 1ull;
  if (t < B) {
    if (sel) {
      trow[t] = tok;
      mrow[t] = 0;
    }
    if (a.decoded_pos) {
      // selected rows in ascending order at [0, n_sel), -1 after them
      if (sel) a.decoded_pos[(size_t)i * B + __popcll(bal_s & ((1ull << t) - 1ull))] = t;
      if (t >= n_sel) a.decoded_pos[(size_t)i * B + t] = -1;
    }
    if (a.conf) a.conf[(size_t)i * B + t] = mk ? conf : __longlong_as_double(0x7ff8000000000000ll);
  }
  if (t == 0) {
    a.n_decoded[i] = n_sel;
    if ((a.flags & 1u) && done && a.sq.bidx) {
      const int k = a.sq.bidx[i];
      if (k + 1 < a.sq.G / a.sq.B) a.sq.bidx[i] = k + 1;
    }
    a.seq_cnt[(size_t)i * kSeqCntStride] = 0u;
  }
  if (!want_list) return;
  // the last sequence to finish writes the ascending list of finished ones
  const auto lane0 = [](uint64_t v) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), 0) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 0);
  };
  const uint64_t old_all = lane0(old);
  if ((int)(old_all >> 48) != b - 1) return;
  const uint64_t bits = (old_all + lane0(add)) & ((1ull << 48) - 1ull);
  const bool fl = t < b && ((bits >> t) & 1ull);
  const uint64_t bal = __ballot(fl);
  if (fl && a.done_seqs) a.done_seqs[__popcll(bal & ((1ull << t) - 1ull))] = t;
  if (t == 0) {
    if (a.n_done) *a.n_done = __popcll(bal);
    __hip_atomic_store(a.glob, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <class RowMerge>
__device__ void unmask_finalize(const UnmaskArgs& a, int i, int start, const RowMerge& merge) {
  __shared__ double s_conf[kMaxBlockSize];  // fixed-step rule: conf of masked rows, -1 otherwise
  __shared__ int s_cnt[kUWaves][2];
  __shared__ double s_bc[kUWaves];
  __shared__ int s_bt[kUWaves];
  __shared__ int s_rank[kUWaves];
  __shared__ int s_done, s_count, s_last;
  __shared__ uint64_t s_bits;
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
    if (p < np && t < B) {
      const bool mk = mrow[t] != 0;
      double Z;
      int tk;
      merge(t, Z, tk);
      // unmasked rows carry stale partials: computed, then discarded
      msk[p] = mk;
      conf[p] = mk ? 1.0 / Z : 0.0;
      tok[p] = tk;
      if (mk) best_of(bc, bt, conf[p], t);
      if (a.topk > 0) s_conf[t] = mk ? conf[p] : -1.0;
    }
    n_masked += msk[p];
    n_pass += msk[p] && conf[p] > tau;
  }
  {
    const auto add = [](int x, int y) { return x + y; };
    n_masked = wave_reduce(n_masked, add);
    n_pass = wave_reduce(n_pass, add);
    best_of_wave(bc, bt);
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
    bool sel = msk[p] && (fallback ? (t == bt) : (conf[p] > tau));
    if (a.topk > 0) {
      // fixed-step rule: fewer than k masked rows outrank row t (unmasked
      // rows hold -1 and never do); s_conf is complete after the barrier
      // that follows pass 1.  k = 1 is the best row bt, k >= n_masked every
      // masked row.
      if (a.topk == 1) {
        sel = msk[p] && t == bt;
      } else if (a.topk >= n_masked) {
        sel = msk[p];
      } else {
        int rank = 0;
        if (msk[p])
          for (int j = 0; j < B; ++j) {
            const double cj = s_conf[j];
            rank += (cj > conf[p] || (cj == conf[p] && j < t)) ? 1 : 0;
          }
        sel = msk[p] && rank < a.topk;
      }
    }
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
  const bool want_list = a.done_seqs || a.n_done;
  const int b = a.sq.b;
  if (tid == 0) {
    a.n_decoded[i] = n_sel;
    const int done = (n_masked == n_sel) ? 1 : 0;
    if ((a.flags & 1u) && done && a.sq.bidx) {
      const int k = a.sq.bidx[i];
      if (k + 1 < a.sq.G / a.sq.B) a.sq.bidx[i] = k + 1;
    }
    a.seq_cnt[(size_t)i * kSeqCntStride] = 0u;
    s_done = done;
    s_count = 0;
    if (want_list && b <= kBitsSeqs) {
      // count in the top 16 bits, finished flags below: adding distinct
      // bits is an or, so the last arriver holds every flag
      const uint64_t add = (1ull << 48) | ((uint64_t)done << i);
      const uint64_t old = __hip_atomic_fetch_add(a.glob, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (int)(old >> 48) == b - 1;
      s_bits = (old + add) & ((1ull << 48) - 1ull);
    }
  }
  if (!want_list) return;
  // the last sequence to finish writes the ascending list of finished ones
  if (b <= kBitsSeqs) {
    __syncthreads();
    if (!s_last || tid >= 64) return;
    const bool fl = tid < b && ((s_bits >> tid) & 1ull);
    const uint64_t bal = __ballot(fl);
    if (fl && a.done_seqs) a.done_seqs[__popcll(bal & ((1ull << lane) - 1ull))] = tid;
    if (tid == 0) {
      if (a.n_done) *a.n_done = __popcll(bal);
      __hip_atomic_store(a.glob, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  uint32_t* cnt = (uint32_t*)(a.glob + 1);
  __syncthreads();
  if (tid == 0) st_coherent((uint64_t*)(a.done_flag + 2 * i), (uint64_t)s_done);
  if (!block_arrive(cnt, (unsigned)b, &s_last)) return;
  for (int q = 0; q < b; q += kUT) {
    const int s = q + tid;
    const bool fl = s < b && ld_coherent((const uint64_t*)(a.done_flag + 2 * s)) != 0;
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
    *cnt = 0u;
  }
}

// A row's mask byte through the scalar cache (its aligned dword, so the
// read stays in the byte's page).  The kernel writes mask bytes only in the
// finalisation of a sequence, after every workgroup of that sequence has
// read its own, so the scalar cache never holds a stale byte.
__device__ __forceinline__ int load_mask_byte(const uint8_t* p) {
  typedef const __attribute__((address_space(4))) uint32_t* ConstU32;
  const uintptr_t addr = (uintptr_t)p;
  const uint32_t w = *(ConstU32)(addr & ~(uintptr_t)3);
  return (int)((w >> (8u * (uint32_t)(addr & 3u))) & 0xffu);
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
  const uint8_t* mptr = a.mask + (size_t)i * a.sq.Lcap + start + t;

  __shared__ float s_f[kUWaves];
  __shared__ double s_d[kUWaves];
  __shared__ int s_i[kUWaves];
  __shared__ int s_flag;

  const size_t esz = BF16 ? 2 : 4;
  const char* row = (const char*)a.logits + ((size_t)i * a.seq_stride + (size_t)t * a.row_stride) * esz;
  const int e0 = c * a.chunk;                        // first vocab id of the chunk
  const int e1 = min(a.V, e0 + a.chunk);
  RowAcc acc{-INFINITY, -1, 0, INT_MAX, 0.0};
  const int nfull = a.vec ? (e1 - e0) / W : 0;       // full vectors (vector path)
  // Vector loads are unconditional and clamped to the chunk's last full
  // vector; a chunk without one (vocab tail shorter than a vector) points
  // them at the workspace, whose values are never used.
  const uint4* rv = nfull > 0 ? (const uint4*)(row + (size_t)e0 * esz) : (const uint4*)a.part;
  const int vlast = max(nfull - 1, 0);
  bool masked;
  if (a.vec) {
    const int n_it = (nfull + kIterVec - 1) / kIterVec;
    // Past the chunk the loads re-read its last vector, so the loads in
    // flight are the same on every path and reducing one buffer never waits
    // for the other.  The logits are read once: non-temporal loads.
    uint4 va[kU], vb[kU];
    auto load = [&](uint4 (&buf)[kU], int it) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const u32x4 w = __builtin_nontemporal_load((const u32x4*)(rv + min(it * kIterVec + u * kUT + tid, vlast)));
        buf[u] = make_uint4(w.x, w.y, w.z, w.w);
      }
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
      fold<N, kU>(acc, x, it);
    };
    // Small grids: the first two iterations are requested before the mask
    // byte is looked at, and the first runs whatever it says (an unmasked
    // row reduces it and discards the result), so nothing between these
    // loads and the loop waits for the mask.  With a thousand workgroups or
    // more, those waiting for their mask byte are covered by the others and
    // the bytes matter more: the byte is read (scalar) before any load, and
    // an unmasked row loads nothing.
    const bool mask_first = gridDim.x * gridDim.y * gridDim.z >= 1024u;
    if (n_it > 0 && mask_first) masked = load_mask_byte(mptr) != 0;
    if (n_it > 0 && (!mask_first || masked)) {
      int n_run = n_it;
      if (mask_first) {
        load(va, 0);
        load(vb, 1);
      } else {
        // mask byte first: loads return in order, so it is in before va
        const int mv = *mptr;
        __builtin_amdgcn_sched_barrier(0);
        load(va, 0);
        load(vb, 1);
        __builtin_amdgcn_sched_barrier(0);
        masked = __builtin_amdgcn_readfirstlane(mv) != 0;
        n_run = masked ? n_it : 1;
      }
      // va holds iteration it and vb iteration it + 1.  The last one or two
      // iterations are reduced after the loop, so no load is issued that
      // only the code after the loop would wait for (its registers are
      // reused there); at most one half-iteration of clamped loads past the
      // chunk is in flight, issued before the last reduction.
      int it = 0;
      while (it + 2 < n_run) {
        reduce(va, it);
        load(va, it + 2);
        reduce(vb, it + 1);
        load(vb, it + 3);
        it += 2;
      }
      reduce(va, it);
      if (it + 1 < n_run) reduce(vb, it + 1);
    } else if (n_it == 0) {
      masked = load_mask_byte(mptr) != 0;  // no full vector: only the scalar tail below
    }
    // vocab entries past the last full vector of the chunk (fewer than W)
    if (masked && tid == 0) {
      for (int e = e0 + nfull * W; e < e1; ++e) {
        float x1[1] = {VT::scalar(row, e)};
        const float before = acc.m;
        fold<1, 1>(acc, x1, -2);
        if (acc.m > before) acc.idx = e;
      }
    }
  } else {
    masked = load_mask_byte(mptr) != 0;
    if (masked) {
      // unaligned rows: one logit per load, same iteration blocking
      for (int it = 0, base = e0; base < e1; ++it, base += N * kUT) {
        float x[N];
#pragma unroll
        for (int k = 0; k < N; ++k) {
          const int e = base + k * kUT + tid;
          const float v = VT::scalar(row, min(e, e1 - 1));  // unconditional, clamped
          x[k] = (e < e1) ? v : -INFINITY;
        }
        fold<N, N>(acc, x, it);
      }
    }
  }

  if (masked) {
    // chunk max, then its lowest index: every thread re-reads the slot where
    // it first saw its own max (the load overlaps the workgroup max), and
    // the threads holding the chunk max search it
    const int vi = min(max(acc.it, 0) * kIterVec + acc.u * kUT + tid, vlast);
    const uint4 wv = rv[vi];
    const float M = block_max(acc.m, s_f);
    int idx = INT_MAX;
    if (acc.m == M && M != -INFINITY) {
      if (acc.it == -2) {
        idx = acc.idx;
      } else if (a.vec) {
        float x[W];
        VT::unpack(wv, x);
#pragma unroll
        for (int e = W - 1; e >= 0; --e)
          if (x[e] == M) idx = e0 + vi * W + e;
      } else {
        idx = e0 + (acc.it * N + acc.u) * kUT + tid;
      }
    }
    const double zt = (acc.m == -INFINITY) ? 0.0 : acc.z * (double)exp2_fast((acc.m - M) * kLog2e);
    double Z;
    int I;
    block_sum_min(zt, idx, s_d, s_i, Z, I);
    if (tid == 0) put_partial(a.part + ((size_t)i * a.nchunk + c) * B + t, M, I, Z);
  }

  // the last of the sequence's B x nchunk workgroups finalises it
  if (!block_arrive(&a.seq_cnt[(size_t)i * kSeqCntStride], (unsigned)(B * a.nchunk), &s_flag)) return;
  const ChunkMerge merge{make_rsrc(a.part + (size_t)i * B * a.nchunk), a.nchunk, B};
  if (B <= 64 && a.sq.b <= kBitsSeqs) {
    if (tid < 64) unmask_finalize_wave(a, i, start, merge);
    return;
  }
  unmask_finalize(a, i, start, merge);
}

// ---- finalisation of the fused vocabulary projection (lmhead.hip)
//
// One workgroup per sequence.  The projection kernel left one partial
// (max, lowest argmax, sum of exp(logit - max)) per (row, vocabulary
// workgroup) in part[row][n_vwg]; up to 32 threads merge a row's partials (in
// fp64, rescaling the running sum whenever the maximum grows), the row
// results go through LDS, and the selection, commit and done list are the
// vocabulary pass's finalisation.
struct LdsMerge {
  const double* z;
  const int* tok;
  __device__ __forceinline__ void operator()(int t, double& Z, int& tk) const {
    Z = z[t];
    tk = tok[t];
  }
};

__device__ __forceinline__ void merge_partial(float& M, double& Z, int& I, float m, double z, int idx) {
  if (m > M) {
    Z = (M == -INFINITY ? 0.0 : Z * (double)exp2_fast((M - m) * kLog2e)) + z;
    M = m;
    I = idx;
  } else if (m == M) {
    Z += z;
    I = min(I, idx);
  } else if (m != -INFINITY) {
    Z += z * (double)exp2_fast((m - M) * kLog2e);
  }
}

// NT threads: 1024 when the one-wave finalisation applies (blocks of up to
// 64 rows), so that up to 32 threads share a row's partials; 256 otherwise.
template <int NT>
__global__ __launch_bounds__(NT) void lmhead_finalize_kernel(UnmaskArgs a, const UnmaskPartial* part, int nv) {
  __shared__ double s_z[kMaxBlockSize];
  __shared__ int s_tok[kMaxBlockSize];
  const int i = blockIdx.x, tid = threadIdx.x;
  const int B = a.sq.B;
  const int start = seq_prompt(a.sq, i) + seq_block(a.sq, i) * B;
  // threads per row: the largest power of two up to 32 with tpr * B <= NT
  int tpr = 1;
  while (tpr < 32 && 2 * tpr * B <= NT) tpr *= 2;
  const int j = tid & (tpr - 1);
  constexpr int kU8 = 8;  // partials in flight per thread
  for (int t0 = 0; t0 < B; t0 += NT / tpr) {
    const int t = t0 + tid / tpr;
    float M = -INFINITY;
    double Z = 0.0;
    int I = INT_MAX;
    if (t < B) {
      const UnmaskPartial* p = part + ((size_t)i * B + t) * nv;
      for (int c0 = j; c0 < nv; c0 += tpr * kU8) {
        UnmaskPartial q[kU8];
#pragma unroll
        for (int u = 0; u < kU8; ++u) q[u] = p[min(c0 + tpr * u, nv - 1)];
#pragma unroll
        for (int u = 0; u < kU8; ++u)
          if (c0 + tpr * u < nv) merge_partial(M, Z, I, q[u].m, q[u].z, q[u].idx);
      }
    }
    // merge the tpr lanes of a row (merge_partial is symmetric)
    const auto merge_lanes = [&](auto oc) __attribute__((always_inline)) {
      constexpr int O = decltype(oc)::value;
      if (O < tpr) {
        float m1, m2;
        double z1, z2;
        int i1, i2;
        lane_pair<O>(M, m1, m2);
        lane_pair<O>(Z, z1, z2);
        lane_pair<O>(I, i1, i2);
        M = m1;
        Z = z1;
        I = i1;
        merge_partial(M, Z, I, m2, z2, i2);
      }
    };
    merge_lanes(std::integral_constant<int, 1>{});
    merge_lanes(std::integral_constant<int, 2>{});
    merge_lanes(std::integral_constant<int, 4>{});
    merge_lanes(std::integral_constant<int, 8>{});
    merge_lanes(std::integral_constant<int, 16>{});
    if (t < B && j == 0) {
      s_z[t] = Z;
      s_tok[t] = I;
    }
  }
  __syncthreads();
  const LdsMerge merge{s_z, s_tok};
  if (B <= 64 && a.sq.b <= kBitsSeqs) {
    if (tid < 64) unmask_finalize_wave(a, i, start, merge);
    return;
  }
  if constexpr (NT == kUT) unmask_finalize(a, i, start, merge);  // the launch picks 256 threads here
}

hipError_t launch_lmhead_finalize(const UnmaskArgs& a, const UnmaskPartial* part, int n_vwg, hipStream_t st,
                                  hipEvent_t ev_stop) {
  hipEvent_t none = nullptr;
  if (a.sq.B <= 64 && a.sq.b <= kBitsSeqs)
    return launch_kernel(lmhead_finalize_kernel<1024>, dim3((unsigned)a.sq.b), dim3(1024), 0, st, none, ev_stop, a,
                         part, n_vwg);
  return launch_kernel(lmhead_finalize_kernel<kUT>, dim3((unsigned)a.sq.b), dim3(kUT), 0, st, none, ev_stop, a, part,
                       n_vwg);
}

// Workgroups the vocab split aims for when the environment variable
// FDLLM_UNMASK_TARGET_WGS sets it (for tuning; 0 when unset).
static long unmask_target_workgroups() {
  static long v = [] {
    const char* e = getenv("FDLLM_UNMASK_TARGET_WGS");
    const long t = e ? atol(e) : 0;
    return t > 0 ? t : 0;
  }();
  return v;
}

static thread_local int g_unmask_wgs = 0;  // fdllm_set_tuning override (0: automatic), per host thread
void set_unmask_tuning(int wgs) { g_unmask_wgs = wgs; }

UnmaskPlan plan_unmask(int dtype, int V, int rows) {
  UnmaskPlan p{};
  const int W = dtype == 0 ? 8 : 4;
  const int iter_elems = kU * kUT * W;           // one workgroup iteration
  // Chunks per row: one, and four for batches of at most 64 rows (one or
  // two blocks), whose few workgroups per sequence stream too little with
  // one.  The logits are loaded non-temporally, which favours long
  // streams per workgroup.  Measured per call on MI355X with 126k-152k
  // logits per row: 32 rows 11.8 / 10.1 / 11.3 us at 2 / 4 / 8 chunks; 256
  // rows 19.3 / 21.6 / 24.8 us at 1 / 2 / 4; 1024 rows 49.5 / 64 us at 1 /
  // 4; 2048 rows of which 59 % masked 79 / 90 us at 1 / 4.  (With cached
  // loads two chunks were best at 256 and 2048 rows: 25.5 and 84 us.)  A
  // target workgroup count set for tuning overrides the rule (at most one
  // chunk per iteration and at most 16 chunks per row).
  const long target = g_unmask_wgs > 0 ? g_unmask_wgs : unmask_target_workgroups();
  int want = rows <= 64 ? 4 : 1;
  if (target > 0) want = (int)((target + rows - 1) / rows);
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

// Workspace: the 16-byte finished-sequence counter, the per-sequence done
// flags and arrival counters first (their place depends only on the batch),
// then the chunk partials.  Zeroed once; every counter is reset by its last
// user, so the unmask calls and the fused LM-head calls of one batch can
// share a workspace whatever their vocabulary split.
static size_t unmask_seq_cnt_offset(int b) {
  return (16 + (size_t)b * 8 + 127) & ~(size_t)127;  // after the global counter and the done flags
}
static size_t unmask_counter_bytes(int b) {
  return unmask_seq_cnt_offset(b) + (size_t)b * 4 * kSeqCntStride;  // one line per sequence counter
}

size_t unmask_workspace_bytes(int b, int B, int nchunk) {
  const size_t part = (size_t)b * B * nchunk * sizeof(UnmaskPartial);  // chunk partials
  return unmask_counter_bytes(b) + ((part + 255) & ~(size_t)255);
}

void unmask_bind_workspace(UnmaskArgs& a, void* workspace) {
  char* w = (char*)workspace;
  a.glob = (uint64_t*)w;
  a.done_flag = (int32_t*)(w + 16);
  a.seq_cnt = (uint32_t*)(w + unmask_seq_cnt_offset(a.sq.b));
  a.part = (UnmaskPartial*)(w + unmask_counter_bytes(a.sq.b));
}

hipError_t launch_unmask(const UnmaskArgs& a, int dtype, hipStream_t st) {
  dim3 grid((unsigned)a.nchunk, (unsigned)a.sq.B, (unsigned)a.sq.b);
  dim3 block(kUT);
  const LaunchEvents ev = take_launch_events();
  return dtype == 0 ? launch_kernel(unmask_kernel<true>, grid, block, 0, st, ev.start, ev.stop, a)
                    : launch_kernel(unmask_kernel<false>, grid, block, 0, st, ev.start, ev.stop, a);
}

}  // namespace fdllm
