// Block attention: the current block's queries attend bidirectionally over
// [cached prefix K/V | fresh block K/V | cached suffix K/V].
//
// Fast-dLLM (project README "Key techniques" item 1; aibase news
// "Innovations" item 1 and "The Challenges and Opportunities"): the model
// attends bidirectionally (no causal mask); K/V of the rows recomputed this
// step are fresh, all other rows come from the block-wise cache written at
// the last refresh.  Which rows are fresh depends on the cache mode
// (none / prefix / DualCache).
//
// bf16, d = 128 (MFMA path).  A workgroup of 4 waves owns one (sequence,
// query head, 32-row query tile, key chunk).  Each wave streams 32-key
// sub-tiles of the chunk:
//   * K rows go straight from HBM into MFMA A-operand registers (16-byte
//     loads; the head dimension is split into 16-byte column pairs, the same
//     split is used for Q so the contraction over d is unchanged);
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys x queries, fp32);
//   * online softmax per query column (exp2 with a log2(e) pre-scale);
//   * V rows are loaded with 16-byte loads, transposed into a wave-private
//     LDS tile (d-major, 4 keys per 8-byte write), and read back as the
//     A operand of O^T += V^T P^T (P in bf16, taken directly from the S^T
//     accumulator layout, so no shuffle of P is needed).
// The 4 waves merge (max, sum, O) through LDS.  When the key range is split
// over several workgroups, each publishes an fp32 partial with agent-scope
// (write-through) 16-byte stores and bumps a counter; the last one to arrive
// reads every partial with agent-scope loads, merges them and writes the
// output, then resets the counter.
//
// Work items are ordered so that the query heads sharing a KV head are
// adjacent, and the grid is remapped so adjacent items land on the same XCD
// (workgroups are dealt round-robin over the 8 XCDs): the g heads of a GQA
// group then read the same K/V rows through one L2.
//
// f32 (any mode, d = 64 or 128): a plain VALU kernel, one wave per query
// row, fp32 throughout.
#include <float.h>
#include <stdlib.h>

#include <type_traits>

#include "fdllm_device.h"
#include "fdllm_internal.h"

namespace fdllm {

constexpr int kNW = 4;                 // waves per workgroup
constexpr int kThreads = kNW * 64;
constexpr int kQT = 32;                // query rows per tile
constexpr int kKT = 32;                // keys per wave sub-tile
constexpr int kD = 128;                // head dim (bf16 path)
constexpr int kVtStride = 36;          // bf16 per d-row of the transposed V tile
constexpr int kRedStride = 65;         // floats per query row of the merge buffer
constexpr int kPartFloats = kQT * kD + 2 * kQT;  // one split partial: O, m, l
constexpr int kMaxSplit = 8;           // key chunks per (sequence, head, query tile)

struct Geo {
  int i, h, hk, qt, s;
  int L, a0, a1, nq, kb, ke, n_act;
};

__device__ __forceinline__ void fresh_range(int mode, int P, int G, int B, int k, int& a0, int& a1) {
  const int L = P + G;
  if (mode == MODE_NONE) {
    a0 = 0;
    a1 = L;
  } else if (mode == MODE_PREFIX) {
    a0 = P + k * B;
    a1 = L;
  } else {
    a0 = P + k * B;
    a1 = a0 + B;
  }
}

// Decode a work item; false if it has nothing to do.
__device__ __forceinline__ bool decode_item(const AttnArgs& a, int item, Geo& g) {
  int rest = item;
  const int hg = rest % a.g;
  rest /= a.g;
  g.s = rest % a.n_split;
  rest /= a.n_split;
  g.qt = rest % a.n_qt;
  rest /= a.n_qt;
  g.hk = rest % a.Hkv;
  g.i = rest / a.Hkv;
  g.h = g.hk * a.g + hg;
  const int P = seq_prompt(a.sq, g.i);
  const int k = seq_block(a.sq, g.i);
  g.L = P + a.sq.G;
  fresh_range(a.mode, P, a.sq.G, a.sq.B, k, g.a0, g.a1);
  g.nq = g.a1 - g.a0;
  if (g.qt * kQT >= g.nq) return false;
  g.n_act = (g.L + a.kchunk - 1) / a.kchunk;
  if (g.s >= g.n_act) return false;
  g.kb = g.s * a.kchunk;
  g.ke = min(g.L, g.kb + a.kchunk);
  return true;
}

// Address of K/V row j: the fresh tensor inside [a0, a1), the cache
// elsewhere.  Branch-free (an integer select), so that loads issued for
// different rows stay in one basic block and in flight together.
template <typename T>
__device__ __forceinline__ const T* kv_row(const AttnArgs& a, const T* fresh, const T* cache, const Geo& g,
                                           int j, int d) {
  const bool fr = (unsigned)(j - g.a0) < (unsigned)(g.a1 - g.a0);
  const uintptr_t pf = (uintptr_t)(fresh + (((size_t)g.i * a.fresh_rows + (j - g.a0)) * a.Hkv + g.hk) * d);
  const uintptr_t pc = (uintptr_t)(cache + (((size_t)g.i * a.Hkv + g.hk) * a.sq.Lcap + j) * d);
  return (const T*)(fr ? pf : pc);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// ------------------------------------------------------------------ bf16 MFMA
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnArgs a) {
  // XCD-aware remap: blockIdx.x is dealt round-robin over 8 XCDs; give each
  // XCD a contiguous range of work items.
  const int bid = blockIdx.x;
  const int item = (bid & 7) * a.per_xcd + (bid >> 3);
  if (item >= a.n_items) return;
  Geo g;
  if (!decode_item(a, item, g)) return;

  __shared__ __attribute__((aligned(16))) uint16_t s_vt_raw[kNW * kD * kVtStride];
  __shared__ float s_m[kNW][kQT], s_l[kNW][kQT];
  __shared__ float s_L[kQT];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lq = lane & 31, hh = lane >> 5;
  const float c = a.scale_log2;
  const int q0 = g.qt * kQT;

  const uint16_t* qp = (const uint16_t*)a.q;
  const uint16_t* knp = (const uint16_t*)a.kn;
  const uint16_t* vnp = (const uint16_t*)a.vn;
  const uint16_t* kcp = (const uint16_t*)a.kc;
  const uint16_t* vcp = (const uint16_t*)a.vc;

  // Q as the B operand of S^T = K Q^T: lane (lq, hh) holds query row lq,
  // columns [16 ks + 8 hh, +8) for ks = 0..7.  Rows past nq are zero.
  bf16x8 qop[8];
  {
    const int r = q0 + lq;
    const uint16_t* qrow = qp + (((size_t)g.i * a.fresh_rows + min(r, g.nq - 1)) * a.Hq + g.h) * kD;
    const bool live = r < g.nq;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 w = *(const uint4*)(qrow + 16 * ks + 8 * hh);
      qop[ks] = as_bf16x8(live ? w : make_uint4(0, 0, 0, 0));
    }
  }

  // K rows of a sub-tile go to A-operand registers; V rows (keys 16 n +
  // 4 (lane / 16) + kk, columns 8 (lane % 16) + [0, 8)) to registers for the
  // LDS transpose.  Rows past the chunk end re-read its last row (masked
  // later), so every load is unconditional.
  bf16x8 kop[8];
  uint4 vr[2][4];
  auto load_tile = [&](int t0) {
    const uint16_t* krow = kv_row(a, knp, kcp, g, min(t0 + lq, g.ke - 1), kD);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kop[ks] = as_bf16x8(*(const uint4*)(krow + 16 * ks + 8 * hh));
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int j = min(t0 + 16 * n + 4 * (lane >> 4) + kk, g.ke - 1);
        vr[n][kk] = *(const uint4*)(kv_row(a, vnp, vcp, g, j, kD) + 8 * (lane & 15));
      }
  };

  f32x16 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  uint16_t* vt = s_vt_raw + wid * (kD * kVtStride);

  // One 32-key sub-tile; with `prefetch` the next sub-tile's loads are
  // issued as soon as this one's K and V registers are consumed.  The last
  // sub-tile of a wave runs without a prefetch (nothing is left to fetch).
  auto tile_step = [&](int kt, auto prefetch) {
    f32x16 S;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[ks], S, 0, 0, 0);

    // V transposed into LDS: vt[d][key], 4 keys per 8-byte write
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const uint32_t* w0 = (const uint32_t*)&vr[n][0];
      const uint32_t* w1 = (const uint32_t*)&vr[n][1];
      const uint32_t* w2 = (const uint32_t*)&vr[n][2];
      const uint32_t* w3 = (const uint32_t*)&vr[n][3];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) ? 16 : 0;
        const uint32_t b0 = (w0[e >> 1] >> sh) & 0xffffu;
        const uint32_t b1 = (w1[e >> 1] >> sh) & 0xffffu;
        const uint32_t b2 = (w2[e >> 1] >> sh) & 0xffffu;
        const uint32_t b3 = (w3[e >> 1] >> sh) & 0xffffu;
        uint2 v2;
        v2.x = b0 | (b1 << 16);
        v2.y = b2 | (b3 << 16);
        *(uint2*)(vt + (8 * (lane & 15) + e) * kVtStride + 16 * n + 4 * (lane >> 4)) = v2;
      }
    }
    // K and V of this sub-tile are consumed: fetch the next one while the
    // softmax and the PV product run
    if constexpr (decltype(prefetch)::value) load_tile(kt + kKT * kNW);

    // lane holds query column lq, keys kt + 8 (r / 4) + 4 hh + (r % 4)
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (key >= g.ke) S[r] = -INFINITY;
      mx = fmaxf(mx, S[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2_fast((m_run - m_new) * c);
    const float mc = m_new * c;
    float p[16];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = exp2_fast(fmaf(S[r], c, -mc));
      ps += p[r];
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;

    bf16x8 pop[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      uint4 w;
      w.x = pack_bf16x2(p[8 * h2 + 0], p[8 * h2 + 1]);
      w.y = pack_bf16x2(p[8 * h2 + 2], p[8 * h2 + 3]);
      w.z = pack_bf16x2(p[8 * h2 + 4], p[8 * h2 + 5]);
      w.w = pack_bf16x2(p[8 * h2 + 6], p[8 * h2 + 7]);
      pop[h2] = as_bf16x8(w);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const uint16_t* base = vt + (lq + 32 * dt) * kVtStride + 16 * k2 + 4 * hh;
        const uint2 u0 = *(const uint2*)base;
        const uint2 u1 = *(const uint2*)(base + 8);
        const bf16x8 vop = as_bf16x8(make_uint4(u0.x, u0.y, u1.x, u1.y));
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[k2], O[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  int kt = g.kb + kKT * wid;
  if (kt < g.ke) {
    load_tile(kt);
    for (; kt + kKT * kNW < g.ke; kt += kKT * kNW) tile_step(kt, std::true_type{});
    tile_step(kt, std::false_type{});
  }

  // ---- merge the 4 waves (per query column lq)
  const float l_full = l_run + __shfl_xor(l_run, 32, 64);
  if (hh == 0) {
    s_m[wid][lq] = m_run;
    s_l[wid][lq] = l_full;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kNW; ++w) M = fmaxf(M, s_m[w][lq]);
  float Lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kNW; ++w) Lsum += s_l[w][lq] * exp2_fast((s_m[w][lq] - M) * c);
  const float f = exp2_fast((m_run - M) * c);
  if (wid == 0 && hh == 0) s_L[lq] = Lsum;

  float* red = (float*)s_vt_raw;  // [kNW][kQT][kRedStride], reuses the V tiles
  const bool split = a.n_split > 1;
  const size_t slot = (((size_t)g.i * a.Hq + g.h) * a.n_qt + g.qt) * a.n_split + g.s;  // (i, h, qt, s)
  const auto prs = make_rsrc(split ? a.part + slot * kPartFloats : a.part);
  const int oq = tid >> 3;          // query row handled in the output phase
  const int od = 8 * (tid & 7);     // 8 columns within the 64-column half

#pragma unroll
  for (int ph = 0; ph < 2; ++ph) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int dt = 2 * ph + u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dl = 32 * u + 8 * (r >> 2) + 4 * hh + (r & 3);
        red[(wid * kQT + lq) * kRedStride + dl] = O[dt][r] * f;
      }
    }
    __syncthreads();
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) acc += red[(w * kQT + oq) * kRedStride + od + e];
      o[e] = acc;
    }
    if (!split) {
      if (q0 + oq < g.nq) {
        const float inv = 1.f / s_L[oq];
        uint4 w;
        w.x = pack_bf16x2(o[0] * inv, o[1] * inv);
        w.y = pack_bf16x2(o[2] * inv, o[3] * inv);
        w.z = pack_bf16x2(o[4] * inv, o[5] * inv);
        w.w = pack_bf16x2(o[6] * inv, o[7] * inv);
        uint16_t* orow = (uint16_t*)a.out + (((size_t)g.i * a.fresh_rows + q0 + oq) * a.Hq + g.h) * kD;
        *(uint4*)(orow + 64 * ph + od) = w;
      }
    } else {
      const int off = (oq * kD + 64 * ph + od) * 4;
      st_coherent_b128(prs, off, make_float4(o[0], o[1], o[2], o[3]));
      st_coherent_b128(prs, off + 16, make_float4(o[4], o[5], o[6], o[7]));
    }
    __syncthreads();
  }
  if (!split) return;

  if (wid == 0 && hh == 0) {
    st_coherent_b32(prs, (kQT * kD + lq) * 4, M);
    st_coherent_b32(prs, (kQT * kD + kQT + lq) * 4, Lsum);
  }
  uint32_t* cnt = a.cnt + ((size_t)g.i * a.Hq + g.h) * a.n_qt + g.qt;
  if (!block_arrive(cnt, (unsigned)g.n_act, &s_last)) return;

  // ---- last workgroup of this tile: merge the n_act split partials.  Every
  // partial load is issued before any is used (clamped index, weight 0 past
  // n_act), so the merge costs one memory round trip.
  const float* part0 = a.part + (slot - g.s) * kPartFloats;
  const int cq = tid >> 3;            // query row
  const int cd = 16 * (tid & 7);      // 16 columns
  if (q0 + cq < g.nq) {
    float ms[kMaxSplit], ls[kMaxSplit];
    float4 xs[kMaxSplit][4];
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
      const auto r = make_rsrc(part0 + min(s, g.n_act - 1) * kPartFloats);
      ms[s] = ld_coherent_b32(r, (kQT * kD + cq) * 4);
      ls[s] = ld_coherent_b32(r, (kQT * kD + kQT + cq) * 4);
#pragma unroll
      for (int v = 0; v < 4; ++v) xs[s][v] = ld_coherent_b128(r, (cq * kD + cd + 4 * v) * 4);
    }
    float Mg = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) Mg = fmaxf(Mg, ms[s]);
    float wsum = 0.f;
    float ov[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) ov[e] = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
      const float w = (s < g.n_act) ? exp2_fast((ms[s] - Mg) * c) : 0.f;
      wsum += ls[s] * w;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        ov[4 * v + 0] += xs[s][v].x * w;
        ov[4 * v + 1] += xs[s][v].y * w;
        ov[4 * v + 2] += xs[s][v].z * w;
        ov[4 * v + 3] += xs[s][v].w * w;
      }
    }
    const float inv = 1.f / wsum;
    uint16_t* orow = (uint16_t*)a.out + (((size_t)g.i * a.fresh_rows + q0 + cq) * a.Hq + g.h) * kD;
    uint4 w0, w1;
    w0.x = pack_bf16x2(ov[0] * inv, ov[1] * inv);
    w0.y = pack_bf16x2(ov[2] * inv, ov[3] * inv);
    w0.z = pack_bf16x2(ov[4] * inv, ov[5] * inv);
    w0.w = pack_bf16x2(ov[6] * inv, ov[7] * inv);
    w1.x = pack_bf16x2(ov[8] * inv, ov[9] * inv);
    w1.y = pack_bf16x2(ov[10] * inv, ov[11] * inv);
    w1.z = pack_bf16x2(ov[12] * inv, ov[13] * inv);
    w1.w = pack_bf16x2(ov[14] * inv, ov[15] * inv);
    *(uint4*)(orow + cd) = w0;
    *(uint4*)(orow + cd + 8) = w1;
  }
  if (tid == 0) *cnt = 0u;
}

// ------------------------------------------------------------------ f32 VALU
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  constexpr int U = D / 64;
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wid;
  Geo g;
  g.i = blockIdx.z;
  g.h = blockIdx.y;
  g.hk = g.h / a.g;
  const int P = seq_prompt(a.sq, g.i);
  const int k = seq_block(a.sq, g.i);
  g.L = P + a.sq.G;
  fresh_range(a.mode, P, a.sq.G, a.sq.B, k, g.a0, g.a1);
  g.nq = g.a1 - g.a0;
  __shared__ float s_q[4][D];
  if (r >= g.nq) return;

  const float* qrow = (const float*)a.q + (((size_t)g.i * a.fresh_rows + r) * a.Hq + g.h) * D;
#pragma unroll
  for (int u = 0; u < U; ++u) s_q[wid][lane + 64 * u] = qrow[lane + 64 * u];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const float* kn = (const float*)a.kn;
  const float* vn = (const float*)a.vn;
  const float* kc = (const float*)a.kc;
  const float* vc = (const float*)a.vc;
  float acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int j0 = 0; j0 < g.L; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j < g.L) {
      const float4* krow = (const float4*)kv_row(a, kn, kc, g, j, D);
      float dot = 0.f;
#pragma unroll 8
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float4 kv = krow[d4];
        dot = fmaf(s_q[wid][4 * d4 + 0], kv.x, dot);
        dot = fmaf(s_q[wid][4 * d4 + 1], kv.y, dot);
        dot = fmaf(s_q[wid][4 * d4 + 2], kv.z, dot);
        dot = fmaf(s_q[wid][4 * d4 + 3], kv.w, dot);
      }
      s = dot * a.scale;
    }
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = exp2_fast((m - m_new) * kLog2e);
    const float p = (j < g.L) ? exp2_fast((s - m_new) * kLog2e) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] *= alpha;
    m = m_new;
    const int nk = min(64, g.L - j0);
    for (int jj = 0; jj < nk; ++jj) {
      const float pj = __shfl(p, jj, 64);
      const float* vrow = kv_row(a, vn, vc, g, j0 + jj, D);
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = fmaf(pj, vrow[lane + 64 * u], acc[u]);
    }
  }
  float* orow = (float*)a.out + (((size_t)g.i * a.fresh_rows + r) * a.Hq + g.h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int u = 0; u < U; ++u) orow[lane + 64 * u] = acc[u] * inv;
}

// ------------------------------------------------------------------ planning
// Workgroups the key-split aims for (about two per CU by default; the
// environment variable FDLLM_ATTN_TARGET_WGS overrides it for tuning).
static long attn_target_workgroups() {
  static long v = [] {
    const char* e = getenv("FDLLM_ATTN_TARGET_WGS");
    long t = e ? atol(e) : 512;
    return t > 0 ? t : 512;
  }();
  return v;
}

AttnPlan plan_block_attn(int dtype, int b, int Hq, int Hkv, int d, int nq_max, int L_max) {
  (void)Hkv;
  (void)d;
  AttnPlan p{};
  if (dtype != 0) {
    p.n_qt = (nq_max + 3) / 4;
    p.n_split = 1;
    p.kchunk = L_max;
    p.n_items = b * Hq * p.n_qt;
    p.grid = p.n_qt;
    p.ws_bytes = 0;
    return p;
  }
  p.n_qt = (nq_max + kQT - 1) / kQT;
  const long base = (long)b * Hq * p.n_qt;
  const int unit = kKT * kNW;  // 128 keys: one sub-tile per wave
  const int max_split = (L_max + unit - 1) / unit;
  const long target = attn_target_workgroups();
  int ns = (int)((target + base - 1) / base);
  if (ns < 1) ns = 1;
  if (ns > max_split) ns = max_split;
  if (ns > kMaxSplit) ns = kMaxSplit;
  int kchunk = (L_max + ns - 1) / ns;
  kchunk = ((kchunk + unit - 1) / unit) * unit;
  ns = (L_max + kchunk - 1) / kchunk;
  p.n_split = ns;
  p.kchunk = kchunk;
  p.n_items = (int)(base * ns);
  p.per_xcd = (p.n_items + 7) / 8;
  p.grid = p.per_xcd * 8;
  if (ns > 1) {
    const size_t slots = (size_t)base * ns;
    size_t bytes = slots * kPartFloats * sizeof(float);
    bytes += (size_t)base * sizeof(uint32_t);  // one counter per (sequence, head, query tile)
    p.ws_bytes = (bytes + 255) & ~(size_t)255;
  }
  return p;
}

hipError_t launch_block_attn(const AttnArgs& a, const AttnPlan& p, int dtype, int d, hipStream_t st) {
  const LaunchEvents ev = take_launch_events();
  if (dtype == 0)
    return launch_kernel(attn_bf16_kernel, dim3((unsigned)p.grid), dim3(kThreads), 0, st, ev.start, ev.stop, a);
  dim3 grid((unsigned)p.n_qt, (unsigned)a.Hq, (unsigned)a.sq.b);
  return d == 64 ? launch_kernel(attn_f32_kernel<64>, grid, dim3(256), 0, st, ev.start, ev.stop, a)
                 : launch_kernel(attn_f32_kernel<128>, grid, dim3(256), 0, st, ev.start, ev.stop, a);
}

}  // namespace fdllm
