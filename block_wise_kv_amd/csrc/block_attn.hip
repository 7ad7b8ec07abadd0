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
// bf16, d = 128 (MFMA path).  A workgroup of 4 waves owns QT query tiles
// (32 rows each) of one (sequence, KV head) -- the query heads of a GQA
// group and/or several query tiles of one head -- and one chunk of keys.
// K/V stream through an LDS ring in 32-key tiles:
//   * tiles go from HBM straight into LDS (16-byte global_load_lds, no
//     register staging), several rounds ahead of the compute; every wave
//     issues its share and waits for its own loads, one barrier per round
//     makes the round visible to all waves;
//   * rows are stored row-major with the 16-byte chunks of row r permuted
//     by an XOR with ((r & 3) << 2 | (r >> 2) & 3), which makes both LDS
//     read patterns below free of bank conflicts;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K rows are the A operand
//     (16-byte LDS reads), Q stays in registers as the B operand;
//   * online softmax per query column (exp2 with a log2(e) pre-scale; the
//     accumulator is rescaled only when some column's max grew);
//   * O^T += V^T P^T: P^T comes straight from the S^T accumulator layout,
//     and the V^T operand is read with ds_read_b64_tr_b16, which gathers
//     4 keys x 4 head-dim columns across each 16-lane group, so V never
//     needs a transposed copy.
// With QT = 4 every wave owns one query tile and consumes every K/V tile;
// with QT = 2 or 1 the 2 or 4 waves of a query tile take alternate tiles
// and merge (max, sum, O) through LDS at the end.  When the keys are split
// over several workgroups, each publishes its partial (O, m, l: fp32 here,
// fp16 O with a power-of-two row scale in the split-key kernel and the
// 8-wave ring) with agent-scope (write-through) 16-byte stores and bumps a
// counter; the last one to arrive reads every partial with agent-scope
// loads, merges them and writes the output, then resets the counter (the
// 8-wave ring leaves the merge to a second kernel).
//
// Work items are ordered so that the groups sharing a KV head (and key
// chunk) are adjacent, and the grid is remapped so adjacent items land on
// the same XCD (workgroups are dealt round-robin over the 8 XCDs): they
// then read the same K/V rows through one L2.
//
// f32 (any mode, d = 64 or 128) and bf16 with d = 64: a plain vector-ALU
// kernel, one wave per query row, fp32 arithmetic.
#include <float.h>
#include <stdlib.h>

#include <type_traits>

#include "fdllm_device.h"
#include "fdllm_internal.h"

namespace fdllm {

constexpr int kThreads = 256;          // 4 waves
constexpr int kQT = 32;                // query rows per tile
constexpr int kKT = 32;                // keys per K/V tile
constexpr int kD = 128;                // head dim (bf16 path)
constexpr int kTileBytes = kKT * kD * 2;         // one K or V tile: 8 KB
constexpr int kPartFloats = kQT * kD + 2 * kQT;  // one split partial: O, m, l
// One split partial of the 8-wave ring: O as fp16 rows of 256 bytes, then
// m, l and the rows' power-of-two scales in fp32.
constexpr int kPart16Bytes = kQT * kD * 2 + 3 * kQT * 4;
constexpr int kMaxSplit = 8;           // key chunks per group
constexpr int kCntStride = 32;         // uint32 per arrival counter: one 128-byte line each (atomics on one line serialise)
constexpr int kVtStride = 36;          // bf16 per d-row of the split kernel's transposed V tile
// Split kernel's wave-merge buffer: [4 waves][32 query rows][32 chunks of 4
// floats]; chunk k of row r sits at k ^ red_swizzle(r), which keeps both the
// writes (16 rows, one chunk) and the reads (2 rows, 8 chunks) on distinct banks.
__device__ __forceinline__ int red_swizzle(int r) { return ((r & 1) << 3) | ((r >> 1) & 7); }
constexpr int kSplitLdsBytes = 4 * kQT * kD * 4;  // also holds the 4 transposed V tiles
static_assert(kSplitLdsBytes >= 4 * kD * kVtStride * 2, "V tiles fit the merge buffer");

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
__device__ __forceinline__ bool decode_split_item(const AttnArgs& a, int item, Geo& g) {
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

// 16-byte chunk c of K/V tile row r is stored at chunk c ^ ring_swizzle(r).
__device__ __forceinline__ int ring_swizzle(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

typedef short short4v __attribute__((ext_vector_type(4)));

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Eight 16-byte LDS reads at addr[i], completed before the block ends (see
// lds_read_tr16_x16 for why the ring's reads are hidden from the compiler).
__device__ __forceinline__ void lds_read_b128_x8(const uint32_t* addr, bf16x8* o) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
        "v"(addr[7]));
}

// Sixteen transpose reads (ds_read_b64_tr_b16) at addr[i] + OFF0 and
// addr[i] + OFF1 (both halves of a V tile), completed before the block ends:
// the loads' destinations are valid only after the wait, so it sits in the
// same asm statement.  The ring's LDS reads are asm blocks with their own
// wait: the compiler does not see them, so it does not order them after the
// ring's LDS loads still in flight into other sets (it would wait for every
// load in flight); the explicit counter waits and barriers of the ring loop
// order them instead.
template <int OFF0, int OFF1>
__device__ __forceinline__ void lds_read_tr16_x16(const uint32_t (&addr)[8], short4v (&o)[8], short4v (&p)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
      "ds_read_b64_tr_b16 %1, %17 offset:%24\n\t"
      "ds_read_b64_tr_b16 %2, %18 offset:%24\n\t"
      "ds_read_b64_tr_b16 %3, %19 offset:%24\n\t"
      "ds_read_b64_tr_b16 %4, %20 offset:%24\n\t"
      "ds_read_b64_tr_b16 %5, %21 offset:%24\n\t"
      "ds_read_b64_tr_b16 %6, %22 offset:%24\n\t"
      "ds_read_b64_tr_b16 %7, %23 offset:%24\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:%25\n\t"
      "ds_read_b64_tr_b16 %9, %17 offset:%25\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:%25\n\t"
      "ds_read_b64_tr_b16 %11, %19 offset:%25\n\t"
      "ds_read_b64_tr_b16 %12, %20 offset:%25\n\t"
      "ds_read_b64_tr_b16 %13, %21 offset:%25\n\t"
      "ds_read_b64_tr_b16 %14, %22 offset:%25\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]),
        "=&v"(p[0]), "=&v"(p[1]), "=&v"(p[2]), "=&v"(p[3]), "=&v"(p[4]), "=&v"(p[5]), "=&v"(p[6]), "=&v"(p[7])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
        "v"(addr[7]), "i"(OFF0), "i"(OFF1));
}

// Merge the NS key-chunk partials (O, m, l in fp32) of one query tile, whose
// partial s starts at float s * kPartFloats of resource r: query row cq,
// head-dim columns c0 + 32 v + 4 j + [0, 4) for v = 0..NV-1, written to orow
// in bf16.  The 8 lanes of a row read one whole 128-byte line per load, and
// every load is issued before any is used, so the merge costs one memory
// round trip.
template <int NS, int NV = 4>
__device__ __forceinline__ void merge_partials_n(__amdgpu_buffer_rsrc_t r, int cq, int j, float c, uint16_t* orow,
                                                 int c0 = 0) {
  float ms[NS], ls[NS];
  float4 xs[NS][NV];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int o = s * kPartFloats;
    ms[s] = ld_coherent_b32(r, (o + kQT * kD + cq) * 4);
    ls[s] = ld_coherent_b32(r, (o + kQT * kD + kQT + cq) * 4);
#pragma unroll
    for (int v = 0; v < NV; ++v) xs[s][v] = ld_coherent_b128(r, (o + cq * kD + c0 + 32 * v + 4 * j) * 4);
  }
  __builtin_amdgcn_sched_barrier(0);
  float Mg = ms[0];
#pragma unroll
  for (int s = 1; s < NS; ++s) Mg = fmaxf(Mg, ms[s]);
  float wsum = 0.f;
  float4 ov[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) ov[v] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float w = exp2_fast((ms[s] - Mg) * c);
    wsum += ls[s] * w;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      ov[v].x += xs[s][v].x * w;
      ov[v].y += xs[s][v].y * w;
      ov[v].z += xs[s][v].z * w;
      ov[v].w += xs[s][v].w * w;
    }
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    uint2 w;
    w.x = pack_bf16x2(ov[v].x * inv, ov[v].y * inv);
    w.y = pack_bf16x2(ov[v].z * inv, ov[v].w * inv);
    *(uint2*)(orow + c0 + 32 * v + 4 * j) = w;
  }
}
// n (wave-uniform, 1..kMaxSplit) partials: only those are read.
__device__ __forceinline__ void merge_partials(int n, __amdgpu_buffer_rsrc_t r, int cq, int j, float c, uint16_t* orow) {
  switch (n) {
    case 1: merge_partials_n<1>(r, cq, j, c, orow); break;
    case 2: merge_partials_n<2>(r, cq, j, c, orow); break;
    case 3: merge_partials_n<3>(r, cq, j, c, orow); break;
    case 4: merge_partials_n<4>(r, cq, j, c, orow); break;
    case 5: merge_partials_n<5>(r, cq, j, c, orow); break;
    case 6: merge_partials_n<6>(r, cq, j, c, orow); break;
    case 7: merge_partials_n<7>(r, cq, j, c, orow); break;
    default: merge_partials_n<8>(r, cq, j, c, orow); break;
  }
}

// Merge NS key-chunk partials of one query tile in the fp16 format (O rows
// of 256 bytes in fp16, then m, l and the rows' power-of-two scales in
// fp32; partial s starts at byte s * kPart16Bytes of resource r): query row
// cq, head-dim columns c0 + 64 h + 8 j + [0, 8) for h = 0..NH-1, written to
// orow in bf16.  The 8 lanes of a row read one whole 128-byte line per
// partial and half, and every load is issued before any is used, so the
// merge costs one memory round trip.
template <int NS, int NH>
__device__ __forceinline__ void merge_partials16_n(__amdgpu_buffer_rsrc_t r, int cq, int j, float c, uint16_t* orow,
                                                   int c0) {
  float ms[NS], ls[NS], ss[NS];
  float4 xs[NS][NH];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int o = s * kPart16Bytes;
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) xs[s][hf] = ld_coherent_b128(r, o + cq * kD * 2 + (c0 + 64 * hf + 8 * j) * 2);
    ms[s] = ld_coherent_b32(r, o + kQT * kD * 2 + cq * 4);
    ls[s] = ld_coherent_b32(r, o + kQT * kD * 2 + (kQT + cq) * 4);
    ss[s] = ld_coherent_b32(r, o + kQT * kD * 2 + (2 * kQT + cq) * 4);
  }
  __builtin_amdgcn_sched_barrier(0);
  float Mg = ms[0];
#pragma unroll
  for (int s = 1; s < NS; ++s) Mg = fmaxf(Mg, ms[s]);
  float wsum = 0.f;
  float ov[NH][8];
#pragma unroll
  for (int hf = 0; hf < NH; ++hf)
#pragma unroll
    for (int k = 0; k < 8; ++k) ov[hf][k] = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float w = exp2_fast((ms[s] - Mg) * c);
    wsum += ls[s] * w;
    const float ws = w * ss[s];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      const uint32_t u[4] = {__float_as_uint(xs[s][hf].x), __float_as_uint(xs[s][hf].y), __float_as_uint(xs[s][hf].z),
                             __float_as_uint(xs[s][hf].w)};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float lo, hi;
        unpack_f16x2(u[k], lo, hi);
        ov[hf][2 * k] = fmaf(lo, ws, ov[hf][2 * k]);
        ov[hf][2 * k + 1] = fmaf(hi, ws, ov[hf][2 * k + 1]);
      }
    }
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
    uint4 w;
    w.x = pack_bf16x2(ov[hf][0] * inv, ov[hf][1] * inv);
    w.y = pack_bf16x2(ov[hf][2] * inv, ov[hf][3] * inv);
    w.z = pack_bf16x2(ov[hf][4] * inv, ov[hf][5] * inv);
    w.w = pack_bf16x2(ov[hf][6] * inv, ov[hf][7] * inv);
    *(uint4*)(orow + c0 + 64 * hf + 8 * j) = w;
  }
}
// n (wave-uniform, 1..kMaxSplit) partials of whole rows: only those are read.
__device__ __forceinline__ void merge_partials16(int n, __amdgpu_buffer_rsrc_t r, int cq, int j, float c,
                                                 uint16_t* orow) {
  switch (n) {
    case 1: merge_partials16_n<1, 2>(r, cq, j, c, orow, 0); break;
    case 2: merge_partials16_n<2, 2>(r, cq, j, c, orow, 0); break;
    case 3: merge_partials16_n<3, 2>(r, cq, j, c, orow, 0); break;
    case 4: merge_partials16_n<4, 2>(r, cq, j, c, orow, 0); break;
    case 5: merge_partials16_n<5, 2>(r, cq, j, c, orow, 0); break;
    case 6: merge_partials16_n<6, 2>(r, cq, j, c, orow, 0); break;
    case 7: merge_partials16_n<7, 2>(r, cq, j, c, orow, 0); break;
    default: merge_partials16_n<8, 2>(r, cq, j, c, orow, 0); break;
  }
}

// ------------------------------------------------------------------ bf16 MFMA, split keys
// One query tile per workgroup (MHA with a single query tile per head):
// the 4 waves take alternate 32-key sub-tiles of the workgroup's key chunk,
// K goes straight from HBM into A-operand registers, V rows are transposed
// through a wave-private LDS tile, and the next sub-tile's loads are issued
// as soon as this one's registers are consumed.
__global__ __launch_bounds__(kThreads, 2) void attn_split_kernel(AttnArgs a) {
  // XCD-aware remap: blockIdx.x is dealt round-robin over 8 XCDs; give each
  // XCD a contiguous range of work items.
  const int bid = blockIdx.x;
  const int item = (bid & 7) * a.per_xcd + (bid >> 3);
  if (item >= a.n_items) return;
  Geo g;
  if (!decode_split_item(a, item, g)) return;

  __shared__ __attribute__((aligned(16))) uint16_t s_vt_raw[kSplitLdsBytes / 2];
  __shared__ float s_m[4][kQT], s_l[4][kQT];
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
    if constexpr (decltype(prefetch)::value) load_tile(kt + kKT * 4);

    // lane holds query column lq, keys kt + 8 (r / 4) + 4 hh + (r % 4)
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (key >= g.ke) S[r] = -INFINITY;
      mx = fmaxf(mx, S[r]);
    }
    mx = xor_combine<32>(mx, [](float x, float y) { return fmaxf(x, y); });
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
    for (; kt + kKT * 4 < g.ke; kt += kKT * 4) tile_step(kt, std::true_type{});
    tile_step(kt, std::false_type{});
  }

  // ---- merge the 4 waves (per query column lq)
  const float l_full = xor_combine<32>(l_run, [](float x, float y) { return x + y; });
  if (hh == 0) {
    s_m[wid][lq] = m_run;
    s_l[wid][lq] = l_full;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][lq]);
  float Lsum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) Lsum += s_l[w][lq] * exp2_fast((s_m[w][lq] - M) * c);
  const float f = exp2_fast((m_run - M) * c);
  if (wid == 0 && hh == 0) s_L[lq] = Lsum;

  // O * f of every wave into the merge buffer (which reuses the V tiles):
  // lane (lq, hh) holds head dims 32 dt + 8 q + 4 hh + [0, 4), chunk
  // 8 dt + 2 q + hh of row lq
  float* red = (float*)s_vt_raw;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = 8 * dt + 2 * q + hh;
      *(float4*)(red + ((wid * kQT + lq) * 32 + (k ^ red_swizzle(lq))) * 4) =
          make_float4(O[dt][4 * q] * f, O[dt][4 * q + 1] * f, O[dt][4 * q + 2] * f, O[dt][4 * q + 3] * f);
    }
  __syncthreads();

  // thread (oq, j) sums head dims 8 j + [0, 8) and 64 + 8 j + [0, 8) of
  // query row oq over the waves (chunks 2 j, 2 j + 1, 16 + 2 j, 17 + 2 j):
  // the 8 lanes of a row then cover whole 128-byte lines of the fp16
  // partial and of the bf16 output
  const bool split = a.n_split > 1;
  const size_t slot = (((size_t)g.i * a.Hq + g.h) * a.n_qt + g.qt) * a.n_split + g.s;  // (i, h, qt, s)
  const int oq = tid >> 3, oj = tid & 7;
  float4 o[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int k = 16 * (v >> 1) + 2 * oj + (v & 1);
    float4 acc = *(const float4*)(red + (oq * 32 + (k ^ red_swizzle(oq))) * 4);
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 x = *(const float4*)(red + ((w * kQT + oq) * 32 + (k ^ red_swizzle(oq))) * 4);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    o[v] = acc;
  }
  if (!split) {
    if (q0 + oq < g.nq) {
      const float inv = 1.f / s_L[oq];
      uint16_t* orow = (uint16_t*)a.out + (((size_t)g.i * a.fresh_rows + q0 + oq) * a.Hq + g.h) * kD;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const float4 x = o[2 * hf], y = o[2 * hf + 1];
        uint4 w;
        w.x = pack_bf16x2(x.x * inv, x.y * inv);
        w.y = pack_bf16x2(x.z * inv, x.w * inv);
        w.z = pack_bf16x2(y.x * inv, y.y * inv);
        w.w = pack_bf16x2(y.z * inv, y.w * inv);
        *(uint4*)(orow + 64 * hf + 8 * oj) = w;
      }
    }
    return;
  }
  // Partial (O, m, l) in attn_gqa_kernel's format: O in fp16 with a
  // power-of-two scale per row, the row's largest |O| stored in [2^14, 2^15).
  float amax = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v)
    amax = fmaxf(fmaxf(amax, fmaxf(fabsf(o[v].x), fabsf(o[v].y))), fmaxf(fabsf(o[v].z), fabsf(o[v].w)));
  amax = xor_combine<1>(amax, [](float x, float y) { return fmaxf(x, y); });
  amax = xor_combine<2>(amax, [](float x, float y) { return fmaxf(x, y); });
  amax = xor_combine<4>(amax, [](float x, float y) { return fmaxf(x, y); });
  const int e = __builtin_amdgcn_frexp_expf(amax) - 15;
  const auto prs = make_rsrc((uint8_t*)a.part + slot * kPart16Bytes);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const float4 x = o[2 * hf], y = o[2 * hf + 1];
    u32x4 w;
    w.x = pack_f16x2(__builtin_amdgcn_ldexpf(x.x, -e), __builtin_amdgcn_ldexpf(x.y, -e));
    w.y = pack_f16x2(__builtin_amdgcn_ldexpf(x.z, -e), __builtin_amdgcn_ldexpf(x.w, -e));
    w.z = pack_f16x2(__builtin_amdgcn_ldexpf(y.x, -e), __builtin_amdgcn_ldexpf(y.y, -e));
    w.w = pack_f16x2(__builtin_amdgcn_ldexpf(y.z, -e), __builtin_amdgcn_ldexpf(y.w, -e));
    __builtin_amdgcn_raw_buffer_store_b128(w, prs, oq * kD * 2 + 128 * hf + 16 * oj, 0, kCoherentAux);
  }
  if (oj == 0) st_coherent_b32(prs, kQT * kD * 2 + (2 * kQT + oq) * 4, __builtin_amdgcn_ldexpf(1.f, e));
  if (wid == 0 && hh == 0) {
    st_coherent_b32(prs, kQT * kD * 2 + lq * 4, M);
    st_coherent_b32(prs, kQT * kD * 2 + (kQT + lq) * 4, Lsum);
  }
  uint32_t* cnt = a.cnt + (((size_t)g.i * a.Hq + g.h) * a.n_qt + g.qt) * kCntStride;
  if (!block_arrive(cnt, (unsigned)g.n_act, &s_last)) return;

  // ---- last workgroup of this tile: merge the n_act split partials
  const auto r = make_rsrc(uniform_ptr((const uint8_t*)a.part + (slot - g.s) * kPart16Bytes));
  const int cq = tid >> 3;            // query row
  if (q0 + cq < g.nq)
    merge_partials16(__builtin_amdgcn_readfirstlane(g.n_act), r, cq, tid & 7, c,
                     (uint16_t*)a.out + (((size_t)g.i * a.fresh_rows + q0 + cq) * a.Hq + g.h) * kD);
  if (tid == 0) *cnt = 0u;
}

constexpr float kRefSlack = 8.f;       // log2 headroom of the softmax exponent reference

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
// Two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}
__device__ __forceinline__ float pairwise_sum16(const float* x) {
  float t[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) t[k] = x[k] + x[k + 8];
#pragma unroll
  for (int k = 0; k < 4; ++k) t[k] += t[k + 4];
  return (t[0] + t[2]) + (t[1] + t[3]);
}

// Online-softmax step of one 32-key tile for the 8-wave kernels, with the
// tile's scores S^T in the MFMA accumulator layout (lane (lq, hh): query
// column lq, 16 keys).  The weights p = 2^(c (S - m_ref)) are taken against
// the running reference m_ref first; only when a column's 16 weights sum
// past 2^kSumCap, or are not finite (the first tile, whose reference is
// -inf), is the reference raised to the column maximum (over both lane
// halves), O and l rescaled and p recomputed.  Exact in either branch: the
// reference only scales the weights, and every weight stays <= 2^kSumCap.
// l_run gains the weights' sum; pop gets them as bf16, the B operand of the
// P V product.
constexpr float kSumCap = 12.f;
__device__ __forceinline__ void softmax_tile(f32x16& S, float c, float& m_ref, float& l_run, f32x16* O,
                                             bf16x8* pop) {
  const float mc = m_ref * c;
  float p[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) p[r] = exp2_fast(fmaf(S[r], c, -mc));
  float sum = pairwise_sum16(p);
  if (__builtin_expect(__ballot(!(sum <= (float)(1 << (int)kSumCap))) != 0, 0)) {
    float mx = S[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
    mx = xor_combine<32>(mx, [](float x, float y) { return fmaxf(x, y); });
    const float m_new = fmaxf(m_ref, mx);
    const float alpha = exp2_fast((m_ref - m_new) * c);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
    m_ref = m_new;
    const float mc2 = m_ref * c;
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = exp2_fast(fmaf(S[r], c, -mc2));
    sum = pairwise_sum16(p);
  }
  l_run += sum;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    uint4 w;
    w.x = cvt_pk_bf16(p[8 * h2 + 0], p[8 * h2 + 1]);
    w.y = cvt_pk_bf16(p[8 * h2 + 2], p[8 * h2 + 3]);
    w.z = cvt_pk_bf16(p[8 * h2 + 4], p[8 * h2 + 5]);
    w.w = cvt_pk_bf16(p[8 * h2 + 6], p[8 * h2 + 7]);
    pop[h2] = as_bf16x8(w);
  }
}

// ------------------------------------------------------------------ bf16 MFMA, LDS ring
template <int QT, int NR>
__global__ __launch_bounds__(kThreads, (QT == 4 && NR <= 4) ? 2 : 1) void attn_ring_kernel(AttnArgs a) {
  constexpr int R = 4 / QT;                         // key tiles per round (one per key phase)
  constexpr int SET = R * 2 * kTileBytes;           // ring set: R tiles of K then V
  constexpr int DPR = 4 * R;                        // 1 KB loads per wave per round
  static_assert(NR >= 3 && NR <= 6, "the pipeline reads two ring sets per round");
  __shared__ __attribute__((aligned(16))) uint8_t ring[NR * SET];
  __shared__ float s_m[4][kQT], s_l[4][kQT];
  __shared__ int s_last;
  auto set_ptr = [&](auto jc) __attribute__((always_inline)) -> uint8_t* {
    return ring + (decltype(jc)::value % NR) * SET;
  };

  // XCD-aware remap: blockIdx.x is dealt round-robin over 8 XCDs; give each
  // XCD a contiguous range of work items.
  const int bid = blockIdx.x;
  const int item = (bid & 7) * a.per_xcd + (bid >> 3);
  if (item >= a.n_items) return;
  // item = ((i * Hkv + hk) * n_split + s) * n_grp + grp
  int rest = item;
  const int grp = rest % a.n_grp;
  rest /= a.n_grp;
  const int sp = rest % a.n_split;
  rest /= a.n_split;
  Geo g;
  g.hk = rest % a.Hkv;
  g.i = rest / a.Hkv;
  const int P = seq_prompt(a.sq, g.i);
  g.L = P + a.sq.G;
  fresh_range(a.mode, P, a.sq.G, a.sq.B, seq_block(a.sq, g.i), g.a0, g.a1);
  g.nq = g.a1 - g.a0;
  g.n_act = (g.L + a.kchunk - 1) / a.kchunk;
  g.kb = sp * a.kchunk;
  g.ke = min(g.L, g.kb + a.kchunk);
  if (g.kb >= g.ke) return;                       // chunk past this sequence's keys
  const int n_live_qt = (g.nq + kQT - 1) / kQT;   // this sequence's query tiles per head
  if (grp * QT >= a.g * a.n_qt) return;
  {
    bool any = false;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int u = grp * QT + t;
      any |= (u < a.g * a.n_qt) && (u % a.n_qt) < n_live_qt;
    }
    if (!any) return;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lq = lane & 31, hh = lane >> 5;
  const int qi = wid % QT, ph = wid / QT;
  const int u = grp * QT + qi;                    // query tile of (i, hk): head-major
  const int hg = min(u / a.n_qt, a.g - 1);
  const int qt = u % a.n_qt;
  const bool live = u < a.g * a.n_qt && qt < n_live_qt;
  const int h = g.hk * a.g + hg;
  const int q0 = qt * kQT;
  const float c = a.scale_log2;

  const uint16_t* knp = (const uint16_t*)a.kn;
  const uint16_t* vnp = (const uint16_t*)a.vn;
  const uint16_t* kcp = (const uint16_t*)a.kc;
  const uint16_t* vcp = (const uint16_t*)a.vc;

  // Q as the B operand of S^T = K Q^T: lane (lq, hh) holds query row lq,
  // columns [16 ks + 8 hh, +8) for ks = 0..7.  Rows past nq are zero.
  bf16x8 qop[8];
  {
    const int r = q0 + lq;
    const uint16_t* qrow =
        (const uint16_t*)a.q + (((size_t)g.i * a.fresh_rows + max(min(r, g.nq - 1), 0)) * a.Hq + h) * kD;
    const bool rl = live && r < g.nq;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 w = *(const uint4*)(qrow + 16 * ks + 8 * hh);
      qop[ks] = as_bf16x8(rl ? w : make_uint4(0, 0, 0, 0));
    }
  }

  const int n_tiles = (g.ke - g.kb + kKT - 1) / kKT;
  const int n_rounds = (n_tiles + R - 1) / R;

  // Round q into ring set J: R tiles x (8 KB K + 8 KB V) = 16 R loads of
  // 1 KB (4 rows each), DPR per wave.  Rows past the chunk re-read its last
  // row (masked in the softmax), so every round issues the same loads and
  // the counter waits below are exact.  Load ii4 of a tile covers rows
  // row_a + 16 (ii4 & 1) of K (ii4 < 2) or V; this lane moves one 16-byte
  // chunk of it.  A tile that lies wholly in the cache or wholly in the
  // fresh rows is addressed from a uniform row base plus a fixed lane offset.
  const int row_a = 4 * wid + (lane >> 4);
  const int chunk_a = (lane & 15) ^ ring_swizzle(row_a);  // row_a + 16: same swizzle
  const uint32_t off_c = (uint32_t)(row_a * 256 + 16 * chunk_a);
  const uint32_t off_f = (uint32_t)(row_a * a.Hkv * 256 + 16 * chunk_a);
  const size_t fstride = (size_t)a.Hkv * 256;  // bytes between fresh rows of one KV head
  const char* kc_row0 = (const char*)kcp + ((size_t)g.i * a.Hkv + g.hk) * a.sq.Lcap * 256;
  const char* vc_row0 = (const char*)vcp + ((size_t)g.i * a.Hkv + g.hk) * a.sq.Lcap * 256;
  const char* kf_row0 = (const char*)knp + ((size_t)g.i * a.fresh_rows * a.Hkv + g.hk) * 256;
  const char* vf_row0 = (const char*)vnp + ((size_t)g.i * a.fresh_rows * a.Hkv + g.hk) * 256;
  auto issue = [&](int q, auto jc) __attribute__((always_inline)) {
    uint8_t* base = set_ptr(jc);
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
      uint8_t* dst = base + rho * 2 * kTileBytes + wid * 1024;
      const int t0 = g.kb + (q * R + rho) * kKT;
      const bool whole = t0 + kKT <= g.ke;
      const bool in_cache = whole && (t0 + kKT <= g.a0 || t0 >= g.a1);
      const bool in_fresh = whole && t0 >= g.a0 && t0 + kKT <= g.a1;
      if (in_cache || in_fresh) {
        const char* kt = in_cache ? kc_row0 + (size_t)t0 * 256 : kf_row0 + (size_t)(t0 - g.a0) * fstride;
        const char* vt = in_cache ? vc_row0 + (size_t)t0 * 256 : vf_row0 + (size_t)(t0 - g.a0) * fstride;
        const size_t r16 = in_cache ? (size_t)16 * 256 : 16 * fstride;
        const uint32_t off = in_cache ? off_c : off_f;
        __builtin_amdgcn_global_load_lds(kt + off, dst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(kt + r16 + off, dst + 4096, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + off, dst + 8192, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + r16 + off, dst + 12288, 16, 0, 0);
      } else {
#pragma unroll
        for (int ii4 = 0; ii4 < 4; ++ii4) {
          const int j = min(t0 + row_a + 16 * (ii4 & 1), g.ke - 1);
          const char* src =
              (const char*)(ii4 >= 2 ? kv_row(a, vnp, vcp, g, j, kD) : kv_row(a, knp, kcp, g, j, kD)) + 16 * chunk_a;
          __builtin_amdgcn_global_load_lds(src, dst + ii4 * 4096, 16, 0, 0);
        }
      }
    }
  };

  f32x16 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;  // exponent reference and sum per column

  // V^T operand of key half k2 and head-dim tile dt: element e of lane l is
  // V[16 k2 + 8 (e / 4) + 4 hh + e % 4][32 dt + lq] (the key order of P^T
  // below).  In a 16-lane group G the transpose read hands lane
  // 16 G + 4 a + b element j of the 8 bytes addressed by lane 16 G + 4 j + a
  // (element b), so lane 16 G + s addresses key 16 k2 + 4 (G / 2) + s / 4
  // (+ 8 for e >= 4), columns 32 dt + 16 (G % 2) + 4 (s % 4) + [0, 4).
  // vt_off[2 dt + hi] is that address within the V tile for k2 = 0 (k2 = 1
  // is 16 rows further, the same swizzle).
  // K operand of product ks: row lq, 16-byte chunk 2 ks + hh (swizzled).
  uint32_t k_off[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) k_off[ks] = (uint32_t)(lq * 256 + 16 * ((2 * ks + hh) ^ ring_swizzle(lq)));
  uint32_t vt_off[8];
  {
    const int G = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = 4 * (G >> 1) + (sl >> 2) + 8 * hi;
        const int col = 32 * dt + 16 * (G & 1) + 4 * (sl & 3);
        vt_off[2 * dt + hi] = (uint32_t)(r * 256 + 16 * ((col >> 3) ^ ring_swizzle(r)) + 8 * ((col >> 2) & 1));
      }
  }

  // S^T of one 32-key tile (K at tb) against this wave's queries.
  auto stage_s = [&](const uint8_t* tb) __attribute__((always_inline)) -> f32x16 {
    const uint32_t base = lds_addr(tb);
    uint32_t ad[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ad[ks] = base + k_off[ks];
    bf16x8 kop[8];
    // all eight K reads before the products (one LDS wait), then one
    // accumulation chain (no final sum of two)
    lds_read_b128_x8(ad, kop);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[0], qop[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < 8; ++ks) S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[ks], S, 0, 0, 0);
    return S;
  };

  // Softmax of S (keys t0..t0+31, V at tb + 8 KB) and O^T += V^T P^T.
  auto stage_pv = [&](const uint8_t* tb, int t0, f32x16 S) __attribute__((always_inline)) {
    // V^T operands (see vt_off)
    bf16x8 vop[2][4];
    {
      const uint32_t base = lds_addr(tb);
      uint32_t ad[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ad[e] = base + vt_off[e];
      short4v t[8], t2[8];
      __builtin_amdgcn_sched_barrier(0);
      lds_read_tr16_x16<kTileBytes, kTileBytes + 16 * 256>(ad, t, t2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        __builtin_memcpy(&vop[0][dt], &t[2 * dt], 8);
        __builtin_memcpy((char*)&vop[0][dt] + 8, &t[2 * dt + 1], 8);
        __builtin_memcpy(&vop[1][dt], &t2[2 * dt], 8);
        __builtin_memcpy((char*)&vop[1][dt] + 8, &t2[2 * dt + 1], 8);
      }
    }
    // lane holds query column lq, keys t0 + 8 (r / 4) + 4 hh + (r % 4)
    if (t0 + kKT > g.ke) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = t0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= g.ke) S[r] = -INFINITY;
      }
    }
    float mx = S[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
    mx = xor_combine<32>(mx, [](float x, float y) { return fmaxf(x, y); });
    // The exponent reference m_ref moves only when some column's max passes
    // it by more than kRefSlack (log2 units): p <= 2^kRefSlack stays well
    // inside bf16 and fp32 range, and the accumulator is rarely rescaled.
    if (__ballot((mx - m_ref) * c > kRefSlack)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = exp2_fast((m_ref - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
      m_ref = m_new;
    }
    const float mc = m_ref * c;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = exp2_fast(fmaf(S[r], c, -mc));
    l_run += pairwise_sum16(p);
    bf16x8 pop[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      uint4 w;
      w.x = cvt_pk_bf16(p[8 * h2 + 0], p[8 * h2 + 1]);
      w.y = cvt_pk_bf16(p[8 * h2 + 2], p[8 * h2 + 3]);
      w.z = cvt_pk_bf16(p[8 * h2 + 4], p[8 * h2 + 5]);
      w.w = cvt_pk_bf16(p[8 * h2 + 6], p[8 * h2 + 7]);
      pop[h2] = as_bf16x8(w);
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[k2][dt], pop[k2], O[dt], 0, 0, 0);
  };

  // Round q of the ring lives in set q % NR.  Step q: wait until round q+1
  // is in (rounds q+2.. may stay in flight), barrier, refill the set round
  // q-1 used, start S^T of this wave's tile of round q+1, then finish the
  // tile of round q (softmax and P V), whose S^T the previous step started.
  // The matrix unit runs the next tile's S^T while the vector unit does the
  // softmax of the current one.
  f32x16 S_cur;
#pragma unroll
  for (int r = 0; r < 16; ++r) S_cur[r] = 0.f;
  auto step = [&](int q, auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    wait_vm<(NR - 3) * DPR, true>();
    ring_barrier();
    issue(q + NR - 1, std::integral_constant<int, (J + NR - 1) % NR>{});
    const int tile_n = (q + 1) * R + ph;
    f32x16 S_nxt = S_cur;
    if (live && tile_n < n_tiles) S_nxt = stage_s(set_ptr(std::integral_constant<int, (J + 1) % NR>{}) + ph * 2 * kTileBytes);
    const int tile = q * R + ph;
    if (live && tile < n_tiles) stage_pv(set_ptr(jc) + ph * 2 * kTileBytes, g.kb + tile * kKT, S_cur);
    S_cur = S_nxt;
  };
  // Q settles together with round 0 (the first product needs both), before
  // the later prologue rounds are issued, so no wait for Q is left inside
  // the loop.
  issue(0, std::integral_constant<int, 0>{});
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qop[ks]));
  issue(1, std::integral_constant<int, 1>{});
  if constexpr (NR > 3) issue(2, std::integral_constant<int, 2>{});
  if constexpr (NR > 4) issue(3, std::integral_constant<int, 3>{});
  if constexpr (NR > 5) issue(4, std::integral_constant<int, 4>{});
  // round 0 in (NR - 2 later rounds in flight): start its S^T
  wait_vm<(NR - 2) * DPR, true>();
  ring_barrier();
  if (live && ph < n_tiles) S_cur = stage_s(ring + ph * 2 * kTileBytes);
  // steps past the last round only wait, meet at the barrier and refill
  // (clamped loads): every path through the loop is the same, which keeps
  // the compiler's view of the loads in flight exact
  for (int q = 0; q < n_rounds; q += NR) {
    step(q, std::integral_constant<int, 0>{});
    step(q + 1, std::integral_constant<int, 1>{});
    step(q + 2, std::integral_constant<int, 2>{});
    if constexpr (NR > 3) step(q + 3, std::integral_constant<int, 3>{});
    if constexpr (NR > 4) step(q + 4, std::integral_constant<int, 4>{});
    if constexpr (NR > 5) step(q + 5, std::integral_constant<int, 5>{});
  }
  // the ring's trailing loads land before its memory is reused
  wait_vm<0, true>();
  ring_barrier();

  // ---- combine the R key phases of each query tile (per column lq)
  const float l_col = xor_combine<32>(l_run, [](float x, float y) { return x + y; });
  float M = m_ref, Lsum = l_col;
  if constexpr (R > 1) {
    if (hh == 0) {
      s_m[wid][lq] = m_ref;
      s_l[wid][lq] = l_col;
    }
    __syncthreads();
    M = -INFINITY;
#pragma unroll
    for (int p2 = 0; p2 < R; ++p2) M = fmaxf(M, s_m[qi + QT * p2][lq]);
    Lsum = 0.f;
#pragma unroll
    for (int p2 = 0; p2 < R; ++p2) Lsum += s_l[qi + QT * p2][lq] * exp2_fast((s_m[qi + QT * p2][lq] - M) * c);
    const float f = exp2_fast((m_ref - M) * c);
    float* red = (float*)ring;  // [(R - 1) QT slots][64 values][64 lanes]
    if (ph > 0) {
      float* slot = red + (size_t)((ph - 1) * QT + qi) * 64 * 64;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) slot[(dt * 16 + r) * 64 + lane] = O[dt][r] * f;
    }
    __syncthreads();
    if (ph == 0) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = O[dt][r] * f;
#pragma unroll
          for (int p2 = 1; p2 < R; ++p2) v += red[((size_t)((p2 - 1) * QT + qi) * 64 + dt * 16 + r) * 64 + lane];
          O[dt][r] = v;
        }
    }
  }

  const bool split = a.n_split > 1;
  const size_t slot = ((((size_t)g.i * a.Hq + h) * a.n_qt + qt) * a.n_split) + sp;  // (i, h, qt, s)
  if (ph == 0 && live) {
    if (!split) {
      // lane holds column q0 + lq, head-dim 32 dt + 8 (r / 4) + 4 hh + [0, 4)
      if (q0 + lq < g.nq) {
        const float inv = 1.f / Lsum;
        uint16_t* orow = (uint16_t*)a.out + (((size_t)g.i * a.fresh_rows + q0 + lq) * a.Hq + h) * kD;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            uint2 w;
            w.x = pack_bf16x2(O[dt][4 * r4 + 0] * inv, O[dt][4 * r4 + 1] * inv);
            w.y = pack_bf16x2(O[dt][4 * r4 + 2] * inv, O[dt][4 * r4 + 3] * inv);
            *(uint2*)(orow + 32 * dt + 8 * r4 + 4 * hh) = w;
          }
      }
    } else {
      const auto prs = make_rsrc(a.part + slot * kPartFloats);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          st_coherent_b128(prs, (lq * kD + 32 * dt + 8 * r4 + 4 * hh) * 4,
                           make_float4(O[dt][4 * r4], O[dt][4 * r4 + 1], O[dt][4 * r4 + 2], O[dt][4 * r4 + 3]));
      if (hh == 0) {
        st_coherent_b32(prs, (kQT * kD + lq) * 4, M);
        st_coherent_b32(prs, (kQT * kD + kQT + lq) * 4, Lsum);
      }
    }
  }
  if (!split) return;
  uint32_t* cnt = a.cnt + (((size_t)g.i * a.Hkv + g.hk) * a.n_grp + grp) * kCntStride;
  if (!block_arrive(cnt, (unsigned)g.n_act, &s_last)) return;

  // ---- last workgroup of this group: merge the n_act split partials of
  // each live query tile
  const int cq = tid >> 3;            // query row
#pragma unroll 1
  for (int t = 0; t < QT; ++t) {
    const int ut = grp * QT + t;
    const int hgt = ut / a.n_qt, qtt = ut % a.n_qt;
    if (ut >= a.g * a.n_qt || qtt >= n_live_qt) continue;
    const int ht = g.hk * a.g + hgt;
    const int q0t = qtt * kQT;
    if (q0t + cq >= g.nq) continue;
    const auto r = make_rsrc(uniform_ptr(a.part + (((size_t)g.i * a.Hq + ht) * a.n_qt + qtt) * a.n_split * kPartFloats));
    merge_partials(__builtin_amdgcn_readfirstlane(g.n_act), r, cq, tid & 7, c,
                   (uint16_t*)a.out + (((size_t)g.i * a.fresh_rows + q0t + cq) * a.Hq + ht) * kD);
  }
  if (tid == 0) *cnt = 0u;
}

// ------------------------------------------------------------------ bf16 MFMA, LDS ring, 8 waves
// The LDS ring above with 8 waves (512 threads) and one K/V tile per round
// shared by 8 query tiles, one per wave: a GQA group of up to 8 heads with
// one query tile each (DualCache) reads every K/V tile once for all its
// heads, and two waves per SIMD hide each other's latency.  Every wave
// moves 2 of a tile's 16 loads of 1 KB.  Split partials are stored with
// plain whole-line stores and merged by attn_merge_kernel (one launch
// later), so no workgroup has to read a whole group's partials.
constexpr int kGqaWaves = 8;
constexpr int kGqaThreads = 64 * kGqaWaves;
constexpr int kNumCUs = 256;  // MI355X compute units: one persistent 8-wave workgroup each
template <int NR>
__global__ __launch_bounds__(kGqaThreads, 1) void attn_gqa_kernel(AttnArgs a) {
  constexpr int QPW = kGqaWaves;                    // query tiles per workgroup
  constexpr int SET = 2 * kTileBytes;               // ring set: one tile of K then V
  constexpr int DPR = 2;                            // 1 KB loads per wave per round
  static_assert(NR == 4 || NR == 6 || NR == 8, "an even number of ring sets, at least four (the epilogue needs 64 KB)");
  // One array per ring set: the compiler then tells the sets apart, so its
  // LDS reads of one set are not held behind the LDS-DMA loads still in
  // flight into another, and it schedules them like any LDS load.
  __shared__ __attribute__((aligned(16))) uint8_t ring0[SET];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[SET];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[SET];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[SET];
  __shared__ __attribute__((aligned(16))) uint8_t ring4[NR > 4 ? SET : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ring5[NR > 4 ? SET : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ring6[NR > 6 ? SET : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ring7[NR > 6 ? SET : 16];
  auto set_ptr = [&](auto jc) __attribute__((always_inline)) -> uint8_t* {
    constexpr int J = decltype(jc)::value % NR;
    if constexpr (J == 0) return ring0;
    if constexpr (J == 1) return ring1;
    if constexpr (J == 2) return ring2;
    if constexpr (J == 3) return ring3;
    if constexpr (J == 4) return ring4;
    if constexpr (J == 5) return ring5;
    if constexpr (J == 6) return ring6;
    return ring7;
  };

  const int bid = blockIdx.x;
  const int item = (bid & 7) * a.per_xcd + (bid >> 3);
  if (item >= a.n_items) return;
  // item = ((i * Hkv + hk) * n_split + s) * n_grp + grp
  int rest = item;
  const int grp = rest % a.n_grp;
  rest /= a.n_grp;
  const int sp = rest % a.n_split;
  rest /= a.n_split;
  Geo g;
  g.hk = rest % a.Hkv;
  g.i = rest / a.Hkv;
  const int P = seq_prompt(a.sq, g.i);
  g.L = P + a.sq.G;
  fresh_range(a.mode, P, a.sq.G, a.sq.B, seq_block(a.sq, g.i), g.a0, g.a1);
  g.nq = g.a1 - g.a0;
  g.kb = sp * a.kchunk;
  g.ke = min(g.L, g.kb + a.kchunk);
  if (g.kb >= g.ke) return;                       // chunk past this sequence's keys
  const int T = a.g * a.n_qt;                     // query tiles of (i, hk), head-major
  const int n_live_qt = (g.nq + kQT - 1) / kQT;
  {
    bool any = false;
    for (int u = grp * QPW; u < min(T, grp * QPW + QPW); ++u) any |= (u % a.n_qt) < n_live_qt;
    if (!any) return;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lq = lane & 31, hh = lane >> 5;
  const int u = grp * QPW + wid;                  // this wave's query tile
  const int qt = u % a.n_qt;
  const bool live = u < T && qt < n_live_qt;
  const int h = g.hk * a.g + min(u / a.n_qt, a.g - 1);
  const int q0 = qt * kQT;
  const float c = a.scale_log2;

  const uint16_t* knp = (const uint16_t*)a.kn;
  const uint16_t* vnp = (const uint16_t*)a.vn;
  const uint16_t* kcp = (const uint16_t*)a.kc;
  const uint16_t* vcp = (const uint16_t*)a.vc;

  // Q as the B operand of S^T = K Q^T: lane (lq, hh) holds query row lq,
  // columns [16 ks + 8 hh, +8) for ks = 0..7.  Rows past nq are zero.
  bf16x8 qop[8];
  {
    const int r = q0 + lq;
    const uint16_t* qrow =
        (const uint16_t*)a.q + (((size_t)g.i * a.fresh_rows + max(min(r, g.nq - 1), 0)) * a.Hq + h) * kD;
    const bool rl = live && r < g.nq;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 w = *(const uint4*)(qrow + 16 * ks + 8 * hh);
      qop[ks] = as_bf16x8(rl ? w : make_uint4(0, 0, 0, 0));
    }
  }

  const int n_tiles = (g.ke - g.kb + kKT - 1) / kKT;

  // Tile q into ring set J: wave w moves rows 4 w + [0, 4) of K and of V
  // (one 1 KB load each); this lane moves one 16-byte chunk, the one that
  // belongs at its LDS position under the ring swizzle.  Rows past the
  // chunk re-read its last row (masked in the softmax), so every round
  // issues the same loads and the counter waits below are exact.
  const int row_a = 4 * wid + (lane >> 4);
  const int chunk_a = (lane & 15) ^ ring_swizzle(row_a);
  const uint32_t off_c = (uint32_t)(row_a * 256 + 16 * chunk_a);
  const uint32_t off_f = (uint32_t)(row_a * a.Hkv * 256 + 16 * chunk_a);
  const size_t fstride = (size_t)a.Hkv * 256;
  const char* kc_row0 = (const char*)kcp + ((size_t)g.i * a.Hkv + g.hk) * a.sq.Lcap * 256;
  const char* kf_row0 = (const char*)knp + ((size_t)g.i * a.fresh_rows * a.Hkv + g.hk) * 256;
  const long long dvc = (const char*)vcp - (const char*)kcp, dvf = (const char*)vnp - (const char*)knp;
  typedef __attribute__((address_space(3))) void* LdsV;
  auto issue = [&](int q, auto jc) __attribute__((always_inline)) {
    // The destination as a plain LDS address, hidden from alias analysis:
    // the compiler otherwise takes the reads of the other ring sets in this
    // round as depending on these loads and waits for all of them (the
    // explicit waits order every hand-off)
    uint32_t dst = lds_addr(set_ptr(jc)) + wid * 1024;
    asm volatile("" : "+s"(dst));
    const LdsV dk = (LdsV)(uintptr_t)dst, dv = (LdsV)(uintptr_t)(dst + kTileBytes);
    const int t0 = g.kb + q * kKT;
    // (branch-free tests: a whole tile is in the cache unless it overlaps
    // [a0, a1), and in the fresh rows if it lies inside [a0, a1))
    const bool whole = t0 + kKT <= g.ke;
    const bool overlaps = (unsigned)(t0 - (g.a0 - kKT + 1)) < (unsigned)(g.a1 - g.a0 + kKT - 1);
    const bool inside = (g.a1 - g.a0 >= kKT) & ((unsigned)(t0 - g.a0) <= (unsigned)(g.a1 - g.a0 - kKT));
    const bool in_cache = whole & !overlaps;
    if (whole & (!overlaps | inside)) {
      const char* kt = in_cache ? kc_row0 + ((size_t)(uint32_t)t0 << 8) : kf_row0 + (size_t)(uint32_t)(t0 - g.a0) * fstride;
      const char* vt = kt + (in_cache ? dvc : dvf);
      const uint32_t off = in_cache ? off_c : off_f;
      __builtin_amdgcn_global_load_lds(kt + off, dk, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vt + off, dv, 16, 0, 0);
    } else {
      const int j = min(t0 + row_a, g.ke - 1);
      __builtin_amdgcn_global_load_lds((const char*)kv_row(a, knp, kcp, g, j, kD) + 16 * chunk_a, dk, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const char*)kv_row(a, vnp, vcp, g, j, kD) + 16 * chunk_a, dv, 16, 0, 0);
    }
  };

  f32x16 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;  // exponent reference and sum per column

  // operand addresses within a tile (as in the LDS ring kernel)
  uint32_t k_off[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) k_off[ks] = (uint32_t)(lq * 256 + 16 * ((2 * ks + hh) ^ ring_swizzle(lq)));
  uint32_t vt_off[8];
  {
    const int G = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = 4 * (G >> 1) + (sl >> 2) + 8 * hi;
        const int col = 32 * dt + 16 * (G & 1) + 4 * (sl & 3);
        vt_off[2 * dt + hi] = (uint32_t)(r * 256 + 16 * ((col >> 3) ^ ring_swizzle(r)) + 8 * ((col >> 2) & 1));
      }
  }

  // K operands as plain LDS loads and V^T operands with the transpose-read
  // builtin: the compiler waits for them (lgkmcnt) itself.  All eight K
  // reads go out before the first product (the empty asm statements keep
  // the compiler from interleaving them with the products), so their
  // latency is paid once, and the eight products accumulate in one chain.
  auto stage_s = [&](const uint8_t* tb, f32x16& S) __attribute__((always_inline)) {
    bf16x8 kop[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kop[ks] = as_bf16x8(*(const uint4*)(tb + k_off[ks]));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(kop[ks]));
    S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[0], qop[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < 8; ++ks) S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[ks], S, 0, 0, 0);
  };

  auto stage_pv = [&](const uint8_t* tb, int t0, f32x16& S) __attribute__((always_inline)) {
    bf16x8 vop[2][4];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        typedef __attribute__((address_space(3))) short4v* LdsS4;
        const uint8_t* vb = tb + kTileBytes + 16 * 256 * k2;
        const short4v t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsS4)(vb + vt_off[2 * dt]));
        const short4v t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsS4)(vb + vt_off[2 * dt + 1]));
        __builtin_memcpy(&vop[k2][dt], &t0, 8);
        __builtin_memcpy((char*)&vop[k2][dt] + 8, &t1, 8);
      }
    if (t0 + kKT > g.ke) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = t0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= g.ke) S[r] = -INFINITY;
      }
    }
    bf16x8 pop[2];
    softmax_tile(S, c, m_ref, l_run, O, pop);
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[k2][dt], pop[k2], O[dt], 0, 0, 0);
  };

  // the LDS ring kernel's pipeline with one tile per round: step q waits
  // until tile q + 1 is in, meets at the barrier, refills the set tile
  // q - 1 used, starts S^T of tile q + 1 and finishes tile q.  S^T of tile
  // q sits in Sb[q % 2] (the loop body has an even number of steps, so the
  // index is known at compile time and nothing is copied).
  f32x16 Sb[2] = {f32x16{}, f32x16{}};
  auto step = [&](int q, auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    wait_vm<(NR - 3) * DPR, true>();
    ring_barrier();
    issue(q + NR - 1, std::integral_constant<int, (J + NR - 1) % NR>{});
    if (live && q + 1 < n_tiles) stage_s(set_ptr(std::integral_constant<int, (J + 1) % NR>{}), Sb[(J + 1) & 1]);
    if (live && q < n_tiles) stage_pv(set_ptr(jc), g.kb + q * kKT, Sb[J & 1]);
  };
  issue(0, std::integral_constant<int, 0>{});
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qop[ks]));
  issue(1, std::integral_constant<int, 1>{});
  issue(2, std::integral_constant<int, 2>{});
  if constexpr (NR > 4) issue(3, std::integral_constant<int, 3>{});
  if constexpr (NR > 5) issue(4, std::integral_constant<int, 4>{});
  if constexpr (NR > 6) issue(5, std::integral_constant<int, 5>{});
  if constexpr (NR > 7) issue(6, std::integral_constant<int, 6>{});
  wait_vm<(NR - 2) * DPR, true>();
  ring_barrier();
  if (live) stage_s(ring0, Sb[0]);
  for (int q = 0; q < n_tiles; q += NR) {
    step(q, std::integral_constant<int, 0>{});
    step(q + 1, std::integral_constant<int, 1>{});
    step(q + 2, std::integral_constant<int, 2>{});
    step(q + 3, std::integral_constant<int, 3>{});
    if constexpr (NR > 4) step(q + 4, std::integral_constant<int, 4>{});
    if constexpr (NR > 5) step(q + 5, std::integral_constant<int, 5>{});
    if constexpr (NR > 6) step(q + 6, std::integral_constant<int, 6>{});
    if constexpr (NR > 7) step(q + 7, std::integral_constant<int, 7>{});
  }
  wait_vm<0, true>();
  ring_barrier();
  if (!live) return;

  const float l_col = xor_combine<32>(l_run, [](float x, float y) { return x + y; });
  if (a.n_split == 1) {
    // lane holds column q0 + lq, head-dim 32 dt + 8 (r / 4) + 4 hh + [0, 4)
    if (q0 + lq < g.nq) {
      const float inv = 1.f / l_col;
      uint16_t* orow = (uint16_t*)a.out + (((size_t)g.i * a.fresh_rows + q0 + lq) * a.Hq + h) * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          uint2 w;
          w.x = pack_bf16x2(O[dt][4 * r4 + 0] * inv, O[dt][4 * r4 + 1] * inv);
          w.y = pack_bf16x2(O[dt][4 * r4 + 2] * inv, O[dt][4 * r4 + 3] * inv);
          *(uint2*)(orow + 32 * dt + 8 * r4 + 4 * hh) = w;
        }
    }
    return;
  }
  // Partial (O, m, l) relative to the tile's exponent reference, O in fp16
  // with a power-of-two scale per query row (O = scale * stored): the row's
  // largest |O| is stored in [2^14, 2^15), so no value overflows and every
  // value keeps fp16's 11 significant bits, half the bytes of fp32.  O goes
  // through 8 KB of LDS per wave so that each global store writes four whole
  // 256-byte rows.
  float amax = 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(O[dt][r]));
  amax = xor_combine<32>(amax, [](float x, float y) { return fmaxf(x, y); });
  const int e = __builtin_amdgcn_frexp_expf(amax) - 15;  // amax < 2^(e + 15)
  uint8_t* part = (uint8_t*)a.part + (((((size_t)g.i * a.Hq + h) * a.n_qt + qt) * a.n_split + sp) * kPart16Bytes);
  // wave w: half w % 2 of ring set w / 2
  uint8_t* wset = (wid >> 1) == 0 ? ring0 : (wid >> 1) == 1 ? ring1 : (wid >> 1) == 2 ? ring2 : ring3;
  uint8_t* wbuf = wset + (wid & 1) * 8192;
  // lane (lq, hh) holds row lq, head dims 32 dt + 8 q4 + 4 hh + [0, 4): half
  // of the row's 16-byte unit 4 dt + q4, placed at unit ^ (lq & 15)
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      uint2 w;
      w.x = pack_f16x2(__builtin_amdgcn_ldexpf(O[dt][4 * q4], -e), __builtin_amdgcn_ldexpf(O[dt][4 * q4 + 1], -e));
      w.y = pack_f16x2(__builtin_amdgcn_ldexpf(O[dt][4 * q4 + 2], -e), __builtin_amdgcn_ldexpf(O[dt][4 * q4 + 3], -e));
      *(uint2*)(wbuf + lq * 256 + 16 * ((4 * dt + q4) ^ (lq & 15)) + 8 * hh) = w;
    }
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int row = 4 * v + (lane >> 4), k = lane & 15;
    *(uint4*)(part + row * 256 + 16 * k) = *(const uint4*)(wbuf + row * 256 + 16 * (k ^ (row & 15)));
  }
  if (hh == 0) {
    float* hdr = (float*)(part + kQT * kD * 2);
    hdr[lq] = m_ref;
    hdr[kQT + lq] = l_col;
    hdr[2 * kQT + lq] = __builtin_amdgcn_ldexpf(1.f, e);
  }
}

// Merge the key-chunk partials written by attn_gqa_kernel in the launch
// before: workgroup (query tile x 2 + column half, query head, sequence)
// merges 64 head-dim columns of the tile's 32 rows, so the partial reads
// spread over twice as many workgroups as query tiles.
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(AttnArgs a) {
  const int qt = blockIdx.x >> 1, half = blockIdx.x & 1, h = blockIdx.y, i = blockIdx.z;
  const int P = seq_prompt(a.sq, i);
  const int L = P + a.sq.G;
  int a0, a1;
  fresh_range(a.mode, P, a.sq.G, a.sq.B, seq_block(a.sq, i), a0, a1);
  const int nq = a1 - a0;
  const int q0 = qt * kQT;
  if (q0 >= nq) return;
  const int n_act = __builtin_amdgcn_readfirstlane((L + a.kchunk - 1) / a.kchunk);
  const auto r = make_rsrc(
      uniform_ptr((const uint8_t*)a.part + (((size_t)i * a.Hq + h) * a.n_qt + qt) * a.n_split * kPart16Bytes));
  const int tid = threadIdx.x;
  const int cq = tid >> 3, j = tid & 7, c0 = 64 * half;
  if (q0 + cq >= nq) return;
  uint16_t* orow = (uint16_t*)a.out + (((size_t)i * a.fresh_rows + q0 + cq) * a.Hq + h) * kD;
  const float c = a.scale_log2;
  switch (n_act) {
    case 1: merge_partials16_n<1, 1>(r, cq, j, c, orow, c0); break;
    case 2: merge_partials16_n<2, 1>(r, cq, j, c, orow, c0); break;
    case 3: merge_partials16_n<3, 1>(r, cq, j, c, orow, c0); break;
    case 4: merge_partials16_n<4, 1>(r, cq, j, c, orow, c0); break;
    case 5: merge_partials16_n<5, 1>(r, cq, j, c, orow, c0); break;
    case 6: merge_partials16_n<6, 1>(r, cq, j, c, orow, c0); break;
    case 7: merge_partials16_n<7, 1>(r, cq, j, c, orow, c0); break;
    default: merge_partials16_n<8, 1>(r, cq, j, c, orow, c0); break;
  }
}

// ------------------------------------------------------------------ bf16 MFMA, 8-wave ring over a stream of tiles
// The 8-wave ring for DualCache GQA batches (one query tile per head), with
// the key tiles of the whole batch dealt evenly over a persistent grid.  The
// tiles of sequence i's KV head hk form segment (i, hk), n_i = ceil(L_i / 32)
// tiles long; the segments laid end to end (sequence-major, KV head within
// a sequence) are cut into gridDim.x equal ranges, one per workgroup.  A
// ragged batch (prompts of 256 to 4096 tokens) then costs every workgroup
// the same number of tiles instead of the longest sequence's.  A workgroup
// walks the segments its range touches: a segment wholly inside the range
// is written to the output directly; a segment cut by range edges is
// computed in parts, whose (O, m, l) partials (the fp16 format of the
// split-key kernel, written through to the device coherence point) go to
// two slots per workgroup in the workspace, and the part that arrives last
// merges them in a fixed order.  Every workgroup derives the partition from
// the prompt lengths itself, so the call stays one launch with no host pass.
// Tiles of sequence i's segment in the tile stream: ceil(L_i / 32) rounded
// up to a multiple of 4, so that segments and ranges start on 4-tile
// boundaries (the padding tiles hold no keys: their loads re-read the
// segment's last row and their compute is skipped).
constexpr int kStreamQuad = 4;
__device__ __forceinline__ int seq_tiles_sq(const SeqArgs& sq, int i) {
  const int n = (seq_prompt(sq, i) + sq.G + kKT - 1) / kKT;
  return (n + kStreamQuad - 1) / kStreamQuad * kStreamQuad;
}
__device__ __forceinline__ int seq_tiles(const AttnArgs& a, int i) {
  const int n = (seq_prompt(a.sq, i) + a.sq.G + kKT - 1) / kKT;
  return (n + kStreamQuad - 1) / kStreamQuad * kStreamQuad;
}
__device__ __forceinline__ int wave_scan_incl(int v) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}
// A value the caller knows to be the same in every lane, moved to scalar
// registers (so that what is computed from it stays scalar: branches,
// per-sequence lookups as scalar loads).
__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long uniform_ll(long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(unsigned long long)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}
// The stream: each segment (sequence, KV head) is its tiles padded to whole
// quads of 4, after kStreamPhantom units that stand for the fixed cost of
// entering and finishing a segment (a segment switch costs about as much as
// a quad of tiles), so that the ranges balance work rather than tile counts.
// The ranges are cut in whole quads: with TQ = T / 4 quads of the stream,
// range u is quads [u TQ / G, (u + 1) TQ / G).  stream_lo is a range's
// first unit; stream_owner the range holding unit x.
constexpr int kStreamPhantom = 4;
__device__ __forceinline__ long long stream_lo(int u, long long T, int G) {
  return (long long)u * (T / kStreamQuad) / G * kStreamQuad;
}
__device__ __forceinline__ int stream_owner(long long x, long long T, int G) {
  const long long xq = x / kStreamQuad, TQ = T / kStreamQuad;
  return (int)((xq * G + G - 1) / TQ);
}

// A workgroup's place in its tile range: the segment (sequence i, KV head
// hk), the tile t within it, this workgroup's part of the segment [tb, te),
// the tiles of the range left from t on (0: past the range), and the
// segment's geometry.  Wave-uniform.
struct StreamCursor {
  int i, hk, t, tb, te, n;
  int left;
  int L, a0, a1, ke;
  const char *kc, *kf;  // row 0 of the segment's cached and fresh K
  long long dvc, dvf;   // V minus K: the same rows of the cached and fresh V
};

template <int NR, bool LOADER>
__global__ __launch_bounds__(kGqaThreads, 1) void attn_gqa_stream_kernel(AttnArgs a) {
  constexpr int SET = 2 * kTileBytes;
  constexpr int NLD = LOADER ? 8 : 1;  // four-row groups of a tile one loading wave moves
  constexpr int DPR = 2 * NLD;         // ring loads per loading wave per tile
  constexpr int QLD = 8;               // Q-prefetch loads per wave (32 rows x 256 bytes)
  constexpr int kLoaderWave = kGqaWaves - 1;
  static_assert(NR == 4, "four ring sets");
  // (the ring sets' larger alignment places them first, in the low 64 KB of
  // LDS, where their base fits a read's immediate offset)
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[SET];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[SET];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[SET];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[SET];
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kGqaWaves * kQT * 256];  // each wave's next Q tile
  __shared__ __attribute__((aligned(16))) uint8_t q_sink[LOADER ? 16 : kGqaWaves * 1024];  // never read (see prefetch_none)
  __shared__ __attribute__((aligned(16))) uint8_t o_stage[LOADER ? kGqaWaves * 4096 : 16];  // finish's staging
  auto set_ptr = [&](auto jc) __attribute__((always_inline)) -> uint8_t* {
    constexpr int J = decltype(jc)::value % NR;
    if constexpr (J == 0) return ring0;
    if constexpr (J == 1) return ring1;
    if constexpr (J == 2) return ring2;
    return ring3;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lq = lane & 31, hh = lane >> 5;
  // XCD-aware: blockIdx.x is dealt round-robin over the 8 XCDs; give each
  // XCD a contiguous run of ranges
  const int w = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  // the arguments the loop reads, as plain scalars (reads through the
  // argument block inside the loop would each wait for every load in flight)
  const int32_t* plens = a.sq.plens;
  const int32_t* bidxp = a.sq.bidx;
  const int b = a.sq.b, Pu = a.sq.P, Ku = a.sq.k, Gl = a.sq.G, Bl = a.sq.B, Lcap = a.sq.Lcap;
  const int Hkv = a.Hkv, Hq = a.Hq, gg = a.g, fresh_rows = a.fresh_rows, mode = a.mode;
  const float c = a.scale_log2;
  const uint16_t* qp = (const uint16_t*)a.q;
  uint16_t* outp = (uint16_t*)a.out;
  uint8_t* partp = (uint8_t*)a.part;
  // per-sequence lookups, uniform (the sequence index is)
  // (scalar loads through the constant address space: they wait on the
  // scalar counter only, not on the ring's loads in flight)
  typedef const __attribute__((address_space(4))) int32_t* ConstI32;
  auto prompt_of = [&](int i) __attribute__((always_inline)) -> int {
    return plens ? ((ConstI32)plens)[uniform_i(i)] : Pu;
  };
  auto block_of = [&](int i) __attribute__((always_inline)) -> int {
    return bidxp ? ((ConstI32)bidxp)[uniform_i(i)] : Ku;
  };
  auto tiles_of_len = [](int L) -> int { return (L + kKT * kStreamQuad - 1) / (kKT * kStreamQuad) * kStreamQuad; };

  // ---- the partition (every wave computes it; the results are uniform).
  // With fewer quads than workgroups only the first TQ take part, so every
  // range holds at least one quad and consecutive owners of a segment's
  // tiles are consecutive workgroups (attn_stream_merge_kernel's part count
  // relies on it); a range of phantom units alone has no tiles.
  // (the first 64 sequences' lengths are loaded once for both passes)
  const int n_first = lane < b ? tiles_of_len((plens ? plens[lane] : Pu) + Gl) + kStreamPhantom : 0;
  long long total = 0;
  for (int i0 = 0; i0 < b; i0 += 64) {
    const int n = i0 == 0 ? n_first : i0 + lane < b ? tiles_of_len((plens ? plens[i0 + lane] : Pu) + Gl) + kStreamPhantom : 0;
    total += __shfl(wave_scan_incl(n), 63, 64);
  }
  const long long T = uniform_ll(total * a.Hkv);
  const long long TQ = T / kStreamQuad;
  const int Gn = (int)((long long)gridDim.x < TQ ? (long long)gridDim.x : TQ);
  if (w >= Gn) return;
  const long long lo = stream_lo(w, T, Gn), hi = stream_lo(w + 1, T, Gn);
  // the sequences holding units lo and hi - 1, and the stream index of
  // their first units
  int i_lo = 0, i_hi = 0;
  long long base = 0, base_hi = 0;
  {
    long long acc = 0;
    bool found_lo = false;
    for (int i0 = 0; i0 < b; i0 += 64) {
      const bool in = i0 + lane < b;
      const int n = i0 == 0 ? n_first : in ? tiles_of_len((plens ? plens[i0 + lane] : Pu) + Gl) + kStreamPhantom : 0;
      const int incl = wave_scan_incl(n);
      const uint64_t m_lo = __ballot(in && acc + (long long)Hkv * incl > lo);
      if (!found_lo && m_lo) {
        const int f = __ffsll((unsigned long long)m_lo) - 1;
        i_lo = i0 + f;
        base = acc + (long long)Hkv * __shfl(incl - n, f, 64);
        found_lo = true;
      }
      const uint64_t m_hi = __ballot(in && acc + (long long)Hkv * incl > hi - 1);
      if (m_hi) {
        const int f = __ffsll((unsigned long long)m_hi) - 1;
        i_hi = i0 + f;
        base_hi = acc + (long long)Hkv * __shfl(incl - n, f, 64);
        break;
      }
      acc += (long long)Hkv * __shfl(incl, 63, 64);
    }
  }

  // segment geometry of a cursor that has just entered segment (i, hk) at tile t
  auto enter = [&](StreamCursor& cu) __attribute__((always_inline)) {
    const int P = prompt_of(cu.i);
    cu.L = P + Gl;
    fresh_range(mode, P, Gl, Bl, block_of(cu.i), cu.a0, cu.a1);
    cu.n = tiles_of_len(cu.L);
    cu.tb = cu.t;
    cu.te = min(cu.n, cu.t + cu.left);
    cu.ke = max(min(cu.L, cu.te * kKT), cu.tb * kKT + 1);  // at least one key row to clamp to
    const size_t cb = ((size_t)cu.i * Hkv + cu.hk) * Lcap * 256;
    const size_t fb = ((size_t)cu.i * fresh_rows * Hkv + cu.hk) * 256;
    cu.kc = (const char*)a.kc + cb;
    cu.kf = (const char*)a.kn + fb;
    cu.dvc = (const char*)a.vc - (const char*)a.kc;
    cu.dvf = (const char*)a.vn - (const char*)a.kn;
  };
  // one tile on: past the part's end the cursor enters the next segment
  // (while the range lasts; past it, it stays on its last tile)
  auto advance = [&](StreamCursor& cu) __attribute__((always_inline)) {
    if (cu.left <= 1) {
      cu.left = 0;
      return;
    }
    --cu.left;
    if (++cu.t == cu.te) {
      cu.t = 0;
      if (++cu.hk == Hkv) {
        cu.hk = 0;
        ++cu.i;
      }
      enter(cu);
    }
  };
  i_lo = uniform_i(i_lo);
  i_hi = uniform_i(i_hi);
  base = uniform_ll(base);
  base_hi = uniform_ll(base_hi);
  StreamCursor ic;  // issue cursor, three tiles ahead of the compute cursor
  {
    const int nv0 = tiles_of_len(prompt_of(i_lo) + Gl) + kStreamPhantom;
    const int nv1 = tiles_of_len(prompt_of(i_hi) + Gl) + kStreamPhantom;
    const int o = (int)((lo - base) % nv0);  // a multiple of 4: 0 is the phantom quad
    ic.i = i_lo;
    ic.hk = (int)((lo - base) / nv0);
    ic.t = o < kStreamPhantom ? 0 : o - kStreamPhantom;
    // the range's tiles: its units less the phantoms of the segments that
    // start in it (those after the first segment's, and that one's if the
    // range starts at it)
    const int seg_lo = i_lo * Hkv + ic.hk, seg_hi = i_hi * Hkv + (int)((hi - 1 - base_hi) / nv1);
    ic.left = (int)(hi - lo) - kStreamPhantom * (seg_hi - seg_lo + (o == 0 ? 1 : 0));
  }
  if (ic.left <= 0) return;  // phantom units alone
  enter(ic);
  StreamCursor cc = ic;  // compute cursor
  const int n_quads = ic.left / NR;

  // K/V tile at the issue cursor into ring set J, as 1 KB LDS-DMA loads of
  // four rows each: row group v is rows 4 v + [0, 4) of K and of V, and this
  // lane moves the 16-byte chunk that belongs at its LDS position under the
  // ring swizzle.  Wave w moves group w; with a loader wave, that wave moves
  // all eight.  Rows past the part (and every tile once the cursor is past
  // the range) re-read the part's last row, so every step issues the same
  // loads.
  const size_t fstride = (size_t)Hkv * 256;
  typedef __attribute__((address_space(3))) void* LdsV;
  auto issue_tile = [&](auto jc, int tile) __attribute__((always_inline)) {
    // The destination as a plain LDS address, hidden from alias analysis:
    // the compiler otherwise takes the reads of the other ring sets in this
    // step as depending on these loads and waits for all of them (the
    // explicit waits order every hand-off)
    uint32_t dst = lds_addr(set_ptr(jc)) + (LOADER ? 0 : wid * 1024);
    asm volatile("" : "+s"(dst));
    const int t0 = tile * kKT;
    // (branch-free tests: a whole tile is in the cache unless it overlaps
    // [a0, a1), and in the fresh rows if it lies inside [a0, a1))
    const bool whole = t0 + kKT <= ic.ke;
    const bool overlaps = (unsigned)(t0 - (ic.a0 - kKT + 1)) < (unsigned)(ic.a1 - ic.a0 + kKT - 1);
    const bool inside = (ic.a1 - ic.a0 >= kKT) & ((unsigned)(t0 - ic.a0) <= (unsigned)(ic.a1 - ic.a0 - kKT));
    const bool in_cache = whole & !overlaps;
    if (whole & (!overlaps | inside)) {
      const char* kt = in_cache ? ic.kc + ((size_t)(uint32_t)t0 << 8) : ic.kf + (size_t)(uint32_t)(t0 - ic.a0) * fstride;
      const char* vt = kt + (in_cache ? ic.dvc : ic.dvf);
#pragma unroll
      for (int v = 0; v < NLD; ++v) {
        const int row = 4 * (LOADER ? v : wid) + (lane >> 4);
        const int chunk = (lane & 15) ^ ring_swizzle(row);
        const uint32_t off = (uint32_t)(row * (in_cache ? 256 : Hkv * 256) + 16 * chunk);
        __builtin_amdgcn_global_load_lds(kt + off, (LdsV)(uintptr_t)(dst + v * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + off, (LdsV)(uintptr_t)(dst + v * 1024 + kTileBytes), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int v = 0; v < NLD; ++v) {
        const int row = 4 * (LOADER ? v : wid) + (lane >> 4);
        const int chunk = (lane & 15) ^ ring_swizzle(row);
        const int j = min(t0 + row, ic.ke - 1);
        const bool fr = (unsigned)(j - ic.a0) < (unsigned)(ic.a1 - ic.a0);
        const char* kt = fr ? ic.kf + (size_t)(uint32_t)(j - ic.a0) * fstride : ic.kc + ((size_t)(uint32_t)j << 8);
        const char* vt = kt + (fr ? ic.dvf : ic.dvc);
        __builtin_amdgcn_global_load_lds(kt + 16 * chunk, (LdsV)(uintptr_t)(dst + v * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + 16 * chunk, (LdsV)(uintptr_t)(dst + v * 1024 + kTileBytes), 16, 0, 0);
      }
    }
  };
  auto issue = [&](auto jc) __attribute__((always_inline)) {
    issue_tile(jc, ic.left > 0 ? ic.t : ic.te - 1);
  };
  // This wave's Q tile of the segment after the compute cursor's current one
  // (query head hk * g + wid of that segment) into its 8 KB of q_lds: row r
  // of the tile, 16-byte chunk k at chunk k ^ (r & 15) (conflict-free reads
  // below); rows past the block re-read its last row (zeroed on reading).
  // QLD loads per wave, whatever the wave or segment.
  auto prefetch_q = [&](int i, int hk) __attribute__((always_inline)) {
    const int P = prompt_of(i);
    int a0, a1;
    fresh_range(mode, P, Gl, Bl, block_of(i), a0, a1);
    const int nq = a1 - a0;
    const int h = hk * gg + min(wid, gg - 1);
    uint8_t* dst = q_lds + wid * (kQT * 256);
    // (the lane's offsets are recomputed here rather than kept live across
    // the loop: a uniform base plus a 32-bit lane offset per load)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const char* qb = (const char*)(qp + ((size_t)i * fresh_rows * Hq + h) * kD);
#pragma unroll
    for (int v = 0; v < QLD; ++v) {
      const int r = 4 * v + (ln >> 4);
      const int k = (ln & 15) ^ (r & 15);
      const uint32_t off = (uint32_t)(max(min(r, nq - 1), 0) * Hq * kD * 2 + 16 * k);
      __builtin_amdgcn_global_load_lds(qb + off, dst + v * 1024, 16, 0, 0);
    }
  };
  // The same number of loads with next to nothing to fetch: every lane
  // copies the first byte of Q into this wave's part of q_sink.  Every quad
  // of steps issues QLD Q-side loads per wave, a prefetch or these, so the
  // count of loads in flight at each wait is the same on every path.
  auto prefetch_none = [&]() __attribute__((always_inline)) {
    uint8_t* dst = q_sink + wid * 1024;
#pragma unroll
    for (int v = 0; v < QLD; ++v) __builtin_amdgcn_global_load_lds((const char*)qp, dst, 1, 0, 0);
  };
  // Q as the B operand of S^T = K Q^T from q_lds: lane (lq, hh) holds query
  // row lq, columns [16 ks + 8 hh, +8) for ks = 0..7; rows past nq are zero
  bf16x8 qop[8];
  auto read_q = [&](int nq) __attribute__((always_inline)) {
    const uint8_t* src = q_lds + wid * (kQT * 256) + lq * 256;
    const bool rl = lq < nq;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 v = *(const uint4*)(src + 16 * ((2 * ks + hh) ^ (lq & 15)));
      qop[ks] = as_bf16x8(rl ? v : make_uint4(0, 0, 0, 0));
    }
  };

  // operand addresses within a tile (as in the LDS ring kernel)
  uint32_t k_off[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) k_off[ks] = (uint32_t)(lq * 256 + 16 * ((2 * ks + hh) ^ ring_swizzle(lq)));
  uint32_t vt_off[8];
  {
    const int G = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int hi2 = 0; hi2 < 2; ++hi2) {
        const int r = 4 * (G >> 1) + (sl >> 2) + 8 * hi2;
        const int col = 32 * dt + 16 * (G & 1) + 4 * (sl & 3);
        vt_off[2 * dt + hi2] = (uint32_t)(r * 256 + 16 * ((col >> 3) ^ ring_swizzle(r)) + 8 * ((col >> 2) & 1));
      }
  }

  const bool live = wid < gg;  // wave wid owns query head hk * g + wid
  f32x16 O[4];
  float m_ref, l_run;
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
    m_ref = -INFINITY;
    l_run = 0.f;
  };
  reset();

  auto stage_s = [&](const uint8_t* tb, f32x16& S) __attribute__((always_inline)) {
    bf16x8 kop[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kop[ks] = as_bf16x8(*(const uint4*)(tb + k_off[ks]));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(kop[ks]));
    S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[0], qop[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < 8; ++ks) S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[ks], S, 0, 0, 0);
  };
  auto stage_pv = [&](const uint8_t* tb, int t0, int ke, f32x16& S) __attribute__((always_inline)) {
    bf16x8 vop[2][4];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        typedef __attribute__((address_space(3))) short4v* LdsS4;
        const uint8_t* vb = tb + kTileBytes + 16 * 256 * k2;
        const short4v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsS4)(vb + vt_off[2 * dt]));
        const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsS4)(vb + vt_off[2 * dt + 1]));
        __builtin_memcpy(&vop[k2][dt], &v0, 8);
        __builtin_memcpy((char*)&vop[k2][dt] + 8, &v1, 8);
      }
    if (t0 + kKT > ke) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = t0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= ke) S[r] = -INFINITY;
      }
    }
    bf16x8 pop[2];
    softmax_tile(S, c, m_ref, l_run, O, pop);
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[k2][dt], pop[k2], O[dt], 0, 0, 0);
  };

  // The end of the compute cursor's part: the output rows when the part is
  // the whole segment, else the partial (O, m, l: fp16 O with a power-of-two
  // row scale) in slot (w, first ? 0 : 1): a workgroup's first segment holds
  // its range start, a later cut segment its range end.  Lane (lq, hh) holds
  // row lq, head dims 32 dt + 8 q4 + 4 hh + [0, 4).  With a loader wave, O
  // goes through this wave's 4 KB of o_stage, half the head dims at a time
  // (16-byte unit 4 (dt % 2) + q4 of the 128-byte half row at unit ^ (lq &
  // 7)), so that each global store writes eight whole 128-byte half rows;
  // stores straight from the accumulator layout touch 32 rows each.
  auto finish = [&](bool first) __attribute__((always_inline)) {
    if (!live) return;
    const int h = cc.hk * gg + wid;
    const int nq = cc.a1 - cc.a0;
    const float l_col = xor_combine<32>(l_run, [](float x, float y) { return x + y; });
    const bool whole = cc.tb == 0 && cc.te == cc.n;
    float inv = 0.f;
    int e = 0;
    if (whole) {
      inv = 1.f / l_col;
    } else {
      float amax = 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(O[dt][r]));
      amax = xor_combine<32>(amax, [](float x, float y) { return fmaxf(x, y); });
      e = __builtin_amdgcn_frexp_expf(amax) - 15;  // amax < 2^(e + 15)
    }
    // four values of O as 8 bytes: bf16 O / l, or fp16 O 2^-e
    auto pack4 = [&](int dt, int q4) __attribute__((always_inline)) -> uint2 {
      uint2 u;
      if (whole) {
        u.x = pack_bf16x2(O[dt][4 * q4 + 0] * inv, O[dt][4 * q4 + 1] * inv);
        u.y = pack_bf16x2(O[dt][4 * q4 + 2] * inv, O[dt][4 * q4 + 3] * inv);
      } else {
        u.x = pack_f16x2(__builtin_amdgcn_ldexpf(O[dt][4 * q4], -e), __builtin_amdgcn_ldexpf(O[dt][4 * q4 + 1], -e));
        u.y = pack_f16x2(__builtin_amdgcn_ldexpf(O[dt][4 * q4 + 2], -e), __builtin_amdgcn_ldexpf(O[dt][4 * q4 + 3], -e));
      }
      return u;
    };
    uint16_t* obase = outp + ((size_t)cc.i * fresh_rows * Hq + h) * kD;
    uint8_t* part = partp + ((size_t)(2 * w + (first ? 0 : 1)) * kGqaWaves + wid) * kPart16Bytes;
    if constexpr (LOADER) {
      uint8_t* wbuf = o_stage + wid * 4096;
#pragma unroll
      for (int hd = 0; hd < 2; ++hd) {
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *(uint2*)(wbuf + lq * 128 + 16 * ((4 * d2 + q4) ^ (lq & 7)) + 8 * hh) = pack4(2 * hd + d2, q4);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // (the reads below are of other lanes' writes)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 8 * v + (lane >> 3), k = lane & 7;
          const uint4 x = *(const uint4*)(wbuf + row * 128 + 16 * (k ^ (row & 7)));
          if (whole) {
            if (row < nq) *(uint4*)(obase + (size_t)row * Hq * kD + 64 * hd + 8 * k) = x;
          } else {
            *(uint4*)(part + row * 256 + 128 * hd + 16 * k) = x;
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read back before the next half is written
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint2 u = pack4(dt, q4);
          if (whole) {
            if (lq < nq) *(uint2*)(obase + (size_t)lq * Hq * kD + 32 * dt + 8 * q4 + 4 * hh) = u;
          } else {
            *(uint2*)(part + lq * 256 + 2 * (32 * dt + 8 * q4 + 4 * hh)) = u;
          }
        }
    }
    if (!whole && hh == 0) {
      float* hdr = (float*)(part + kQT * kD * 2);
      hdr[lq] = m_ref;
      hdr[kQT + lq] = l_col;
      hdr[2 * kQT + lq] = __builtin_amdgcn_ldexpf(1.f, e);
    }
  };

  // ---- the pipeline.  Step x (the compute cursor's tile): wait until tile
  // x + 1 is in (later tiles may stay in flight), barrier, refill the ring
  // set tile x - 1 used with the issue cursor's tile x + 3, start S^T of
  // tile x + 1 when it is in the same segment, finish tile x (softmax and
  // P V).  After each quad of steps: at the end of a segment part, write its
  // output or partial, take the next segment's Q from q_lds and start S^T of
  // its first tile; then QLD Q-side loads (the following segment's Q when a
  // segment has just been entered, else prefetch_none).  Those loads are
  // younger than tiles x + 1 and x + 2 at the first two steps of a quad (the
  // waits there leave them in flight) and older than the tiles waited for at
  // the last two, so a prefetch has landed one quad after it was issued, and
  // a segment part spans at least one quad.
  f32x16 Sb[2] = {f32x16{}, f32x16{}};
  bool first = true;  // the compute cursor is in this workgroup's first segment
  // the segment after the compute cursor's current one (if the range reaches it)
  auto next_seg = [&](int& i2, int& hk2) __attribute__((always_inline)) -> bool {
    if (cc.te - cc.t >= cc.left) return false;
    i2 = cc.i;
    hk2 = cc.hk + 1;
    if (hk2 == Hkv) {
      hk2 = 0;
      ++i2;
    }
    return true;
  };
  auto step = [&](auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    wait_vm<(NR - 3) * DPR + (J < 2 ? QLD : 0), true>();
    ring_barrier();
    issue(std::integral_constant<int, (J + NR - 1) % NR>{});
    advance(ic);
    if (cc.left <= 0) return;  // past the range: the loads above keep the counts exact
    // segment parts are whole quads: tile x + 1 leaves the part only after
    // the quad's last step, which boundary() handles
    const bool more = J < NR - 1 || cc.t + 1 < cc.te;
    const bool keys = cc.t * kKT < cc.L;  // a padding tile holds none
    if (live && more && (cc.t + 1) * kKT < cc.L)
      stage_s(set_ptr(std::integral_constant<int, (J + 1) % NR>{}), Sb[(J + 1) & 1]);
    if (live && keys) stage_pv(set_ptr(jc), cc.t * kKT, cc.ke, Sb[J & 1]);
    if (more) advance(cc);
  };
  auto boundary = [&]() __attribute__((always_inline)) {
    bool entered = false;
    if (cc.left > 0 && cc.t + 1 == cc.te) {
      finish(first);
      reset();
      first = false;
      if (cc.left <= 1) {
        cc.left = 0;
      } else {
        advance(cc);
        read_q(cc.a1 - cc.a0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // q_lds read before the next prefetch lands
        if (live) stage_s(set_ptr(std::integral_constant<int, 0>{}), Sb[0]);
        entered = true;
      }
    }
    int i2, hk2;
    if (entered && next_seg(i2, hk2))
      prefetch_q(i2, hk2);
    else
      prefetch_none();
  };

  if constexpr (LOADER) {
    // With a loader wave (g < 8: wave 7 has no query head), that wave alone
    // moves the ring: per step it waits for its own loads of tile x + 1,
    // meets the others at the barrier and refills the set tile x - 1 used
    // with tile x + 3.  The compute waves issue no ring loads: their only
    // vector-memory operations are their own Q prefetches and output
    // stores, so they wait for nothing at the ring's barriers but their
    // LDS reads, and the stores at a segment's end hold back no ring wait.
    if (wid == kLoaderWave) {
      issue(std::integral_constant<int, 0>{});
      advance(ic);
      issue(std::integral_constant<int, 1>{});
      advance(ic);
      issue(std::integral_constant<int, 2>{});
      advance(ic);
      wait_vm<(NR - 2) * DPR, false>();
      ring_barrier();
      auto lstep = [&](auto jc) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        wait_vm<(NR - 3) * DPR, false>();
        ring_barrier();
        issue(std::integral_constant<int, (J + NR - 1) % NR>{});
        advance(ic);
      };
      for (int qd = n_quads; qd > 0; --qd) {
        lstep(std::integral_constant<int, 0>{});
        lstep(std::integral_constant<int, 1>{});
        lstep(std::integral_constant<int, 2>{});
        lstep(std::integral_constant<int, 3>{});
      }
      wait_vm<0, false>();
      return;
    }
    auto cstep = [&](auto jc) __attribute__((always_inline)) {
      constexpr int J = decltype(jc)::value;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's reads of the set to be refilled are done
      ring_barrier();
      if (cc.left <= 0) return;
      const bool more = J < NR - 1 || cc.t + 1 < cc.te;
      const bool keys = cc.t * kKT < cc.L;
      if (live && more && (cc.t + 1) * kKT < cc.L)
        stage_s(set_ptr(std::integral_constant<int, (J + 1) % NR>{}), Sb[(J + 1) & 1]);
      if (live && keys) stage_pv(set_ptr(jc), cc.t * kKT, cc.ke, Sb[J & 1]);
      if (more) advance(cc);
    };
    auto cboundary = [&]() __attribute__((always_inline)) {
      if (cc.left > 0 && cc.t + 1 == cc.te) {
        wait_vm<0, false>();  // the next segment's Q, prefetched at least a quad ago
        finish(first);
        reset();
        first = false;
        if (cc.left <= 1) {
          cc.left = 0;
        } else {
          advance(cc);
          read_q(cc.a1 - cc.a0);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // q_lds read before the next prefetch lands
          if (live) stage_s(set_ptr(std::integral_constant<int, 0>{}), Sb[0]);
          int i2, hk2;
          if (live && next_seg(i2, hk2)) prefetch_q(i2, hk2);
        }
      }
    };
    if (live) prefetch_q(cc.i, cc.hk);
    ring_barrier();
    wait_vm<0, false>();
    read_q(cc.a1 - cc.a0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (live) stage_s(ring0, Sb[0]);
    {
      int i2, hk2;
      if (live && next_seg(i2, hk2)) prefetch_q(i2, hk2);
    }
    for (int qd = n_quads; qd > 0; --qd) {
      cstep(std::integral_constant<int, 0>{});
      cstep(std::integral_constant<int, 1>{});
      cstep(std::integral_constant<int, 2>{});
      cstep(std::integral_constant<int, 3>{});
      cboundary();
    }
    wait_vm<0, false>();
    return;
  }

  // prologue: Q of the first segment and tiles 0..2 in flight; then Q in
  // registers, S^T of tile 0, the next segment's Q prefetched
  prefetch_q(cc.i, cc.hk);
  issue(std::integral_constant<int, 0>{});
  advance(ic);
  issue(std::integral_constant<int, 1>{});
  advance(ic);
  issue(std::integral_constant<int, 2>{});
  advance(ic);
  wait_vm<(NR - 2) * DPR, true>();
  ring_barrier();
  read_q(cc.a1 - cc.a0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (live) stage_s(ring0, Sb[0]);
  {
    int i2, hk2;
    if (next_seg(i2, hk2))
      prefetch_q(i2, hk2);
    else
      prefetch_none();
  }
  for (int qd = n_quads; qd > 0; --qd) {
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    boundary();
  }
  wait_vm<0, true>();
}

// Merge the parts of every cut segment written by attn_gqa_stream_kernel in
// the launch before: workgroup (sequence i, KV head hk) recomputes the
// partition, returns at once when its segment was not cut, and otherwise
// wave wid merges query head hk * g + wid over the segment's parts in
// workgroup order.  Lane (row, half) merges head-dim columns 64 half +
// [0, 64) of query row `row`; the parts go in pairs whose loads are all
// issued before any is used (a segment cut once is one memory round trip),
// and the running (M, L, O) is rescaled pair by pair.
__global__ __launch_bounds__(kGqaThreads) void attn_stream_merge_kernel(AttnArgs a) {
  const int i = blockIdx.x / a.Hkv, hk = blockIdx.x % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wid >= a.g) return;
  const int b = a.sq.b;
  // this sequence's prompt length and block index, loaded together with the
  // partition's prompt lengths (one memory round trip for both)
  const int P = seq_prompt(a.sq, i);
  const int kblk = seq_block(a.sq, i);
  long long total = 0, before = 0;
  for (int i0 = 0; i0 < b; i0 += 64) {
    const int n = i0 + lane < b ? seq_tiles(a, i0 + lane) + kStreamPhantom : 0;
    total += __shfl(wave_scan_incl(n), 63, 64);
    const int nb = i0 + lane < i ? n : 0;
    before += __shfl(wave_scan_incl(nb), 63, 64);
  }
  const long long T = uniform_ll(total * a.Hkv);
  const long long TQ = T / kStreamQuad;
  const int Gn = (int)((long long)kNumCUs < TQ ? (long long)kNumCUs : TQ);
  const int n_i = ((P + a.sq.G + kKT - 1) / kKT + kStreamQuad - 1) / kStreamQuad * kStreamQuad;  // seq_tiles
  // the segment's first unit (its phantom quad) and its tiles
  const long long seg0 = uniform_ll(before * a.Hkv + (long long)hk * (n_i + kStreamPhantom));
  const long long t0 = seg0 + kStreamPhantom;
  const int u0 = stream_owner(t0, T, Gn), u1 = stream_owner(t0 + n_i - 1, T, Gn);
  if (u0 == u1) return;  // written whole by its workgroup
  int a0, a1;
  fresh_range(a.mode, P, a.sq.G, a.sq.B, kblk, a0, a1);
  const int nq = a1 - a0;
  const int h = hk * a.g + wid;
  const float c = a.scale_log2;
  // Lane l merges, for v = 0..7, the 16-byte piece k = l % 16 (head dims
  // 8 k + [0, 8)) of row 4 v + l / 16, so each load and store moves four
  // whole 256-byte rows; lane r < 32 keeps row r's running (M, L) and hands
  // the row's factors to the lanes holding its pieces.
  const int k = lane & 15, rq = lane >> 4;
  float M = -INFINITY, Lsum = 0.f;  // of row `lane` (lanes < 32)
  float acc[8][8];
#pragma unroll
  for (int v = 0; v < 8; ++v)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[v][t] = 0.f;
#pragma unroll 1
  for (int ub = u0; ub <= u1; ub += 2) {
    float4 x[2][8];
    float mp[2], lp[2], sp[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int u = min(ub + e, u1);  // past the last part: re-read it (weight 0 below)
      const int slot = (u == u0 && stream_lo(u, T, Gn) < seg0) ? 1 : 0;
      const uint8_t* part = (const uint8_t*)a.part + ((size_t)(2 * u + slot) * kGqaWaves + wid) * kPart16Bytes;
#pragma unroll
      for (int v = 0; v < 8; ++v) x[e][v] = *(const float4*)(part + (4 * v + rq) * 256 + 16 * k);
      const float* hdr = (const float*)(part + kQT * kD * 2);
      const int r = lane & 31;
      mp[e] = hdr[r];
      lp[e] = hdr[kQT + r];
      sp[e] = hdr[2 * kQT + r];
    }
    if (ub + 1 > u1) mp[1] = -INFINITY;  // a re-read part adds nothing
    // row factors (lane r < 32 for row r; lanes 32..63 hold copies)
    const float Mn = fmaxf(M, fmaxf(mp[0], mp[1]));
    const float fo = exp2_fast((M - Mn) * c);
    const float f0 = exp2_fast((mp[0] - Mn) * c), f1 = exp2_fast((mp[1] - Mn) * c);
    Lsum = fmaf(lp[1], f1, fmaf(lp[0], f0, Lsum * fo));
    const float w0 = f0 * sp[0], w1 = f1 * sp[1];
    M = Mn;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int src = 4 * v + rq;
      const float fov = __shfl(fo, src, 64), w0v = __shfl(w0, src, 64), w1v = __shfl(w1, src, 64);
      const float4 xs[2] = {x[0][v], x[1][v]};
      float lo0[4], hi0[4], lo1[4], hi1[4];
      const uint32_t u0w[4] = {__float_as_uint(xs[0].x), __float_as_uint(xs[0].y), __float_as_uint(xs[0].z),
                               __float_as_uint(xs[0].w)};
      const uint32_t u1w[4] = {__float_as_uint(xs[1].x), __float_as_uint(xs[1].y), __float_as_uint(xs[1].z),
                               __float_as_uint(xs[1].w)};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        unpack_f16x2(u0w[t], lo0[t], hi0[t]);
        unpack_f16x2(u1w[t], lo1[t], hi1[t]);
        acc[v][2 * t] = fmaf(lo1[t], w1v, fmaf(lo0[t], w0v, acc[v][2 * t] * fov));
        acc[v][2 * t + 1] = fmaf(hi1[t], w1v, fmaf(hi0[t], w0v, acc[v][2 * t + 1] * fov));
      }
    }
  }
  const float inv = 1.f / Lsum;
  uint16_t* obase = (uint16_t*)a.out + ((size_t)i * a.fresh_rows * a.Hq + h) * kD;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int row = 4 * v + rq;
    const float iv = __shfl(inv, row, 64);
    uint4 u;
    u.x = pack_bf16x2(acc[v][0] * iv, acc[v][1] * iv);
    u.y = pack_bf16x2(acc[v][2] * iv, acc[v][3] * iv);
    u.z = pack_bf16x2(acc[v][4] * iv, acc[v][5] * iv);
    u.w = pack_bf16x2(acc[v][6] * iv, acc[v][7] * iv);
    if (row < nq) *(uint4*)(obase + (size_t)row * a.Hq * kD + 8 * k) = u;
  }
}

// ------------------------------------------------------------------ vector ALU
// fp32 inputs (d = 64 or 128) and bf16 inputs with d = 64: one wave per
// query row, every product and sum in fp32; the lanes take 64 keys at a
// time for the scores, then every lane accumulates its head-dim columns of
// P V over those keys.  The output is stored in the input dtype.
__device__ __forceinline__ float4 load4(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 w = *(const uint2*)p;
  return make_float4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y));
}
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_bits_to_f32(*p); }
__device__ __forceinline__ void store1(float* p, float v) { *p = v; }
__device__ __forceinline__ void store1(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16_bits(v); }

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs a) {
  constexpr int U = D / 64;
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wid;
  Geo g;
  g.i = blockIdx.z;
  const int h = blockIdx.y;
  g.hk = h / a.g;
  const int P = seq_prompt(a.sq, g.i);
  const int k = seq_block(a.sq, g.i);
  g.L = P + a.sq.G;
  fresh_range(a.mode, P, a.sq.G, a.sq.B, k, g.a0, g.a1);
  g.nq = g.a1 - g.a0;
  __shared__ float s_q[4][D];
  if (r >= g.nq) return;

  const T* qrow = (const T*)a.q + (((size_t)g.i * a.fresh_rows + r) * a.Hq + h) * D;
#pragma unroll
  for (int u = 0; u < U; ++u) s_q[wid][lane + 64 * u] = load1(qrow + lane + 64 * u);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const T* kn = (const T*)a.kn;
  const T* vn = (const T*)a.vn;
  const T* kc = (const T*)a.kc;
  const T* vc = (const T*)a.vc;
  float acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int j0 = 0; j0 < g.L; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j < g.L) {
      const T* krow = kv_row(a, kn, kc, g, j, D);
      float dot = 0.f;
#pragma unroll 8
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float4 kv = load4(krow + 4 * d4);
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
      const T* vrow = kv_row(a, vn, vc, g, j0 + jj, D);
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = fmaf(pj, load1(vrow + lane + 64 * u), acc[u]);
    }
  }
  T* orow = (T*)a.out + (((size_t)g.i * a.fresh_rows + r) * a.Hq + h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int u = 0; u < U; ++u) store1(orow + lane + 64 * u, acc[u] * inv);
}

// ------------------------------------------------------------------ planning
static long env_long(const char* name, long dflt) {
  const char* e = getenv(name);
  const long v = e ? atol(e) : dflt;
  return v > 0 ? v : dflt;
}

// fdllm_set_tuning overrides (0: automatic), per host thread: a workspace
// query and the call it sizes see the same plan when made on one thread.
static thread_local int g_attn_qt = 0, g_attn_wgs = 0;
void set_attn_tuning(int qt, int wgs) {
  g_attn_qt = qt;
  g_attn_wgs = wgs;
}

static long attn_env_target() {
  static const long v = env_long("FDLLM_ATTN_TARGET_WGS", 0);
  return v;
}

// Kernel and work split (see the choice of QT below).  The key split fills
// the GPU when there are few work items.  The environment
// variables FDLLM_ATTN_QT (1: split-key kernel, 2, 4: LDS ring, 8: LDS ring
// with 8 waves of one query tile each, 16: that ring over the batch's tile
// stream) and FDLLM_ATTN_TARGET_WGS override the defaults for tuning.
AttnPlan plan_block_attn(int dtype, int b, int Hq, int Hkv, int d, int nq_max, int L_max, bool ragged) {
  AttnPlan p{};
  if (dtype != 0 || d != kD) {  // vector-ALU kernel: four query rows per workgroup
    p.n_qt = (nq_max + 3) / 4;
    p.n_grp = 1;
    p.n_split = 1;
    p.kchunk = L_max;
    p.n_items = b * Hq * p.n_qt;
    p.grid = p.n_qt;
    return p;
  }
  const int g = Hq / Hkv;
  p.n_qt = (nq_max + kQT - 1) / kQT;
  const int T = g * p.n_qt;  // query tiles per (sequence, KV head)
  static const long qt_env = env_long("FDLLM_ATTN_QT", 0);
  int QT = g_attn_qt > 0 ? g_attn_qt : (int)qt_env;
  // One query tile per head (DualCache): the split-key kernel (sharing K/V
  // across the heads of a GQA group would need a key split whose merge
  // costs more than the shared loads save).  Several query tiles per head
  // (prefix / no cache): the ring, four query tiles per K/V tile.
  // A GQA group of 4 or more heads with one query tile each: the 8-wave
  // ring (8 query tiles per workgroup), so the group's heads share every K/V
  // tile; with per-sequence prompt lengths and at least half as many
  // (sequence, KV head) segments as CUs, that ring over the batch's tile
  // stream, which gives every CU the same number of tiles (one workgroup
  // per segment would last as long as the longest sequence).
  if (QT != 1 && QT != 2 && QT != 4 && QT != 8 && QT != 16)
    QT = p.n_qt == 1 ? (g >= 4 ? (ragged && g <= kGqaWaves && (long)b * Hkv >= kNumCUs / 2 ? 16 : 8) : 1)
                     : (T >= 4 ? 4 : 2);
  if (QT == 16 && !(p.n_qt == 1 && g <= kGqaWaves)) QT = 8;  // the tile stream needs one query tile per wave
  p.qt_per_wg = QT;
  if (QT == 16) {
    // 8-wave ring over the batch's tile stream: one persistent workgroup per
    // CU, two partial slots of 8 query tiles each per workgroup
    p.n_grp = 1;
    p.n_split = 1;
    p.kchunk = L_max;
    p.grid = kNumCUs;
    p.n_items = p.grid;
    p.per_xcd = p.grid / 8;
    p.part_bytes = (size_t)p.grid * 2 * kGqaWaves * kPart16Bytes;
    return p;
  }
  long base;
  int unit;
  if (QT == 1) {  // split-key kernel: one item per (sequence, query head, query tile, key chunk)
    p.n_grp = 1;
    base = (long)b * Hq * p.n_qt;
    unit = kKT * 4;  // one sub-tile per wave
  } else if (QT == 8) {
    p.n_grp = (T + 7) / 8;
    base = (long)b * Hkv * p.n_grp;
    unit = kKT;  // one tile per ring round
  } else {
    p.n_grp = (T + QT - 1) / QT;
    base = (long)b * Hkv * p.n_grp;
    unit = kKT * (4 / QT);  // keys per ring round
  }
  const long target_env = attn_env_target();
  const long target = g_attn_wgs > 0 ? g_attn_wgs : target_env > 0 ? target_env : (QT == 4 ? 512 : 256);
  const int max_split = (L_max + unit - 1) / unit;
  int ns = (int)((target + base / 2) / base);  // nearest: one chunk unless the items fall well short
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
    const size_t slots = (size_t)b * Hq * p.n_qt * ns;
    const size_t slot_bytes = (QT == 8 || QT == 1) ? (size_t)kPart16Bytes : kPartFloats * sizeof(float);
    p.part_bytes = ((slots * slot_bytes) + 255) & ~(size_t)255;
  }
  return p;
}

// Workspace layout: the arrival counters of the in-kernel merges first, one
// per (sequence, query head, query tile) of the largest query-row count the
// geometry allows (nq_bound: the block size with DualCache, the generation
// length with the prefix cache, prompt + generation without a cache), then
// the split partials.  The counters therefore sit at the same place, and
// only ever hold zeros between calls, whatever the block index, the
// per-call row count or the kernel the planner picks: one workspace zeroed
// once serves every block index of a geometry.  Each kernel's counter index
// is below b * Hq * n_qt (the 4-wave ring's groups, b * Hkv * n_grp, are
// fewer; the 8-wave ring uses none).
size_t attn_counter_bytes(int b, int Hq, int nq_bound) {
  const size_t n = (size_t)b * Hq * ((nq_bound + kQT - 1) / kQT);
  return (n * sizeof(uint32_t) * kCntStride + 255) & ~(size_t)255;
}

// Bytes of a workspace that serves every call of the geometry: the counters
// and the largest partial area over every query-row count up to nq_bound.
// A plan has one key chunk (no partials) once its work items reach the
// workgroup target, and every kernel's item count is at least
// b * Hq * n_qt / 8, so the scan stops there.
size_t attn_workspace_bytes(int dtype, int b, int Hq, int Hkv, int d, int nq_bound, int L_max, bool ragged) {
  if (dtype != 0 || d != kD) return 0;
  const long target_env = attn_env_target();
  const long tmax = g_attn_wgs > 0 ? g_attn_wgs : target_env > 0 ? target_env : 512;
  const int nqt_bound = (nq_bound + kQT - 1) / kQT;
  size_t part = 0;
  for (int t = 1; t <= nqt_bound; ++t) {
    const AttnPlan p = plan_block_attn(dtype, b, Hq, Hkv, d, t < nqt_bound ? t * kQT : nq_bound, L_max, ragged);
    if (p.part_bytes > part) part = p.part_bytes;
    if ((long)b * Hq * t >= 8 * tmax) break;
  }
  return part > 0 ? attn_counter_bytes(b, Hq, nq_bound) + part : 0;
}

void attn_bind_workspace(AttnArgs& a, const AttnPlan& p, void* workspace, size_t counter_bytes) {
  a.n_qt = p.n_qt;
  a.n_grp = p.n_grp;
  a.n_split = p.n_split;
  a.kchunk = p.kchunk;
  a.n_items = p.n_items;
  a.per_xcd = p.per_xcd;
  if (p.part_bytes > 0) {
    a.cnt = (uint32_t*)workspace;
    a.part = (float*)((char*)workspace + counter_bytes);
  }
}

hipError_t launch_block_attn(const AttnArgs& a, const AttnPlan& p, int dtype, int d, hipStream_t st) {
  const LaunchEvents ev = take_launch_events();
  if (dtype == 0 && d == kD) {
    const dim3 grid((unsigned)p.grid), block(kThreads);
    if (p.qt_per_wg == 16) {
      auto* kern = a.g < kGqaWaves ? attn_gqa_stream_kernel<4, true> : attn_gqa_stream_kernel<4, false>;
      const hipError_t e = launch_kernel(kern, grid, dim3(kGqaThreads), 0, st, ev.start, (hipEvent_t) nullptr, a);
      if (e != hipSuccess) return e;
      return launch_kernel(attn_stream_merge_kernel, dim3((unsigned)(a.sq.b * a.Hkv)), dim3(kGqaThreads), 0, st,
                           (hipEvent_t) nullptr, ev.stop, a);
    }
    if (p.qt_per_wg == 8) {
      auto* kern = attn_gqa_kernel<4>;
      const dim3 gblock(kGqaThreads);
      if (p.n_split == 1) return launch_kernel(kern, grid, gblock, 0, st, ev.start, ev.stop, a);
      const hipError_t e = launch_kernel(kern, grid, gblock, 0, st, ev.start, (hipEvent_t) nullptr, a);
      if (e != hipSuccess) return e;
      const dim3 mgrid((unsigned)p.n_qt * 2, (unsigned)a.Hq, (unsigned)a.sq.b);
      return launch_kernel(attn_merge_kernel, mgrid, block, 0, st, (hipEvent_t) nullptr, ev.stop, a);
    }
    if (p.qt_per_wg == 4) return launch_kernel(attn_ring_kernel<4, 4>, grid, block, 0, st, ev.start, ev.stop, a);
    if (p.qt_per_wg == 2) return launch_kernel(attn_ring_kernel<2, 4>, grid, block, 0, st, ev.start, ev.stop, a);
    return launch_kernel(attn_split_kernel, grid, block, 0, st, ev.start, ev.stop, a);
  }
  dim3 grid((unsigned)p.n_qt, (unsigned)a.Hq, (unsigned)a.sq.b);
  if (dtype == 0) return launch_kernel(attn_valu_kernel<uint16_t, 64>, grid, dim3(256), 0, st, ev.start, ev.stop, a);
  return d == 64 ? launch_kernel(attn_valu_kernel<float, 64>, grid, dim3(256), 0, st, ev.start, ev.stop, a)
                 : launch_kernel(attn_valu_kernel<float, 128>, grid, dim3(256), 0, st, ev.start, ev.stop, a);
}

}  // namespace fdllm
