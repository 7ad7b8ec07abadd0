// Vocabulary projection fused with the confidence pass: the logits of the
// current block's rows are computed on the matrix cores and reduced in
// registers, never written.
//
// Fast-dLLM (project README "Key techniques" item 2; aibase news
// "Innovations" item 2): a masked position's confidence is the largest
// softmax probability of its logits and its token their argmax (lowest id
// on a tie).  The logits are the projection of the row's final hidden state
// onto the vocabulary, logits[v] = sum_k x[k] w[v][k].  Each workgroup
// reduces its slice of the vocabulary to one partial (max, lowest argmax,
// sum of exp(logit - max)) per row -- 16 bytes instead of 2 bytes per logit
// -- and a small second kernel (unmask.hip) merges the partials of each
// sequence and applies the threshold or fixed-step rule.
//
// Packed weight (fdllm_lmhead_pack, once per model): the vocabulary is cut
// into tiles of 32 rows and the hidden dimension into steps of 16; fragment
// (tile, step) is 1 KB holding, for lane l, the 8 values
// w[32 tile + l % 32][16 step + 8 (l / 32) + 0..7] -- the A operand of one
// v_mfma_f32_32x32x16_bf16.  A wave loads a fragment with one 16-byte load
// per lane (1 KB contiguous per instruction, every cache line fully used,
// no LDS staging).  The hidden dimension is zero-padded to a multiple of
// 512 and the vocabulary to a multiple of 32.
//
// Workgroup: 8 waves; each wave owns VT vocabulary tiles and every wave
// multiplies them with the same RT row tiles (32 rows each) of hidden
// states.  The hidden states are staged through LDS in phases of 512 / RT
// hidden dims (128 at 8 row tiles; two buffers laid out as B-operand
// fragments, read from global memory a whole line per 8 lanes, one
// barrier per phase, no memory fence: the weight loads in flight are not
// waited for).  Each wave keeps kLDepth MFMA steps of weight fragments in
// flight across phase boundaries.  logits^T = W x^T: lane (c, h) of the
// accumulator holds row c and the 16 vocabulary entries 8 (r / 4) + 4 h +
// r % 4 of the tile.
#include <limits.h>
#include <math.h>
#include <stdlib.h>

#include "fdllm_device.h"
#include "fdllm_internal.h"

namespace fdllm {

constexpr int kLWaves = 8;
constexpr int kLThreads = kLWaves * 64;
constexpr int kLDepth = 8;  // MFMA steps of weight fragments in flight per wave

// Hidden dims per phase: 32 RT rows x KC dims x 2 bytes = 32 KB per buffer up
// to 4 row tiles; at 8 row tiles 128 dims (64 KB per buffer, 8 MFMA steps
// per phase: 4-step phases were measured 3-7 % slower).
template <int RT>
struct LPhase {
  static constexpr int KC = RT >= 8 ? 128 : 512 / RT;
};

template <int RT, int VT>
__global__ __launch_bounds__(kLThreads, 1) void lmhead_kernel(LmheadArgs a) {
  constexpr int KC = LPhase<RT>::KC;
  constexpr int NKS = KC / 16;             // MFMA steps per phase
  constexpr int BUF = NKS * RT * 64;       // 16-byte slots per phase buffer
  constexpr int PIECES = BUF / kLThreads;  // slots each thread fills per phase
  constexpr int D = kLDepth;
  static_assert(NKS % D == 0, "a phase holds whole prefetch windows (slot = step % D)");
  static_assert(BUF % kLThreads == 0, "phase buffer must split evenly over the threads");
  // the two phase buffers; after the main loop the epilogue's per-wave
  // partials reuse the same memory
  __shared__ uint4 s_h[2 * BUF];
  static_assert(kLWaves * RT * 32 * 16 <= 2 * BUF * 16, "epilogue partials must fit the phase buffers");
  float(*s_m)[RT * 32] = reinterpret_cast<float(*)[RT * 32]>(s_h);
  int(*s_i)[RT * 32] = reinterpret_cast<int(*)[RT * 32]>(s_m + kLWaves);
  double(*s_z)[RT * 32] = reinterpret_cast<double(*)[RT * 32]>(s_i + kLWaves);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int bid = blockIdx.x;
  // adjacent work items (the row groups of one vocabulary slice) share an XCD
  const int item = (bid & 7) * a.per_xcd + (bid >> 3);
  if (item >= a.n_items) return;
  const int vwg = item / a.n_rg;
  const int rg = item - vwg * a.n_rg;
  const int row0 = rg * RT * 32;
  const int nph = a.Hp / KC;
  const int nks = a.Hp >> 4;  // MFMA steps per vocabulary tile

  // this wave's vocabulary tiles; a tile past the vocabulary re-reads the
  // last one and its logits are discarded
  int vt[VT];
  const uint4* wsrc[VT];
#pragma unroll
  for (int v = 0; v < VT; ++v) {
    vt[v] = vwg * a.tiles_per_wg + wid * VT + v;
    wsrc[v] = a.wp + (size_t)min(vt[v], a.nvt - 1) * nks * 64 + lane;
  }
  // the weight is read once per call: non-temporal loads (measured 10 %
  // faster than cached ones on the LLaDA-8B vocabulary)
  auto wload = [&](int v, int gs) {
    const u32x4 w4 = __builtin_nontemporal_load((const u32x4*)(wsrc[v] + (size_t)min(gs, nks - 1) * 64));
    bf16x8 r;
    __builtin_memcpy(&r, &w4, 16);
    return r;
  };

  // Hidden-state pieces of this thread, read row-major so that 8 lanes
  // cover one 128-byte line: piece q = j * 512 + tid is dims 8 c + [0, 8) of
  // row q / (KC / 8) of the workgroup's rows (c = q % (KC / 8)).  It belongs
  // to B fragment (step c / 2, row tile), lane (row % 32) + 32 (c % 2); in
  // LDS that lane's slot is XORed with (c % 16), which keeps the 8 writes
  // of a line on distinct banks and each fragment 1 KB contiguous.
  constexpr int PR = KC / 8;  // pieces per row and phase
  const uint16_t* xrow[PIECES];
  int koff[PIECES];
  int slot[PIECES];
  bool rok[PIECES];
#pragma unroll
  for (int j = 0; j < PIECES; ++j) {
    const int q = j * kLThreads + tid;
    const int rl = q / PR, c = q - (q / PR) * PR;
    const int rt = rl >> 5, lane_f = (rl & 31) + 32 * (c & 1);
    slot[j] = ((c >> 1) * RT + rt) * 64 + (lane_f ^ (c & 15));
    const int r = row0 + rl;
    rok[j] = r < a.M;
    const int rr = rok[j] ? r : 0;
    const int i = rr / a.B, t = rr - (rr / a.B) * a.B;
    xrow[j] = a.x + (size_t)i * a.seq_stride + (size_t)t * a.row_stride;
    koff[j] = 8 * c;
  }
  // Loads are unconditional and in bounds (clamped); slots of rows past the
  // batch or dims past the hidden size are zeroed with a mask applied when
  // they are stored, so no branch waits for a load in flight.
  auto load_h = [&](uint4 (&hv)[PIECES], uint32_t (&keep)[PIECES], int ph) {
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
      const int k = ph * KC + koff[j];
      hv[j] = *(const uint4*)(xrow[j] + min(k, a.H - 8));
      keep[j] = (rok[j] && k < a.H) ? ~0u : 0u;
    }
  };
  auto store_h = [&](const uint4 (&hv)[PIECES], const uint32_t (&keep)[PIECES], int buf) {
#pragma unroll
    for (int j = 0; j < PIECES; ++j)
      s_h[buf * BUF + slot[j]] = make_uint4(hv[j].x & keep[j], hv[j].y & keep[j], hv[j].z & keep[j], hv[j].w & keep[j]);
  };

  f32x16 acc[VT][RT];
#pragma unroll
  for (int v = 0; v < VT; ++v)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[v][rt][r] = 0.f;
  bf16x8 wa[D][VT];
  {
    uint4 hv[PIECES];
    uint32_t keep[PIECES];
    load_h(hv, keep, 0);
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
      for (int v = 0; v < VT; ++v) wa[d][v] = wload(v, d);
    store_h(hv, keep, 0);
  }
  wait_vm<63, true>();
  ring_barrier();

  for (int ph = 0; ph < nph; ++ph) {
    {
      const int buf = ph & 1;
      // the next phase's hidden states, stored after this phase's steps
      uint4 hv[PIECES];
      uint32_t keep[PIECES];
      load_h(hv, keep, min(ph + 1, nph - 1));
      const uint4* hb = s_h + buf * BUF;
      // Each step is fenced off from the scheduler so the weight loads stay
      // D steps ahead of their use (left alone it sinks them next to the
      // MFMAs and waits for every load); up to 4 row tiles the LDS operand
      // is read one step ahead (8 row tiles have no registers for it: the
      // two waves of a SIMD hide each other's LDS latency instead).
      constexpr bool kAhead = RT <= 4;
      // this lane's slot in the fragments of step s: lane ^ ((2 s + lane / 32) % 16)
      auto bslot = [&](int s) { return lane ^ ((2 * s + (lane >> 5)) & 15); };
      bf16x8 bf[RT];
      if (kAhead) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) bf[rt] = as_bf16x8(hb[rt * 64 + bslot(0)]);
      }
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const int slot = s % D;
        bf16x8 bn[RT];
        if (!kAhead) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) bf[rt] = as_bf16x8(hb[(s * RT + rt) * 64 + bslot(s)]);
        } else if (s + 1 < NKS) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) bn[rt] = as_bf16x8(hb[((s + 1) * RT + rt) * 64 + bslot(s + 1)]);
        }
#pragma unroll
        for (int v = 0; v < VT; ++v)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            acc[v][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[slot][v], bf[rt], acc[v][rt], 0, 0, 0);
        // refill the slot just consumed, D steps ahead (clamped to the tile)
#pragma unroll
        for (int v = 0; v < VT; ++v) wa[slot][v] = wload(v, ph * NKS + s + D);
        if (kAhead && s + 1 < NKS) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) bf[rt] = bn[rt];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // the other buffer was last read before the previous barrier
      store_h(hv, keep, buf ^ 1);
      wait_vm<63, true>();
      ring_barrier();
    }
  }

  // epilogue: per row of each row tile, (max, lowest argmax, sum of exp)
  // over this wave's tiles, then over the two half-waves, then over the
  // workgroup's waves (fp64 sums)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float xv[VT * 16];
    float m = -INFINITY;
    int idx = INT_MAX;
#pragma unroll
    for (int v = 0; v < VT; ++v)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // vocabulary ids increase with (v, r), so '>' keeps the lowest id of a tie
        const int vid = vt[v] * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const float x = (vid < a.V) ? acc[v][rt][r] : -INFINITY;
        xv[v * 16 + r] = x;
        if (x > m) {
          m = x;
          idx = vid;
        }
      }
    float e[VT * 16];
#pragma unroll
    for (int n = 0; n < VT * 16; ++n) e[n] = exp2_fast((xv[n] - m) * kLog2e);
#pragma unroll
    for (int w = VT * 8; w > 0; w >>= 1)
#pragma unroll
      for (int n = 0; n < w; ++n) e[n] += e[n + w];
    float z = (m == -INFINITY) ? 0.f : e[0];
    // the two half-waves hold the same rows: (m1, z1, i1) and (m2, z2, i2)
    // are this lane's and lane ^ 32's, in a lane-pair order
    float m1, m2, z1, z2;
    int i1, i2;
    lane_pair<32>(m, m1, m2);
    lane_pair<32>(z, z1, z2);
    lane_pair<32>(idx, i1, i2);
    const float M = fmaxf(m1, m2);
    const float za = (m1 == -INFINITY) ? 0.f : z1 * exp2_fast((m1 - M) * kLog2e);
    const float zb = (m2 == -INFINITY) ? 0.f : z2 * exp2_fast((m2 - M) * kLog2e);
    const int I = min(m1 == M ? i1 : INT_MAX, m2 == M ? i2 : INT_MAX);
    if (lane < 32) {
      s_m[wid][rt * 32 + lane] = M;
      s_z[wid][rt * 32 + lane] = (double)za + (double)zb;
      s_i[wid][rt * 32 + lane] = I;
    }
  }
  __syncthreads();
  if (tid < RT * 32) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kLWaves; ++w) M = fmaxf(M, s_m[w][tid]);
    double Z = 0.0;
    int I = INT_MAX;
#pragma unroll
    for (int w = 0; w < kLWaves; ++w) {
      const float mw = s_m[w][tid];
      if (mw != -INFINITY) Z += s_z[w][tid] * (double)exp2_fast((mw - M) * kLog2e);
      if (mw == M) I = min(I, s_i[w][tid]);
    }
    const int r = row0 + tid;
    if (r < a.M) {
      UnmaskPartial p;
      p.m = M;
      p.idx = I;
      p.z = Z;
      a.part[(size_t)r * a.n_vwg + vwg] = p;
    }
  }
}

// Weight packing: one thread per 16-byte slot of the packed layout.
__global__ __launch_bounds__(256) void lmhead_pack_kernel(const uint4* w, uint4* wp, int V, int H, int Hp,
                                                          size_t total) {
  const int nks = Hp >> 4;
  for (size_t p = (size_t)blockIdx.x * 256 + threadIdx.x; p < total; p += (size_t)gridDim.x * 256) {
    const int lane = (int)(p & 63);
    const size_t f = p >> 6;
    const size_t tile = f / (size_t)nks;
    const int ks = (int)(f - tile * nks);
    const size_t v = tile * 32 + (lane & 31);
    const int k = ks * 16 + 8 * (lane >> 5);
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (v < (size_t)V && k < H) val = w[(v * (size_t)H + k) >> 3];
    wp[p] = val;
  }
}

size_t lmhead_packed_bytes(int V, int H) {
  const size_t Hp = ((size_t)H + kLmheadHpad - 1) / kLmheadHpad * kLmheadHpad;
  return ((size_t)V + 31) / 32 * 32 * Hp * 2;
}

hipError_t launch_lmhead_pack(const void* w, void* wp, int V, int H, hipStream_t st) {
  const int Hp = (H + kLmheadHpad - 1) / kLmheadHpad * kLmheadHpad;
  const size_t total = lmhead_packed_bytes(V, H) / 16;
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(lmhead_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint4*)w, (uint4*)wp, V,
                     H, Hp, total);
  return hipGetLastError();
}

// Vocabulary tiles per wave: the environment variable FDLLM_LMHEAD_VT or
// fdllm_set_lmhead_tuning (1 or 2) overrides the default.
static thread_local int g_lmhead_vt = 0;  // per host thread, like the other tuning overrides
void set_lmhead_tuning(int vt) { g_lmhead_vt = vt; }
static int lmhead_env_vt() {
  static int v = [] {
    const char* e = getenv("FDLLM_LMHEAD_VT");
    return e ? atoi(e) : 0;
  }();
  return v;
}

LmheadPlan plan_lmhead(int M, int V) {
  LmheadPlan p{};
  // row tiles per workgroup: every CU streams the weight once per row group
  p.rt = M <= 32 ? 1 : M <= 64 ? 2 : M <= 128 ? 4 : 8;
  int vt = g_lmhead_vt > 0 ? g_lmhead_vt : lmhead_env_vt();
  if (vt != 1 && vt != 2) vt = p.rt == 2 ? 2 : 1;
  if (p.rt >= 4) vt = 1;  // register budget: RT x 16 accumulators
  p.vt = vt;
  const int nvt = (V + 31) / 32;
  p.tiles_per_wg = kLWaves * vt;
  p.n_vwg = (nvt + p.tiles_per_wg - 1) / p.tiles_per_wg;
  p.n_rg = (M + 32 * p.rt - 1) / (32 * p.rt);
  p.n_items = p.n_vwg * p.n_rg;
  p.per_xcd = (p.n_items + 7) / 8;
  p.grid = p.per_xcd * 8;
  return p;
}

hipError_t launch_lmhead(const LmheadArgs& a, const LmheadPlan& p, hipStream_t st, hipEvent_t ev_start) {
  const dim3 grid((unsigned)p.grid), block(kLThreads);
  hipEvent_t none = nullptr;
  if (p.rt == 1)
    return p.vt == 2 ? launch_kernel(lmhead_kernel<1, 2>, grid, block, 0, st, ev_start, none, a)
                     : launch_kernel(lmhead_kernel<1, 1>, grid, block, 0, st, ev_start, none, a);
  if (p.rt == 2)
    return p.vt == 2 ? launch_kernel(lmhead_kernel<2, 2>, grid, block, 0, st, ev_start, none, a)
                     : launch_kernel(lmhead_kernel<2, 1>, grid, block, 0, st, ev_start, none, a);
  if (p.rt == 4) return launch_kernel(lmhead_kernel<4, 1>, grid, block, 0, st, ev_start, none, a);
  return launch_kernel(lmhead_kernel<8, 1>, grid, block, 0, st, ev_start, none, a);
}

}  // namespace fdllm
