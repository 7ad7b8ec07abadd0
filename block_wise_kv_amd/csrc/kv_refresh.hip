// Cache refresh at a block boundary: scatter the token-major K/V of a full
// forward into the head-major caches.
//
// Fast-dLLM (ICLR reviews, review 4; aibase news "Innovations" item 1): once
// a block is decoded, the K/V of every position are recomputed and stored,
// and the steps of the next block read them.  DualCache keeps rows [0, L),
// the prefix cache keeps rows before the new block, no-cache keeps nothing.
//
// Pure data movement.  The source of one sequence is contiguous over
// (row j, head h, 16-byte column c); each thread moves one 16-byte vector of
// K and one of V per iteration, so reads are fully linear and every 16
// consecutive threads write one contiguous 256-byte cache row.
#include "fdllm_device.h"
#include "fdllm_internal.h"

namespace fdllm {

constexpr int kRefreshThreads = 256;

// VPT: vectors of K (and of V) per thread.  One work item moves chunk c
// (kRefreshThreads x VPT vectors) of sequence i's rows from one layer's
// sources (ks0, vs0: [b][Lcap][Hkv][d]) to its caches (kd0, vd0).
template <int VPT>
__device__ __forceinline__ void refresh_rows(const RefreshArgs& a, int i, int c, const uint4* ks0, const uint4* vs0,
                                             uint4* kd0, uint4* vd0) {
  const int P = seq_prompt(a.sq, i);
  int rows = 0;
  if (a.mode == MODE_DUAL) rows = P + a.sq.G;
  else if (a.mode == MODE_PREFIX) rows = P + seq_block(a.sq, i) * a.sq.B;
  const uint32_t vpr_shift = a.row_vec_shift;
  const uint32_t vpr_mask = (1u << vpr_shift) - 1u;
  const uint32_t nvec = ((uint32_t)rows * (uint32_t)a.Hkv) << vpr_shift;
  const size_t seq_vecs = ((size_t)a.sq.Lcap * a.Hkv) << vpr_shift;
  const u32x4* ks = (const u32x4*)ks0 + (size_t)i * seq_vecs;
  const u32x4* vs = (const u32x4*)vs0 + (size_t)i * seq_vecs;
  u32x4* kd = (u32x4*)kd0 + (size_t)i * seq_vecs;
  u32x4* vd = (u32x4*)vd0 + (size_t)i * seq_vecs;

  const uint32_t base = (uint32_t)c * (kRefreshThreads * VPT) + threadIdx.x;
  if (nvec == 0 || base - threadIdx.x >= nvec) return;
  // loads are unconditional (clamped to the last vector), so all of a
  // thread's loads are in flight together; only the stores are guarded
  u32x4 kv[VPT], vv[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const uint32_t v = min(base + u * kRefreshThreads, nvec - 1u);
    kv[u] = __builtin_nontemporal_load(ks + v);
    vv[u] = __builtin_nontemporal_load(vs + v);
  }
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const uint32_t v = base + u * kRefreshThreads;
    if (v < nvec) {
      const uint32_t c4 = v & vpr_mask;
      const uint32_t jh = v >> vpr_shift;
      const uint32_t j = fdiv(jh, a.hkv_div);
      const uint32_t h = jh - j * (uint32_t)a.Hkv;
      const size_t dst = ((((size_t)h * a.sq.Lcap) + j) << vpr_shift) + c4;
      // Non-temporal stores: the refreshed rows go out to HBM during this
      // kernel instead of sitting dirty in the memory-side cache, where the
      // next kernel's streaming reads would evict them and pay for their
      // write-back (1.34 GB refreshed ahead of the LLaDA-8B batch-32
      // attention: that kernel took 296 us after a refresh with ordinary
      // stores, 233 us after one with these, 236 us with no refresh)
      __builtin_nontemporal_store(kv[u], kd + dst);
      __builtin_nontemporal_store(vv[u], vd + dst);
    }
  }
}

// Work items (chunk c fastest, then layer, then the j-th refreshed
// sequence): workgroup w takes items w, w + grid, ...  Without a sequence
// list every item is real and the grid has one workgroup per item; with a
// device list (a few finished sequences out of a large batch) the host
// cannot size the grid to the list, and a workgroup per possible item would
// mostly read the list's length and exit (a 64-sequence, 28-layer refresh
// of 2 sequences: 516k workgroups, 158 us), so a bounded grid walks the
// listed sequences' items instead.
struct LayerPtrs1 {
  const RefreshArgs& a;
  __device__ const uint4* ks(int) const { return a.k_src; }
  __device__ const uint4* vs(int) const { return a.v_src; }
  __device__ uint4* kd(int) const { return a.k_cache; }
  __device__ uint4* vd(int) const { return a.v_cache; }
};
struct LayerPtrsN {
  const RefreshLayerPtrs& p;
  __device__ const uint4* ks(int l) const { return p.k_src[l]; }
  __device__ const uint4* vs(int l) const { return p.v_src[l]; }
  __device__ uint4* kd(int l) const { return p.k_cache[l]; }
  __device__ uint4* vd(int l) const { return p.v_cache[l]; }
};
template <int VPT, class Ptrs>
__device__ __forceinline__ void refresh_items(const RefreshArgs& a, int n_layers, int gx, const Ptrs& ptrs) {
  // (a list never names more than the batch: the list holds b entries)
  const int n = a.seq_ids ? min(__builtin_amdgcn_readfirstlane(*a.n_seq), a.sq.b) : a.sq.b;
  const long long items = (long long)n * n_layers * gx;
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
    const int c = (int)(it % gx);
    const long long r = it / gx;
    const int l = (int)(r % n_layers);
    const int j = (int)(r / n_layers);
    const int i = a.seq_ids ? __builtin_amdgcn_readfirstlane(a.seq_ids[j]) : j;
    refresh_rows<VPT>(a, i, c, ptrs.ks(l), ptrs.vs(l), ptrs.kd(l), ptrs.vd(l));
  }
}

template <int VPT>
__global__ __launch_bounds__(kRefreshThreads) void kv_refresh_kernel(RefreshArgs a, int gx) {
  refresh_items<VPT>(a, 1, gx, LayerPtrs1{a});
}

// Every layer of a block boundary's refresh in one launch: the per-layer
// calls of a small refresh (a few finished sequences) each last about one
// memory round trip plus a launch; together they fill the GPU.
template <int VPT>
__global__ __launch_bounds__(kRefreshThreads) void kv_refresh_layers_kernel(RefreshArgs a, RefreshLayerPtrs p,
                                                                           int n_layers, int gx) {
  refresh_items<VPT>(a, n_layers, gx, LayerPtrsN{p});
}

// Vectors per thread: the choice that gives the least work to the busiest
// CU when the workgroups are dealt evenly over 256 CUs (4 unless the
// refresh fits in about one round: 6 for the LLaDA-8B single-sequence
// refresh, one workgroup per CU instead of one or two).
static int refresh_vpt(size_t nvec, int b, int n_layers) {
  const int cand[3] = {4, 6, 3};
  int vpt = 4;
  size_t best = ~(size_t)0;
  for (int k = 0; k < 3; ++k) {
    const size_t per_block = (size_t)kRefreshThreads * cand[k];
    const size_t wgs = ((nvec + per_block - 1) / per_block) * (size_t)b * (size_t)n_layers;
    const size_t cost = ((wgs + 255) / 256) * (size_t)cand[k];
    if (cost < best) {
      best = cost;
      vpt = cand[k];
    }
  }
  return vpt;
}

// Workgroups of a launch over a sequence list: 8 per CU (each keeps VPT x 8
// KB of loads in flight), never more than the items could need; without a
// list, one per item up to 4M (then the workgroups take several items).
constexpr long long kRefreshListWgs = 8LL * 256;
constexpr long long kRefreshMaxWgs = 1LL << 22;

struct RefreshGrid {
  int vpt, gx;
  unsigned wgs;
};
static RefreshGrid refresh_grid(const RefreshArgs& a, int n_layers, int max_rows) {
  RefreshGrid g{};
  const size_t nvec = ((size_t)max_rows * a.Hkv) << a.row_vec_shift;
  if (nvec == 0) return g;
  g.vpt = refresh_vpt(nvec, a.sq.b, n_layers);
  const size_t per_block = (size_t)kRefreshThreads * g.vpt;
  g.gx = (int)((nvec + per_block - 1) / per_block);
  long long wgs = (long long)g.gx * a.sq.b * n_layers;
  const long long cap = a.seq_ids ? kRefreshListWgs : kRefreshMaxWgs;
  g.wgs = (unsigned)(wgs < cap ? wgs : cap);
  return g;
}

hipError_t launch_kv_refresh(const RefreshArgs& a, int max_rows, hipStream_t st) {
  const RefreshGrid g = refresh_grid(a, 1, max_rows);
  if (g.wgs == 0) return hipSuccess;
  const LaunchEvents ev = take_launch_events();
  auto* kern = g.vpt == 6 ? kv_refresh_kernel<6> : g.vpt == 3 ? kv_refresh_kernel<3> : kv_refresh_kernel<4>;
  return launch_kernel(kern, dim3(g.wgs), dim3(kRefreshThreads), 0, st, ev.start, ev.stop, a, g.gx);
}

hipError_t launch_kv_refresh_layers(const RefreshArgs& a, const RefreshLayerPtrs& p, int n_layers, int max_rows,
                                    hipStream_t st) {
  const RefreshGrid g = refresh_grid(a, n_layers, max_rows);
  if (g.wgs == 0) return hipSuccess;
  const LaunchEvents ev = take_launch_events();
  auto* kern = g.vpt == 6   ? kv_refresh_layers_kernel<6>
               : g.vpt == 3 ? kv_refresh_layers_kernel<3>
                            : kv_refresh_layers_kernel<4>;
  return launch_kernel(kern, dim3(g.wgs), dim3(kRefreshThreads), 0, st, ev.start, ev.stop, a, p, n_layers, g.gx);
}

// ------------------------------------------------------------------ zero fill
__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, size_t n) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  for (; i < n; i += stride) p[i] = 0u;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  const LaunchEvents ev = take_launch_events();
  return launch_kernel(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, ev.start, ev.stop, (uint32_t*)p, n);
}

}  // namespace fdllm
