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

// VPT: vectors of K (and of V) per thread
template <int VPT>
__global__ __launch_bounds__(kRefreshThreads) void kv_refresh_kernel(RefreshArgs a) {
  int i = blockIdx.y;
  if (a.seq_ids) {
    if ((int)blockIdx.y >= *a.n_seq) return;
    i = a.seq_ids[blockIdx.y];
  }
  const int P = seq_prompt(a.sq, i);
  int rows = 0;
  if (a.mode == MODE_DUAL) rows = P + a.sq.G;
  else if (a.mode == MODE_PREFIX) rows = P + seq_block(a.sq, i) * a.sq.B;
  const uint32_t vpr_shift = a.row_vec_shift;
  const uint32_t vpr_mask = (1u << vpr_shift) - 1u;
  const uint32_t nvec = ((uint32_t)rows * (uint32_t)a.Hkv) << vpr_shift;
  const size_t seq_vecs = ((size_t)a.sq.Lcap * a.Hkv) << vpr_shift;
  const u32x4* ks = (const u32x4*)a.k_src + (size_t)i * seq_vecs;
  const u32x4* vs = (const u32x4*)a.v_src + (size_t)i * seq_vecs;
  u32x4* kd = (u32x4*)a.k_cache + (size_t)i * seq_vecs;
  u32x4* vd = (u32x4*)a.v_cache + (size_t)i * seq_vecs;

  const uint32_t base = blockIdx.x * (kRefreshThreads * VPT) + threadIdx.x;
  if (nvec == 0) return;
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
      const uint32_t c = v & vpr_mask;
      const uint32_t jh = v >> vpr_shift;
      const uint32_t j = fdiv(jh, a.hkv_div);
      const uint32_t h = jh - j * (uint32_t)a.Hkv;
      const size_t dst = ((((size_t)h * a.sq.Lcap) + j) << vpr_shift) + c;
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

// Vectors per thread: the choice that gives the least work to the busiest
// CU when the workgroups are dealt evenly over 256 CUs (4 unless the
// refresh fits in about one round: 6 for the LLaDA-8B single-sequence
// refresh, one workgroup per CU instead of one or two).
hipError_t launch_kv_refresh(const RefreshArgs& a, int max_rows, hipStream_t st) {
  const size_t nvec = ((size_t)max_rows * a.Hkv) << a.row_vec_shift;
  if (nvec == 0) return hipSuccess;
  const int cand[3] = {4, 6, 3};
  int vpt = 4;
  size_t best = ~(size_t)0;
  for (int k = 0; k < 3; ++k) {
    const size_t per_block = (size_t)kRefreshThreads * cand[k];
    const size_t wgs = ((nvec + per_block - 1) / per_block) * (size_t)a.sq.b;
    const size_t cost = ((wgs + 255) / 256) * (size_t)cand[k];
    if (cost < best) {
      best = cost;
      vpt = cand[k];
    }
  }
  const size_t per_block = (size_t)kRefreshThreads * vpt;
  const unsigned gx = (unsigned)((nvec + per_block - 1) / per_block);
  dim3 grid(gx, (unsigned)a.sq.b, 1);
  const LaunchEvents ev = take_launch_events();
  auto* kern = vpt == 6 ? kv_refresh_kernel<6> : vpt == 3 ? kv_refresh_kernel<3> : kv_refresh_kernel<4>;
  return launch_kernel(kern, grid, dim3(kRefreshThreads), 0, st, ev.start, ev.stop, a);
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
