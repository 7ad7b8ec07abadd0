// Debug-mode validation of the device-resident per-sequence arrays
// (prompt lengths, block indices, a refresh list), run before a call's
// kernels when debug checks are on.  Outside debug mode these arrays are
// trusted.
#include <limits.h>

#include <mutex>

#include "fdllm_device.h"
#include "fdllm_internal.h"

namespace fdllm {

// The first problem found: (sequence or list index) * 8 + code, minimised
// over threads (INT_MAX: none).  A module-scope word, so the check needs no
// allocation; a host mutex held from its reset to the synchronisation that
// reads it back makes concurrent debug-mode calls from several host threads
// take turns.
__device__ int g_validate_key;
static std::mutex g_validate_mu;

__global__ __launch_bounds__(256) void validate_kernel(SeqArgs sq, int max_P, const int32_t* seq_ids,
                                                      const int32_t* n_seq) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  int key = INT_MAX;
  if (i < sq.b) {
    const int nblocks = sq.G / sq.B;
    if (sq.plens) {
      const int P = sq.plens[i];
      if (P < 0 || P > max_P) key = min(key, i * 8 + VALIDATE_PROMPT);
    }
    if (sq.bidx) {
      const int k = sq.bidx[i];
      if (k < 0 || k >= nblocks) key = min(key, i * 8 + VALIDATE_BLOCK);
    }
  }
  if (n_seq) {
    const int n = *n_seq;
    if (i == 0 && (n < 0 || n > sq.b)) key = min(key, VALIDATE_NSEQ);
    if (seq_ids && i < min(max(n, 0), sq.b)) {
      const int s = seq_ids[i];
      if (s < 0 || s >= sq.b) key = min(key, i * 8 + VALIDATE_SEQID);
    }
  }
  if (key != INT_MAX) atomicMin(&g_validate_key, key);
}

hipError_t run_validate(const SeqArgs& sq, int max_P, const int32_t* seq_ids, const int32_t* n_seq, hipStream_t st,
                        int* key_out) {
  std::lock_guard<std::mutex> lock(g_validate_mu);
  const int none = INT_MAX;
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_validate_key), &none, sizeof(int), 0, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return e;
  const int n = sq.b > 1 ? sq.b : 1;
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, sq, max_P, seq_ids, n_seq);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbolAsync(key_out, HIP_SYMBOL(g_validate_key), sizeof(int), 0, hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(st);
}

}  // namespace fdllm
