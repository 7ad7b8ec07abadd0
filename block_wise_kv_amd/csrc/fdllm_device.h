// Device helpers for the gfx950 kernels of libfdllm (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fdllm {

constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// bf16 bit patterns <-> float.  A bf16 value is the top half of a float.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Two floats as IEEE fp16 (round to nearest even) in one word, low first,
// and back.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 v = {(_Float16)lo, (_Float16)hi};
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}
__device__ __forceinline__ void unpack_f16x2(uint32_t u, float& lo, float& hi) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 v;
  __builtin_memcpy(&v, &u, 4);
  lo = (float)v.x;
  hi = (float)v.y;
}

// 16 bytes as the 8 bf16 values of an MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// 2^x on the hardware exp unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt on the vector-memory counter only (vmcnt <= N), plus lgkmcnt(0)
// when `LDS` is set.
template <int N, bool LDS>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | ((LDS ? 0 : 15) << 8));
}

// Workgroup barrier without a memory fence: hand-offs through LDS are
// ordered by explicit counter waits (a fence here would wait for every load
// in flight, including the ones being prefetched).
__device__ __forceinline__ void ring_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- cross-lane exchange without LDS (gfx950).  lane_pair<O>(v, a, b)
// sets {a, b} = {v of this lane, v of lane ^ O}, in an order that depends
// only on the lane: O = 1, 2 by DPP quad permutations, 4 and 8 by DPP row
// shifts and a select, 16 and 32 by v_permlane16_swap / v_permlane32_swap
// (each swaps rows of 16 or halves of 32 lanes between two copies of v, so
// the two results hold both lanes' values).  Every use combines a and b
// with a commutative operation, so both lanes of a pair end with the same
// bits, as with a butterfly through LDS.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int O>
__device__ __forceinline__ void lane_pair_u32(uint32_t v, uint32_t& a, uint32_t& b) {
  static_assert(O == 1 || O == 2 || O == 4 || O == 8 || O == 16 || O == 32, "lane offset");
  if constexpr (O == 1 || O == 2) {
    a = v;
    b = dpp_u32<O == 1 ? 0xB1 : 0x4E>(v);  // quad_perm [1,0,3,2] / [2,3,0,1]
  } else if constexpr (O == 4 || O == 8) {
    const uint32_t lo = dpp_u32<0x110 + O>(v);  // row_shr:O, lane - O
    const uint32_t hi = dpp_u32<0x100 + O>(v);  // row_shl:O, lane + O
    a = v;
    b = (__lane_id() & O) ? lo : hi;
  } else if constexpr (O == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  }
}
template <int O, typename T>
__device__ __forceinline__ void lane_pair(T v, T& a, T& b) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    uint32_t x, y;
    lane_pair_u32<O>(__builtin_bit_cast(uint32_t, v), x, y);
    a = __builtin_bit_cast(T, x);
    b = __builtin_bit_cast(T, y);
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    uint32_t al, bl, ah, bh;
    lane_pair_u32<O>((uint32_t)u, al, bl);
    lane_pair_u32<O>((uint32_t)(u >> 32), ah, bh);
    a = __builtin_bit_cast(T, ((uint64_t)ah << 32) | al);
    b = __builtin_bit_cast(T, ((uint64_t)bh << 32) | bl);
  }
}
// v combined with lane (lane ^ O)'s v by a commutative op.
template <int O, typename T, typename F>
__device__ __forceinline__ T xor_combine(T v, F op) {
  T a, b;
  lane_pair<O>(v, a, b);
  return op(a, b);
}

// Workgroup barrier for data exchanged through LDS only: it waits for this
// wave's LDS operations, not for its global loads still in flight (which
// __syncthreads' full fence would).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wave64 reductions (every lane gets the result).
template <typename T, typename F>
__device__ __forceinline__ T wave_reduce(T v, F op) {
  v = xor_combine<32>(v, op);
  v = xor_combine<16>(v, op);
  v = xor_combine<8>(v, op);
  v = xor_combine<4>(v, op);
  v = xor_combine<2>(v, op);
  return xor_combine<1>(v, op);
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
}
__device__ __forceinline__ double wave_sum_d(double v) {
  return wave_reduce(v, [](double x, double y) { return x + y; });
}
__device__ __forceinline__ int wave_min_i(int v) {
  return wave_reduce(v, [](int x, int y) { return min(x, y); });
}

// ---- cross-workgroup publication without cache write-back / invalidate.
// Data published to other workgroups is written with agent-scope atomic
// stores (write-through to the device coherence point), the writer waits for
// their completion, then bumps a relaxed agent-scope counter; the last
// arriver reads the data back with agent-scope atomic loads.
__device__ __forceinline__ void st_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coherent(const uint64_t* p) {
  return __hip_atomic_load((uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent_f2(float* p, float a, float b) {
  st_coherent((uint64_t*)p, (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32));
}
__device__ __forceinline__ void ld_coherent_f2(const float* p, float& a, float& b) {
  const uint64_t w = ld_coherent((const uint64_t*)p);
  a = __uint_as_float((uint32_t)w);
  b = __uint_as_float((uint32_t)(w >> 32));
}
// 16-byte and 4-byte accesses with the same agent-scope cache policy (sc1),
// through a raw buffer resource: full-line write-through for bulk partials.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7fffffff, 0x00020000);
}
// A pointer the caller knows to be the same in every lane, moved to scalar
// registers (so that a buffer resource built from it needs no per-lane loop).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
constexpr int kCoherentAux = 16;  // sc1
__device__ __forceinline__ void st_coherent_b128(__amdgpu_buffer_rsrc_t r, int byte_off, float4 v) {
  u32x4 w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, byte_off, 0, kCoherentAux);
}
__device__ __forceinline__ void st_coherent_b32(__amdgpu_buffer_rsrc_t r, int byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, kCoherentAux);
}
__device__ __forceinline__ float4 ld_coherent_b128(__amdgpu_buffer_rsrc_t r, int byte_off) {
  const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCoherentAux);
  return make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w));
}
__device__ __forceinline__ float ld_coherent_b32(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kCoherentAux));
}

// Wait until this thread's memory operations have completed, then add 1 to
// the counter; returns the previous count.
__device__ __forceinline__ unsigned arrive(uint32_t* cnt) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every thread of the workgroup waits for its own stores, then thread 0
// arrives; returns (to all threads) whether this workgroup was the last of
// `expected` arrivals.
__device__ __forceinline__ bool block_arrive(uint32_t* cnt, unsigned expected, int* s_flag) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) *s_flag = (arrive(cnt) == expected - 1u);
  __syncthreads();
  return *s_flag != 0;
}

}  // namespace fdllm
