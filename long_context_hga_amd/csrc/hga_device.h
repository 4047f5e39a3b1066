// Device-side helpers shared by the HGA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hga.h"

namespace hga {

constexpr int kMaxPairs = 64;       // head_dim <= 128
constexpr int kGroupTokens = 16;    // tokens per group (C = 64, G = 4)
constexpr int kChunk = 64;
constexpr int kGroups = 4;
// Workspace: a fixed counter area (one 32-bit arrival counter per unit and
// kernel), then data.  Counters return to zero at the end of every call.
constexpr size_t kCounterBytes = size_t(1) << 20;
constexpr int kRouteCounterBase = 0;
constexpr int kAttendCounterBase = 1 << 17;

// Everything a kernel needs to know about the configuration, passed by value.
struct KCfg {
  int d, hq, hkv, hg;
  int n_sink, n_local, topk_c, topk_g;
  int dtype;                       // hga_dtype
  float qscale_log2;               // log2(e) / sqrt(d)
  double inv_sqrt_d;
  unsigned long long hf_mask;      // bit j: pair j is high-frequency
  double omega[kMaxPairs];         // theta^(-2j/d), computed on the host in fp64
};

// ------------------------------------------------------------ numerics
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp64 -> bf16, round to nearest even, without double rounding: first to
// fp32 rounding toward zero with a sticky bit (round-to-odd keeps every bit
// the second rounding needs), then fp32 -> bf16 RNE on the bit pattern.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  float f = __double2float_rz(x);
  uint32_t u = __float_as_uint(f);
  if ((double)f != x) u |= 1u;
  uint32_t bias = 0x7fffu + ((u >> 16) & 1u);
  return uint16_t((u + bias) >> 16);
}

// Angle p*omega (fp64) -> (cos, sin) in fp64.
__device__ __forceinline__ void rope_cs(double pos, double omega, double* c, double* s) {
  sincos(pos * omega, s, c);
}

// ------------------------------------------------ cross-lane reductions
// DPP row controls (gfx9): quad_perm [1,0,3,2] / [2,3,0,1], half-row and row
// mirrors.  Applied in this order they form an all-reduce over 4, 8 or 16
// consecutive lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Sum over groups of N consecutive lanes (N in {8, 16}); every lane of the
// group ends with the group's total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  if constexpr (N == 16) x += dpp_f<kDppMirror>(x);
  static_assert(N == 8 || N == 16, "group size");
  return x;
}

__device__ __forceinline__ double shfl_xor_d(double x, int m) {
  return __shfl_xor(x, m, 64);
}

// Arrival counter of a "last workgroup finishes the job" pattern.  Every
// thread's global writes are released at agent scope before the count; the
// workgroup that brings the count to `total` resets it to zero and acquires
// the others' writes.  Returns true in every thread of that last workgroup.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned total, int* lds_flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    int last = (prev + 1 == total);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = last;
  }
  __syncthreads();
  bool last = *lds_flag != 0;
  if (last) __threadfence();
  return last;
}

// The visible windows of a query chunk ct: sink chunks [0, sink_end),
// candidates [cand_lo, cand_hi), local chunks [local_begin, ct).
struct Windows {
  int sink_end, cand_lo, cand_hi, local_begin;
};
__device__ __host__ inline Windows windows_of(int ct, int n_sink, int n_local) {
  Windows w;
  w.sink_end = ct < n_sink ? ct : n_sink;
  w.cand_lo = n_sink;
  w.cand_hi = ct - n_local;
  if (w.cand_hi < w.cand_lo) w.cand_hi = w.cand_lo;
  int lb = ct - n_local;
  w.local_begin = lb > w.sink_end ? lb : w.sink_end;
  return w;
}

}  // namespace hga
