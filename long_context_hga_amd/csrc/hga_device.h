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

// The same controls on an fp64 value (each 32-bit half moved by DPP).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const unsigned long long u = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(u & 0xffffffffu), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
// Sum over 8 consecutive lanes (fp64); every lane of the group gets it.
__device__ __forceinline__ double group8_sum_d(double x) {
  x += dpp_d<kDppXor1>(x);
  x += dpp_d<kDppXor2>(x);
  x += dpp_d<kDppHalfMirror>(x);
  return x;
}

// Keeps the compiler from consuming a loaded value before this point: the
// empty asm takes the registers as in/out operands, so uses (and the wait for
// the load) cannot be hoisted above it.  It emits no instruction.
__device__ __forceinline__ void hold(float4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
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
