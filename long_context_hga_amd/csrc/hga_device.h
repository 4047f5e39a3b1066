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
  // Selected lists: `lists` per sequence, each shared by `lhg` query heads and
  // reading KV head (list index) / kvdiv.  One list per KV head (lists = hkv,
  // lhg = hg, kvdiv = 1) or, routing per query head, one per query head
  // (lists = hq, lhg = 1, kvdiv = hg).
  int lists, lhg, kvdiv;
  int interleaved;                 // RoPE pairs (2j, 2j+1) instead of (j, j + d/2)
  int pool8;                       // K/V pool of E4M3FN codes with per-row scales
  int route_max;                   // routing score: the largest of the lhg heads' scores
  int n_sink, n_local, topk_c, topk_g;
  int dtype;                       // hga_dtype
  float qscale_log2;               // log2(e) / sqrt(d)
  double inv_sqrt_d;
  unsigned long long hf_mask;      // bit j: pair j is high-frequency
  double rep_shift;                // representative position a + (n-1)/2 + rep_shift
  double omega[kMaxPairs];         // theta^(-2j/d), computed on the host in fp64
};

// FP8 pool rows (OCP E4M3FN: sign, 4 exponent bits with bias 7, 3 mantissa
// bits; largest finite value 448): a row's scale is the smallest power of two
// s with max|x| <= 448 s (1 for a zero row), its codes x / s (exact) rounded
// to nearest even.
__device__ __forceinline__ double fp8_row_scale(double amax) {
  if (!(amax > 0.0)) return 1.0;
  int e;
  const double f = 2.0 * frexp(amax, &e);  // amax = f 2^(e-1), f in [1, 2)
  e -= 1;
  return ldexp(1.0, f <= 1.75 ? e - 8 : e - 7);
}
__device__ __forceinline__ uint32_t fp8_code(double y) {  // |y| <= 448
  const uint32_t sign = y < 0.0 ? 0x80u : 0u;
  const double a = fabs(y);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  e -= 1;                                  // a in [2^e, 2^(e+1))
  if (e < -6) {                            // subnormal codes: steps of 2^-9
    const double m = rint(a * 512.0);
    return sign | (m >= 8.0 ? 8u : (uint32_t)m);  // 8 = the smallest normal code
  }
  double q = rint(ldexp(a, 3 - e));        // 8 .. 16
  if (q >= 16.0) {
    q = 8.0;
    e += 1;
  }
  return sign | ((uint32_t)(e + 7) << 3) | ((uint32_t)q - 8u);
}

// Dims of the two members of RoPE pair j.
__host__ __device__ __forceinline__ int pair_a(const KCfg& c, int j) { return c.interleaved ? 2 * j : j; }
__host__ __device__ __forceinline__ int pair_b(const KCfg& c, int j) {
  return c.interleaved ? 2 * j + 1 : j + c.d / 2;
}

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

// sin and cos of x radians in fp64, |x| < 2^31, with short straight-line code
// (it runs cold, once per workgroup, on the routing and summary paths).
// x = k pi/2 + r with k = rint(2x / pi); r = x - k pi/2 from a two-part pi/2
// (fused multiply-adds keep each product k p exact; the dropped third part
// is below 1.5e-33 k), so |r| <= pi/4 to ~2e-16.  Then Taylor series in r^2:
// sin to r^17 / 17!, cos to r^16 / 16! (truncation below 5e-17 at pi/4), and
// the quadrant k mod 4 picks the signs and the swap.
__device__ __forceinline__ void sincos_rad(double x, double* s, double* c) {
  const double k = rint(x * 0.63661977236758134308);       // 2 / pi
  double r = fma(-k, 1.5707963267948966192, x);             // pi/2 rounded to double
  r = fma(-k, 6.123233995736766036e-17, r);                 // pi/2 minus that
  const double r2 = r * r;
  double ps = 1.0 / 355687428096000.0;                      // 1 / 17!
  ps = fma(ps, r2, -1.0 / 1307674368000.0);                 // 1 / 15!
  ps = fma(ps, r2, 1.0 / 6227020800.0);
  ps = fma(ps, r2, -1.0 / 39916800.0);
  ps = fma(ps, r2, 1.0 / 362880.0);
  ps = fma(ps, r2, -1.0 / 5040.0);
  ps = fma(ps, r2, 1.0 / 120.0);
  ps = fma(ps, r2, -1.0 / 6.0);
  const double sr = fma(ps * r2, r, r);
  double pc = 1.0 / 20922789888000.0;                       // 1 / 16!
  pc = fma(pc, r2, -1.0 / 87178291200.0);                   // 1 / 14!
  pc = fma(pc, r2, 1.0 / 479001600.0);
  pc = fma(pc, r2, -1.0 / 3628800.0);
  pc = fma(pc, r2, 1.0 / 40320.0);
  pc = fma(pc, r2, -1.0 / 720.0);
  pc = fma(pc, r2, 1.0 / 24.0);
  pc = fma(pc, r2, -0.5);
  const double cr = fma(pc, r2, 1.0);
  const int q = (int)((long long)k & 3);
  const double ss = (q & 1) ? cr : sr, cc = (q & 1) ? sr : cr;
  *s = (q & 2) ? -ss : ss;
  *c = ((q + 1) & 2) ? -cc : cc;
}

// Angle p*omega (fp64) -> (cos, sin) in fp64.
__device__ __forceinline__ void rope_cs(double pos, double omega, double* c, double* s) {
  sincos_rad(pos * omega, s, c);
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
// Inclusive prefix sum over the 64 lanes of a wave: DPP row_shr:1,2,4,8
// within each 16-lane row (zero fill), then row_bcast:15 / row_bcast:31
// carry the row totals into the later rows.
template <int CTRL, int ROWS, bool ZERO>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, ZERO);
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i<0x111, 0xF, true>(v);
  v += dpp_i<0x112, 0xF, true>(v);
  v += dpp_i<0x114, 0xF, true>(v);
  v += dpp_i<0x118, 0xF, true>(v);
  v += dpp_i<0x142, 0xA, false>(v);
  v += dpp_i<0x143, 0xC, false>(v);
  return v;
}

// fp64 max / min over the wave: DPP inside 16-lane rows, then
// v_permlane16_swap / v_permlane32_swap across rows (each swap returns the
// lane's own value and its partner's, in some order).
template <bool MAX>
__device__ __forceinline__ double wave_ext_d(double x) {
  auto op = [](double a, double b) { return MAX ? fmax(a, b) : fmin(a, b); };
  x = op(x, dpp_d<kDppXor1>(x));
  x = op(x, dpp_d<kDppXor2>(x));
  x = op(x, dpp_d<kDppHalfMirror>(x));
  x = op(x, dpp_d<kDppMirror>(x));
  {
    const unsigned long long u = __double_as_longlong(x);
    auto lo = __builtin_amdgcn_permlane16_swap((unsigned)u, (unsigned)u, false, false);
    auto hi = __builtin_amdgcn_permlane16_swap((unsigned)(u >> 32), (unsigned)(u >> 32), false, false);
    x = op(__longlong_as_double(((unsigned long long)hi[0] << 32) | lo[0]),
           __longlong_as_double(((unsigned long long)hi[1] << 32) | lo[1]));
  }
  {
    const unsigned long long u = __double_as_longlong(x);
    auto lo = __builtin_amdgcn_permlane32_swap((unsigned)u, (unsigned)u, false, false);
    auto hi = __builtin_amdgcn_permlane32_swap((unsigned)(u >> 32), (unsigned)(u >> 32), false, false);
    x = op(__longlong_as_double(((unsigned long long)hi[0] << 32) | lo[0]),
           __longlong_as_double(((unsigned long long)hi[1] << 32) | lo[1]));
  }
  return x;
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0));
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
