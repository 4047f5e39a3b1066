// Declarations shared by the decode and the chunked-prefill attention
// kernels: split geometry, the per-split partial layout that the merge kernel
// reads, list-part helpers and cross-row reductions.
#pragma once

#include "hga_internal.h"

namespace hga {

constexpr int kSplitGroups = 8;   // selected groups per workgroup
constexpr int kMaxSplits = 32;    // splits per (unit, query token): max_sel <= 256
constexpr int kPrefillMinLq = 16; // query tokens from which the MFMA prefill kernel runs

struct AttendArgs {
  KCfg cfg;
  AttendLaunch a;
  int n_splits;     // partial records per (unit, query token)
  int grid_splits;  // split workgroups per (unit, column block / head)
};

// Partial of one split: m[HG], l[HG], padding to a 16-byte boundary, o[HG][D].
template <int HG>
__host__ __device__ constexpr int part_head() { return (2 * HG + 3) / 4 * 4; }
template <int D, int HG>
__host__ __device__ constexpr int part_floats() { return part_head<HG>() + HG * D; }

// Virtual group index v of a part -> slot of the unit's selected list.
__device__ __forceinline__ int part_slot(int part, const ListParts& lp, int v) {
  if (part == HGA_PART_ROUTED) return lp.n_head + v;
  if (part == HGA_PART_WINDOWS) return v < lp.n_head ? v : v + lp.n_routed;
  return v;
}
__device__ __forceinline__ int part_count(int part, const ListParts& lp, int n_sel) {
  if (part == HGA_PART_ROUTED) return lp.n_routed;
  if (part == HGA_PART_WINDOWS) return lp.n_head + lp.n_tail;
  return n_sel;
}

// First partial record of this call's splits, and the number of records the
// merge kernel combines, for the one-part and the two-part layouts.
__device__ __forceinline__ int record_base(const AttendLaunch& a, const ListParts& lp) {
  return (a.two_part && a.part_sel == HGA_PART_ROUTED)
             ? (lp.n_head + lp.n_tail + kSplitGroups - 1) / kSplitGroups
             : 0;
}
__device__ __forceinline__ int records_active(const AttendLaunch& a, const ListParts& lp,
                                              int n_sel) {
  if (a.two_part)
    return (lp.n_head + lp.n_tail + kSplitGroups - 1) / kSplitGroups +
           (lp.n_routed + kSplitGroups - 1) / kSplitGroups;
  return (part_count(a.part_sel, lp, n_sel) + kSplitGroups - 1) / kSplitGroups;
}

// Sum / max over the 4 token rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Matrix-core operand types (v_mfma_f32_16x16x32_bf16).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> one register of two bf16, rounded to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// (a, b) -> bf16 pairs hi, lo with a ~= hi.x + lo.x, b ~= hi.y + lo.y: 16
// significant bits of each value in two bf16 operands.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

// The bf16 elements of x whose bit in keep (bit i = element i) is clear
// become +0.
__device__ __forceinline__ uint4 keep_bf16(uint4 x, uint32_t keep) {
  auto m = [&](int i) {
    return ((keep >> (2 * i)) & 1u ? 0x0000FFFFu : 0u) | ((keep >> (2 * i + 1)) & 1u ? 0xFFFF0000u : 0u);
  };
  return make_uint4(x.x & m(0), x.y & m(1), x.z & m(2), x.w & m(3));
}

// Split kernels; the merge kernel of hga_attend.hip combines their partials.
void launch_decode(const AttendArgs& x, hipStream_t st);   // 1..15 query tokens
void launch_prefill(const AttendArgs& x, hipStream_t st);  // 16..64 query tokens
// The host tier's one-launch front: the first win_splits splits of the decode
// split grid x beside a persistent gather (hga_decode.hip).
struct GatherArgs;
void launch_tier_front(const AttendArgs& x, int win_splits, const GatherArgs& g, int n_items,
                       hipStream_t st);

}  // namespace hga
