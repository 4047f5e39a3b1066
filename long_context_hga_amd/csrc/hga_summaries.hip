// Pool append and RoPE-aware chunk/group key summaries.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 3: summaries
// come from the projected keys with no new layers; high-frequency RoPE pairs
// are rotated per token and then averaged, low-frequency pairs are averaged
// raw and then rotated to the span's representative position (taken as the
// midpoint a + (n-1)/2).  Item 4: the pool keeps the exact token keys, here
// stored already rotated and rounded once to the pool dtype, and the exact
// values, stored per 16-token group as a transposed [d][16] block (the layout
// in which the attention kernels feed V to the matrix cores).
//
// One workgroup per (chunk overlapping the range, KV head, sequence).  256
// threads = P pairs x S token slices (P = d/2).  Each thread loads its pair
// for all tokens of its slice at once, then rotates them in fp64 (fp64 vector
// math runs at the fp32 non-packed rate on gfx950), stepping the angle by one
// fp64 rotation per token from a single sincos, writes the rounded pool rows
// and keeps fp64 slice sums.  Slices are then combined through LDS into the
// group and chunk summaries (fp32 stores).
#include "hga_build_dev.h"

namespace hga {

struct BuildArgs {
  KCfg cfg;
  const void* k_raw;
  const void* v_new;
  void* k_pool;
  void* v_pool;
  float* chunk_sum;
  float* group_sum;
  int pos0, n_tok, pool_cap, max_chunks, B;
};

template <int D, bool BF16>
__global__ __launch_bounds__(256) void build_kernel(BuildArgs a) {
  constexpr int P = D / 2;
  constexpr int S = 256 / P;
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  __shared__ double part[S * P * 2];
  const int h = blockIdx.y, b = blockIdx.z;
  const int unit = b * a.cfg.hkv + h;
  const int chunk = a.pos0 / kChunk + blockIdx.x;
  const T* kr = static_cast<const T*>(a.k_raw) + (size_t)unit * a.n_tok * D;
  const T* vr = static_cast<const T*>(a.v_new) + (size_t)unit * a.n_tok * D;
  const int lo = a.pos0;
  // a plain pool, or the FP8 pool (codes and row scales)
  const bool pool = a.k_pool != nullptr, f8 = pool && a.cfg.pool8;
  T* kp = pool && !f8 ? static_cast<T*>(a.k_pool) + (size_t)unit * a.pool_cap * D : nullptr;
  T* vp = pool && !f8 ? static_cast<T*>(a.v_pool) + (size_t)unit * a.pool_cap * D : nullptr;
  const Fp8Rows rows8 = f8 ? fp8_rows_of(a.k_pool, a.v_pool, a.B * a.cfg.hkv, a.pool_cap, D, unit)
                           : Fp8Rows{};
  float* cs = a.chunk_sum ? a.chunk_sum + ((size_t)unit * a.max_chunks + chunk) * D : nullptr;
  float* gs = a.chunk_sum ? a.group_sum + ((size_t)unit * a.max_chunks + chunk) * kGroups * D : nullptr;
  build_span<D, BF16>(
      a.cfg, chunk * kChunk, lo, lo + a.n_tok, [&](int p) { return kr + (size_t)(p - lo) * D; },
      [&](int p) { return vr + (size_t)(p - lo) * D; }, kp, vp, cs, gs, part, nullptr, rows8);
}

hipError_t launch_build(const KCfg& cfg, int B, const void* k_raw, const void* v_new, int pos0,
                        int n_tok, void* k_pool, void* v_pool, int pool_cap, float* chunk_sum,
                        float* group_sum, int max_chunks, hipStream_t st) {
  BuildArgs a{cfg, k_raw, v_new, k_pool, v_pool, chunk_sum, group_sum, pos0, n_tok, pool_cap,
              max_chunks, B};
  const int first = pos0 / kChunk, last = (pos0 + n_tok - 1) / kChunk;
  dim3 grid(last - first + 1, cfg.hkv, B);
  const bool bf = cfg.dtype == HGA_BF16;
  if (cfg.d == 128) {
    if (bf) hipLaunchKernelGGL((build_kernel<128, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((build_kernel<128, false>), grid, dim3(256), 0, st, a);
  } else {
    if (bf) hipLaunchKernelGGL((build_kernel<64, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((build_kernel<64, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace hga
