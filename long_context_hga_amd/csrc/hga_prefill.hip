// Exact softmax attention over the selected token K/V, chunked-prefill shape:
// 16..64 query tokens of one chunk against the selected groups, on the
// matrix cores.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 4: after
// routing, the output is softmax attention over the exact token K/V of the
// selected set; the "Experimentele Resultaten" section reports the prefill speed-up
// of fusing this step.  Within the query's own chunk a key at position p is
// visible to query token tau only if p <= tau; every routed and window key
// precedes the chunk and is visible to all of its tokens.
//
// Work split: grid = (splits of 8 selected groups, query head, sequence),
// 256 threads.  Wave w owns query tokens 16w .. 16w+15 of the chunk; all four
// waves share the split's 128 keys, staged once in LDS.
//
// The split's 128 keys are one tile of hga_mfma_tile.h (LDS layouts, the
// two contractions on the matrix cores; the FP8 pool's codes and row
// scales).  The hi/lo split (x = hi + lo, both
// bf16) carries 16 significant bits of the query and of the probabilities;
// K and V enter unrounded (they are bf16), so the products carry about
// 2^-17 relative error before fp32 accumulation.
//
// Softmax in two passes over registers: a lane's 32 scores of the split stay
// in registers; the row maximum is taken once, then the probabilities, then
// O^T.  The partial carries that maximum (no online rescaling inside a
// split).
//
// The result of each split is a partial (max m in log2 units, sum l,
// unnormalised o) per query token in the decode kernel's layout; the merge
// kernel of the decode path combines the splits exactly.
#include "hga_mfma_tile.h"

namespace hga {

template <int D, int HG, bool FP8 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attend_prefill_kernel(AttendArgs args) {
  static_assert(D == 128, "staging maps assume 16 chunks of 16 bytes per key row");
  constexpr int KS = D / 32;              // k-steps of the QK^T contraction
  constexpr int NB = D / 16;              // 16-dim blocks of the output
  __shared__ __align__(16) uint16_t ks[kTileKeys * D];   // [128 keys][D], swizzled
  __shared__ __align__(16) uint16_t vt[D * kTileKeys];   // [D][128 keys], swizzled
  __shared__ __align__(16) float sc_k[FP8 ? kTileKeys : 1];  // FP8: row scales of the keys
  __shared__ __align__(16) float sc_v[FP8 ? kTileKeys : 1];

  const KCfg& c = args.cfg;
  const AttendLaunch& a = args.a;
  // every kernel argument used below, read from the argument segment at once
  // (one scalar round trip, instead of one at each first use)
  asm volatile("" ::"s"(c.lists), "s"(c.kvdiv), "s"(c.hq), "s"(c.hkv), "s"(c.n_sink),
               "s"(c.n_local), "s"(c.interleaved), "s"(c.qscale_log2), "s"(a.lq), "s"(a.max_sel),
               "s"(a.src_layout), "s"(a.src_cap), "s"(a.part_sel), "s"(a.two_part),
               "s"(args.n_splits), "s"(a.B), "s"(a.q), "s"(a.q_pos0), "s"(a.k), "s"(a.v),
               "s"(a.sel), "s"(a.n_sel), "s"(a.part));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sp = blockIdx.x, qh = blockIdx.y, b = blockIdx.z;
  const int lst = qh / HG, hj = qh % HG;        // HG = query heads per list
  const int unit = b * c.lists + lst;           // the list (and its partial records)
  const int unit_p = b * c.hkv + lst / c.kvdiv;  // the pool rows of its KV head
  const int rl = lane & 15, qg = lane >> 4;  // C-layout column (query row) and row group
  const int row = wave * 16 + rl;            // query token of this lane
  const int pos0 = a.q_pos0[b];
  const int n_sel = a.n_sel[unit];
  const int* sel = a.sel + (size_t)unit * a.max_sel;
  const int v0 = sp * kSplitGroups;
  int sel_spec[kSplitGroups];
#pragma unroll
  for (int g = 0; g < kSplitGroups; ++g) {
    const int v = v0 + g;
    sel_spec[g] = sel[v < a.max_sel ? v : a.max_sel - 1];
  }
  uint4 qraw[KS];
  double om[16];
  {
    const int tq = row < a.lq ? row : a.lq - 1;
    load_q_raw<D>(static_cast<const uint16_t*>(a.q) + ((size_t)(b * c.hq + qh) * a.lq + tq) * D, qg, qraw);
    load_q_omega<D>(c, qg, om);
  }

  bool bad = n_sel < 0 || n_sel > a.max_sel || pos0 < 0 || (pos0 % kChunk) + a.lq > kChunk;
  ListParts lp{0, 0, 0};
  if (!bad) {
    lp = list_parts(n_sel, pos0 + a.lq - 1, pos0, c.n_sink, c.n_local);
    bad = lp.n_routed < 0;
  }
  if (bad) return;  // the merge kernel writes NaN for this unit
  const int n_part = part_count(a.part_sel, lp, n_sel);
  if (v0 >= n_part) return;  // an empty split: the merge kernel skips it
  const int pos_last = pos0 + a.lq - 1;

  // ---- the split's groups: source rows and first positions (-1: no group)
  int gpos[kSplitGroups];
  size_t gbase[kSplitGroups];
  {
    const int max_gid = a.src_cap / kGroupTokens - 1;
#pragma unroll
    for (int g = 0; g < kSplitGroups; ++g) {
      const int v = v0 + g;
      const int slot = part_slot(a.part_sel, lp, v < n_part ? v : v0);
      int gid = a.part_sel == HGA_PART_ALL ? sel_spec[g] : sel[slot];
      const bool in_range = gid >= 0 && (a.src_layout == HGA_SRC_WORKING_SET || gid <= max_gid);
      gpos[g] = (v < n_part && in_range) ? gid * kGroupTokens : -1;
      gid = gid < 0 ? 0 : (gid > max_gid ? max_gid : gid);
      gbase[g] = a.src_layout == HGA_SRC_WORKING_SET
                     ? ((size_t)unit * a.max_sel + slot) * kGroupTokens * D
                     : ((size_t)unit_p * a.src_cap + (size_t)gid * kGroupTokens) * D;
    }
  }
  // ---- every K/V load of the split, issued before any is used; the query
  // is rotated while they are in flight
  u32x4 kraw[kSplitGroups], vraw[kSplitGroups];
  float sc = 0.f;
  const float* k_sc = nullptr;
  const float* v_sc = nullptr;
  if constexpr (FP8) {  // the row scales follow the codes of every pool (or working-set) unit
    const size_t codes =
        (size_t)a.B * (a.src_layout == HGA_SRC_WORKING_SET ? c.lists : c.hkv) * a.src_cap * D;
    k_sc = reinterpret_cast<const float*>(static_cast<const uint8_t*>(a.k) + codes);
    v_sc = reinterpret_cast<const float*>(static_cast<const uint8_t*>(a.v) + codes);
  }
  load_tile<D, 256, FP8>(a.k, a.v, gbase, tid, kraw, vraw, k_sc, v_sc, &sc);
  bf16x8 qop_hi[KS], qop_lo[KS];
  rotate_q<D>(c, qraw, om, pos0 + row, qop_hi, qop_lo);
  bool all_before = true;  // every group present and before the query chunk (uniform)
#pragma unroll
  for (int g = 0; g < kSplitGroups; ++g) all_before = all_before && gpos[g] >= 0 && gpos[g] + kGroupTokens <= pos0;
  stage_tile<D, 256, FP8>(ks, vt, kraw, vraw, gpos, pos_last, tid, all_before, sc, sc_k, sc_v);
  __syncthreads();
  if (wave * 16 >= a.lq) return;  // no query rows in this wave

  // ---- softmax in two passes over registers: the row maximum of the
  // split's 128 scores first, then the probabilities and O^T (no running
  // rescale inside a split)
  f32x4 s[4][2];
  const float m =
      rows_max(tile_scores<D, FP8>(ks, qop_hi, qop_lo, gpos, pos0 + row, rl, qg, s, all_before, sc_k));
  const float mref = m == -INFINITY ? 0.f : m;  // a row with no visible key: p = 0
  float l = 0.f;
  f32x4 o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  tile_pv<D, FP8>(vt, s, mref, rl, qg, l, o, sc_v);
  l = rows_sum(l);
  const int ri = sp + record_base(a, lp);  // < n_splits for lists hga_route can write
  if (row < a.lq && ri < args.n_splits) {
    float* rec = a.part + ((size_t)(unit * a.lq + row) * args.n_splits + ri) * part_floats<D, HG>();
    if (qg == 0) {
      rec[hj] = m;
      rec[HG + hj] = l;
    }
    float* orow = rec + part_head<HG>() + hj * D;
#pragma unroll
    for (int n = 0; n < NB; ++n)
      *reinterpret_cast<float4*>(orow + 16 * n + 4 * qg) = make_float4(o[n][0], o[n][1], o[n][2], o[n][3]);
  }
}

void launch_prefill(const AttendArgs& x, hipStream_t st) {
  const dim3 grid(x.grid_splits, x.cfg.hq, x.a.B);
  if (x.cfg.pool8) {
    switch (x.cfg.lhg) {
      case 1: hipLaunchKernelGGL((attend_prefill_kernel<128, 1, true>), grid, dim3(256), 0, st, x); break;
      case 2: hipLaunchKernelGGL((attend_prefill_kernel<128, 2, true>), grid, dim3(256), 0, st, x); break;
      case 4: hipLaunchKernelGGL((attend_prefill_kernel<128, 4, true>), grid, dim3(256), 0, st, x); break;
      default: hipLaunchKernelGGL((attend_prefill_kernel<128, 8, true>), grid, dim3(256), 0, st, x); break;
    }
    return;
  }
  switch (x.cfg.lhg) {
    case 1: hipLaunchKernelGGL((attend_prefill_kernel<128, 1>), grid, dim3(256), 0, st, x); break;
    case 2: hipLaunchKernelGGL((attend_prefill_kernel<128, 2>), grid, dim3(256), 0, st, x); break;
    case 4: hipLaunchKernelGGL((attend_prefill_kernel<128, 4>), grid, dim3(256), 0, st, x); break;
    default: hipLaunchKernelGGL((attend_prefill_kernel<128, 8>), grid, dim3(256), 0, st, x); break;
  }
}

}  // namespace hga
