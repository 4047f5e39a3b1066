// Whole-prompt chunked prefill: every 64-token query chunk of a prompt is
// routed and attended in one pass over the prompt.
//
// HGA technical summary (gist.science), "Kernmechanisme" items 2-4: each
// query chunk routes over the summaries of the complete chunks before it and
// attends the exact K/V of its selected set; the "Experimentele Resultaten"
// section reports the prefill speed-up of fusing these steps.  A query chunk
// only ever reads chunks before it (and its own, causally), so once the
// prompt's pool and summaries exist all query chunks are independent: they
// are routed as virtual sequences (sequence b, chunk qc) and attended by one
// launch.
//
// attend_prompt_kernel: one workgroup per (two query heads of a KV head,
// query chunk), 512 threads, wave w owning query tokens 16(w%4) .. +15 of the
// chunk for head w/4 of the pair, so each staged tile serves both heads.  It
// walks the chunk's selected list in tiles of 8 groups (hga_mfma_tile.h):
// the next tile's K/V loads are in flight while the current tile is
// computed, and the softmax runs online over the tiles (running maximum and
// sum per row, output rescaled when the maximum grows), so the normalised
// output is written directly, with no partials to merge.
//
// Workgroups are dispatched to the 8 XCDs of the chip in turn (workgroup i
// on XCD i % 8).  The launch index is remapped so that consecutive work
// items - the head pairs of one KV head and chunk, which read the same K/V -
// run on the same XCD and share its L2.  The mapping only orders the
// work; any dispatch policy gives the same results.
#include "hga_mfma_tile.h"

namespace hga {

struct PromptArgs {
  KCfg cfg;
  const uint16_t* q;   // [Bp][Hq][T][d] bf16 raw queries
  const void* k;       // pool [Bp][Hkv][cap][d] (FP8: codes, then row scales)
  const void* v;       // pool [Bp][Hkv][cap/16][d][16]
  int Bp;              // pool sequences
  const int* sel;      // [Bv][Hkv][max_sel], Bv = Bp * nq virtual sequences
  const int* n_sel;    // [Bv][Hkv]
  float* out;          // [Bp][Hq][T][d]
  float* lse;          // [Bp][Hq][T] or null
  int nq, T, cap, max_sel, n_items;  // n_items = Bv * Hkv * (Hg / HPW)
};

constexpr int kXcds = 8;

// HPW query heads per workgroup (2, or 1 when a KV head has one query head).
template <int D, int HG, int HPW, bool FP8 = false>
__global__ __launch_bounds__(256 * HPW) __attribute__((amdgpu_waves_per_eu(2))) void attend_prompt_kernel(PromptArgs a) {
  static_assert(D == 128, "staging maps assume 16 chunks of 16 bytes per key row");
  static_assert(HG % HPW == 0, "head pairs");
  constexpr int KS = D / 32;
  constexpr int NB = D / 16;
  constexpr int NTHR = 256 * HPW;
  constexpr int GPT = TileStaging<NTHR>::GPT;
  __shared__ __align__(16) uint16_t ks[kTileKeys * D];
  __shared__ __align__(16) uint16_t vt[D * kTileKeys];
  __shared__ __align__(16) float sc_k[FP8 ? kTileKeys : 1];  // FP8: row scales of the keys
  __shared__ __align__(16) float sc_v[FP8 ? kTileKeys : 1];

  const KCfg& c = a.cfg;
  const int per_xcd = (a.n_items + kXcds - 1) / kXcds;
  const int item = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
  if (item >= a.n_items) return;  // uniform: the whole workgroup leaves
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hp = item % (HG / HPW), uv = item / (HG / HPW);  // uv = virtual unit (bv, kvh)
  const int kvh = uv % c.hkv, bv = uv / c.hkv;
  const int qh = kvh * HG + hp * HPW + wave / 4;  // this wave's query head
  const int bp = bv / a.nq, qc = bv % a.nq;
  const int unit_p = bp * c.hkv + kvh;

  const int rl = lane & 15, qg = lane >> 4;
  const int row = (wave % 4) * 16 + rl;  // query token of this lane within the chunk
  const size_t tok = (size_t)(bp * c.hq + qh) * a.T + (size_t)qc * kChunk + row;
  const int pos0 = qc * kChunk;  // the chunk's first position
  const int n_sel = a.n_sel[uv];
  // the unit's list in registers: lane l holds slots l, 64 + l, 128 + l, 192 + l
  int selr[4];
  {
    const int* sel = a.sel + (size_t)uv * a.max_sel;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int v = 64 * r + lane;
      selr[r] = sel[v < a.max_sel ? v : a.max_sel - 1];
    }
  }
  uint4 qraw[KS];
  double om[16];
  load_q_raw<D>(a.q + tok * D, qg, qraw);
  load_q_omega<D>(c, qg, om);
  const float* k_sc = nullptr;
  const float* v_sc = nullptr;
  if constexpr (FP8) {  // the row scales follow the codes of every pool unit
    const size_t codes = (size_t)a.Bp * c.hkv * a.cap * D;
    k_sc = reinterpret_cast<const float*>(static_cast<const uint8_t*>(a.k) + codes);
    v_sc = reinterpret_cast<const float*>(static_cast<const uint8_t*>(a.v) + codes);
  }
  float sc = 0.f;

  if (n_sel < 0 || n_sel > a.max_sel) {  // uniform: no usable list
    const float nan = __builtin_nanf("");
    float* orow = a.out + tok * D;
#pragma unroll
    for (int n = 0; n < NB; ++n)
      *reinterpret_cast<float4*>(orow + 16 * n + 4 * qg) = make_float4(nan, nan, nan, nan);
    if (a.lse && qg == 0) a.lse[tok] = nan;
    return;
  }
  const int pos_last = pos0 + kChunk - 1;
  const int tau = pos0 + row;
  const int max_gid = a.cap / kGroupTokens - 1;
  // slot v (wave-uniform) of the list
  auto sel_at = [&](int v) {
    const int x = v < 64 ? selr[0] : (v < 128 ? selr[1] : (v < 192 ? selr[2] : selr[3]));
    return __builtin_amdgcn_readlane(x, v & 63);
  };
  auto tile_groups = [&](int t, int (&gpos)[kTileGroups], size_t (&gbase)[kTileGroups]) {
#pragma unroll
    for (int it = 0; it < kTileGroups; ++it) {
      const int v = kTileGroups * t + it;
      int gid = v < n_sel ? sel_at(v) : -1;
      gpos[it] = (gid >= 0 && gid <= max_gid) ? gid * kGroupTokens : -1;
      gid = gid < 0 ? 0 : (gid > max_gid ? max_gid : gid);
      gbase[it] = ((size_t)unit_p * a.cap + (size_t)gid * kGroupTokens) * D;
    }
  };

  const int n_tiles = (n_sel + kTileGroups - 1) / kTileGroups;
  int gpos[kTileGroups];
  size_t gbase[kTileGroups];
  u32x4 kraw[GPT], vraw[GPT];
  if (n_tiles > 0) {
    tile_groups(0, gpos, gbase);
    load_tile<D, NTHR, FP8>(a.k, a.v, gbase, tid, kraw, vraw, k_sc, v_sc, &sc);
  }
  bf16x8 qop_hi[KS], qop_lo[KS];
  rotate_q<D>(c, qraw, om, tau, qop_hi, qop_lo);

  f32x4 o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  for (int t = 0; t < n_tiles; ++t) {
    if (t > 0) __syncthreads();  // every wave is done with the previous tile
    bool all_before = true;  // every group present and before the chunk (uniform)
#pragma unroll
    for (int it = 0; it < kTileGroups; ++it)
      all_before = all_before && gpos[it] >= 0 && gpos[it] + kGroupTokens <= pos0;
    stage_tile<D, NTHR, FP8>(ks, vt, kraw, vraw, gpos, pos_last, tid, all_before, sc, sc_k, sc_v);
    __syncthreads();
    int gcur[kTileGroups];
#pragma unroll
    for (int it = 0; it < kTileGroups; ++it) gcur[it] = gpos[it];
    if (t + 1 < n_tiles) {  // the next tile's loads fly during this tile
      tile_groups(t + 1, gpos, gbase);
      load_tile<D, NTHR, FP8>(a.k, a.v, gbase, tid, kraw, vraw, k_sc, v_sc, &sc);
    }
    f32x4 s[4][2];
    const float tmax =
        rows_max(tile_scores<D, FP8>(ks, qop_hi, qop_lo, gcur, tau, rl, qg, s, all_before, sc_k));
    const float mn = fmaxf(m, tmax);
    const float mref = mn == -INFINITY ? 0.f : mn;
    if (__ballot(mn != m)) {  // some row's maximum grew: rescale (by 1 where it did not)
      const float al = __builtin_amdgcn_exp2f(m - mref);  // 0 while the row had no visible key
      l *= al;
#pragma unroll
      for (int n = 0; n < NB; ++n) o[n] *= al;
    }
    m = mn;
    tile_pv<D, FP8>(vt, s, mref, rl, qg, l, o, sc_v);
  }
  l = rows_sum(l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* orow = a.out + tok * D;
#pragma unroll
  for (int n = 0; n < NB; ++n)
    *reinterpret_cast<float4*>(orow + 16 * n + 4 * qg) =
        make_float4(o[n][0] * inv, o[n][1] * inv, o[n][2] * inv, o[n][3] * inv);
  if (a.lse && qg == 0)
    a.lse[tok] = l > 0.f ? (m + log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

__global__ void prompt_positions_kernel(int* pos, int n, int nq) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) pos[i] = (i % nq) * kChunk;
}

hipError_t launch_prompt_positions(int* pos, int n_virtual, int nq, hipStream_t st) {
  hipLaunchKernelGGL(prompt_positions_kernel, dim3((n_virtual + 255) / 256), dim3(256), 0, st, pos,
                     n_virtual, nq);
  return hipGetLastError();
}

hipError_t launch_prompt_attend(const KCfg& cfg, const PromptLaunch& p, hipStream_t st) {
  PromptArgs a;
  a.cfg = cfg;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = p.k;
  a.v = p.v;
  a.Bp = p.B;
  a.sel = p.sel;
  a.n_sel = p.n_sel;
  a.out = p.out;
  a.lse = p.lse;
  a.nq = p.nq;
  a.T = p.T;
  a.cap = p.cap;
  a.max_sel = p.max_sel;
  const int hpw = cfg.hg >= 2 ? 2 : 1;
  a.n_items = p.B * p.nq * cfg.hkv * (cfg.hg / hpw);
  const dim3 grid((unsigned)((a.n_items + kXcds - 1) / kXcds * kXcds));
  if (cfg.pool8) {
    switch (cfg.hg) {
      case 1: hipLaunchKernelGGL((attend_prompt_kernel<128, 1, 1, true>), grid, dim3(256), 0, st, a); break;
      case 2: hipLaunchKernelGGL((attend_prompt_kernel<128, 2, 2, true>), grid, dim3(512), 0, st, a); break;
      case 4: hipLaunchKernelGGL((attend_prompt_kernel<128, 4, 2, true>), grid, dim3(512), 0, st, a); break;
      default: hipLaunchKernelGGL((attend_prompt_kernel<128, 8, 2, true>), grid, dim3(512), 0, st, a); break;
    }
    return hipGetLastError();
  }
  switch (cfg.hg) {
    case 1: hipLaunchKernelGGL((attend_prompt_kernel<128, 1, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((attend_prompt_kernel<128, 2, 2>), grid, dim3(512), 0, st, a); break;
    case 4: hipLaunchKernelGGL((attend_prompt_kernel<128, 4, 2>), grid, dim3(512), 0, st, a); break;
    default: hipLaunchKernelGGL((attend_prompt_kernel<128, 8, 2>), grid, dim3(512), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace hga
