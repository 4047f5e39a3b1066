// Device body of the group gather (hga_gather, the host tier), shared by the
// gather kernel and the host tier's one-launch front (copy workgroups next to
// window-attention workgroups).
//
// HGA technical summary (gist.science), "Kernmechanisme" item 4 and
// "Geheugenarchitectuur": only the routed working set moves to accelerator
// memory; the full token K/V may stay in host RAM.  The gather copies whole
// 16-token groups (one contiguous 4 KiB row block per group, KV head and
// tensor at d = 128, bf16; the same block size for the transposed V
// groups), 16 bytes per lane, from device memory or directly from pinned host
// memory over PCIe.
#pragma once

#include "hga_internal.h"

namespace hga {

struct GatherArgs {
  const uint4* k_pool;
  const uint4* v_pool;
  uint4* k_ws;
  uint4* v_ws;
  const int* sel;
  const int* n_sel;
  const int* q_pos0;
  int lists, kvdiv, hkv, n_sink, n_local, pool_cap, max_sel, part, row_vecs;  // row_vecs: uint4 per token row
  // FP8 pool: the row scales after the codes, of the pool and of the working
  // set (null otherwise)
  const float* k_sc;
  const float* v_sc;
  float* k_sc_ws;
  float* v_sc_ws;
};

// A persistent grid of at most kGatherWgs workgroups walks the (slot, KV
// head, sequence) items; each item copies one group of K and of V (4 KiB
// each at d = 128, bf16; 2 KiB of codes and 64 bytes of row scales from the
// FP8 pool), 16 bytes per lane.  Reading a pinned host pool,
// the workgroups spend their time waiting on PCIe, so the grid is kept small
// enough to leave CUs to other work.
constexpr int kGatherWgs = 256;

inline GatherArgs make_gather_args(const KCfg& cfg, int B, const void* k_pool, const void* v_pool,
                                   int pool_cap, const int* sel, const int* n_sel, int max_sel,
                                   const int* q_pos0, int part, void* k_ws, void* v_ws) {
  GatherArgs a;
  a.k_pool = static_cast<const uint4*>(k_pool);
  a.v_pool = static_cast<const uint4*>(v_pool);
  a.k_ws = static_cast<uint4*>(k_ws);
  a.v_ws = static_cast<uint4*>(v_ws);
  a.sel = sel;
  a.n_sel = n_sel;
  a.q_pos0 = q_pos0;
  a.lists = cfg.lists;
  a.kvdiv = cfg.kvdiv;
  a.hkv = cfg.hkv;
  a.n_sink = cfg.n_sink;
  a.n_local = cfg.n_local;
  a.pool_cap = pool_cap;
  a.max_sel = max_sel;
  a.part = part;
  a.row_vecs = cfg.d * (cfg.pool8 ? 1 : (cfg.dtype == HGA_BF16 ? 2 : 4)) / 16;
  a.k_sc = a.v_sc = nullptr;
  a.k_sc_ws = a.v_sc_ws = nullptr;
  if (cfg.pool8) {  // codes of every unit, then the row scales
    const size_t pool_codes = (size_t)B * cfg.hkv * pool_cap * cfg.d;
    const size_t ws_codes = (size_t)B * cfg.lists * max_sel * kGroupTokens * cfg.d;
    a.k_sc = reinterpret_cast<const float*>(static_cast<const char*>(k_pool) + pool_codes);
    a.v_sc = reinterpret_cast<const float*>(static_cast<const char*>(v_pool) + pool_codes);
    a.k_sc_ws = reinterpret_cast<float*>(static_cast<char*>(k_ws) + ws_codes);
    a.v_sc_ws = reinterpret_cast<float*>(static_cast<char*>(v_ws) + ws_codes);
  }
  return a;
}

// Workgroup wg of n_wg copies items wg, wg + n_wg, ... (256 threads).
__device__ __forceinline__ void gather_items(const GatherArgs& a, int n_items, int wg, int n_wg) {
  for (int item = wg; item < n_items; item += n_wg) {
    const int slot = item % a.max_sel;
    const int unit = item / a.max_sel;  // b * lists + list
    const int b = unit / a.lists;
    const int unit_p = b * a.hkv + (unit % a.lists) / a.kvdiv;  // pool rows of its KV head
    // the list length and the slot's group id are read together (the slot
    // index is always inside the list buffer; the empty asm keeps the
    // compiler from issuing the second load after the first has returned);
    // the id is used only if the slot is listed
    int n_sel = a.n_sel[unit];
    int gid = a.sel[(size_t)unit * a.max_sel + slot];
    asm volatile("" : "+v"(n_sel), "+v"(gid));
    if (n_sel < 0 || slot >= n_sel) continue;  // uniform over the workgroup
    if (a.part != HGA_PART_ALL) {
      const int pos0 = a.q_pos0[b];
      // the list covers query tokens of one chunk; the last listed group holds
      // the last query token
      const int last_gid = a.sel[(size_t)unit * a.max_sel + n_sel - 1];
      const ListParts lp = list_parts(n_sel, last_gid * kGroupTokens, pos0, a.n_sink, a.n_local);
      const bool routed = slot >= lp.n_head && slot < lp.n_head + lp.n_routed;
      if ((a.part == HGA_PART_ROUTED) != routed) continue;
    }
    if (gid < 0 || (size_t)(gid + 1) * kGroupTokens > (size_t)a.pool_cap) continue;
    const int n = kGroupTokens * a.row_vecs;  // uint4 per group
    const size_t src = ((size_t)unit_p * a.pool_cap + (size_t)gid * kGroupTokens) * a.row_vecs;
    const size_t dst = ((size_t)unit * a.max_sel + slot) * kGroupTokens * a.row_vecs;
    for (int i = threadIdx.x; i < n; i += 256) {
      const uint4 kv = a.k_pool[src + i];
      const uint4 vv = a.v_pool[src + i];
      a.k_ws[dst + i] = kv;
      a.v_ws[dst + i] = vv;
    }
    if (a.k_sc && threadIdx.x < kGroupTokens) {  // FP8: the group's 16 row scales of K and V
      const size_t ss = (size_t)unit_p * a.pool_cap + (size_t)gid * kGroupTokens + threadIdx.x;
      const size_t sd = ((size_t)unit * a.max_sel + slot) * kGroupTokens + threadIdx.x;
      a.k_sc_ws[sd] = a.k_sc[ss];
      a.v_sc_ws[sd] = a.v_sc[ss];
    }
  }
}

}  // namespace hga
