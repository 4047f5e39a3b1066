// Warm tier of a host-memory pool: a bounded LRU cache in device memory of
// recently routed groups.
//
// HGA technical summary (gist.science), "Geheugenarchitectuur": summaries and
// the always-visible windows are hot in accelerator memory, a bounded LRU
// cache in accelerator memory keeps the chunks routing picked lately (warm), and the
// full token K/V history stays in host RAM (cold).  The cache holds the unit
// the routing delivers and the attention reads, the 16-token group, so a miss
// moves only the selected group across PCIe.
//
// Per (sequence, list) unit the cache has n_warm slots, each one group of K
// (4 KiB at d = 128, bf16; with the FP8 pool its codes, the cache's row
// scales following the codes of every slot) and its V^T block, with a tag
// (group id, -1 = empty) and the step that last used it.  One call:
//   warm_update_kernel (one workgroup per unit): the tags go into an LDS
//     hash table; the routed groups of the unit's list found there are hits
//     (their stamps renewed); the i-th miss in list order takes the i-th
//     least recently used slot that is not a hit this step (stamp order,
//     ties by slot index, empty slots first); tags and stamps are rewritten
//     and the fill plan (slot and source of every routed list position) goes
//     to the workspace;
//   warm_fill_kernel (persistent grid): a miss copies its group from the
//     pinned host pool over PCIe into its cache slot and into the working
//     set, a hit copies its cache slot into the working set.
// The working set then holds the routed part of every list, as hga_gather
// with HGA_PART_ROUTED would leave it.
#include "hga_internal.h"

namespace hga {

struct WarmArgs {
  const int* sel;      // [units][max_sel]
  const int* n_sel;    // [units]
  const int* q_pos0;   // [B]
  const uint4* k_cold;  // pinned host pool (device mapping), [units_kv][cap][row]
  const uint4* v_cold;
  uint4* k_warm;        // [units][W][16 rows]
  uint4* v_warm;
  uint4* k_ws;          // [units][max_sel * 16 rows]
  uint4* v_ws;
  int* tags;           // [units][W]
  int* used;           // [units][W]
  int* hits;           // [units] or null
  int* slot_of;        // workspace [units][max_sel]: cache slot of a routed list position, else -1
  int* src_of;         // workspace [units][max_sel]: group to fetch (miss), -1 for a hit
  int lists, hkv, kvdiv, n_sink, n_local, cap, max_sel, W, step, row_vecs;
  // FP8 pool: the row scales after the codes of the host pool, the cache and
  // the working set (null otherwise)
  const float* k_sc_cold;
  const float* v_sc_cold;
  float* k_sc_warm;
  float* v_sc_warm;
  float* k_sc_ws;
  float* v_sc_ws;
};

constexpr int kMaxWarm = 1024;  // slots per unit
constexpr int kWarmHash = 2048; // open-addressing table of the tags (>= 2 * kMaxWarm)

__device__ __forceinline__ int warm_hash(int gid) {
  return (int)(((uint32_t)gid * 2654435761u) >> 21);  // 11 bits
}

__global__ __launch_bounds__(256) void warm_update_kernel(WarmArgs a) {
  __shared__ int s_tag[kMaxWarm];
  __shared__ int s_used[kMaxWarm];
  __shared__ int s_hit[kMaxWarm];      // 1 if the slot is a hit this step
  __shared__ int s_victim[kMaxWarm];    // s_victim[r]: the r-th least recently used free slot
  __shared__ __align__(16) int s_key[kMaxWarm];  // victim order key of a slot
  __shared__ int wave_miss[4];
  __shared__ int s_hkey[kWarmHash];    // tag hash: group id (-1 = empty)
  __shared__ int s_hval[kWarmHash];    // its slot
  __shared__ int s_sel[256];            // the unit's list (max_sel <= 256)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = blockIdx.x;
  const int b = unit / a.lists;
  const int W = a.W;
  int* slot_of = a.slot_of + (size_t)unit * a.max_sel;
  int* src_of = a.src_of + (size_t)unit * a.max_sel;
  // every load the unit needs goes out at once: its list, count and position,
  // the tags and the stamps
  const int* sel = a.sel + (size_t)unit * a.max_sel;
  const int n_sel = a.n_sel[unit];
  const int pos0 = a.q_pos0[b];
  if (tid < a.max_sel) s_sel[tid] = sel[tid];
  for (int s = tid; s < W; s += 256) {
    s_tag[s] = a.tags[(size_t)unit * W + s];
    s_used[s] = a.used[(size_t)unit * W + s];
    s_hit[s] = 0;
  }
  for (int h = tid; h < kWarmHash; h += 256) s_hkey[h] = -1;
  for (int i = tid; i < a.max_sel; i += 256) {
    slot_of[i] = -1;
    src_of[i] = -1;
  }
  if (n_sel <= 0 || n_sel > a.max_sel) {  // no usable list: nothing routed (uniform)
    if (a.hits && tid == 0) a.hits[unit] = 0;
    return;
  }
  __syncthreads();
  const ListParts lp = list_parts(n_sel, s_sel[n_sel - 1] * kGroupTokens, pos0, a.n_sink, a.n_local);
  const int n_routed = lp.n_routed < 0 ? 0 : lp.n_routed;
  // the cached tags into the hash table (tags are distinct; linear probing)
  for (int s = tid; s < W; s += 256) {
    const int t = s_tag[s];
    if (t < 0) continue;
    int h = warm_hash(t);
    while (atomicCAS(&s_hkey[h], -1, t) != -1) h = (h + 1) & (kWarmHash - 1);
    s_hval[h] = s;
  }
  __syncthreads();
  // hits: routed list position n_head + i (thread i) scans the tags
  int my_gid = -1, my_slot = -1;
  // (a group id outside the pool is not routed data: it is neither cached nor
  // fetched, and its working-set slot is left as it was)
  bool routed = false;
  if (tid < n_routed) {
    my_gid = s_sel[lp.n_head + tid];
    routed = my_gid >= 0 && (size_t)(my_gid + 1) * kGroupTokens <= (size_t)a.cap;
    if (routed) {
      for (int h = warm_hash(my_gid); s_hkey[h] != -1; h = (h + 1) & (kWarmHash - 1))
        if (s_hkey[h] == my_gid) {
          my_slot = s_hval[h];
          break;
        }
      if (my_slot >= 0) s_hit[my_slot] = 1;
    }
  }
  const bool miss = routed && my_slot < 0;
  // misses in list order: exclusive scan of the miss flags
  const int incl = wave_incl_scan(miss ? 1 : 0);
  if (lane == 63) wave_miss[wave] = incl;
  __syncthreads();
  int m = 0, before = 0;
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? wave_miss[w] : 0;
    m += wave_miss[w];
  }
  const int my_rank = before + incl - (miss ? 1 : 0);
  // victims: the non-hit slots ranked by (stamp, slot index) -- empty slots
  // carry stamp 0 and every stamp is below this call's step -- and the m
  // first taken.  A slot's rank is the count of slots before it in that
  // order; hits carry the key INT_MAX and are never counted.  The keys are
  // read 16 bytes at a time by every thread at once (LDS broadcasts).
  const int W4 = (W + 3) / 4;
  for (int s = tid; s < 4 * W4; s += 256) s_key[s] = (s >= W || s_hit[s]) ? 0x7FFFFFFF : s_used[s];
  __syncthreads();
  const int4* key4 = reinterpret_cast<const int4*>(s_key);
  for (int s = tid; s < W; s += 256) {
    const int key = s_key[s];
    if (key == 0x7FFFFFFF) continue;
    int r = 0;
#pragma unroll 8
    for (int t4 = 0; t4 < W4; ++t4) {
      const int4 v = key4[t4];
      const int t = 4 * t4;
      r += (v.x < key || (v.x == key && t < s)) ? 1 : 0;
      r += (v.y < key || (v.y == key && t + 1 < s)) ? 1 : 0;
      r += (v.z < key || (v.z == key && t + 2 < s)) ? 1 : 0;
      r += (v.w < key || (v.w == key && t + 3 < s)) ? 1 : 0;
    }
    if (r < m) s_victim[r] = s;
  }
  __syncthreads();
  if (miss) {
    const int slot = s_victim[my_rank];
    s_tag[slot] = my_gid;
    s_used[slot] = a.step;
    slot_of[lp.n_head + tid] = slot;
    src_of[lp.n_head + tid] = my_gid;
  } else if (routed) {
    s_used[my_slot] = a.step;
    slot_of[lp.n_head + tid] = my_slot;
  }
  __syncthreads();
  for (int s = tid; s < W; s += 256) {
    a.tags[(size_t)unit * W + s] = s_tag[s];
    a.used[(size_t)unit * W + s] = s_used[s];
  }
  if (a.hits) {  // routed groups found in the cache
    const int h = wave_incl_scan(routed && !miss ? 1 : 0);
    if (lane == 63) wave_miss[wave] = h;  // every wave read wave_miss before the top-k barriers
    __syncthreads();
    if (tid == 0) a.hits[unit] = wave_miss[0] + wave_miss[1] + wave_miss[2] + wave_miss[3];
  }
}

// Persistent grid: item = (list position, unit).
__global__ __launch_bounds__(256) void warm_fill_kernel(WarmArgs a, int n_items) {
  const int n = kGroupTokens * a.row_vecs;  // uint4 per group and tensor
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int p = item % a.max_sel, unit = item / a.max_sel;
    const int slot = a.slot_of[(size_t)unit * a.max_sel + p];
    if (slot < 0) continue;  // uniform over the workgroup
    const int src = a.src_of[(size_t)unit * a.max_sel + p];
    const size_t wdst = ((size_t)unit * a.W + slot) * n;
    const size_t dst = ((size_t)unit * a.max_sel + p) * n;
    // FP8: the 16 row scales of K and V of the group (token rows of the slot)
    const size_t wsd = ((size_t)unit * a.W + slot) * kGroupTokens + threadIdx.x;
    const size_t sd = ((size_t)unit * a.max_sel + p) * kGroupTokens + threadIdx.x;
    const bool scales = a.k_sc_cold && threadIdx.x < kGroupTokens;
    if (src >= 0) {  // miss: host pool -> cache slot and working set
      const int unit_p = (unit / a.lists) * a.hkv + (unit % a.lists) / a.kvdiv;
      const size_t from = ((size_t)unit_p * a.cap + (size_t)src * kGroupTokens) * a.row_vecs;
      for (int i = threadIdx.x; i < n; i += 256) {
        const uint4 kv = a.k_cold[from + i];
        const uint4 vv = a.v_cold[from + i];
        a.k_warm[wdst + i] = kv;
        a.v_warm[wdst + i] = vv;
        a.k_ws[dst + i] = kv;
        a.v_ws[dst + i] = vv;
      }
      if (scales) {
        const size_t ss = (size_t)unit_p * a.cap + (size_t)src * kGroupTokens + threadIdx.x;
        const float ks = a.k_sc_cold[ss], vs = a.v_sc_cold[ss];
        a.k_sc_warm[wsd] = ks;
        a.v_sc_warm[wsd] = vs;
        a.k_sc_ws[sd] = ks;
        a.v_sc_ws[sd] = vs;
      }
    } else {  // hit: cache slot -> working set
      for (int i = threadIdx.x; i < n; i += 256) {
        const uint4 kv = a.k_warm[wdst + i];
        const uint4 vv = a.v_warm[wdst + i];
        a.k_ws[dst + i] = kv;
        a.v_ws[dst + i] = vv;
      }
      if (scales) {
        a.k_sc_ws[sd] = a.k_sc_warm[wsd];
        a.v_sc_ws[sd] = a.v_sc_warm[wsd];
      }
    }
  }
}

hipError_t launch_warm(const KCfg& cfg, int B, const void* k_cold, const void* v_cold, int cap,
                       const int* sel, const int* n_sel, int max_sel, const int* q_pos0,
                       void* k_warm, void* v_warm, int* tags, int* used, int n_warm, int step,
                       void* k_ws, void* v_ws, int* hits, int* plan, hipStream_t st) {
  WarmArgs a;
  a.sel = sel;
  a.n_sel = n_sel;
  a.q_pos0 = q_pos0;
  a.k_cold = static_cast<const uint4*>(k_cold);
  a.v_cold = static_cast<const uint4*>(v_cold);
  a.k_warm = static_cast<uint4*>(k_warm);
  a.v_warm = static_cast<uint4*>(v_warm);
  a.k_ws = static_cast<uint4*>(k_ws);
  a.v_ws = static_cast<uint4*>(v_ws);
  a.tags = tags;
  a.used = used;
  a.hits = hits;
  const int units = B * cfg.lists;
  a.slot_of = plan;
  a.src_of = plan + (size_t)units * max_sel;
  a.lists = cfg.lists;
  a.hkv = cfg.hkv;
  a.kvdiv = cfg.kvdiv;
  a.n_sink = cfg.n_sink;
  a.n_local = cfg.n_local;
  a.cap = cap;
  a.max_sel = max_sel;
  a.W = n_warm;
  a.step = step;
  a.row_vecs = cfg.d * (cfg.pool8 ? 1 : (cfg.dtype == HGA_BF16 ? 2 : 4)) / 16;
  a.k_sc_cold = a.v_sc_cold = nullptr;
  a.k_sc_warm = a.v_sc_warm = a.k_sc_ws = a.v_sc_ws = nullptr;
  if (cfg.pool8) {  // codes of every unit, then the row scales
    auto after = [&](const void* p, size_t codes) {
      return reinterpret_cast<const float*>(static_cast<const char*>(p) + codes);
    };
    const size_t cold = (size_t)B * cfg.hkv * cap * cfg.d;
    const size_t warm = (size_t)units * n_warm * kGroupTokens * cfg.d;
    const size_t wset = (size_t)units * max_sel * kGroupTokens * cfg.d;
    a.k_sc_cold = after(k_cold, cold);
    a.v_sc_cold = after(v_cold, cold);
    a.k_sc_warm = const_cast<float*>(after(k_warm, warm));
    a.v_sc_warm = const_cast<float*>(after(v_warm, warm));
    a.k_sc_ws = const_cast<float*>(after(k_ws, wset));
    a.v_sc_ws = const_cast<float*>(after(v_ws, wset));
  }
  hipLaunchKernelGGL(warm_update_kernel, dim3(units), dim3(256), 0, st, a);
  const int n_items = units * max_sel;
  const int n_wg = n_items < 256 ? n_items : 256;
  hipLaunchKernelGGL(warm_fill_kernel, dim3(n_wg), dim3(256), 0, st, a, n_items);
  return hipGetLastError();
}

size_t warm_ws_bytes(const KCfg& cfg, int B, int max_sel) {
  return (size_t)2 * B * cfg.lists * max_sel * sizeof(int);
}

}  // namespace hga
