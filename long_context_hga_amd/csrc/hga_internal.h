// Host-side declarations shared by the HGA translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "hga_device.h"

namespace hga {

hipError_t launch_build(const KCfg& cfg, int B, const void* k_raw, const void* v_new, int pos0,
                        int n_tok, void* k_pool, void* v_pool, int pool_cap, float* chunk_sum,
                        float* group_sum, int max_chunks, hipStream_t st);

struct RouteLaunch {
  const void* q;
  const int* q_pos0;
  const float* chunk_sum;
  const float* group_sum;
  int* sel;
  int* n_sel;
  double* chunk_scores;
  double* scores;       // workspace [B*Hkv][max_cand]
  double* qbar;         // workspace [B*Hkv][d]
  int B, lq, max_chunks, max_sel;
  // B counts virtual sequences: virtual sequence b routes query chunk b % nq
  // of pool sequence b / nq (nq = 1 outside whole-prompt prefill).  Its lq
  // query tokens are rows (b % nq) * lq .. of q [B/nq][Hq][q_tokens][d];
  // positions, lists and workspace rows are per virtual sequence, summaries
  // per pool sequence.
  int nq, q_tokens;
  // 1: the multi-token pooled query of each unit is formed by a launch of
  // its own and read by the tile workgroups (many units, many tiles each)
  int pool_once;
  // > 0 (a fused step): tokens per unit of the pool the step appends to; a
  // position whose tokens do not fit is unusable (n_sel = -1)
  int pool_cap = 0;
};
// The token work of a fused decode step, run by extra workgroups of the
// selection launch: the new token's pool append, its raw key into the chunk
// staging rows, and the summaries of the chunk it completes.
struct StepFront {
  const void* k_new;  // [B][Hkv][d] raw key of the new token (position q_pos0[b])
  const void* v_new;  // [B][Hkv][d]
  void* k_stage;      // [B][Hkv][C][d] raw keys of the current chunk
  void* k_pool;
  void* v_pool;
  int pool_cap;
  float* chunk_sum;   // written for a completed chunk
  float* group_sum;
};
hipError_t launch_route(const KCfg& cfg, const RouteLaunch& r, hipStream_t st,
                        const StepFront* front = nullptr);
size_t route_ws_bytes(const KCfg& cfg, int B, int max_chunks);
// Row stride of the level-1 scores in the route workspace; the pooled query
// rows follow B * lists * route_score_ld doubles from the start.
int route_score_ld(const KCfg& cfg, int max_chunks);
size_t route_select_lds(const KCfg& cfg, int max_chunks);

struct AttendLaunch {
  const void* q;
  const int* q_pos0;
  const void* k;
  const void* v;
  const int* sel;
  const int* n_sel;
  float* out;
  float* lse;
  float* part;          // workspace partials
  int B, lq, src_layout, src_cap, max_sel, part_sel;
  // Two-part record layout (host tier): the window part's splits are records
  // [0, ceil(n_w/8)), the routed part's follow; rec_splits records per
  // (unit, query token).  two_part = 0: one part, ceil(max_sel/8) records.
  int two_part, rec_splits;
};
hipError_t launch_attend(const KCfg& cfg, const AttendLaunch& a, hipStream_t st);
hipError_t launch_attend_split(const KCfg& cfg, const AttendLaunch& a, hipStream_t st);
hipError_t launch_attend_merge(const KCfg& cfg, const AttendLaunch& a, hipStream_t st);
// Host tier in one stream: the window part's decode splits (win, lq <= 15)
// and the gather g of n_items (slot, KV head, sequence) items in one launch.
struct GatherArgs;
hipError_t launch_tiered_front(const KCfg& cfg, const AttendLaunch& win, const GatherArgs& g,
                               int n_items, hipStream_t st);
size_t attend_ws_bytes(const KCfg& cfg, int B, int lq, int max_sel);

// Whole-prompt prefill: attention of every query chunk of the prompt over
// its selected list (virtual sequence b * nq + qc = chunk qc of sequence b).
struct PromptLaunch {
  const void* q;       // [B][Hq][T][d]
  const void* k;       // pool
  const void* v;
  const int* sel;      // [B*nq][Hkv][max_sel]
  const int* n_sel;    // [B*nq][Hkv]
  float* out;          // [B][Hq][T][d]
  float* lse;          // [B][Hq][T] or null
  int B, nq, T, cap, max_sel;
};
hipError_t launch_prompt_positions(int* pos, int n_virtual, int nq, hipStream_t st);
hipError_t launch_prompt_attend(const KCfg& cfg, const PromptLaunch& p, hipStream_t st);

// from_host: the pool is pinned host memory read over PCIe (a small
// persistent grid); otherwise one workgroup per copied group.
// Warm tier: LRU update of the routed groups of every list over n_warm
// cache slots per unit, then the fill of the working set (misses over PCIe
// from the pinned pool, hits from the cache).  plan: workspace of
// warm_ws_bytes.
hipError_t launch_warm(const KCfg& cfg, int B, const void* k_cold, const void* v_cold, int cap,
                       const int* sel, const int* n_sel, int max_sel, const int* q_pos0,
                       void* k_warm, void* v_warm, int* tags, int* used, int n_warm, int step,
                       void* k_ws, void* v_ws, int* hits, int* plan, hipStream_t st);
size_t warm_ws_bytes(const KCfg& cfg, int B, int max_sel);

hipError_t launch_gather(const KCfg& cfg, int B, const void* k_pool, const void* v_pool,
                         int pool_cap, const int* sel, const int* n_sel, int max_sel,
                         const int* q_pos0, int part, void* k_ws, void* v_ws, bool from_host,
                         hipStream_t st);

hipError_t launch_merge(int B, int hq, int lq, int d, const float* oa, const float* la,
                        const float* ob, const float* lb, float* out, float* lse, hipStream_t st);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

// Position of list slots by part: the selected list of a unit is ordered
// sink groups | routed groups | local groups | current-chunk groups.
struct ListParts {
  int n_head;    // sink groups
  int n_routed;  // routed groups
  int n_tail;    // local + current groups
};
__device__ __host__ inline ListParts list_parts(int n_sel, int pos_last, int lq_first_pos,
                                                int n_sink, int n_local) {
  const int ct = lq_first_pos / kChunk;
  const Windows w = windows_of(ct, n_sink, n_local);
  ListParts lp;
  lp.n_head = w.sink_end * kGroups;
  const int cur = pos_last / kGroupTokens - ct * kGroups + 1;
  lp.n_tail = (ct - w.local_begin) * kGroups + cur;
  lp.n_routed = n_sel - lp.n_head - lp.n_tail;
  return lp;
}

}  // namespace hga
