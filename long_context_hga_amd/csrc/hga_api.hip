// C ABI of the HGA hot path: host-side validation, workspace layout and
// launches.  Every check runs before anything is enqueued; no entry point
// allocates, frees or synchronises.  The one piece of library state is the
// per-device address of the static scratch array of hga_decode_step_noalloc.
#include <math.h>

#include <mutex>

#include "hga_internal.h"
#include "hga_gather_dev.h"

using namespace hga;

namespace {

constexpr int kMaxLqDecode = 15;
constexpr int kMaxListDecode = 256;  // 32 splits of 8 groups
constexpr int kMaxUnits = 1 << 20;
constexpr size_t kMaxRouteLds = 60 * 1024;
constexpr int64_t kMaxGridZ = 65535;

// Third grid dimension of the attention split kernels: B * (16-row column
// blocks of Hg*lq query rows) for decode, B for prefill.
// Selected lists per sequence: one per KV head, or one per query head.
int64_t lists_of(const hga_config* c) { return c->route_per_head ? c->n_q_heads : c->n_kv_heads; }

int64_t grid_z_of(const hga_config* c, int B, int lq) {
  if (lq >= 16) return B;
  const int rows = (c->route_per_head ? 1 : c->n_q_heads / c->n_kv_heads) * lq;
  return (int64_t)B * ((rows + 15) / 16);
}

hga_status check_cfg(const hga_config* c) {
  if (!c) return HGA_ERR_INVALID_ARGUMENT;
  if (c->head_dim <= 0 || c->head_dim % 2 != 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->n_q_heads % c->n_kv_heads != 0 || c->chunk_size <= 0 || c->groups_per_chunk <= 0 ||
      c->chunk_size % c->groups_per_chunk != 0 || c->n_sink_chunks < 0 || c->n_local_chunks < 0 ||
      c->topk_chunks < 0 || c->topk_groups < 0 || !(c->rope_theta > 1.0) ||
      !(c->hf_wavelength >= 0.0) || (c->qkv_dtype != HGA_F32 && c->qkv_dtype != HGA_BF16) ||
      (c->rep_position != 0 && c->rep_position != 1) ||
      (c->route_per_head != 0 && c->route_per_head != 1) ||
      (c->rope_style != 0 && c->rope_style != 1) || (c->pool_dtype != 0 && c->pool_dtype != 1) ||
      (c->route_pool != 0 && c->route_pool != 1))
    return HGA_ERR_INVALID_ARGUMENT;
  const int hg = c->n_q_heads / c->n_kv_heads;
  if ((c->head_dim != 64 && c->head_dim != 128) || c->chunk_size != kChunk ||
      c->groups_per_chunk != kGroups || (hg != 1 && hg != 2 && hg != 4 && hg != 8))
    return HGA_ERR_UNSUPPORTED;
  if (c->pool_dtype == 1 && (c->qkv_dtype != HGA_BF16 || c->head_dim != 128))
    return HGA_ERR_UNSUPPORTED;  // the FP8 pool: bf16 inputs, head_dim 128
  return HGA_OK;
}

KCfg make_kcfg(const hga_config* c) {
  KCfg k{};
  k.d = c->head_dim;
  k.hq = c->n_q_heads;
  k.hkv = c->n_kv_heads;
  k.hg = c->n_q_heads / c->n_kv_heads;
  k.lists = c->route_per_head ? c->n_q_heads : c->n_kv_heads;
  k.lhg = c->route_per_head ? 1 : k.hg;
  k.kvdiv = c->route_per_head ? k.hg : 1;
  k.n_sink = c->n_sink_chunks;
  k.n_local = c->n_local_chunks;
  k.topk_c = c->topk_chunks;
  k.topk_g = c->topk_groups;
  k.dtype = c->qkv_dtype;
  k.inv_sqrt_d = 1.0 / sqrt((double)c->head_dim);
  k.qscale_log2 = (float)(1.4426950408889634 / sqrt((double)c->head_dim));
  k.rep_shift = c->rep_position == 1 ? 0.5 : 0.0;
  k.interleaved = c->rope_style == 1;
  k.route_max = c->route_pool == 1 && k.lhg > 1;  // one head per list: the mean is the max
  k.pool8 = c->pool_dtype == 1;
  k.hf_mask = 0;
  for (int j = 0; j < c->head_dim / 2; ++j) {
    k.omega[j] = pow(c->rope_theta, -2.0 * (double)j / (double)c->head_dim);
    if (2.0 * M_PI / k.omega[j] < c->hf_wavelength) k.hf_mask |= 1ull << j;
  }
  return k;
}

int max_selected(const hga_config* c) {
  return (c->n_sink_chunks + c->n_local_chunks + 1) * c->groups_per_chunk + c->topk_groups;
}

hga_status hip_status(hipError_t e) { return e == hipSuccess ? HGA_OK : HGA_ERR_HIP; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Device address of pinned host memory (hipHostMalloc / pinned allocations);
// false if p is not pinned host memory.
bool pinned_device_ptr(const void* p, const void** dev) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (at.type != hipMemoryTypeHost || !at.devicePointer) return false;
  *dev = at.devicePointer;
  return true;
}

// Partial records per (unit, query token) of hga_attend_tiered: the window
// part's splits, then the routed part's.
int tiered_rec_splits(const hga_config* c) {
  const int w = (c->n_sink_chunks + c->n_local_chunks + 1) * c->groups_per_chunk;
  return (w + 7) / 8 + (c->topk_groups + 7) / 8;
}
size_t tiered_ws_bytes(const hga_config* c, const KCfg& k, int B, int lq) {
  const int pf = ((2 * k.lhg + 3) / 4 * 4) + k.lhg * k.d;
  return (size_t)B * k.lists * lq * tiered_rec_splits(c) * pf * sizeof(float);
}

}  // namespace

extern "C" {

hga_status hga_validate(const hga_config* cfg) { return check_cfg(cfg); }

hga_status hga_max_selected(const hga_config* cfg, int32_t max_lq, int32_t* out) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (!out || max_lq <= 0 || max_lq > kChunk) return HGA_ERR_INVALID_ARGUMENT;
  *out = max_selected(cfg);
  return HGA_OK;
}

hga_status hga_workspace_bytes(const hga_config* cfg, int32_t B, int32_t max_ctx, int32_t max_lq,
                               size_t* bytes) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (!bytes || B <= 0 || max_ctx <= 0 || max_lq <= 0 || max_lq > kChunk)
    return HGA_ERR_INVALID_ARGUMENT;
  const KCfg k = make_kcfg(cfg);
  const int max_chunks = (max_ctx + kChunk - 1) / kChunk;
  const size_t r = route_ws_bytes(k, B, max_chunks);
  size_t a = attend_ws_bytes(k, B, max_lq, max_selected(cfg));
  const size_t t = tiered_ws_bytes(cfg, k, B, max_lq);
  a = a > t ? a : t;
  *bytes = round_up(r > a ? r : a, 256);
  return HGA_OK;
}

hga_status hga_workspace_reset(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return HGA_ERR_INVALID_ARGUMENT;
  return hip_status(launch_fill_zero(ws, ws_bytes, (hipStream_t)stream));
}

hga_status hga_build_summaries(const hga_config* cfg, int32_t B, const void* k_raw,
                               const void* v_new, int32_t pos0, int32_t n_tok, void* k_pool,
                               void* v_pool, int32_t pool_cap, float* chunk_sum,
                               float* group_sum, int32_t max_chunks, void* stream) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (B <= 0 || !k_raw || pos0 < 0 || n_tok <= 0) return HGA_ERR_INVALID_ARGUMENT;
  const bool append = k_pool || v_pool;
  const bool summ = chunk_sum || group_sum;
  if (append && (!k_pool || !v_pool || !v_new || pool_cap <= 0 || pool_cap % kGroupTokens != 0))
    return HGA_ERR_INVALID_ARGUMENT;
  if (summ && (!chunk_sum || !group_sum || max_chunks <= 0)) return HGA_ERR_INVALID_ARGUMENT;
  const int64_t end = (int64_t)pos0 + n_tok;
  if (end > INT32_MAX) return HGA_ERR_OUT_OF_RANGE;
  if (append && end > pool_cap) return HGA_ERR_OUT_OF_RANGE;
  if (summ) {
    const int64_t last_complete = end / kChunk - 1;  // highest chunk that can complete here
    if (last_complete >= max_chunks) return HGA_ERR_OUT_OF_RANGE;
  }
  if (!append && !summ) return HGA_OK;
  const KCfg k = make_kcfg(cfg);
  if (append) {  // a pinned host pool is written through its device mapping
    const void* kd = nullptr;
    const void* vd = nullptr;
    if (pinned_device_ptr(k_pool, &kd)) k_pool = const_cast<void*>(kd);
    if (pinned_device_ptr(v_pool, &vd)) v_pool = const_cast<void*>(vd);
  }
  return hip_status(launch_build(k, B, k_raw, v_new, pos0, n_tok, append ? k_pool : nullptr,
                                 append ? v_pool : nullptr, pool_cap, summ ? chunk_sum : nullptr,
                                 summ ? group_sum : nullptr, max_chunks, (hipStream_t)stream));
}

hga_status hga_route(const hga_config* cfg, int32_t B, const void* q_raw, int32_t lq,
                     const int32_t* q_pos0, const float* chunk_sum, const float* group_sum,
                     int32_t max_chunks, int32_t* sel_groups, int32_t* n_sel, int32_t max_sel,
                     double* chunk_scores_opt, void* ws, size_t ws_bytes, void* stream) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (B <= 0 || !q_raw || lq <= 0 || lq > kChunk || !q_pos0 || !chunk_sum || !group_sum ||
      max_chunks <= 0 || !sel_groups || !n_sel || !ws)
    return HGA_ERR_INVALID_ARGUMENT;
  if (max_sel < max_selected(cfg)) return HGA_ERR_OUT_OF_RANGE;
  if ((int64_t)B * lists_of(cfg) > kMaxUnits) return HGA_ERR_UNSUPPORTED;
  const KCfg k = make_kcfg(cfg);
  if (route_select_lds(k, max_chunks) > kMaxRouteLds) return HGA_ERR_UNSUPPORTED;
  const size_t need = route_ws_bytes(k, B, max_chunks);
  if (ws_bytes < need) return HGA_ERR_WORKSPACE_TOO_SMALL;
  RouteLaunch r;
  r.q = q_raw;
  r.q_pos0 = q_pos0;
  r.chunk_sum = chunk_sum;
  r.group_sum = group_sum;
  r.sel = sel_groups;
  r.n_sel = n_sel;
  r.chunk_scores = chunk_scores_opt;
  const int max_cand = route_score_ld(k, max_chunks);  // padded score rows
  r.scores = static_cast<double*>(ws);
  r.qbar = r.scores + (size_t)B * k.lists * max_cand;
  r.B = B;
  r.lq = lq;
  r.nq = 1;
  r.q_tokens = lq;
  r.pool_once = 0;
  r.max_chunks = max_chunks;
  r.max_sel = max_sel;
  return hip_status(launch_route(k, r, (hipStream_t)stream));
}

hga_status hga_gather(const hga_config* cfg, int32_t B, const void* k_pool, const void* v_pool,
                      int32_t pool_cap, int32_t pool_is_host, const int32_t* sel_groups,
                      const int32_t* n_sel, int32_t max_sel, const int32_t* q_pos0, int32_t part,
                      void* k_ws, void* v_ws, void* stream) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (B <= 0 || !k_pool || !v_pool || pool_cap <= 0 || pool_cap % kGroupTokens != 0 ||
      !sel_groups || !n_sel || max_sel <= 0 ||
      !k_ws || !v_ws || part < HGA_PART_ALL || part > HGA_PART_ROUTED ||
      (part != HGA_PART_ALL && !q_pos0))
    return HGA_ERR_INVALID_ARGUMENT;
  if ((int64_t)max_sel * lists_of(cfg) * B > INT32_MAX) return HGA_ERR_UNSUPPORTED;
  const void* kp = k_pool;
  const void* vp = v_pool;
  if (pool_is_host && (!pinned_device_ptr(k_pool, &kp) || !pinned_device_ptr(v_pool, &vp)))
    return HGA_ERR_INVALID_ARGUMENT;
  const KCfg k = make_kcfg(cfg);
  return hip_status(launch_gather(k, B, kp, vp, pool_cap, sel_groups, n_sel, max_sel, q_pos0, part,
                                  k_ws, v_ws, pool_is_host != 0, (hipStream_t)stream));
}

hga_status hga_attend(const hga_config* cfg, int32_t B, const void* q_raw, int32_t lq,
                      const int32_t* q_pos0, const void* k_src, const void* v_src,
                      int32_t src_layout, int32_t src_cap, const int32_t* sel_groups,
                      const int32_t* n_sel, int32_t max_sel, int32_t part, float* out,
                      float* lse_opt, void* ws, size_t ws_bytes, void* stream) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (B <= 0 || !q_raw || lq <= 0 || lq > kChunk || !q_pos0 || !k_src || !v_src ||
      (src_layout != HGA_SRC_POOL && src_layout != HGA_SRC_WORKING_SET) || !sel_groups ||
      !n_sel || max_sel <= 0 || part < HGA_PART_ALL || part > HGA_PART_ROUTED || !out || !ws)
    return HGA_ERR_INVALID_ARGUMENT;
  if (src_layout == HGA_SRC_POOL && (src_cap <= 0 || src_cap % kGroupTokens != 0))
    return HGA_ERR_INVALID_ARGUMENT;
  // 16..64 query tokens run the MFMA prefill kernel: head_dim 128, bf16 (it
  // takes K/V as bf16 operands unrounded; an fp32 pool would need a
  // three-product split)
  if (lq > kMaxLqDecode && (cfg->qkv_dtype != HGA_BF16 || cfg->head_dim != 128))
    return HGA_ERR_UNSUPPORTED;
  if (max_sel > kMaxListDecode) return HGA_ERR_UNSUPPORTED;
  if ((int64_t)B * lists_of(cfg) * lq > kMaxUnits || grid_z_of(cfg, B, lq) > kMaxGridZ)
    return HGA_ERR_UNSUPPORTED;
  const KCfg k = make_kcfg(cfg);
  if (ws_bytes < attend_ws_bytes(k, B, lq, max_sel)) return HGA_ERR_WORKSPACE_TOO_SMALL;
  AttendLaunch a;
  a.q = q_raw;
  a.q_pos0 = q_pos0;
  a.k = k_src;
  a.v = v_src;
  a.sel = sel_groups;
  a.n_sel = n_sel;
  a.out = out;
  a.lse = lse_opt;
  a.part = static_cast<float*>(ws);
  a.B = B;
  a.lq = lq;
  a.src_layout = src_layout;
  a.src_cap = src_layout == HGA_SRC_POOL ? src_cap : max_sel * kGroupTokens;
  a.max_sel = max_sel;
  a.part_sel = part;
  a.two_part = 0;
  a.rec_splits = 0;
  return hip_status(launch_attend(k, a, (hipStream_t)stream));
}

// The fused step for lq query tokens of one chunk per sequence (decode:
// lq = 1; chunked prefill: up to a chunk).
static hga_status fused_step(const hga_config* cfg, int32_t B, const void* q_raw, int32_t lq,
                             const void* k_new, const void* v_new, const int32_t* q_pos0,
                             void* k_pool, void* v_pool, int32_t pool_cap, void* k_stage,
                             float* chunk_sum, float* group_sum, int32_t max_chunks,
                             int32_t* sel_groups, int32_t* n_sel, int32_t max_sel, float* out,
                             float* lse_opt, void* ws, size_t ws_bytes, void* stream,
                             bool launch = true) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (B <= 0 || lq <= 0 || lq > kChunk || !q_raw || !k_new || !v_new || !q_pos0 || !k_pool ||
      !v_pool || pool_cap <= 0 || pool_cap % kGroupTokens != 0 || !k_stage || !chunk_sum ||
      !group_sum || max_chunks <= 0 || !sel_groups || !n_sel || !out || !ws)
    return HGA_ERR_INVALID_ARGUMENT;
  if (lq > kMaxLqDecode && (cfg->qkv_dtype != HGA_BF16 || cfg->head_dim != 128))
    return HGA_ERR_UNSUPPORTED;
  if (max_sel < max_selected(cfg)) return HGA_ERR_OUT_OF_RANGE;
  if (max_sel > kMaxListDecode) return HGA_ERR_UNSUPPORTED;
  if ((int64_t)B * lists_of(cfg) * lq > kMaxUnits || grid_z_of(cfg, B, lq) > kMaxGridZ)
    return HGA_ERR_UNSUPPORTED;
  const KCfg k = make_kcfg(cfg);
  if (route_select_lds(k, max_chunks) > kMaxRouteLds) return HGA_ERR_UNSUPPORTED;
  const size_t need_r = route_ws_bytes(k, B, max_chunks);
  const size_t need_a = attend_ws_bytes(k, B, lq, max_sel);
  if (ws_bytes < need_r || ws_bytes < need_a) return HGA_ERR_WORKSPACE_TOO_SMALL;
  if (!launch) return HGA_OK;  // the checks only
  hipStream_t st = static_cast<hipStream_t>(stream);

  RouteLaunch r;
  r.q = q_raw;
  r.q_pos0 = q_pos0;
  r.chunk_sum = chunk_sum;
  r.group_sum = group_sum;
  r.sel = sel_groups;
  r.n_sel = n_sel;
  r.chunk_scores = nullptr;
  const int max_cand = route_score_ld(k, max_chunks);  // padded score rows
  r.scores = static_cast<double*>(ws);
  r.qbar = r.scores + (size_t)B * k.lists * max_cand;
  r.B = B;
  r.lq = lq;
  r.nq = 1;
  r.q_tokens = lq;
  r.pool_once = 0;
  r.max_chunks = max_chunks;
  r.max_sel = max_sel;
  r.pool_cap = pool_cap;
  StepFront f;
  f.k_new = k_new;
  f.v_new = v_new;
  f.k_stage = k_stage;
  f.k_pool = k_pool;
  f.v_pool = v_pool;
  f.pool_cap = pool_cap;
  f.chunk_sum = chunk_sum;
  f.group_sum = group_sum;
  hipError_t e = launch_route(k, r, st, &f);
  if (e != hipSuccess) return HGA_ERR_HIP;

  AttendLaunch a;
  a.q = q_raw;
  a.q_pos0 = q_pos0;
  a.k = k_pool;
  a.v = v_pool;
  a.sel = sel_groups;
  a.n_sel = n_sel;
  a.out = out;
  a.lse = lse_opt;
  a.part = static_cast<float*>(ws);
  a.B = B;
  a.lq = lq;
  a.src_layout = HGA_SRC_POOL;
  a.src_cap = pool_cap;
  a.max_sel = max_sel;
  a.part_sel = HGA_PART_ALL;
  a.two_part = 0;
  a.rec_splits = 0;
  return hip_status(launch_attend(k, a, st));
}

hga_status hga_decode_step(const hga_config* cfg, int32_t B, const void* q_raw, const void* k_new,
                           const void* v_new, const int32_t* q_pos0, void* k_pool, void* v_pool,
                           int32_t pool_cap, void* k_stage, float* chunk_sum, float* group_sum,
                           int32_t max_chunks, int32_t* sel_groups, int32_t* n_sel,
                           int32_t max_sel, float* out, float* lse_opt, void* ws, size_t ws_bytes,
                           void* stream) {
  return fused_step(cfg, B, q_raw, 1, k_new, v_new, q_pos0, k_pool, v_pool, pool_cap, k_stage,
                    chunk_sum, group_sum, max_chunks, sel_groups, n_sel, max_sel, out, lse_opt, ws,
                    ws_bytes, stream);
}

// Scratch of hga_decode_step_noalloc: one array per GPU (each device holds
// its own copy from the library's load until the process ends).  Host code
// never uses this name as an address: the device address comes from
// hipGetSymbolAddress, once per device, below.
static __device__ __align__(256) unsigned char scratch[HGA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once known

// Device address of the scratch array on the current device.
hga_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return HGA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return HGA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return HGA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HGA_OK;
}
}  // namespace

hga_status hga_decode_step_noalloc(const hga_config* cfg, int32_t B, const void* q_raw,
                                   const void* k_new, const void* v_new, const int32_t* q_pos0,
                                   void* k_pool, void* v_pool, int32_t pool_cap, void* k_stage,
                                   float* chunk_sum, float* group_sum, int32_t max_chunks,
                                   int32_t* sel_groups, int32_t* n_sel, int32_t max_sel,
                                   float* out, float* lse_opt, void* stream) {
  // every check first, against the scratch size (a stand-in pointer: nothing
  // is launched)
  hga_status s = fused_step(cfg, B, q_raw, 1, k_new, v_new, q_pos0, k_pool, v_pool, pool_cap,
                            k_stage, chunk_sum, group_sum, max_chunks, sel_groups, n_sel, max_sel,
                            out, lse_opt, reinterpret_cast<void*>(uintptr_t(256)),
                            HGA_NOALLOC_SCRATCH_BYTES, stream, false);
  if (s != HGA_OK) return s;
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != HGA_OK) return s;
  return fused_step(cfg, B, q_raw, 1, k_new, v_new, q_pos0, k_pool, v_pool, pool_cap, k_stage,
                    chunk_sum, group_sum, max_chunks, sel_groups, n_sel, max_sel, out, lse_opt, ws,
                    HGA_NOALLOC_SCRATCH_BYTES, stream);
}

hga_status hga_prefill_step(const hga_config* cfg, int32_t B, const void* q_raw, int32_t lq,
                            const void* k_new, const void* v_new, const int32_t* q_pos0,
                            void* k_pool, void* v_pool, int32_t pool_cap, void* k_stage,
                            float* chunk_sum, float* group_sum, int32_t max_chunks,
                            int32_t* sel_groups, int32_t* n_sel, int32_t max_sel, float* out,
                            float* lse_opt, void* ws, size_t ws_bytes, void* stream) {
  return fused_step(cfg, B, q_raw, lq, k_new, v_new, q_pos0, k_pool, v_pool, pool_cap, k_stage,
                    chunk_sum, group_sum, max_chunks, sel_groups, n_sel, max_sel, out, lse_opt, ws,
                    ws_bytes, stream);
}

// Whole-prompt prefill workspace: routing rows of every (sequence, query
// chunk, KV head) and the query chunks' first positions.
static size_t prompt_ws_bytes(const KCfg& k, int B, int T, int max_chunks) {
  const int nq = T / kChunk;
  return round_up(route_ws_bytes(k, B * nq, max_chunks), 256) + (size_t)B * nq * sizeof(int32_t);
}

hga_status hga_prompt_workspace_bytes(const hga_config* cfg, int32_t B, int32_t T,
                                      int32_t max_chunks, size_t* bytes) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (!bytes || B <= 0 || T <= 0 || T % kChunk != 0 || max_chunks < T / kChunk)
    return HGA_ERR_INVALID_ARGUMENT;
  *bytes = round_up(prompt_ws_bytes(make_kcfg(cfg), B, T, max_chunks), 256);
  return HGA_OK;
}

hga_status hga_prefill_prompt(const hga_config* cfg, int32_t B, int32_t T, const void* q_raw,
                              const void* k_raw, const void* v_raw, void* k_pool, void* v_pool,
                              int32_t pool_cap, float* chunk_sum, float* group_sum,
                              int32_t max_chunks, int32_t* sel_groups, int32_t* n_sel,
                              int32_t max_sel, float* out, float* lse_opt, int32_t phases,
                              void* ws, size_t ws_bytes, void* stream) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (B <= 0 || T <= 0 || T % kChunk != 0 || phases <= 0 || (phases & ~HGA_PROMPT_ALL) ||
      !k_pool || !v_pool || pool_cap <= 0 || pool_cap % kGroupTokens != 0 || !chunk_sum ||
      !group_sum || max_chunks <= 0 || !sel_groups || !n_sel || !ws)
    return HGA_ERR_INVALID_ARGUMENT;
  if ((phases & HGA_PROMPT_APPEND) && (!k_raw || !v_raw)) return HGA_ERR_INVALID_ARGUMENT;
  if ((phases & (HGA_PROMPT_ROUTE | HGA_PROMPT_ATTEND)) && !q_raw) return HGA_ERR_INVALID_ARGUMENT;
  if ((phases & HGA_PROMPT_ATTEND) && !out) return HGA_ERR_INVALID_ARGUMENT;
  if (T > pool_cap || T / kChunk > max_chunks) return HGA_ERR_OUT_OF_RANGE;
  if (cfg->qkv_dtype != HGA_BF16 || cfg->head_dim != 128 || cfg->route_per_head)
    return HGA_ERR_UNSUPPORTED;
  if (max_sel < max_selected(cfg)) return HGA_ERR_OUT_OF_RANGE;
  if (max_sel > kMaxListDecode) return HGA_ERR_UNSUPPORTED;
  const int nq = T / kChunk;
  const int64_t n_virtual = (int64_t)B * nq;
  if (n_virtual * cfg->n_kv_heads > kMaxUnits || n_virtual > kMaxGridZ ||
      n_virtual * cfg->n_q_heads > INT32_MAX / 2)
    return HGA_ERR_UNSUPPORTED;
  const KCfg k = make_kcfg(cfg);
  if (route_select_lds(k, max_chunks) > kMaxRouteLds) return HGA_ERR_UNSUPPORTED;
  if (ws_bytes < prompt_ws_bytes(k, B, T, max_chunks)) return HGA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);

  if (phases & HGA_PROMPT_APPEND) {
    const hipError_t e = launch_build(k, B, k_raw, v_raw, 0, T, k_pool, v_pool, pool_cap, chunk_sum,
                                      group_sum, max_chunks, st);
    if (e != hipSuccess) return HGA_ERR_HIP;
  }
  if (phases & HGA_PROMPT_ROUTE) {
    RouteLaunch r;
    r.q = q_raw;
    r.chunk_sum = chunk_sum;
    r.group_sum = group_sum;
    r.sel = sel_groups;
    r.n_sel = n_sel;
    r.chunk_scores = nullptr;
    const int max_cand = route_score_ld(k, max_chunks);  // padded score rows
    r.scores = static_cast<double*>(ws);
    r.qbar = r.scores + (size_t)n_virtual * k.lists * max_cand;
    int* pos = reinterpret_cast<int*>(static_cast<char*>(ws) +
                                      round_up(route_ws_bytes(k, (int)n_virtual, max_chunks), 256));
    r.q_pos0 = pos;
    r.B = (int)n_virtual;
    r.lq = kChunk;
    r.nq = nq;
    r.q_tokens = T;
    r.pool_once = 1;
    r.max_chunks = max_chunks;
    r.max_sel = max_sel;
    hipError_t e = launch_prompt_positions(pos, (int)n_virtual, nq, st);
    if (e != hipSuccess) return HGA_ERR_HIP;
    e = launch_route(k, r, st);
    if (e != hipSuccess) return HGA_ERR_HIP;
  }
  if (phases & HGA_PROMPT_ATTEND) {
    PromptLaunch p;
    p.q = q_raw;
    p.k = k_pool;
    p.v = v_pool;
    p.sel = sel_groups;
    p.n_sel = n_sel;
    p.out = out;
    p.lse = lse_opt;
    p.B = B;
    p.nq = nq;
    p.T = T;
    p.cap = pool_cap;
    p.max_sel = max_sel;
    return hip_status(launch_prompt_attend(k, p, st));
  }
  return HGA_OK;
}

hga_status hga_attend_tiered(const hga_config* cfg, int32_t B, const void* q_raw, int32_t lq,
                             const int32_t* q_pos0, const void* k_hot, const void* v_hot,
                             int32_t hot_cap, const void* k_cold, const void* v_cold,
                             int32_t cold_cap, const int32_t* sel_groups, const int32_t* n_sel,
                             int32_t max_sel, void* k_ws, void* v_ws, float* out, float* lse_opt,
                             void* ws, size_t ws_bytes, void* stream_a, void* stream_b,
                             void* ev_fork, void* ev_join) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (cfg->route_per_head) return HGA_ERR_UNSUPPORTED;
  if (B <= 0 || !q_raw || lq <= 0 || lq > kChunk || !q_pos0 || !k_hot || !v_hot ||
      hot_cap <= 0 || hot_cap % kGroupTokens != 0 || !k_cold || !v_cold || cold_cap <= 0 ||
      cold_cap % kGroupTokens != 0 || !sel_groups || !n_sel ||
      max_sel <= 0 || !k_ws || !v_ws || !out || !ws)
    return HGA_ERR_INVALID_ARGUMENT;
  if (lq > kMaxLqDecode && (cfg->qkv_dtype != HGA_BF16 || cfg->head_dim != 128))
    return HGA_ERR_UNSUPPORTED;
  if (max_sel > kMaxListDecode || tiered_rec_splits(cfg) > kMaxListDecode / 8)
    return HGA_ERR_UNSUPPORTED;
  if ((int64_t)B * lists_of(cfg) * lq > kMaxUnits || grid_z_of(cfg, B, lq) > kMaxGridZ)
    return HGA_ERR_UNSUPPORTED;
  const KCfg k = make_kcfg(cfg);
  if (ws_bytes < tiered_ws_bytes(cfg, k, B, lq)) return HGA_ERR_WORKSPACE_TOO_SMALL;
  if (stream_b && (!ev_fork || !ev_join || ev_fork == ev_join)) return HGA_ERR_INVALID_ARGUMENT;
  const void* kc = nullptr;
  const void* vc = nullptr;
  if (!pinned_device_ptr(k_cold, &kc) || !pinned_device_ptr(v_cold, &vc))
    return HGA_ERR_INVALID_ARGUMENT;
  hipStream_t sa = static_cast<hipStream_t>(stream_a);
  hipStream_t sb = static_cast<hipStream_t>(stream_b);
  const bool one_stream = stream_b == nullptr;

  // one partial buffer: the window part's splits, then the routed part's;
  // one merge over both
  AttendLaunch a;
  a.q = q_raw;
  a.q_pos0 = q_pos0;
  a.sel = sel_groups;
  a.n_sel = n_sel;
  a.out = out;
  a.lse = lse_opt;
  a.part = static_cast<float*>(ws);
  a.B = B;
  a.lq = lq;
  a.max_sel = max_sel;
  a.two_part = 1;
  a.rec_splits = tiered_rec_splits(cfg);
  AttendLaunch ah = a, ac = a;
  ah.k = k_hot;
  ah.v = v_hot;
  ah.src_layout = HGA_SRC_POOL;
  ah.src_cap = hot_cap;
  ah.part_sel = HGA_PART_WINDOWS;
  ac.k = k_ws;
  ac.v = v_ws;
  ac.src_layout = HGA_SRC_WORKING_SET;
  ac.src_cap = max_sel * kGroupTokens;
  ac.part_sel = HGA_PART_ROUTED;

  if (one_stream) {
    // one stream: the window part and the transfer share one launch (decode
    // shapes), then the routed part and the merge follow in order
    hipError_t e;
    if (lq <= kMaxLqDecode) {
      const GatherArgs g = make_gather_args(k, B, kc, vc, cold_cap, sel_groups, n_sel, max_sel,
                                            q_pos0, HGA_PART_ROUTED, k_ws, v_ws);
      e = launch_tiered_front(k, ah, g, max_sel * k.lists * B, sa);
    } else {
      e = launch_attend_split(k, ah, sa);
      if (e == hipSuccess)
        e = launch_gather(k, B, kc, vc, cold_cap, sel_groups, n_sel, max_sel, q_pos0,
                          HGA_PART_ROUTED, k_ws, v_ws, true, sa);
    }
    if (e == hipSuccess) e = launch_attend_split(k, ac, sa);
    if (e == hipSuccess) e = launch_attend_merge(k, a, sa);
    return hip_status(e);
  }

  // fork: stream b starts after everything already queued on stream a (the
  // list written by hga_route); join: the merge on stream a waits for b.  The
  // window part is queued right behind the fork, ahead of the transfer, so
  // its workgroups take their CUs before the copy kernel's waves (which
  // mostly wait on PCIe) fill the rest.  The two events are the caller's.
  hipEvent_t fork = static_cast<hipEvent_t>(ev_fork);
  hipEvent_t join = static_cast<hipEvent_t>(ev_join);
  hipError_t e = hipEventRecord(fork, sa);
  if (e == hipSuccess) e = launch_attend_split(k, ah, sa);
  if (e == hipSuccess) e = hipStreamWaitEvent(sb, fork, 0);
  if (e == hipSuccess)
    e = launch_gather(k, B, kc, vc, cold_cap, sel_groups, n_sel, max_sel, q_pos0, HGA_PART_ROUTED,
                      k_ws, v_ws, true, sb);
  if (e == hipSuccess) e = launch_attend_split(k, ac, sb);
  if (e == hipSuccess) e = hipEventRecord(join, sb);
  if (e == hipSuccess) e = hipStreamWaitEvent(sa, join, 0);
  if (e == hipSuccess) e = launch_attend_merge(k, a, sa);
  return hip_status(e);
}

hga_status hga_warm_workspace_bytes(const hga_config* cfg, int32_t B, int32_t max_sel,
                                    size_t* bytes) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (!bytes || B <= 0 || max_sel <= 0) return HGA_ERR_INVALID_ARGUMENT;
  *bytes = round_up(warm_ws_bytes(make_kcfg(cfg), B, max_sel), 256);
  return HGA_OK;
}

hga_status hga_warm_gather(const hga_config* cfg, int32_t B, const void* k_cold, const void* v_cold,
                           int32_t cold_cap, const int32_t* sel_groups, const int32_t* n_sel,
                           int32_t max_sel, const int32_t* q_pos0, void* k_warm, void* v_warm,
                           int32_t* warm_tags, int32_t* warm_used, int32_t n_warm, int32_t step,
                           void* k_ws, void* v_ws, int32_t* hits_opt, void* ws, size_t ws_bytes,
                           void* stream) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (B <= 0 || !k_cold || !v_cold || cold_cap <= 0 || cold_cap % kGroupTokens != 0 ||
      !sel_groups || !n_sel || max_sel <= 0 || !q_pos0 || !k_warm || !v_warm || !warm_tags ||
      !warm_used || !k_ws || !v_ws || !ws || step <= 0)
    return HGA_ERR_INVALID_ARGUMENT;
  if (max_sel > kMaxListDecode) return HGA_ERR_UNSUPPORTED;
  if (n_warm < cfg->topk_groups || n_warm < 1 || n_warm > 1024) return HGA_ERR_OUT_OF_RANGE;
  if ((int64_t)B * lists_of(cfg) * max_sel > INT32_MAX) return HGA_ERR_UNSUPPORTED;
  const KCfg k = make_kcfg(cfg);
  if (ws_bytes < warm_ws_bytes(k, B, max_sel)) return HGA_ERR_WORKSPACE_TOO_SMALL;
  const void* kc = nullptr;
  const void* vc = nullptr;
  if (!pinned_device_ptr(k_cold, &kc) || !pinned_device_ptr(v_cold, &vc))
    return HGA_ERR_INVALID_ARGUMENT;
  return hip_status(launch_warm(k, B, kc, vc, cold_cap, sel_groups, n_sel, max_sel, q_pos0, k_warm,
                                v_warm, warm_tags, warm_used, n_warm, step, k_ws, v_ws, hits_opt,
                                static_cast<int*>(ws), static_cast<hipStream_t>(stream)));
}

hga_status hga_merge_partials(const hga_config* cfg, int32_t B, int32_t lq, const float* out_a,
                              const float* lse_a, const float* out_b, const float* lse_b,
                              float* out, float* lse_out, void* stream) {
  hga_status s = check_cfg(cfg);
  if (s != HGA_OK) return s;
  if (B <= 0 || lq <= 0 || !out_a || !lse_a || !out_b || !lse_b || !out)
    return HGA_ERR_INVALID_ARGUMENT;
  return hip_status(launch_merge(B, cfg->n_q_heads, lq, cfg->head_dim, out_a, lse_a, out_b, lse_b,
                                 out, lse_out, (hipStream_t)stream));
}

const char* hga_status_string(hga_status s) {
  switch (s) {
    case HGA_OK: return "ok";
    case HGA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case HGA_ERR_UNSUPPORTED: return "unsupported configuration";
    case HGA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case HGA_ERR_OUT_OF_RANGE: return "position or size out of range";
    case HGA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t hga_version(void) { return 1; }

}  // extern "C"
