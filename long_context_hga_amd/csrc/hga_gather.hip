// Gather of the selected token K/V into a compact working set, exact merge of
// two attention partials, and the workspace fill.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 4 and
// "Geheugenarchitectuur": only the routed working set moves to accelerator
// memory; the full token K/V may stay in host RAM.  The gather copies whole
// 16-token groups (one contiguous 4 KiB row block per group, KV head and
// tensor at d = 128, bf16; the same block size for the transposed V
// groups), 16 bytes per lane, from device memory or directly from pinned host
// memory over PCIe.
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
  int hkv, n_sink, n_local, pool_cap, max_sel, part, row_vecs;  // row_vecs: uint4 per token row
};

// A persistent grid of at most kGatherWgs workgroups walks the (slot, KV
// head, sequence) items; each item copies one group of K and of V (4 KiB
// each at d = 128, bf16), 16 bytes per lane.  Reading a pinned host pool,
// the workgroups spend their time waiting on PCIe, so the grid is kept small
// enough to leave CUs to work queued on other streams.
constexpr int kGatherWgs = 256;

__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a, int n_items) {
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int slot = item % a.max_sel;
    const int unit = item / a.max_sel;  // b * Hkv + h
    const int b = unit / a.hkv;
    const int n_sel = a.n_sel[unit];
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
    const int gid = a.sel[(size_t)unit * a.max_sel + slot];
    if (gid < 0 || (size_t)(gid + 1) * kGroupTokens > (size_t)a.pool_cap) continue;
    const int n = kGroupTokens * a.row_vecs;  // uint4 per group
    const size_t src = ((size_t)unit * a.pool_cap + (size_t)gid * kGroupTokens) * a.row_vecs;
    const size_t dst = ((size_t)unit * a.max_sel + slot) * kGroupTokens * a.row_vecs;
    for (int i = threadIdx.x; i < n; i += 256) {
      const uint4 kv = a.k_pool[src + i];
      const uint4 vv = a.v_pool[src + i];
      a.k_ws[dst + i] = kv;
      a.v_ws[dst + i] = vv;
    }
  }
}

hipError_t launch_gather(const KCfg& cfg, int B, const void* k_pool, const void* v_pool,
                         int pool_cap, const int* sel, const int* n_sel, int max_sel,
                         const int* q_pos0, int part, void* k_ws, void* v_ws, hipStream_t st) {
  GatherArgs a;
  a.k_pool = static_cast<const uint4*>(k_pool);
  a.v_pool = static_cast<const uint4*>(v_pool);
  a.k_ws = static_cast<uint4*>(k_ws);
  a.v_ws = static_cast<uint4*>(v_ws);
  a.sel = sel;
  a.n_sel = n_sel;
  a.q_pos0 = q_pos0;
  a.hkv = cfg.hkv;
  a.n_sink = cfg.n_sink;
  a.n_local = cfg.n_local;
  a.pool_cap = pool_cap;
  a.max_sel = max_sel;
  a.part = part;
  a.row_vecs = cfg.d * (cfg.dtype == HGA_BF16 ? 2 : 4) / 16;
  const int n_items = max_sel * cfg.hkv * B;
  const int n_wg = n_items < kGatherWgs ? n_items : kGatherWgs;
  hipLaunchKernelGGL(gather_kernel, dim3(n_wg), dim3(256), 0, st, a, n_items);
  return hipGetLastError();
}

// out = (e^la oa + e^lb ob) / (e^la + e^lb); one thread per output element.
__global__ __launch_bounds__(256) void merge_kernel(const float* oa, const float* la, const float* ob,
                                                    const float* lb, float* out, float* lse,
                                                    long rows, int d) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * d) return;
  const long r = i / d;
  const float a = la[r], b = lb[r];
  const float m = fmaxf(a, b);
  float wa = 0.f, wb = 0.f;
  if (m != -INFINITY) {
    wa = expf(a - m);
    wb = expf(b - m);
  }
  const float den = wa + wb;
  const float x = oa[i], y = ob[i];
  out[i] = den > 0.f ? (wa * x + wb * y) / den : 0.f;
  if (lse && i % d == 0) lse[r] = den > 0.f ? m + logf(den) : -INFINITY;
}

hipError_t launch_merge(int B, int hq, int lq, int d, const float* oa, const float* la,
                        const float* ob, const float* lb, float* out, float* lse, hipStream_t st) {
  const long rows = (long)B * hq * lq;
  const long n = rows * d;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, oa, la, ob,
                     lb, out, lse, rows, d);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0, 0, 0, 0);
  if (i < ntail) tail[i] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  const size_t n = n16 > ntail ? n16 : ntail;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     static_cast<uint4*>(p), n16, static_cast<unsigned char*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace hga
