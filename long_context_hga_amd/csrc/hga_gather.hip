// Gather of the selected token K/V into a compact working set (body in
// hga_gather_dev.h), exact merge of two attention partials, and the workspace
// fill.
#include "hga_gather_dev.h"

namespace hga {

__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a, int n_items) {
  gather_items(a, n_items, blockIdx.x, gridDim.x);
}

hipError_t launch_gather(const KCfg& cfg, int B, const void* k_pool, const void* v_pool,
                         int pool_cap, const int* sel, const int* n_sel, int max_sel,
                         const int* q_pos0, int part, void* k_ws, void* v_ws, bool from_host,
                         hipStream_t st) {
  const GatherArgs a = make_gather_args(cfg, B, k_pool, v_pool, pool_cap, sel, n_sel, max_sel,
                                        q_pos0, part, k_ws, v_ws);
  const int n_items = max_sel * cfg.lists * B;
  // over PCIe a few hundred workgroups keep the link busy and leave CUs to
  // other work; from HBM every group gets its own workgroup so that all its
  // loads are in flight at once
  const int n_wg = from_host ? (n_items < kGatherWgs ? n_items : kGatherWgs) : n_items;
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
