// Calibration kernels for the benchmark (not part of the HGA path): the rate
// of a plain device-to-device copy on this device, in a few shapes, to set
// the attainable ceiling next to the 8 TB/s published HBM peak for the
// gather (which reads and writes every selected byte once).  The caller owns
// both buffers; nothing is allocated here.
#include <hip/hip_runtime.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// U uint4 per thread, all loads issued before the stores; block b covers
// the U * 256 consecutive uint4 starting at b * U * 256 (lane-contiguous per
// step).  NT: non-temporal loads and stores.
template <int U, bool NT>
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   size_t n) {
  const size_t base = (size_t)blockIdx.x * U * 256 + threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = base + (size_t)u * 256;
    if (i < n) v[u] = NT ? __builtin_nontemporal_load(src + i) : src[i];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = base + (size_t)u * 256;
    if (i < n) {
      if (NT) __builtin_nontemporal_store(v[u], dst + i);
      else dst[i] = v[u];
    }
  }
}

// Grid-stride form: a fixed grid of `blocks` workgroups walks the buffer.
__global__ __launch_bounds__(256) void copy_stride_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    dst[i] = src[i];
}

// Per-workgroup read rate: workgroup w reads its own `per_wg` bytes (16
// uint4 per thread in flight), folding them into one word per thread so the
// loads stay.  With few workgroups this is the rate one CU pulls on its own.
template <int NT>
__global__ __launch_bounds__(NT) void cu_read_kernel(const u32x4* __restrict__ src, size_t per_wg,
                                                     uint32_t* __restrict__ out) {
  const u32x4* base = src + (size_t)blockIdx.x * (per_wg / 16);
  const size_t n = per_wg / 16;
  uint32_t acc = 0;
  for (size_t i0 = 0; i0 < n; i0 += (size_t)16 * NT) {
    u32x4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const size_t i = i0 + (size_t)u * NT + threadIdx.x;
      v[u] = i < n ? base[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[(size_t)blockIdx.x * NT + threadIdx.x] = acc;
}

}  // namespace

// Read rate of n_wg workgroups of `threads` (256 or 1024) threads, each
// reading its own per_wg bytes of src (a multiple of 16); out holds n_wg *
// threads words.  *gbps: total bytes read / time, *ms: one launch (mean of
// reps back to back).
extern "C" int hga_calib_cu_read_rate(const void* src, size_t per_wg, int n_wg, int threads,
                                      void* out, int reps, double* gbps, double* ms) {
  if (!src || !out || per_wg == 0 || per_wg % 16 || n_wg <= 0 || (threads != 256 && threads != 1024) ||
      reps <= 0 || !gbps || !ms)
    return 1;
  const u32x4* s = static_cast<const u32x4*>(src);
  uint32_t* o = static_cast<uint32_t*>(out);
  auto launch = [&]() {
    if (threads == 256) hipLaunchKernelGGL(cu_read_kernel<256>, dim3(n_wg), dim3(256), 0, 0, s, per_wg, o);
    else hipLaunchKernelGGL(cu_read_kernel<1024>, dim3(n_wg), dim3(1024), 0, 0, s, per_wg, o);
  };
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return 2;
  if (hipEventCreate(&e1) != hipSuccess) {
    hipEventDestroy(e0);
    return 2;
  }
  int rc = 0;
  launch();
  (void)hipEventRecord(e0, 0);
  for (int r = 0; r < reps; ++r) launch();
  (void)hipEventRecord(e1, 0);
  if (hipEventSynchronize(e1) != hipSuccess) rc = 3;
  float t = 0.f;
  if (!rc && hipEventElapsedTime(&t, e0, e1) != hipSuccess) rc = 4;
  if (!rc) {
    *ms = t / reps;
    *gbps = (double)per_wg * n_wg / (*ms * 1e-3) / 1e9;
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return rc;
}

// variant 0: one uint4 per thread; 1: 4 per thread; 2: 4 per thread,
// non-temporal; 3: 8 per thread; 4: grid-stride over 8 workgroups per CU
// (n_cus of them).  bytes: a multiple of 16.  Times `reps` back-to-back
// launches between two events; returns 0 on success.
extern "C" int hga_calib_copy_rate(const void* src, void* dst, size_t bytes, int variant, int reps,
                                   int n_cus, double* gbps, double* ms) {
  if (!src || !dst || bytes == 0 || bytes % 16 || variant < 0 || variant > 4 || reps <= 0 ||
      n_cus <= 0 || !gbps || !ms)
    return 1;
  const size_t n = bytes / 16;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  auto launch = [&]() {
    switch (variant) {
      case 0: hipLaunchKernelGGL((copy_kernel<1, false>), dim3((n + 255) / 256), dim3(256), 0, 0, s, d, n); break;
      case 1: hipLaunchKernelGGL((copy_kernel<4, false>), dim3((n + 1023) / 1024), dim3(256), 0, 0, s, d, n); break;
      case 2: hipLaunchKernelGGL((copy_kernel<4, true>), dim3((n + 1023) / 1024), dim3(256), 0, 0, s, d, n); break;
      case 3: hipLaunchKernelGGL((copy_kernel<8, false>), dim3((n + 2047) / 2048), dim3(256), 0, 0, s, d, n); break;
      default: hipLaunchKernelGGL(copy_stride_kernel, dim3(8 * n_cus), dim3(256), 0, 0, s, d, n); break;
    }
  };
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return 2;
  if (hipEventCreate(&e1) != hipSuccess) {
    hipEventDestroy(e0);
    return 2;
  }
  int rc = 0;
  launch();  // warm
  hipEventRecord(e0, 0);
  for (int r = 0; r < reps; ++r) launch();
  hipEventRecord(e1, 0);
  if (hipEventSynchronize(e1) != hipSuccess) rc = 3;
  float t = 0.f;
  if (!rc && hipEventElapsedTime(&t, e0, e1) != hipSuccess) rc = 4;
  if (!rc) {
    *ms = t / reps;
    *gbps = 2.0 * bytes / (*ms * 1e-3) / 1e9;  // read + write
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return rc;
}
