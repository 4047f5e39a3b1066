// Calibration kernel for the benchmark (not part of the HGA path): the issue
// rate of v_mfma_f32_16x16x32_bf16 on this device.  Each wave runs n rounds
// of K independent products on K accumulators and folds the accumulators
// into one store, so nothing is optimised away.  Reported as dense bf16
// TFLOP/s, next to the published peak, to read the matrix-core utilisation
// of the attention kernels.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int K>
__global__ __launch_bounds__(256) void mfma_rate_kernel(float* out, int n) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
  f32x4 c[K];
  for (int k = 0; k < K; ++k) c[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < n; ++r) {
#pragma unroll
    for (int k = 0; k < K; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
  for (int k = 0; k < K; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// waves_per_simd in 1..4: 256 CUs x 4 SIMDs are filled with that many waves
// each (256-thread workgroups).  Returns 0 on success; *tflops = dense bf16
// rate of the timed launch, *ms its duration.
extern "C" int hga_calib_mfma_rate(int n_cus, int waves_per_simd, int rounds, double* tflops,
                                   double* ms) {
  if (n_cus <= 0 || waves_per_simd < 1 || waves_per_simd > 4 || rounds <= 0 || !tflops || !ms)
    return 1;
  const int blocks = n_cus * waves_per_simd;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)) != hipSuccess) return 2;
  hipEvent_t e0, e1;
  int rc = 0;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) rc = 3;
  if (!rc) {
    hipLaunchKernelGGL(mfma_rate_kernel<8>, dim3(blocks), dim3(256), 0, 0, out, rounds);  // warm
    hipEventRecord(e0, 0);
    hipLaunchKernelGGL(mfma_rate_kernel<8>, dim3(blocks), dim3(256), 0, 0, out, rounds);
    hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) != hipSuccess) rc = 4;
  }
  if (!rc) {
    float t = 0.f;
    if (hipEventElapsedTime(&t, e0, e1) != hipSuccess) rc = 5;
    const double flops = (double)blocks * 4 /* waves */ * rounds * 8 /* K */ * 16384.0;
    *ms = t;
    *tflops = flops / (t * 1e-3) / 1e12;
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  hipFree(out);
  return rc;
}
