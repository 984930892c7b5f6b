// Measured matrix-core peak: back-to-back independent bf16 32x32x16 MFMAs, one wave per SIMD (one
// 256-thread workgroup per CU), eight accumulators per wave so no MFMA waits for another's result.
// The figure it gives is what the hardware sustains under full matrix load (clock included), the
// practical ceiling the product kernels are compared with beside the nominal 2.5 PFLOP/s.
#include "common.h"
#include "kernels.h"

namespace wam {

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) mfma_peak_kernel(float* out, int iters) {
  floatx16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = floatx16{};
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)((threadIdx.x + i) & 15));
    b[i] = (__bf16)(1e-3f * (float)i);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) s += acc[m][threadIdx.x & 15];
  out[(long)blockIdx.x * 256 + threadIdx.x] = s;   // keeps the products live
}

hipError_t launch_mfma_peak(float* out, int workgroups, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(workgroups), dim3(256), 0, s, out, iters);
  return hipGetLastError();
}

}  // namespace wam
