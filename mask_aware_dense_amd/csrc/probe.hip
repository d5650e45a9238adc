// probe.hip -- sustained MFMA rate probe (a measurement aid).
//
// The attention kernels are dense contractions bounded by the bf16 matrix
// cores.  The published peak assumes the top clock; under a sustained matrix
// load the clock drops, so the rate a kernel can actually reach is measured
// here: every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on register
// operands, four independent accumulator chains, no memory traffic.
#include "kernel_common.hpp"

namespace mad {

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 x, y;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = (bf16)(0.001f * (lane + e));
    y[e] = (bf16)(0.002f * (lane - e));
  }
  f32x16 a0{}, a1{}, a2{}, a3{};
  for (int i = 0; i < iters; ++i) {
    a0 = mfma32(x, y, a0);
    a1 = mfma32(y, x, a1);
    a2 = mfma32(x, x, a2);
    a3 = mfma32(y, y, a3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += a0[r] + a1[r] + a2[r] + a3[r];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;  // keeps the products live
}

}  // namespace mad

using namespace mad;

extern "C" mad_status mad_probe_mfma(int32_t n_workgroups, int32_t iters, float* sink, hipStream_t stream) {
  clear_error();
  if (n_workgroups <= 0 || iters <= 0 || !sink) return fail(MAD_ERR_INVALID, "mad_probe_mfma: bad arguments");
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(n_workgroups), dim3(256), 0, stream, iters, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MAD_ERR_HIP, std::string("mad_probe_mfma: ") + hipGetErrorString(e));
  return MAD_OK;
}
