// attn_dkdv.hip -- dK / dV launches for head dims 64 and 128 (the kernel is
// in attn_dkdv.hpp; head dim 256 launches from attn_dkdv256.hip), and the
// fp32 column-chunk sums' zeroing and rounding kernels.
#include "attn_dkdv.hpp"

namespace mad {

// Column chunks: zero the fp32 sums before, round them to bf16 after.
__global__ __launch_bounds__(256) void zero2_kernel(float* a, float* b, int64_t n4) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n4; x += (int64_t)gridDim.x * 256) {
    reinterpret_cast<float4*>(a)[x] = float4{0.f, 0.f, 0.f, 0.f};
    reinterpret_cast<float4*>(b)[x] = float4{0.f, 0.f, 0.f, 0.f};
  }
}
__global__ __launch_bounds__(256) void round2_kernel(const float* a, const float* b, bf16* ra, bf16* rb, int64_t n4) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n4; x += (int64_t)gridDim.x * 256) {
    const float4 u = reinterpret_cast<const float4*>(a)[x], v = reinterpret_cast<const float4*>(b)[x];
    bf16x4 y, z;
    y[0] = (bf16)u.x; y[1] = (bf16)u.y; y[2] = (bf16)u.z; y[3] = (bf16)u.w;
    z[0] = (bf16)v.x; z[1] = (bf16)v.y; z[2] = (bf16)v.z; z[3] = (bf16)v.w;
    reinterpret_cast<bf16x4*>(ra)[x] = y;
    reinterpret_cast<bf16x4*>(rb)[x] = z;
  }
}

// Head dim 256 has a kernel of its own (attn_dkdv256.hip).
hipError_t launch_dkdv_d256(const AttnParams& P, int n_items, bool hm, hipStream_t stream);

hipError_t launch_dkdv(const AttnParams& P, int D, int n_items, hipStream_t stream) {
  const int S = P.kv_splits;
  const int64_t n4 = (int64_t)P.Tk * P.Hkv * D / 4;  // D is a multiple of 4
  const int nb = (int)std::min<int64_t>((n4 + 255) / 256, 4096);
  if (S > 1 && n4 > 0) hipLaunchKernelGGL(zero2_kernel, dim3(nb), dim3(256), 0, stream, P.dk_acc, P.dv_acc, n4);
  const dim3 grid(n_items * S);
  auto run = [&](auto k, int nw) { hipLaunchKernelGGL(k, grid, dim3(64 * nw), 0, stream, P); };
  const bool hm = P.R == 1 && (P.m.mode == MODE_BLOCKS || P.t.uniform);
  const bool fine = P.t.BN == BN1_FINE;
  if (D == 256) {
    const hipError_t e = launch_dkdv_d256(P, n_items, hm, stream);
    if (e != hipSuccess) return e;
  } else if (D == 128) {
    if (fine) hm ? run(dkdv_kernel<128, 2, true>, 2) : run(dkdv_kernel<128, 2, false>, 2);
    else hm ? run(dkdv_kernel<128, 4, true>, 4) : run(dkdv_kernel<128, 4, false>, 4);
  } else {
    if (fine) hm ? run(dkdv_kernel<64, 2, true>, 2) : run(dkdv_kernel<64, 2, false>, 2);
    else hm ? run(dkdv_kernel<64, 4, true>, 4) : run(dkdv_kernel<64, 4, false>, 4);
  }
  if (S > 1 && n4 > 0)
    hipLaunchKernelGGL(round2_kernel, dim3(nb), dim3(256), 0, stream, P.dk_acc, P.dv_acc, P.dk, P.dv, n4);
  return hipGetLastError();
}

}  // namespace mad
