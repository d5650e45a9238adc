// attn_dkdv256.hip -- dK / dV launches for head dim 256 (the kernel is in
// attn_dkdv.hpp).  A file of its own so that these instances keep the default
// instruction scheduling: the strategy the 64 / 128 instances are built with
// changes their register allocation.
#include "attn_dkdv.hpp"

namespace mad {

hipError_t launch_dkdv_d256(const AttnParams& P, dim3 grid, bool fine, bool hm, hipStream_t stream) {
  auto run = [&](auto k, int nw) { hipLaunchKernelGGL(k, grid, dim3(64 * nw), 0, stream, P); };
  if (fine) hm ? run(dkdv_kernel<256, 2, true>, 2) : run(dkdv_kernel<256, 2, false>, 2);
  else hm ? run(dkdv_kernel<256, 4, true>, 4) : run(dkdv_kernel<256, 4, false>, 4);
  return hipGetLastError();
}

}  // namespace mad
