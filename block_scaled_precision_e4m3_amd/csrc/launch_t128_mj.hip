// 128x128-tile kernel instantiations with m-major A and/or n-major B: bf16
// datapath, float32 n-major C, 8-bit formats.
#include "gemm_launch.hpp"
#include "mxgemm_big.hpp"

namespace mxg {

hipError_t launch_bf16_mj_t128(const Params& p, int sf, int fa, int fb, int mj, int64_t grid, hipStream_t s) {
  if (fa == 2 || fb == 2 || mj < 1 || mj > 3) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b(2 * big::kThreads);  // 4 compute + 4 DMA waves
  return dispatch_formats(sf, fa, fb, [&](auto SFc, auto FAc, auto FBc) {
    constexpr int SF = decltype(SFc)::value, FA = decltype(FAc)::value, FB = decltype(FBc)::value;
    if constexpr (FA == 2) {
      return hipErrorInvalidValue;
    } else {
      if (mj == 1)
        hipLaunchKernelGGL((big::mxgemm_amax_big_kernel<SF, FA, FB, kModeBf16, 0, 128, 1, 8>), g, b, 0, s, p);
      else if (mj == 2)
        hipLaunchKernelGGL((big::mxgemm_amax_big_kernel<SF, FA, FB, kModeBf16, 0, 128, 2, 8>), g, b, 0, s, p);
      else
        hipLaunchKernelGGL((big::mxgemm_amax_big_kernel<SF, FA, FB, kModeBf16, 0, 128, 3, 8>), g, b, 0, s, p);
      return hipGetLastError();
    }
  });
}

}  // namespace mxg
