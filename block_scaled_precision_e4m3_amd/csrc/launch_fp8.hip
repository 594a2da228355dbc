// Tile-kernel instantiations of the scaled-FP8 datapath (float32 C), both tile sizes.
#include "gemm_launch.hpp"
#include "mxgemm_big.hpp"

namespace mxg {

hipError_t launch_fp8(const Params& p, int sf, int fa, int fb, int bt, int64_t grid, hipStream_t s) {
  if (fa == 2) return hipErrorInvalidValue;  // packed FP4 runs on the bf16 datapath only
  const dim3 g((unsigned)grid), b(big::kThreads);
  return dispatch_formats(sf, fa, fb, [&](auto SFc, auto FAc, auto FBc) {
    constexpr int SF = decltype(SFc)::value, FA = decltype(FAc)::value, FB = decltype(FBc)::value;
    if constexpr (FA == 2) {
      return hipErrorInvalidValue;
    } else {
      if (bt == 256)
        hipLaunchKernelGGL((big::mxgemm_amax_big_kernel<SF, FA, FB, kModeFp8, 0, 256>), g, b, 0, s, p);
      else
        hipLaunchKernelGGL((big::mxgemm_amax_big_kernel<SF, FA, FB, kModeFp8, 0, 128>), g, b, 0, s, p);
      return hipGetLastError();
    }
  });
}

}  // namespace mxg
