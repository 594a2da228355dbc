// 128x128 kernel instantiations: both datapaths, float32 / bfloat16 / float16 C.
#include "gemm_launch.hpp"
#include "mxgemm_kernel.hpp"

namespace mxg {

hipError_t launch_small(const Params& p, int fp8, int sf, int fa, int fb, int ct, int64_t grid, hipStream_t s) {
  if (fa == 2) return hipErrorInvalidValue;  // packed FP4 runs on the 256x256 kernel only
  const dim3 g((unsigned)grid), b(kThreads);
  return dispatch_formats(sf, fa, fb, [&](auto SFc, auto FAc, auto FBc) {
    constexpr int SF = decltype(SFc)::value, FA = decltype(FAc)::value, FB = decltype(FBc)::value;
    if constexpr (FA == 2) {
      return hipErrorInvalidValue;
    } else {
      if (fp8)
        hipLaunchKernelGGL((mxgemm_amax_kernel<SF, FA, FB, kModeFp8, 0>), g, b, 0, s, p);
      else if (ct == 1)
        hipLaunchKernelGGL((mxgemm_amax_kernel<SF, FA, FB, kModeBf16, 1>), g, b, 0, s, p);
      else if (ct == 2)
        hipLaunchKernelGGL((mxgemm_amax_kernel<SF, FA, FB, kModeBf16, 2>), g, b, 0, s, p);
      else
        hipLaunchKernelGGL((mxgemm_amax_kernel<SF, FA, FB, kModeBf16, 0>), g, b, 0, s, p);
      return hipGetLastError();
    }
  });
}

}  // namespace mxg
