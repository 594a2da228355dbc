// 256x256-tile kernel instantiations: bf16 datapath, float32 C (n-major and m-major).
#include "gemm_launch.hpp"
#include "mxgemm_big.hpp"

namespace mxg {

hipError_t launch_bf16_f32_t256(const Params& p, int sf, int fa, int fb, int ct, int64_t grid, hipStream_t s) {
  const dim3 g((unsigned)grid), b(big::kThreads);
  return dispatch_formats(sf, fa, fb, [&](auto SFc, auto FAc, auto FBc) {
    constexpr int SF = decltype(SFc)::value, FA = decltype(FAc)::value, FB = decltype(FBc)::value;
    if constexpr (FA == 2 && SF == 16) {
      return hipErrorInvalidValue;  // FP4 at sf = 16: 128x128 tiles only
    } else {
      if (ct == 3)
        hipLaunchKernelGGL((big::mxgemm_amax_big_kernel<SF, FA, FB, kModeBf16, 3, 256>), g, b, 0, s, p);
      else
        hipLaunchKernelGGL((big::mxgemm_amax_big_kernel<SF, FA, FB, kModeBf16, 0, 256>), g, b, 0, s, p);
      return hipGetLastError();
    }
  });
}

}  // namespace mxg
