// 256x256-tile kernel instantiations with the projection epilogue (RoPE and
// dual-direction MXFP8 of the float32 accumulators): 8-bit formats, bf16
// datapath.
#include "gemm_launch.hpp"
#include "mxgemm_big.hpp"

namespace mxg {

hipError_t launch_proj_t256(const Params& p, int sf, int fa, int fb, int64_t grid, hipStream_t s) {
  if (fa == 2 || fb == 2) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b(big::kThreads);
  return dispatch_formats(sf, fa, fb, [&](auto SFc, auto FAc, auto FBc) {
    constexpr int SF = decltype(SFc)::value, FA = decltype(FAc)::value, FB = decltype(FBc)::value;
    if constexpr (FA == 2) {
      return hipErrorInvalidValue;
    } else {
      hipLaunchKernelGGL((big::mxgemm_amax_big_kernel<SF, FA, FB, kModeBf16, 4, 256>), g, b, 0, s, p);
      return hipGetLastError();
    }
  });
}

}  // namespace mxg
