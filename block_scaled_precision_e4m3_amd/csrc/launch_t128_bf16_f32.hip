// 128x128-tile kernel instantiations: bf16 datapath, float32 C (n-major and m-major).
#include "gemm_launch.hpp"
#include "mxgemm_big.hpp"

namespace mxg {

hipError_t launch_bf16_f32_t128(const Params& p, int sf, int fa, int fb, int ct, int64_t grid, hipStream_t s) {
  const dim3 g((unsigned)grid);
  return dispatch_formats(sf, fa, fb, [&](auto SFc, auto FAc, auto FBc) {
    constexpr int SF = decltype(SFc)::value, FA = decltype(FAc)::value, FB = decltype(FBc)::value;
    // the 4-stage ring runs with 4 DMA waves beside the 4 compute waves; FP4
    // at sf = 16 keeps two stages and 4 waves
    constexpr int NW = (FA == 2 && SF == 16) ? 4 : 8;
    const dim3 b(64 * NW);
    if (ct == 3)
      hipLaunchKernelGGL((big::mxgemm_amax_big_kernel<SF, FA, FB, kModeBf16, 3, 128, 0, NW>), g, b, 0, s, p);
    else
      hipLaunchKernelGGL((big::mxgemm_amax_big_kernel<SF, FA, FB, kModeBf16, 0, 128, 0, NW>), g, b, 0, s, p);
    return hipGetLastError();
  });
}

}  // namespace mxg
