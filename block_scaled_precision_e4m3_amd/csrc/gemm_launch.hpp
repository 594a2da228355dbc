// Launchers of the GEMM kernels, one per translation unit so that the many
// template instantiations compile in parallel.  Each returns the HIP error of
// its launch (hipErrorInvalidValue for a combination it does not hold).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxgemm_common.hpp"

namespace mxg {

// 256x256 kernel, bf16 datapath, float32 C (ct 0: n-major, 3: m-major)
hipError_t launch_big_bf16_f32(const Params& p, int sf, int fa, int fb, int ct, int64_t grid, hipStream_t s);
// 256x256 kernel, bf16 datapath, 16-bit C (ct 1: bfloat16, 2: float16)
hipError_t launch_big_bf16_c16(const Params& p, int sf, int fa, int fb, int ct, int64_t grid, hipStream_t s);
// 256x256 kernel, scaled-FP8 datapath, float32 C
hipError_t launch_big_fp8(const Params& p, int sf, int fa, int fb, int64_t grid, hipStream_t s);
// 128x128 kernel, either datapath (fp8 != 0: scaled FP8), ct 0 / 1 / 2
hipError_t launch_small(const Params& p, int fp8, int sf, int fa, int fb, int ct, int64_t grid, hipStream_t s);

// The format dispatch shared by those launchers: K(SF, FA, FB) names the
// kernel to launch with hipLaunchKernelGGL(kernel, grid, block, 0, s, p).
template <typename Launch>
hipError_t dispatch_formats(int sf, int fa, int fb, Launch&& launch) {
  if (fa == 2 || fb == 2) {
    if (fa == 2 && fb == 2 && sf == 32) return launch(std::integral_constant<int, 32>{}, std::integral_constant<int, 2>{},
                                                      std::integral_constant<int, 2>{});
    return hipErrorInvalidValue;
  }
#define MXG_DISPATCH(SF)                                                                                         \
  if (fa == 0 && fb == 0) return launch(std::integral_constant<int, SF>{}, std::integral_constant<int, 0>{},     \
                                        std::integral_constant<int, 0>{});                                       \
  if (fa == 0 && fb == 1) return launch(std::integral_constant<int, SF>{}, std::integral_constant<int, 0>{},     \
                                        std::integral_constant<int, 1>{});                                       \
  if (fa == 1 && fb == 0) return launch(std::integral_constant<int, SF>{}, std::integral_constant<int, 1>{},     \
                                        std::integral_constant<int, 0>{});                                       \
  return launch(std::integral_constant<int, SF>{}, std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
  if (sf == 32) {
    MXG_DISPATCH(32)
  }
  MXG_DISPATCH(16)
#undef MXG_DISPATCH
}

}  // namespace mxg
