// Launchers of the GEMM kernels, one per translation unit so that the many
// template instantiations compile in parallel.  Each returns the HIP error of
// its launch (hipErrorInvalidValue for a combination it does not hold).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxgemm_common.hpp"

namespace mxg {

// Tile kernel (mxgemm_big.hpp), bf16 datapath, float32 C (ct 0: n-major, 3:
// m-major), 256x256 or 128x128 tiles
hipError_t launch_bf16_f32_t256(const Params& p, int sf, int fa, int fb, int ct, int64_t grid, hipStream_t s);
hipError_t launch_bf16_f32_t128(const Params& p, int sf, int fa, int fb, int ct, int64_t grid, hipStream_t s);
// the same with a 16-bit C (ct 1: bfloat16, 2: float16)
hipError_t launch_bf16_c16_t256(const Params& p, int sf, int fa, int fb, int ct, int64_t grid, hipStream_t s);
hipError_t launch_bf16_c16_t128(const Params& p, int sf, int fa, int fb, int ct, int64_t grid, hipStream_t s);
// 256x256 tiles, bf16 datapath, the projection epilogue in place of C
// (Params' rope / code / scale fields); 8-bit formats
hipError_t launch_proj_t256(const Params& p, int sf, int fa, int fb, int64_t grid, hipStream_t s);
// scaled-FP8 datapath, float32 C; bt = 256 or 128
hipError_t launch_fp8(const Params& p, int sf, int fa, int fb, int bt, int64_t grid, hipStream_t s);
// bf16 datapath, float32 n-major C, m-major A (mj bit 0) and/or n-major B (bit 1); 8-bit formats
hipError_t launch_bf16_mj_t256(const Params& p, int sf, int fa, int fb, int mj, int64_t grid, hipStream_t s);
hipError_t launch_bf16_mj_t128(const Params& p, int sf, int fa, int fb, int mj, int64_t grid, hipStream_t s);

// The format dispatch shared by those launchers: K(SF, FA, FB) names the
// kernel to launch with hipLaunchKernelGGL(kernel, grid, block, 0, s, p).
template <typename Launch>
hipError_t dispatch_formats(int sf, int fa, int fb, Launch&& launch) {
  if (fa == 2 || fb == 2) {
    if (fa != 2 || fb != 2) return hipErrorInvalidValue;
    if (sf == 32)
      return launch(std::integral_constant<int, 32>{}, std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
    return launch(std::integral_constant<int, 16>{}, std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
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
