// Measurement probes for MI355X (gfx950): what the hardware under the GEMM
// sustains, timed by the caller around one launch.  Each probe has a C entry
// point in include/mxgemm_probe.h.
//
// * mfma: every wave issues `iters` rounds of 8 independent MFMAs (bf16
//   32x32x16 or scaled FP8 32x32x64), four waves per CU; reports the
//   workgroup's shader-clock and 100 MHz-clock spans, so the caller gets the
//   MFMA rate and the clock it ran at.
// * copy_lds: the GEMM's operand staging without its math -- every wave
//   moves `per_step` 1 KB blocks per step from a source region into an LDS
//   ring with buffer_load_dwordx4 ... lds, waits, and meets the other waves
//   at a barrier; or (vgpr != 0) the same blocks with buffer_load_dwordx4
//   into registers.
// * hbm_read / hbm_write: streaming 16-byte loads (folded into one value per
//   thread) or stores over a buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxgemm_probe.h"
#include "mxgemm_common.hpp"

namespace mxg {
namespace probe {

template <int KIND>
__global__ __launch_bounds__(256, 1) void mfma_kernel(int iters, unsigned long long* spans) {
  v16f acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  const int lane = threadIdx.x & 63;
  v8bf a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1.0f + (float)((lane + e) & 3) * 0.25f);
    b[e] = (__bf16)(1.0f - (float)((lane * 3 + e) & 3) * 0.125f);
  }
  v8i fa, fb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    fa[e] = 0x38383838 ^ (lane & e);
    fb[e] = 0x30303030 ^ ((lane >> 1) & e);
  }
  __syncthreads();
  const unsigned long long c0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (KIND == 0)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
      else
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[i], 0, 0, 0, 127, 0, 127);
    }
  }
  __syncthreads();
  const unsigned long long c1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float keep = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) keep += acc[i][e];
  if (threadIdx.x == 0) {
    spans[2 * blockIdx.x] = c1 - c0;
    spans[2 * blockIdx.x + 1] = r1 - r0;
  }
  if (keep == 12345.678f) spans[0] = 0;  // keeps the accumulators live
}

// LDS ring of 4 stages of 64 KB would not fit; the ring is 2 x (4 waves x
// per_step KB) <= 2 x 64 KB.
constexpr int kMaxPerStep = 16;

__global__ __launch_bounds__(256, 1) void copy_lds_kernel(const uint8_t* src, unsigned src_bytes, int steps,
                                                          int per_step, int vgpr, unsigned row_stride,
                                                          unsigned* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * 4 * kMaxPerStep * 1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, src_bytes);
  const unsigned lds0 = lds_addr(ring);
  // block j of step s of workgroup b starts at a 1 KB slot that walks the
  // source region (wrapping); with row_stride == 0 a block is those 1024
  // contiguous bytes, 16 per lane; otherwise it is 8 rows of 128 bytes at
  // row_stride apart (lane l: row l / 8, 16-byte chunk l % 8), as the GEMM
  // reads its operand tiles
  const unsigned slots = (row_stride ? src_bytes / (8u * row_stride) : src_bytes >> 10);
  unsigned acc = 0u;
  for (int s = 0; s < steps; ++s) {
    const unsigned base = (unsigned)((blockIdx.x * 131u + (unsigned)s * 4u * (unsigned)per_step) % slots);
    for (int j = 0; j < per_step; ++j) {
      const unsigned slot = (base + (unsigned)(wave * per_step + j)) % slots;
      const unsigned voff = row_stride ? slot * 8u * row_stride + (unsigned)(lane >> 3) * row_stride +
                                             16u * (unsigned)(lane & 7)
                                       : (slot << 10) + 16u * (unsigned)lane;
      if (vgpr) {
        const v4u v = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, 0, 0));
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      } else {
        const unsigned dst = lds0 + (unsigned)(((s & 1) * 4 + wave) * kMaxPerStep + j) * 1024u;
        dma16_at(rs, voff, dst);
      }
    }
    wait_vm<0>();
    barrier();
  }
  if (acc == 0x12345678u) sink[0] = acc;
}

__global__ void hbm_read_kernel(const uint4* x, int64_t n16, unsigned* sink) {
  unsigned acc = 0u;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 v = x[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ void hbm_write_kernel(uint4* y, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    y[i] = make_uint4((unsigned)i, 0u, 0u, 0u);
}

}  // namespace probe
}  // namespace mxg

extern "C" {

int mxprobe_mfma(int kind, int workgroups, int iters, unsigned long long* spans, void* stream) {
  if ((kind != 0 && kind != 1) || workgroups <= 0 || iters <= 0 || !spans) return -1;
  if (kind == 0)
    hipLaunchKernelGGL(mxg::probe::mfma_kernel<0>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, iters, spans);
  else
    hipLaunchKernelGGL(mxg::probe::mfma_kernel<1>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, iters, spans);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int mxprobe_copy_lds(const void* src, uint64_t src_bytes, int workgroups, int steps, int per_step, int vgpr,
                     unsigned row_stride, unsigned* sink, void* stream) {
  if (!src || !sink || workgroups <= 0 || steps <= 0 || per_step <= 0 || per_step > mxg::probe::kMaxPerStep)
    return -1;
  if (src_bytes < 64 * 1024 || src_bytes > (1ull << 31) || (src_bytes & 1023) != 0) return -2;
  if (row_stride != 0 && (row_stride < 128 || row_stride % 16 != 0 || src_bytes / (8ull * row_stride) < 64)) return -3;
  hipLaunchKernelGGL(mxg::probe::copy_lds_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint8_t*>(src), (unsigned)src_bytes, steps, per_step, vgpr, row_stride, sink);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int mxprobe_hbm(int write, void* buf, uint64_t bytes, int workgroups, unsigned* sink, void* stream) {
  if (!buf || workgroups <= 0 || (bytes & 15) != 0 || (!write && !sink)) return -1;
  const int64_t n16 = (int64_t)(bytes / 16);
  if (write)
    hipLaunchKernelGGL(mxg::probe::hbm_write_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       static_cast<uint4*>(buf), n16);
  else
    hipLaunchKernelGGL(mxg::probe::hbm_read_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
