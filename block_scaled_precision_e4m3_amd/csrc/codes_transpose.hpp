// m-major element codes -> the k-major rows the GEMM kernels read.
//
// "GEMM + Amax (SM100)", section "Parameters": A may be m-major, shape
// (M, K, L) with strides (1, M, M*K), and B n-major likewise; byte (mn, k, l)
// then sits at mn + MN*k + MN*K*l.  The GEMM kernels move whole 128-byte
// runs of K per row into LDS, so they read (l, mn, k) at k + K*mn + MN*K*l.
// This kernel rewrites one layout into the other, one byte per element (the
// pages allow m-major operands for the 8-bit formats only).
//
// One workgroup of 256 threads per 64 x 64-byte tile.  Thread (r, c) =
// (t / 4, t % 4) loads the 16 bytes mn [16c, +16) of K row r (coalesced: 4
// threads cover 64 contiguous bytes), parks them in LDS (rows of 68 bytes),
// then gathers the 16 bytes k [16c, +16) of mn row r from 16 LDS rows and
// stores them as one 16-byte run of the k-major row.  With a row pitch of 17
// dwords the gathers of a wave hit 64 different banks or the same dword.
// MN % 16 == 0 and K % 16 == 0 (the host checks), so every 16-byte run lies
// wholly inside or outside the matrix.
#pragma once

#include "mxgemm_common.hpp"

namespace mxg {
namespace transpose {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kPitch = 68;  // LDS bytes per parked K row

struct TParams {
  const uint8_t* S;  // (L, K, MN) codes, MN contiguous
  uint8_t* D;        // (L, MN, K) codes, K contiguous
  int MN, K;
  int tiles_mn, tiles_k;
  int num_tiles;
};

__global__ __launch_bounds__(kThreads) void codes_to_kmajor_kernel(TParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t park[kTile * kPitch];
  const int t = threadIdx.x;
  const int r = t >> 2, c = t & 3;
  for (int a = blockIdx.x; a < p.num_tiles; a += gridDim.x) {
    const int tk = a % p.tiles_k;
    const int rest = a / p.tiles_k;
    const int tmn = rest % p.tiles_mn;
    const int l = rest / p.tiles_mn;
    const int k0 = tk * kTile, mn0 = tmn * kTile;
    uint4 v = {0u, 0u, 0u, 0u};
    const int k = k0 + r, mn = mn0 + 16 * c;
    if (k < p.K && mn < p.MN) v = *reinterpret_cast<const uint4*>(p.S + ((int64_t)l * p.K + k) * p.MN + mn);
    __syncthreads();  // the previous tile's gathers are done
    unsigned* row = reinterpret_cast<unsigned*>(park + r * kPitch + 16 * c);
    row[0] = v.x;
    row[1] = v.y;
    row[2] = v.z;
    row[3] = v.w;
    __syncthreads();
    unsigned w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      unsigned x = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) x |= (unsigned)park[(16 * c + 4 * i + j) * kPitch + r] << (8 * j);
      w[i] = x;
    }
    const int mn2 = mn0 + r, k2 = k0 + 16 * c;
    if (mn2 < p.MN && k2 < p.K)
      *reinterpret_cast<uint4*>(p.D + ((int64_t)l * p.MN + mn2) * p.K + k2) = uint4{w[0], w[1], w[2], w[3]};
  }
}

}  // namespace transpose
}  // namespace mxg
