// Per-head RoPE and dual-direction MXFP8 quantisation of a projection output
// ("GEMM + RoPE + MXFP8 Projection (SM100)", sections "Overview", "Shapes"
// and "Equations"), applied to the float32 C of the GEMM:
//
//   Y (tokens, H * D) viewed as (tokens, H, D);
//   RoPE on the trailing QR features of each head, interleaved in, halves
//   out: with (a_i, b_i) = (y[2i], y[2i+1]) of the rotary part and R = QR/2,
//       out[i]     = a_i * cos[i]     - b_i * sin[i]
//       out[R + i] = b_i * cos[R + i] + a_i * sin[R + i]
//   (bf16 cos / sin rows of the token; float32 products and sum, each
//   rounded on its own, no fused multiply-add);
//   MXFP8 (E4M3 codes, one E8M0 scale per 32 values) along D (row codes
//   (tokens, H, D), scales (tokens, H, D/32)) and along tokens (column codes
//   (tokens, H, D), scales (tokens/32, H, D)), with the scale rule of the MX
//   quantiser (mx_quantize.hpp): e the smallest integer with 448 * 2^e >= the
//   block's largest magnitude, codes rounded to nearest, ties to even.
//
// One workgroup of 256 threads per (32-token block, head).  The 32 x D tile
// is read with 16-byte loads (each token's D floats are contiguous) and
// parked in LDS at a pitch of D + 1 floats, so that a column read by 32
// lanes hits 32 banks.  RoPE runs in place after a barrier.  Row blocks:
// one thread per (token, block) quantises 32 consecutive values and stores
// 32 codes.  Column blocks: one thread per feature quantises its 32 tokens
// into an LDS byte tile, which then leaves as whole rows.
#pragma once

#include "mx_quantize.hpp"

namespace mxg {
namespace rope {

constexpr int kThreads = 256;
constexpr int kMaxD = 256;

struct RParams {
  const float* Y;           // (tokens, H * D)
  const uint16_t* cs;       // cos, (tokens, QR) bf16 bits
  const uint16_t* sn;       // sin, (tokens, QR) bf16 bits
  uint8_t* row_codes;       // (tokens, H, D)
  uint8_t* row_scales;      // (tokens, H, D / 32)
  uint8_t* col_codes;       // (tokens, H, D)
  uint8_t* col_scales;      // (tokens / 32, H, D)
  int H, D, QR;
  int num_tiles;            // tokens / 32 * H
};

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) { return __uint_as_float((unsigned)b << 16); }

// 32 floats at stride `step` (in floats) from LDS -> block exponent and 32 codes
__device__ __forceinline__ int quantize32(const float* src, int step, unsigned (&w)[8]) {
  float bm = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) bm = fmaxf(bm, fabsf(src[j * step]));
  const int e = quant::block_exponent<0>(bm);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    w[q] = quant::codes4<0>(ldexpf(src[(4 * q) * step], -e), ldexpf(src[(4 * q + 1) * step], -e),
                            ldexpf(src[(4 * q + 2) * step], -e), ldexpf(src[(4 * q + 3) * step], -e));
  return e;
}

__global__ __launch_bounds__(kThreads) void proj_rope_mxfp8_kernel(RParams p) {
  __shared__ float z[32 * (kMaxD + 1)];
  __shared__ __attribute__((aligned(16))) uint8_t qc[32 * kMaxD];
  const int t = threadIdx.x;
  const int D = p.D, P = p.D + 1, HD = p.H * p.D;
  const int nope = p.D - p.QR, R = p.QR / 2, nb = p.D / 32;
  for (int a = blockIdx.x; a < p.num_tiles; a += gridDim.x) {
    const int h = a % p.H, tb = a / p.H;
    const int64_t row0 = (int64_t)tb * 32;
    __syncthreads();  // the previous tile's LDS reads are done
    // load: 32 rows of D floats (D / 4 float4 per row)
    const int q4 = D / 4;
    for (int f = t; f < 32 * q4; f += kThreads) {
      const int r = f / q4, c = f - r * q4;
      const float4 v = *reinterpret_cast<const float4*>(p.Y + (row0 + r) * HD + (int64_t)h * D + 4 * c);
      float* dst = z + r * P + 4 * c;
      dst[0] = v.x;
      dst[1] = v.y;
      dst[2] = v.z;
      dst[3] = v.w;
    }
    __syncthreads();
    // RoPE: pair i of row r, results held in registers until every pair has
    // been read (a fixed trip count keeps them out of scratch)
    constexpr int kPairsPerThread = 32 * (kMaxD / 2) / kThreads;
    float o1[kPairsPerThread], o2[kPairsPerThread];
#pragma unroll
    for (int k = 0; k < kPairsPerThread; ++k) {
      const int f = t + k * kThreads;
      if (f < 32 * R) {
        const int r = f / R, i = f - r * R;
        const float av = z[r * P + nope + 2 * i], bv = z[r * P + nope + 2 * i + 1];
        const uint16_t* cr = p.cs + (row0 + r) * p.QR;
        const uint16_t* sr = p.sn + (row0 + r) * p.QR;
        const float c1 = bf16_bits_to_float(cr[i]), s1 = bf16_bits_to_float(sr[i]);
        const float c2 = bf16_bits_to_float(cr[R + i]), s2 = bf16_bits_to_float(sr[R + i]);
        o1[k] = __fsub_rn(__fmul_rn(av, c1), __fmul_rn(bv, s1));
        o2[k] = __fadd_rn(__fmul_rn(bv, c2), __fmul_rn(av, s2));
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPairsPerThread; ++k) {
      const int f = t + k * kThreads;
      if (f < 32 * R) {
        const int r = f / R, i = f - r * R;
        z[r * P + nope + i] = o1[k];
        z[r * P + nope + R + i] = o2[k];
      }
    }
    __syncthreads();
    // row blocks: thread (r, blk)
    for (int f = t; f < 32 * nb; f += kThreads) {
      const int r = f / nb, blk = f - r * nb;
      unsigned w[8];
      const int e = quantize32(z + r * P + 32 * blk, 1, w);
      const int64_t o = ((row0 + r) * p.H + h) * (int64_t)D + 32 * blk;
      *reinterpret_cast<uint4*>(p.row_codes + o) = uint4{w[0], w[1], w[2], w[3]};
      *reinterpret_cast<uint4*>(p.row_codes + o + 16) = uint4{w[4], w[5], w[6], w[7]};
      p.row_scales[((row0 + r) * p.H + h) * nb + blk] = (uint8_t)(e + 127);
    }
    // column blocks: thread d quantises its 32 tokens into the LDS byte tile
    for (int d = t; d < D; d += kThreads) {
      unsigned w[8];
      const int e = quantize32(z + d, P, w);
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) qc[(4 * q + j) * D + d] = (uint8_t)(w[q] >> (8 * j));
      p.col_scales[((int64_t)tb * p.H + h) * D + d] = (uint8_t)(e + 127);
    }
    __syncthreads();
    const int d4 = D / 4;
    for (int f = t; f < 32 * d4; f += kThreads) {
      const int r = f / d4, c = f - r * d4;
      *reinterpret_cast<unsigned*>(p.col_codes + ((row0 + r) * p.H + h) * (int64_t)D + 4 * c) =
          *reinterpret_cast<const unsigned*>(qc + r * D + 4 * c);
    }
  }
}

}  // namespace rope
}  // namespace mxg
