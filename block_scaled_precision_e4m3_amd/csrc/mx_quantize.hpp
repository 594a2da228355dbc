// MX block quantisation on gfx950: float32 (L, MN, K) -> E4M3 or E5M2 codes
// (L, MN, K) plus one E8M0 scale byte per (row, block of sf K elements),
// written straight into the physical scale-factor atom buffer
// (L, ceil(MN/128), ceil(K/(4 sf)), 32, 4, 4) that the GEMM reads.
//
// "GEMM + RoPE + MXFP8 Projection (SM100)", section "Equations": MXFP8
// quantisation with an E8M0 scale per block and E4M3 data; the atom layout
// is that of "GEMM + Amax (SM100)", sections "Shapes" and "Using JAX arrays".
// The scale of a block with largest magnitude bm is 2^e, e the smallest
// integer with FMAX * 2^e >= bm (FMAX = 448 for E4M3, 57344 for E5M2),
// clamped to [-127, 127], and e = 0 for an all-zero block; codes are x * 2^-e
// rounded to nearest, ties to even (|x * 2^-e| <= FMAX by the choice of e).
//
// Work: one workgroup per 512-byte atom, i.e. 128 rows x 4 blocks (4 sf
// K elements).  A lane holds 4 consecutive floats of a row (one 16-byte
// load); the sf/4 lanes of a block are consecutive, so the block maximum is
// an xor-shuffle reduction inside them.  Rows past MN and K chunks past K read
// as zero (the buffer resource ends at the atom's last valid row; chunks past
// K get an offset of 2^31 or more) and are not stored; their scale bytes,
// like those of all-zero blocks, are 127.  The atom's bytes are gathered in
// LDS and leave as one 512-byte store.
#pragma once

#include "mxgemm_common.hpp"

namespace mxg {
namespace quant {

constexpr int kThreads = 256;

struct QParams {
  const float* X;
  uint8_t* Q;
  uint8_t* SF;
  int MN, K;
  int MNb, Kg;
  int num_atoms;
};

template <int FMT>
__device__ __forceinline__ unsigned codes4(float a, float b, float c, float d) {
  int w;
  if constexpr (FMT == 0) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (unsigned)w;
}

// E4M3 codes of a * 2^-e .. d * 2^-e in one go: v_cvt_scalef32_pk_fp8_f32
// divides by the power of two in its scale operand's exponent field before
// rounding, bitwise what ldexpf(x, -e) then v_cvt_pk_fp8_f32 give (measured on
// MI355X over 2.2 M value pairs: every code, the midpoints and their f32
// neighbours, both signs, e = -127 .. 120).
__device__ __forceinline__ unsigned codes4_e4m3_exp(float a, float b, float c, float d, int e) {
  typedef short v2s_t __attribute__((ext_vector_type(2)));
  const float s = __uint_as_float((unsigned)(e + 127) << 23);
  const v2s_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((v2s_t){0, 0}, a, b, s, false);
  const v2s_t w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, c, d, s, true);
  return __builtin_bit_cast(unsigned, w);
}

// Smallest e with FMAX * 2^e >= bm (bm >= 0 finite), clamped; 0 for bm = 0.
// FMAX = 1.75 * 2^EF (EF = 8 for E4M3, 15 for E5M2).  For a normal bm =
// (1 + m/2^23) * 2^(E - 127): e = E - 127 - EF, plus one when the mantissa
// exceeds that of 1.75.  A subnormal bm (< 2^-126) needs e < -127: clamped.
template <int FMT>
__device__ __forceinline__ int block_exponent(float bm) {
  constexpr int EF = FMT == 0 ? 8 : 15;
  const unsigned bits = __float_as_uint(bm);
  const int E = (int)(bits >> 23);
  const int m = (int)(bits & 0x7FFFFFu);
  int e = E - 127 - EF + (m > 0x600000 ? 1 : 0);
  e = E == 0 ? -127 : e;
  e = min(max(e, -127), 127);
  return bits == 0u ? 0 : e;
}

template <int SF, int FMT>
__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(QParams p) {
  constexpr int kCpr = SF;                // 16-byte chunks per atom row (4 sf floats)
  constexpr int kRpp = kThreads / kCpr;   // rows per pass: 8 (sf=32) or 16 (sf=16)
  constexpr int kPasses = 128 / kRpp;
  constexpr int kBlk = SF / 4;            // lanes per block
  __shared__ __attribute__((aligned(16))) uint8_t atom[512];

  const int t = threadIdx.x;
  const int c = t % kCpr;                 // chunk of the row: K offset 4c within the atom
  const int rr = t / kCpr;                // row within a pass
  const int kbl = c / kBlk;               // block within the atom (0..3)
  constexpr unsigned kOob = 0x80000000u;

  for (int a = blockIdx.x; a < p.num_atoms; a += gridDim.x) {
    const int kg = a % p.Kg;
    const int rest = a / p.Kg;
    const int mb = rest % p.MNb;
    const int l = rest / p.MNb;
    const int r0 = 128 * mb, k0 = 4 * SF * kg;
    const int rows = min(128, p.MN - r0);
    const int64_t base = ((int64_t)l * p.MN + r0) * p.K + k0;
    const unsigned bytes = (unsigned)rows * (unsigned)p.K;  // < 2^30: K < 2^23 (checked on the host)
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.X + base, bytes * 4u);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.Q + base, bytes);
    const bool kin = k0 + 4 * c < p.K;

    v4f v[kPasses];
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
      const int r = i * kRpp + rr;
      const unsigned off = kin ? ((unsigned)r * (unsigned)p.K + 4u * (unsigned)c) * 4u : kOob;
      v[i] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
      const int r = i * kRpp + rr;
      float bm = fmaxf(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])), fmaxf(fabsf(v[i][2]), fabsf(v[i][3])));
#pragma unroll
      for (int s = 1; s < kBlk; s <<= 1) bm = fmaxf(bm, __shfl_xor(bm, s));
      const int e = block_exponent<FMT>(bm);
      const unsigned w = codes4<FMT>(ldexpf(v[i][0], -e), ldexpf(v[i][1], -e), ldexpf(v[i][2], -e),
                                     ldexpf(v[i][3], -e));
      const unsigned off = kin ? (unsigned)r * (unsigned)p.K + 4u * (unsigned)c : kOob;
      __builtin_amdgcn_raw_buffer_store_b32(w, rq, (int)off, 0, 0);
      // row r's byte of block kbl: atom offset 16 (r % 32) + 4 ((r / 32) % 4) + kbl
      if (c % kBlk == 0) atom[16 * (r & 31) + 4 * ((r >> 5) & 3) + kbl] = (uint8_t)(e + 127);
    }
    __syncthreads();
    if (t < 32) {
      const uint4 d = *reinterpret_cast<const uint4*>(atom + 16 * t);
      *reinterpret_cast<uint4*>(p.SF + (int64_t)a * 512 + 16 * t) = d;
    }
    __syncthreads();  // the atom buffer is reused by the next atom
  }
}

}  // namespace quant
}  // namespace mxg
