// Row-wise E8M0 scales -> the physical scale-factor atom layout.
//
// "GEMM + RoPE + MXFP8 Projection (SM100)", section "Shapes": the MXFP8 input
// path carries its block scales row-wise, x_scale (tokens, Q_LORA / 32) and
// w_scale (rows of w, Q_LORA / 32), one byte per (row, block of 32 K).  The
// GEMM reads scales in the atom layout of "GEMM + Amax (SM100)", sections
// "Shapes" and "Using JAX arrays": 512-byte atom (l, mn / 128, kb / 4) holds
// row mn's block kb at byte 16 (mn % 32) + 4 ((mn / 32) % 4) + kb % 4.
//
// One workgroup of 128 threads per atom; thread t handles row 128 mb + t and
// writes that row's 4 bytes of the atom as one dword.  Rows past MN and
// blocks past ceil(K / sf) are padding: 127 (a scale of 1).
#pragma once

#include "mxgemm_common.hpp"

namespace mxg {
namespace repack {

constexpr int kThreads = 128;

struct RParams {
  const uint8_t* R;  // (L, MN, Kb) row-wise scale bytes
  uint8_t* SF;       // physical atoms
  int MN, Kb;
  int MNb, Kg;
  int num_atoms;
};

__global__ __launch_bounds__(kThreads) void rowwise_to_atoms_kernel(RParams p) {
  const int t = threadIdx.x;
  for (int a = blockIdx.x; a < p.num_atoms; a += gridDim.x) {
    const int kg = a % p.Kg;
    const int rest = a / p.Kg;
    const int mb = rest % p.MNb;
    const int l = rest / p.MNb;
    const int row = 128 * mb + t;
    unsigned w = 0x7F7F7F7Fu;
    if (row < p.MN) {
      const uint8_t* src = p.R + ((int64_t)l * p.MN + row) * p.Kb + 4 * kg;
      const int n = min(4, p.Kb - 4 * kg);  // >= 1: atom kg covers block 4 kg
      unsigned v = 0x7F7F7F7Fu;
      for (int j = 0; j < n; ++j) v = (v & ~(0xFFu << (8 * j))) | ((unsigned)src[j] << (8 * j));
      w = v;
    }
    *reinterpret_cast<unsigned*>(p.SF + (int64_t)a * 512 + 16 * (t & 31) + 4 * (t >> 5)) = w;
  }
}

}  // namespace repack
}  // namespace mxg
