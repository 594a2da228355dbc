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
//   rounded on its own: no fused multiply-add);
//   MXFP8 (E4M3 codes, one E8M0 scale per 32 values) along D (row codes
//   (tokens, H, D), scales (tokens, H, D/32)) and along tokens (column codes
//   (tokens, H, D), scales (tokens/32, H, D)), with the scale rule of the MX
//   quantiser (mx_quantize.hpp): e the smallest integer with 448 * 2^e >= the
//   block's largest magnitude, codes rounded to nearest, ties to even.
//
// One workgroup of 512 threads per (32-token block, head), in runs of
// consecutive heads.  The 32 x D tile is read with 16-byte loads (each
// token's D floats are contiguous), one tile ahead into registers, and parked
// in LDS at a pitch of D + 4 floats (rows stay 16-byte aligned, and a column
// read by 64 lanes hits 64 banks).  The tokens' cos / sin rows come in with
// 16-byte loads, once per token block.  A 4-feature group holds whole rotary
// pairs, so the thread that loaded it rotates them on the way into LDS (a_i
// to position i of the rotary part, b_i to R + i).  Then one thread per
// feature finds its column block's exponent, and finally thread (token r,
// features 16q .. 16q + 15) makes both directions' codes: the row block's
// maximum from one xor shuffle with the neighbouring lane, the column
// exponents from LDS; each direction's 16 codes leave as one 16-byte store.
// Row scale bytes collect in LDS over the workgroup's run of heads and leave
// at its end, a token's bytes for the whole run contiguous (scattered single
// bytes cost about 15% of the time).  The phases meet at barriers that wait
// for LDS operations only.
#pragma once

#include "mx_quantize.hpp"

namespace mxg {
namespace rope {

constexpr int kThreads = 512;  // 8 waves per workgroup
constexpr int kMaxD = 256;
constexpr int kMaxQR = 128;

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
  int per_wg;               // consecutive tiles per workgroup
};

// bytes of dynamic LDS for head size D and rotary width QR (34 KB for 192 / 64:
// four workgroups per CU)
inline size_t lds_bytes(int D, int QR, int per_wg) {
  return (size_t)32 * (D + 4) * 4 + (size_t)D * 4 + (size_t)64 * QR * 2 + (size_t)32 * per_wg * (D / 32);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) { return __uint_as_float((unsigned)b << 16); }

// DC, QC: the head size and rotary width as compile-time constants (the
// projection page's 192 and 64), so that the index arithmetic divides by
// constants; 0, 0 takes both from p.
template <int DC, int QC>
__global__ __launch_bounds__(kThreads) void proj_rope_mxfp8_kernel(RParams p) {
  // dynamic LDS, lds_bytes(D, QR): the tile (32 x (D + 4) floats), the column
  // exponents (D ints), the cos and sin rows (32 x QR bf16 each); every part
  // starts 16-byte aligned (D % 32 == 0, QR even)
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  float* z = reinterpret_cast<float*>(dyn);
  const int D = DC ? DC : p.D, QR = DC ? QC : p.QR;
  int* ecol = reinterpret_cast<int*>(z + 32 * (D + 4));
  uint16_t* csl = reinterpret_cast<uint16_t*>(ecol + D);
  uint16_t* snl = csl + 32 * QR;
  uint8_t* rsl = reinterpret_cast<uint8_t*>(snl + 32 * QR);  // the run's row scale bytes, (32, per_wg * nb)
  const int t = threadIdx.x;
  const int P = D + 4, HD = p.H * D;
  const int nope = D - QR, R = QR / 2, nb = D / 32;
  const int q4 = D / 4;  // float4 groups per token (a multiple of 8: D % 32 == 0)
  // a contiguous run of tiles per workgroup: consecutive heads of one token
  // block, so that a workgroup writes whole 128-byte lines of the code rows
  // (a head's row is D bytes) instead of sharing them with workgroups on
  // other XCDs
  // workgroups go round-robin over the 8 XCDs; with the grid a multiple of 8
  // the runs are renumbered so that consecutive runs (the heads of one token
  // block, which share the 128-byte lines of its row scales) run on one XCD
  // and meet in one L2
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  const int w = (G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b;
  const int a0 = w * p.per_wg, a1 = min(a0 + p.per_wg, p.num_tiles);
  const int run_bytes = (a1 - a0) * nb;  // a token's row scale bytes over the run (per_wg divides H)
  // thread t takes the tile's 16-byte groups f = t + kThreads k (token
  // f / q4, features 4 (f % q4) ..), the same in every tile, so their
  // offsets are worked out once: in Y and in the code arrays (both (tokens,
  // H * D) elements) relative to the tile's first element, and in LDS.  It
  // loads them one tile ahead: tile a + 1's loads go out right after tile a
  // reaches LDS and land while tile a is processed.  The phases meet at
  // barriers that wait for LDS operations only, so neither those loads nor
  // the code stores hold them.
  constexpr int kMaxF4 = 32 * (kMaxD / 4) / kThreads;
  int fr[kMaxF4], fc[kMaxF4], zo[kMaxF4];
  int64_t go[kMaxF4];
#pragma unroll
  for (int k = 0; k < kMaxF4; ++k) {
    const int f = t + kThreads * k;
    fr[k] = f / q4;
    fc[k] = f - fr[k] * q4;
    zo[k] = fr[k] * P + 4 * fc[k];
    go[k] = (int64_t)fr[k] * HD + 4 * fc[k];
  }
  const int ngroups = 32 * q4;
  float4 nx[kMaxF4];
  auto fetch = [&](int a) {
    const float* y = p.Y + (int64_t)(a / p.H) * 32 * HD + (int64_t)(a % p.H) * D;
#pragma unroll
    for (int k = 0; k < kMaxF4; ++k)
      if (t + kThreads * k < ngroups) nx[k] = *reinterpret_cast<const float4*>(y + go[k]);
  };
  if (a0 < a1) fetch(a0);
  int cs_tb = -1;  // the token block whose cos / sin rows are in LDS
  for (int a = a0; a < a1; ++a) {
    const int h = a % p.H, tb = a / p.H;
    const int64_t row0 = (int64_t)tb * 32;
    const int64_t base = row0 * HD + (int64_t)h * D;  // the tile's first element in Y and the code arrays
    barrier();  // the previous tile's LDS reads are done
    // the 32 tokens' cos / sin rows (32 * QR * 2 contiguous bytes per table),
    // once per token block
    if (tb != cs_tb) {
      for (int f = t; f < 4 * QR; f += kThreads) {
        reinterpret_cast<uint4*>(csl)[f] = reinterpret_cast<const uint4*>(p.cs + row0 * QR)[f];
        reinterpret_cast<uint4*>(snl)[f] = reinterpret_cast<const uint4*>(p.sn + row0 * QR)[f];
      }
      cs_tb = tb;
      barrier();
    }
    // the tile into LDS, RoPE applied on the way: a group of 4 features holds
    // whole pairs (a_i, b_i) = (feature nope + 2i, nope + 2i + 1), since nope
    // is even, and its thread writes the rotated a to position nope + i and b
    // to nope + R + i of the rotary part
#pragma unroll
    for (int k = 0; k < kMaxF4; ++k) {
      if (t + kThreads * k >= ngroups) continue;
      const int r = fr[k], c = fc[k];
      const float4 v = nx[k];
      if (4 * c + 3 < nope) {
        *reinterpret_cast<float4*>(z + zo[k]) = v;
      } else {
        // each product and the sum rounded on its own: a fused multiply-add
        // (which the compiler forms by default, also from __fmul_rn /
        // __fsub_rn, whose own operations carry the contraction flag) rounds
        // a*c - b*s once, and under cancellation that moves the value and
        // can flip a code.  Plain operators here, in a scope where
        // contraction is off.
#pragma clang fp contract(off)
        const float e4[4] = {v.x, v.y, v.z, v.w};
        float* zr = z + r * P;
        const uint16_t* cr = csl + r * QR;
        const uint16_t* sr = snl + r * QR;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 4 * c + j, kk = d - nope;
          if (kk < 0) {
            zr[d] = e4[j];
          } else if ((kk & 1) == 0 && j < 3) {
            const int i = kk >> 1;
            const float av = e4[j], bv = e4[j + 1];
            const float c1 = bf16_bits_to_float(cr[i]), s1 = bf16_bits_to_float(sr[i]);
            const float c2 = bf16_bits_to_float(cr[R + i]), s2 = bf16_bits_to_float(sr[R + i]);
            const float ac = av * c1, bs = bv * s1, bc = bv * c2, as = av * s2;
            zr[nope + i] = ac - bs;
            zr[nope + R + i] = bc + as;
          }
        }
      }
    }
    if (a + 1 < a1) fetch(a + 1);
    barrier();
    // column blocks: the exponent of feature d over the 32 tokens
    for (int d = t; d < D; d += kThreads) {
      float bm = 0.f;
#pragma unroll 8
      for (int r = 0; r < 32; ++r) bm = fmaxf(bm, fabsf(z[r * P + d]));
      const int e = quant::block_exponent<0>(bm);
      ecol[d] = e;
      p.col_scales[((int64_t)tb * p.H + h) * D + d] = (uint8_t)(e + 127);
    }
    barrier();
    // both directions' codes: thread (r, q) takes features 16q .. 16q + 15
    // of token r (D / 16 threads per token, an even count, so a 32-feature
    // row block is the lane pair q, q ^ 1 and one xor shuffle finds its
    // maximum), and each direction's 16 codes leave as one 16-byte store.
    // The row block's values share one exponent and convert with it as the
    // scale operand (bitwise ldexp then convert).
    {
      const int nq = D / 16;
      const int r = t / nq, q = t - r * nq;
      if (r < 32) {
        const float* zr = z + r * P + 16 * q;
        float4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const float4*>(zr + 4 * j);
        float bm = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bm = fmaxf(bm, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
        bm = fmaxf(bm, __shfl_xor(bm, 1));
        const int e = quant::block_exponent<0>(bm);
        uint4 rc, cc;
        const int* ec = ecol + 16 * q;
        unsigned* rcu = reinterpret_cast<unsigned*>(&rc);
        unsigned* ccu = reinterpret_cast<unsigned*>(&cc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rcu[j] = quant::codes4_e4m3_exp(v[j].x, v[j].y, v[j].z, v[j].w, e);
          ccu[j] = quant::codes4<0>(ldexpf(v[j].x, -ec[4 * j]), ldexpf(v[j].y, -ec[4 * j + 1]),
                                    ldexpf(v[j].z, -ec[4 * j + 2]), ldexpf(v[j].w, -ec[4 * j + 3]));
        }
        const int64_t o = base + (int64_t)r * HD + 16 * q;
        *reinterpret_cast<uint4*>(p.row_codes + o) = rc;
        *reinterpret_cast<uint4*>(p.col_codes + o) = cc;
        if ((q & 1) == 0) rsl[r * run_bytes + (a - a0) * nb + (q >> 1)] = (uint8_t)(e + 127);
      }
    }
  }
  // the run's row scales: per token, run_bytes contiguous bytes (heads h0 ..)
  // in one coalesced pass instead of a scattered byte per row block
  if (a0 < a1) {
    barrier();
    const int h0 = a0 % p.H;
    const int64_t row0 = (int64_t)(a0 / p.H) * 32;
    for (int f = t; f < 32 * run_bytes; f += kThreads) {
      const int r = f / run_bytes, b = f - r * run_bytes;
      p.row_scales[((row0 + r) * p.H + h0) * nb + b] = rsl[f];
    }
  }
}

}  // namespace rope
}  // namespace mxg
