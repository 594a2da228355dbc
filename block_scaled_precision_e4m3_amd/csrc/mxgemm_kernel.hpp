// Block-scaled FP8 GEMM with a fused global-amax epilogue for gfx950 (CDNA4).
//
// Computes, per batch l ("GEMM + Amax (SM100)", section "Equations"):
//   C[m,n] = sum_k dec(A[m,k]) 2^(SFA(m,k/sf)-127) * dec(B[n,k]) 2^(SFB(n,k/sf)-127)
//   Amax   = max |C|
//
// Two main-loop modes share everything but the innermost step:
//
// * kModeBf16 (default).  Each FP8 fragment is dequantised in registers with
//   v_cvt_scalef32_pk_bf16_{fp8,bf8} (code * 2^(sf-127) rounded to bf16,
//   exact whenever the value lies in bf16's range: scale bytes 3..246 for
//   E4M3, 10..239 for E5M2) and fed to v_mfma_f32_32x32x16_bf16, whose
//   products are exact and whose sums round like fp32 additions.  This meets
//   a 1e-5 * sum|A_hat||B_hat| error bound for any data.
// * kModeFp8.  The FP8 codes go straight into gfx950's scaled MFMA
//   (v_mfma_scale_f32_32x32x64_f8f6f4), which applies the E8M0 scales itself
//   at twice the bf16 rate.  Measured on MI355X, that instruction aligns the
//   products of each 8-element K group to the largest one and drops bits
//   more than 13 binary places below it, so terms far smaller than their
//   neighbours are truncated; on heavy-tailed data the result can miss the
//   bound above.  Opt-in only.
//
// Operand layouts (lane l, row r = l % 32, half h = l / 32):
//   32x32x64 f8f6f4: bytes 0..15 of a lane hold K [16h, 16h+16) of the 64-K
//     slice and bytes 16..31 hold K [32+16h, +16); lane r's scale covers
//     K [0,32) of row r and lane r+32's covers K [32,64).
//   32x32x16 bf16: 8 elements per lane; any assignment of (h, element) to K
//     works as long as A and B use the same one, because the scale is folded
//     into each element.  We give lane half h the contiguous K range
//     [32h, 32h+32) of the slice and MFMA j (j = 0..3) its bytes [8j, 8j+8).
//   Output (both): lane l, element e holds D[8(e/4) + 4h + e%4][r] for
//     (src0 row, src1 col).  B is src0 and A is src1, so a lane owns one
//     output row m and 4-element runs of n: float4 stores into n-major C.
//
// Workgroup: 256 threads = 4 waves in 2x2; tile BM x BN; wave tile
// (BM/2) x (BN/2) of 32x32 MFMA blocks; BK = 128 K bytes per main-loop step.
// Tiles are staged global -> LDS directly (buffer_load_dwordx4 ... lds),
// double buffered, one barrier per step.  LDS rows are 128 bytes; 16-byte
// chunk c of row r lives at chunk c ^ (r & 7), so the 16-byte fragment reads
// of 8 consecutive rows hit distinct banks.  A wave's load instruction fills
// 1 KB = 8 rows; lane i writes chunk i % 8 of row i / 8 and therefore
// fetches logical chunk (i % 8) ^ (i / 8) of that row.  Rows past M (N) and
// K chunks past K are fetched through an out-of-range buffer offset, which
// the hardware returns as zero.
//
// Scale factors: a lane's SF dword for (row, atom g) is bytes
// [16*(row%32) + 4*((row/32)%4), +4) of atom (l*MNb + row/128)*Kg + g: the 4
// K-blocks of that atom for that row.  sf=32: one atom per 128-K step, slice
// s covers blocks 2s and 2s+1.  sf=16: one atom per 64-K slice (4 blocks of
// 16).  Scale bytes of K-blocks past ceil(K/sf), of atoms past the last and
// of rows past M (N) read as 0x7F (1.0), so padding bytes (which may be
// anything, NaN included) never meet data.
//
// Scheduling: persistent; workgroup w takes tiles w, w+G, ...; tiles are
// ordered batch-major and, inside a batch, in groups of kGroupM tile rows
// walked column-major; with G a multiple of 8, slot w maps to XCD-contiguous
// runs (workgroups are dispatched round-robin over the 8 XCDs).
//
// Amax: each lane keeps max(bits(|c|)) over the outputs it stores, as an
// unsigned integer (the order of non-negative IEEE floats, NaN above +inf),
// reduced across the wave with xor-shuffles, then one atomic max per wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kBK = 128;    // K bytes per main-loop step
constexpr int kGroupM = 8;  // tile rows per raster group

constexpr int kModeBf16 = 0;
constexpr int kModeFp8 = 1;

struct Params {
  const uint8_t* A;
  const uint8_t* B;
  const uint8_t* SFA;
  const uint8_t* SFB;
  float* C;
  unsigned* amax_bits;
  int M, N, K, L;
  int Kb;      // ceil(K / sf): K-blocks
  int Kg;      // ceil(K / (4 sf)): atoms along K
  int MNbA;    // ceil(M / 128)
  int MNbB;    // ceil(N / 128)
  int tilesM, tilesN;
  int ksteps;  // ceil(K / 128)
  int64_t num_tiles;
  int xcd_remap;  // 1 when gridDim.x is a multiple of 8
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// --- tile scheduling ---------------------------------------------------------

__device__ __forceinline__ void tile_coords(const Params& p, int64_t t, int& l, int& tm, int& tn) {
  const int per_batch = p.tilesM * p.tilesN;
  l = (int)(t / per_batch);
  const int r = (int)(t - (int64_t)l * per_batch);
  const int group_size = kGroupM * p.tilesN;
  const int g = r / group_size;
  const int first_m = g * kGroupM;
  const int gm = min(p.tilesM - first_m, kGroupM);
  const int rg = r - g * group_size;
  tm = first_m + rg % gm;
  tn = rg / gm;
}

// --- global -> LDS staging ---------------------------------------------------

// Issue this wave's share of the loads of a ROWS x 128-byte tile.  `rsrc`
// covers the tile's valid rows (rows_valid * K bytes from the tile's first
// row); out-of-range fetches return zeros.
template <int ROWS>
__device__ __forceinline__ void load_tile_lds(uint8_t* lds_tile, __amdgpu_buffer_rsrc_t rsrc, int K, int k0,
                                              int rows_valid, int wave, int lane) {
  const int oob = rows_valid * K;  // first out-of-range byte
  const int rsub = lane >> 3;      // row within the 8-row group
  const int chunk = (lane & 7) ^ rsub;
  const int kk = k0 + (chunk << 4);
#pragma unroll
  for (int q = 0; q < ROWS / 32; ++q) {
    const int grp = wave + 4 * q;  // 8-row group
    const int row = grp * 8 + rsub;
    const int voff = (row < rows_valid && kk < K) ? row * K + kk : oob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds_tile + grp * 1024), 16, voff, 0, 0, 0);
  }
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 32 bytes of one row at chunks c0 and c1 (each 16 bytes).
__device__ __forceinline__ v8i read_frag(const uint8_t* lds, int row, int c0, int c1) {
  const uint8_t* rp = lds + row * kBK;
  const uint4 lo = *reinterpret_cast<const uint4*>(rp + ((c0 ^ (row & 7)) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(rp + ((c1 ^ (row & 7)) << 4));
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// --- scale factors -----------------------------------------------------------

__device__ __forceinline__ unsigned load_sf(const uint8_t* sf, int l, int mnb, int Kg, int Kb, int g, int row,
                                            int rows) {
  if (row >= rows || g >= Kg) return 0x7F7F7F7Fu;
  const int64_t atom = ((int64_t)l * mnb + (row >> 7)) * Kg + g;
  unsigned d = *reinterpret_cast<const unsigned*>(sf + atom * 512 + 16 * (row & 31) + 4 * ((row >> 5) & 3));
  const int valid = Kb - 4 * g;  // >= 1 here
  if (valid < 4) {
    const unsigned keep = (1u << (8 * valid)) - 1u;
    d = (d & keep) | (0x7F7F7F7Fu & ~keep);
  }
  return d;
}

// E8M0 byte -> the fp32 2^(b-127) used by the scaled conversions (byte 0 is
// the fp32 denormal 2^-127, byte 255 is NaN).
__device__ __forceinline__ float e8m0_to_f32(unsigned b) {
  const unsigned bits = b == 0u ? 0x00400000u : (b == 255u ? 0x7FC00000u : (b << 23));
  return __uint_as_float(bits);
}

// --- one 64-K slice ----------------------------------------------------------

template <int OPSEL, int FA, int FB>
__device__ __forceinline__ v16f mfma_f8(const v8i& b, const v8i& a, const v16f& c, unsigned sb, unsigned sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, FB, FA, OPSEL, (int)sb, OPSEL, (int)sa);
}

// Two FP8 codes (bytes 0,1 or 2,3 of `w`) -> two bf16 times `scale`, as one dword.
template <int FMT, bool HI>
__device__ __forceinline__ unsigned cvt2(unsigned w, float scale) {
  v2bf r;
  if constexpr (FMT == 0)
    r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI);
  else
    r = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, scale, HI);
  return __builtin_bit_cast(unsigned, r);
}

// 8 codes (two dwords) -> one bf16 MFMA operand.
template <int FMT>
__device__ __forceinline__ v8bf cvt8(unsigned w0, unsigned w1, float scale) {
  v4u u;
  u[0] = cvt2<FMT, false>(w0, scale);
  u[1] = cvt2<FMT, true>(w0, scale);
  u[2] = cvt2<FMT, false>(w1, scale);
  u[3] = cvt2<FMT, true>(w1, scale);
  return __builtin_bit_cast(v8bf, u);
}

template <int MODE, int S, int SF, int FA, int FB, int TM, int TN>
__device__ __forceinline__ void compute_slice(v16f (&acc)[TM][TN], const uint8_t* ldsA, const uint8_t* ldsB,
                                              int arow0, int brow0, int lane, const unsigned (&sfa)[2][TM],
                                              const unsigned (&sfb)[2][TN]) {
  const int r = lane & 31;
  const int h = lane >> 5;
  if constexpr (MODE == kModeFp8) {
    const int c0 = 4 * S + h;
    v8i af[TM], bf[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = read_frag(ldsA, arow0 + 32 * i + r, c0, c0 + 2);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = read_frag(ldsB, brow0 + 32 * j + r, c0, c0 + 2);
    if constexpr (SF == 32) {
      // scale dwords pre-shifted by 8h: byte 2S selects block 2S + h
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = mfma_f8<2 * S, FA, FB>(bf[j], af[i], acc[i][j], sfb[0][j], sfa[0][i]);
    } else {
      // scale dwords pre-shifted by 16h; split the lane's two 16-K blocks
      const v8i zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const v8i a_even = h ? zero : af[i];
        const v8i a_odd = h ? af[i] : zero;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = mfma_f8<0, FA, FB>(bf[j], a_even, acc[i][j], sfb[S][j], sfa[S][i]);
          acc[i][j] = mfma_f8<1, FA, FB>(bf[j], a_odd, acc[i][j], sfb[S][j], sfa[S][i]);
        }
      }
    }
  } else {
    // lane half h owns K [32h, 32h+32) of the slice: chunks 4S+2h, 4S+2h+1
    const int c0 = 4 * S + 2 * h;
    v8i af[TM], bf[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = read_frag(ldsA, arow0 + 32 * i + r, c0, c0 + 1);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = read_frag(ldsB, brow0 + 32 * j + r, c0, c0 + 1);
    // scale bytes: sf=32 -> block 2S+h (byte 0 of the dword pre-shifted by
    // 8*(2S+h)); sf=16 -> blocks 2h, 2h+1 of this slice's atom (bytes 0, 1 of
    // the dword pre-shifted by 16h).
    float sa0[TM], sa1[TM], sb0[TN], sb1[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const unsigned d = (SF == 32) ? sfa[0][i] >> (16 * S) : sfa[S][i];
      sa0[i] = e8m0_to_f32(d & 0xFFu);
      sa1[i] = (SF == 32) ? sa0[i] : e8m0_to_f32((d >> 8) & 0xFFu);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const unsigned d = (SF == 32) ? sfb[0][j] >> (16 * S) : sfb[S][j];
      sb0[j] = e8m0_to_f32(d & 0xFFu);
      sb1[j] = (SF == 32) ? sb0[j] : e8m0_to_f32((d >> 8) & 0xFFu);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v8bf ab[TM], bb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) ab[i] = cvt8<FA>(af[i][2 * q], af[i][2 * q + 1], q < 2 ? sa0[i] : sa1[i]);
#pragma unroll
      for (int j = 0; j < TN; ++j) bb[j] = cvt8<FB>(bf[j][2 * q], bf[j][2 * q + 1], q < 2 ? sb0[j] : sb1[j]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bb[j], ab[i], acc[i][j], 0, 0, 0);
    }
  }
}

// --- the kernel --------------------------------------------------------------

template <int BM, int BN, int SF, int FA, int FB, int MODE, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void mxgemm_amax_kernel(Params p) {
  constexpr int WM = BM / 2, WN = BN / 2;   // wave tile
  constexpr int TM = WM / 32, TN = WN / 32; // MFMA blocks per wave
  constexpr int STAGE = (BM + BN) * kBK;    // bytes per LDS stage
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31;
  const int h = lane >> 5;
  // scale dword pre-shift per lane half (see compute_slice)
  const int sf_shift = (SF == 32) ? 8 * h : 16 * h;

  unsigned lmax = 0u;

  const int64_t G = gridDim.x;
  int64_t slot = blockIdx.x;
  if (p.xcd_remap) slot = (int64_t)(blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  for (int64_t t = slot; t < p.num_tiles; t += G) {
    int l, tm, tn;
    tile_coords(p, t, l, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int mvalid = min(p.M - m0, BM), nvalid = min(p.N - n0, BN);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.A + ((int64_t)l * p.M + m0) * p.K), (short)0, mvalid * p.K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.B + ((int64_t)l * p.N + n0) * p.K), (short)0, nvalid * p.K, 0x00020000);

    const int arow_g = m0 + wm * WM + r;
    const int brow_g = n0 + wn * WN + r;

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    unsigned sfa[2][TM], sfb[2][TN];

    auto fetch_sf = [&](int kt, unsigned (&fa)[2][TM], unsigned (&fb)[2][TN]) {
#pragma unroll
      for (int s = 0; s < (SF == 32 ? 1 : 2); ++s) {
        const int g = (SF == 32) ? kt : 2 * kt + s;
#pragma unroll
        for (int i = 0; i < TM; ++i)
          fa[s][i] = load_sf(p.SFA, l, p.MNbA, p.Kg, p.Kb, g, arow_g + 32 * i, p.M) >> sf_shift;
#pragma unroll
        for (int j = 0; j < TN; ++j)
          fb[s][j] = load_sf(p.SFB, l, p.MNbB, p.Kg, p.Kb, g, brow_g + 32 * j, p.N) >> sf_shift;
      }
    };

    auto issue_tiles = [&](int kt) {
      uint8_t* st = lds + (kt & 1) * STAGE;
      load_tile_lds<BM>(st, ra, p.K, kt * kBK, mvalid, wave, lane);
      load_tile_lds<BN>(st + BM * kBK, rb, p.K, kt * kBK, nvalid, wave, lane);
    };

    if (p.ksteps > 0) {
      issue_tiles(0);
      fetch_sf(0, sfa, sfb);
    }

    for (int kt = 0; kt < p.ksteps; ++kt) {
      // this step's tiles (issued one step earlier) have landed in LDS, and
      // every wave has finished reading the other stage
      wait_vm_all();
      __syncthreads();
      unsigned nsfa[2][TM], nsfb[2][TN];
      const bool more = kt + 1 < p.ksteps;
      if (more) {
        issue_tiles(kt + 1);
        fetch_sf(kt + 1, nsfa, nsfb);
      }
      const uint8_t* cur = lds + (kt & 1) * STAGE;
      compute_slice<MODE, 0, SF, FA, FB, TM, TN>(acc, cur, cur + BM * kBK, wm * WM, wn * WN, lane, sfa, sfb);
      compute_slice<MODE, 1, SF, FA, FB, TM, TN>(acc, cur, cur + BM * kBK, wm * WM, wn * WN, lane, sfa, sfb);
      if (more) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
          for (int i = 0; i < TM; ++i) sfa[s][i] = nsfa[s][i];
#pragma unroll
          for (int j = 0; j < TN; ++j) sfb[s][j] = nsfb[s][j];
        }
      }
    }
    // all waves are done with LDS before the next tile's first loads land
    __syncthreads();

    // epilogue: C stores and the running |C| maximum
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm * WM + 32 * i + r;
      if (m < p.M) {
        float* crow = p.C + ((int64_t)l * p.M + m) * p.N;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn * WN + 32 * j + 8 * q + 4 * h;
            if (n < p.N) {
              v4f v;
              v[0] = acc[i][j][4 * q];
              v[1] = acc[i][j][4 * q + 1];
              v[2] = acc[i][j][4 * q + 2];
              v[3] = acc[i][j][4 * q + 3];
              __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(crow + n));
              lmax = max(lmax, __float_as_uint(v[0]) & 0x7FFFFFFFu);
              lmax = max(lmax, __float_as_uint(v[1]) & 0x7FFFFFFFu);
              lmax = max(lmax, __float_as_uint(v[2]) & 0x7FFFFFFFu);
              lmax = max(lmax, __float_as_uint(v[3]) & 0x7FFFFFFFu);
            }
          }
        }
      }
    }
  }

#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lmax = max(lmax, (unsigned)__shfl_xor((int)lmax, off));
  if (lane == 0 && lmax != 0u) atomicMax(p.amax_bits, lmax);
}

__global__ void amax_reset_kernel(unsigned* amax_bits) {
  if (threadIdx.x == 0) *amax_bits = 0u;
}

}  // namespace mxg
