// Block-scaled FP8 GEMM with a fused global-amax epilogue for gfx950 (CDNA4).
//
// Computes, per batch l ("GEMM + Amax (SM100)", sections "Equations" and
// "Shapes"):
//   C[m,n] = sum_k dec(A[m,k]) 2^(SFA(m,k/sf)-127) * dec(B[n,k]) 2^(SFB(n,k/sf)-127)
//   Amax   = max |C|
//
// Two datapaths share everything but the innermost step:
//
// * bf16 (default).  Each FP8 (or FP4) code is dequantised in registers with
//   v_cvt_scalef32_pk_bf16_{fp8,bf8,fp4} (code * 2^(byte-127) rounded to
//   bf16, exact whenever the value is a bf16 number) and fed to
//   v_mfma_f32_32x32x16_bf16, whose products are exact and whose sums are
//   fp32 additions.
// * FP8 (opt-in).  The codes go straight into the scaled MFMA
//   v_mfma_scale_f32_32x32x64_f8f6f4, which applies the E8M0 scales itself at
//   twice the bf16 rate but keeps only the bits of each product down to
//   2^-13 of the largest in its 8-element K group, so terms much smaller
//   than their neighbours are truncated.
//
// Work shape: one workgroup per CU, 4 computing waves in 2 x 2, on square C
// tiles of BT x BT (BT = 256: waves of 128 x 128 in 4 x 4 MFMA blocks, all
// 256 matrix-core registers; BT = 128: waves of 64 x 64).  Tiles are taken
// persistently: workgroup w runs tiles w, w+G, ....
//
// * The K loop moves 128 bytes of every operand row per step through an LDS
//   ring (2 stages for BT = 256, 4 for the bf16 datapath at BT = 128) by
//   direct global->LDS DMA, the step's E8M0 atoms beside the tile.  Per
//   128-K step a 256x256 tile moves 64 KB for 8.4 M multiply-adds, a
//   128x128 tile 32 KB for 2.1 M.  The 4-stage ring's DMA comes from 4 more
//   waves that do nothing else, so that a DMA instruction waiting for room in
//   the vector-memory queue holds up no MFMA issue (a 128x128 tile moves
//   twice the bytes per flop of a 256x256 one).  The 256x256 waves hold all
//   512 registers of their SIMD, leaving no room for a second wave.
// * bf16 step: 8 MFMA slices of 16 K; each slice's conversions run under the
//   previous slice's MFMAs (scheduling-group barriers pin the interleave), so
//   one wave per SIMD keeps the matrix core fed; one barrier per step.
// * C stores.  A tile's C is stored at its end, transposed through LDS so
//   that every store writes whole 128-byte lines.  Every CU ends its tiles at
//   about the same time, so the stores drain slowly; the DMA of the next
//   steps is queued before those stores, so that the next tile's first
//   steps wait for their DMA only and the stores drain under their MFMAs (the
//   vector-memory counter retires in issue order).
//
// bf16 datapath, per 32-K chunk c of a step: lane (r, h) reads the 16 bytes
// K [32c + 16h, +16) of its row for each of its A and B fragments; bytes
// 0..7 feed MFMA slice 0 and bytes 8..15 slice 1 (any K assignment is valid
// when A and B share it, since the scale is folded into every element).  The
// chunk lies in one K-block for sf=32 (block c) and for sf=16 (block 2c + h).
// FP8 datapath, per 64-K slice S: bytes 0..15 of a lane are K [16h, +16) and
// bytes 16..31 are K [32 + 16h, +16) of the slice, as the scaled MFMA needs.
// MFMA output layout: lane l, element e holds D[8(e/4) + 4h + e%4][r] for
// (src0 row, src1 col); B is src0 and A src1 (an m-major C swaps them), so
// a lane owns one C row and 4-element runs along the contiguous dimension.
//
// Amax: each lane keeps max(bits(|c|)) over the outputs it stores, as an
// unsigned integer (the order of non-negative IEEE floats, NaN above +inf),
// reduced across the wave with xor-shuffles and across the computing waves in
// LDS; the workgroup then issues one atomic max, and only if its maximum is
// above the value Amax holds. Atomics on one address from every CU serialize
// in the memory system (about 10 ns each): one per wave at the end of a
// one-round grid cost a quarter of the time of a 2048^3 problem.
#pragma once

#include "mx_quantize.hpp"
#include "mxgemm_common.hpp"

namespace mxg {
namespace big {

constexpr int kThreads = 256;
constexpr int kBK = 128;

// Square C tiles of BT x BT (256 or 128): 2 x 2 waves, each (BT/2) x (BT/2) in
// (BT/64) x (BT/64) blocks of 32 x 32.
template <int SF, bool FP4, int BT, int NST>
struct Layout {
  static_assert(BT == 256 || BT == 128, "tile size");
  static constexpr int kStages = NST;                // LDS ring stages
  static constexpr int kBM = BT, kBN = BT;
  static constexpr int KE = FP4 ? 256 : 128;         // K elements per step (128 bytes per row)
  static constexpr int NSF = KE / (4 * SF);          // atoms per 128-row group per step
  static constexpr int kGroups = BT / 128;           // 128-row atom groups per operand tile
  // atom bytes per operand per stage: the atoms of both 128-row groups; for
  // a 128-row tile one kilobyte, which takes the one wave's scale DMA (one
  // group's NSF atoms, or with NSF = 1 its atom and the zeros its other half
  // of the wave reads for a group past the tile), or with NSF = 4 (FP4 at
  // sf = 16) two kilobytes, the scale DMAs of two waves
  static constexpr int kSF = BT == 256 ? 2 * NSF * 512 : (NSF == 4 ? 2048 : 1024);
  static constexpr int kOffB = kBM * kBK;            // A tile: BT rows x 128 bytes
  static constexpr int kOffSFA = kOffB + kBN * kBK;  // B tile: BT rows x 128 bytes
  static constexpr int kOffSFB = kOffSFA + kSF;
  static constexpr int kStage = kOffSFB + kSF;
  static constexpr int kDmaA = kBM / 32;             // A DMA instructions per wave per step
  static constexpr int kDma = (kBM + kBN) / 32;      // A/B DMA instructions per wave per step
  // Per-wave LDS area where the epilogue transposes one 32x32 fp32 block
  // (rows padded to 36 floats) so its stores write whole 128-byte lines.
  static constexpr int kEpiRow = 36;
  static constexpr int kEpiWave = 32 * kEpiRow * 4;
  static constexpr int kEpiBytes = 4 * kEpiWave;
  // Two kilobytes where the scale DMA of a wave that loads no atoms (sf = 32:
  // waves 2 and 3) writes its zeros: every wave issues the same instructions,
  // so a step stays one branch-free block the scheduler can interleave.  It
  // is apart from the epilogue area because that DMA may still be in flight
  // while the epilogue runs.
  static constexpr int kOffEpi = NST * kStage;
  static constexpr int kOffDummy = kOffEpi + kEpiBytes;
  static constexpr int kLds = kOffDummy + 2048;
};

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ unsigned lds4(const uint8_t* p) { return *reinterpret_cast<const unsigned*>(p); }

// Bytes of K-blocks at or past Kb in the dword of atom g become 0x7F (1.0):
// padding bytes past K (possibly NaN) must not meet the zero-filled data.
__device__ __forceinline__ unsigned sf_tail(unsigned d, int g, int Kb) {
  const int valid = Kb - 4 * g;
  const unsigned keep = valid >= 4 ? 0xFFFFFFFFu : (valid <= 0 ? 0u : (1u << (8 * valid)) - 1u);
  return (d & keep) | (0x7F7F7F7Fu & ~keep);
}

// 8 bytes of an m-major tile held in LDS as (K row, M column), read with the
// transposing LDS load: the lanes of each group of 16 give 16 row addresses
// and lane j receives byte (j & 7) of the rows given by lanes 2b + (j >> 3),
// b = 0..7 (measured on MI355X for three address patterns).
__device__ __forceinline__ uint2 lds_tr8(const uint8_t* p) {
  typedef int v2i_t __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;
  const v2i_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(p));
  return make_uint2((unsigned)v[0], (unsigned)v[1]);
}

// MJ: operand majors, bit 0 A m-major ((L, K, M) bytes, M contiguous), bit 1
// B n-major ((L, K, N)); 8-bit codes on the bf16 datapath with a float32
// n-major C.  NW: waves per workgroup, 4, or 8 on the 128x128 ring (every
// format but FP4 at sf = 16), where waves 4..7 only stream the operands into
// the ring (each what wave w - 4 would queue) and waves 0..3 only compute and
// store, so no DMA instruction waiting for room in the vector-memory queue
// holds up the computing waves.
template <int SF, int FA, int FB, int MODE, int CT, int BT, int MJ = 0, int NW = 4>
__global__ __launch_bounds__(64 * NW, 1) void mxgemm_amax_big_kernel(Params p) {
  // FA = FB = 2: packed FP4 (E2M1), bf16 datapath, sf = 32 (the host enforces it)
  constexpr bool kFp4 = FA == 2;
  static_assert(!kFp4 || (FB == 2 && MODE == kModeBf16), "FP4: both operands, bf16 path");
  static_assert(!(kFp4 && SF == 16) || (BT == 128 && CT != 4), "FP4 at sf = 16: 128x128 tiles (LDS)");
  static_assert(!kCMajorM<CT> || MODE == kModeBf16, "m-major C: bf16 path");
  static_assert(CT != 4 || (MODE == kModeBf16 && BT == 256), "projection epilogue: bf16 path, 256x256 tiles");
  constexpr bool kAMaj = (MJ & 1) != 0, kBMaj = (MJ & 2) != 0;
  static_assert(MJ == 0 || (MODE == kModeBf16 && !kFp4 && CT == 0), "m-major operands: 8-bit, bf16 path, f32 C");
  static_assert(NW == 4 || (NW == 8 && BT == 128 && MODE == kModeBf16 && !(kFp4 && SF == 16) && CT != 4),
                "8 waves: the 128x128 ring of the bf16 path");
  // LDS ring stages: a 128x128 tile's steps are short, so its bf16 datapath
  // queues the DMA three steps ahead in four stages; a 256x256 tile's ring
  // fills the LDS with two
  // (FP4 at sf = 16 carries four scale atoms per step and keeps two stages)
  constexpr int kStages = (BT == 128 && MODE == kModeBf16 && !(kFp4 && SF == 16)) ? 4 : 2;
  using Y = Layout<SF, kFp4, BT, kStages>;
  constexpr int kBM = Y::kBM, kBN = Y::kBN;
  constexpr int kTM = BT / 64, kTN = BT / 64;  // 32x32 MFMA blocks per wave
  constexpr int kWM = kBM / 2, kWN = kBN / 2;  // wave tile rows and columns
  static_assert(Y::NSF == 1 || Y::NSF == 2 || (Y::NSF == 4 && BT == 128),
                "one or two scale atoms per 128-row group per step, or four in a 128-row tile");
  constexpr int kEs = kCBytes<CT>;  // bytes per C element
  constexpr int NSF = Y::NSF;
  static_assert(Y::kLds <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Y::kLds];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int dw = NW == 8 ? wave & 3 : wave;  // the wave's share of the DMA
  const bool producer = NW == 8 && wave >= 4;  // 8 waves: this wave only queues DMA
  const int wm = NW == 8 ? (wave >> 1) & 1 : wave >> 1, wn = wave & 1;

  const int G = (int)gridDim.x;
  const int t0 = first_tile(p);
  const int my_tiles = t0 < p.num_tiles ? (p.num_tiles - 1 - t0) / G + 1 : 0;
  const unsigned lds0 = lds_addr(lds);

  // Per-lane geometry.  It is recomputed every step from an opaque copy of the
  // lane id: values the compiler sees as loop-invariant get hoisted out of the
  // K loop and then spilled, and a spill reload inside the loop makes it wait
  // for every DMA in flight.
  struct Geo {
    int r, h;           // fragment row (lane % 32) and lane half
    int xr;             // the swizzle of every fragment row of this lane (see kchunk)
    int a_off, b_off;   // LDS offset of the lane's first A / B fragment row
    unsigned row_k;     // DMA: byte offset of the lane's row in its first 8-row group
    unsigned kchunk;    // DMA: the lane's 16-byte K chunk inside a 128-byte row
    // LDS swizzle: 16-byte chunk c of tile row t sits at slot c ^ f(t), f(t) =
    // (t & 7) ^ ((t >> 3) & 1).  The 16 rows that one pass of a 16-byte read
    // serves then cover all 64 banks (rows t and t+1 differ in the 128-byte
    // half, rows t and t+8 in f), and any 8 consecutive rows cover 32 banks.
    unsigned sf_lane;   // SF DMA: the lane's 16 bytes inside an atom
    int sf_rg, sf_j;    // SF DMA: 128-row group and atom along K of the lane's load
  };
  auto geo = [&](int ln) {
    Geo g;
    g.r = ln & 31;
    g.h = ln >> 5;
    g.xr = (ln & 7) ^ ((ln >> 3) & 1);
    g.a_off = (kWM * wm + g.r) * kBK;
    g.b_off = Y::kOffB + (kWN * wn + g.r) * kBK;
    const int dma_row = ln >> 3;
    g.row_k = (unsigned)(dw * 8 + dma_row) * (unsigned)p.Kbytes;
    g.kchunk = (unsigned)(((ln & 7) ^ dma_row ^ (dw & 1)) << 4);
    g.sf_lane = 16u * (unsigned)(ln & 31);
    g.sf_rg = NSF == 1 ? (ln >> 5) : NSF == 4 ? 0 : (dw >> 1);
    g.sf_j = NSF == 1 ? 0 : NSF == 4 ? 2 * (dw >> 1) + (ln >> 5) : (ln >> 5);
    return g;
  };
  auto lane_opaque = [&]() {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return ln;
  };
  // The lane geometry, computed once: the 128x128 ring's steps and DMA waves,
  // and the 256x256 steps (both datapaths) of k-major 8-bit operands with a
  // stored C, take it from here rather than rebuilding it every step from the
  // opaque lane index (20-28 VALU instructions fewer per step: 2048^3 24.5 ->
  // 23.6 us, 8192x24576x1536 520.6 -> 513.9 us, 4000x7168x2048 at sf = 16
  // 110.7 -> 108.7 us, the FP8 datapath 1.5-4%; at sf = 16 one register then
  // spills, outside the K loop).  The
  // other 256x256 instances (FP4, m-major operands, the projection epilogue)
  // would spill dozens of registers with it held, so they keep rebuilding it.
  const Geo g_lane = geo(lane);
  constexpr bool kHoistGeo = BT == 128 || (!kFp4 && MJ == 0 && CT != 4);

  // --- DMA of one stage ------------------------------------------------------
  // A/B: wave w fills the 8-row groups w, w+4, ... of each tile, one
  // instruction (1 KB) per group: 8 for A, 8 for B.  A lane's offset is
  // row*K + k; rows past the tile's valid rows fall past the resource
  // (num_records = valid rows * K) and K chunks past K get an offset of 2^31
  // or more: both read as zero.  A and B rows use the same offsets, only the
  // resources differ.  SF: sf=32 -> waves 0 and 1 load the A and B atoms of
  // both 128-row groups (lanes 0-31 group 0, 32-63 group 1); sf=16 (or FP4)
  // -> waves 0,1 (A,B) load row group 0's two atoms, waves 2,3 row group
  // 1's (256-row tiles only); four atoms per step (FP4 at sf=16, 128-row
  // tiles) -> waves 0,1 (A,B) atoms 0 and 1, waves 2,3 atoms 2 and 3.  Groups
  // past the matrix or the tile read as zero.  Waves that load no atoms issue the same instruction on an empty
  // resource into their own kilobyte of the dummy area (no branch in the
  // step).
  constexpr unsigned kOob = 0x80000000u;
  const bool sf_wave = (NSF == 2 && BT == 256) || NSF == 4 || dw < 2;
  const bool sf_is_b = (dw & 1) != 0;
  // An m-major operand (MJ) is staged as 128 K rows of BT bytes (its tile's
  // columns), 16-byte chunk u of K row k at slot u ^ sw(k), sw(k) = 2 (k & 7)
  // for BT = 256 and 2 ((k >> 1) & 3) for BT = 128: the transposing reads of
  // a pass then cover every bank once.  DMA instruction q of wave w fills K
  // rows (BT == 256 ? 4 : 8) * (w + 4q) onward, one kilobyte, lane l taking
  // row (BT == 256 ? l / 16 : l / 8) of those and slot l % (BT / 16); chunks
  // past the matrix's columns or K rows past K read as zero (the host
  // requires columns in whole chunks).
  constexpr int kMjRowsPerQ = BT == 256 ? 16 : 32;  // K rows between a wave's DMA instructions
  struct Dma {
    __amdgpu_buffer_rsrc_t ra, rb, rs;
    unsigned voff_a, voff_b;  // lane's offset for instruction 0 (or >= 2^31)
    int left_a, left_b;       // m-major: K rows from the lane's first to K (0 if none valid)
    unsigned sf_voff;  // lane's SF offset
    unsigned dst;      // LDS address of the stage
  };
  // m-major operand X (MN columns) of tile columns mn0..: resource, lane offset, rows left
  auto mj_setup = [&](const Geo& g, const uint8_t* X, int MN, int mn0, int l, int kt, bool live,
                      __amdgpu_buffer_rsrc_t& rsrc, unsigned& voff, int& left) {
    const int ln = g.r + 32 * g.h;
    const int64_t base = (int64_t)l * MN * p.K + mn0;
    rsrc = make_rsrc(X + base, live ? (unsigned)((int64_t)MN * p.K - mn0) : 0u);
    const int row = BT == 256 ? 4 * dw + (ln >> 4) : 8 * dw + (ln >> 3);
    const int sw = BT == 256 ? 2 * ((4 * (dw & 1) + (ln >> 4)) & 7) : 2 * ((ln >> 4) & 3);
    const int u = (BT == 256 ? (ln & 15) : (ln & 7)) ^ sw;
    const int krow = kt * kBK + row;
    const bool ok = mn0 + 16 * u < MN && krow < p.K;
    voff = ok ? (unsigned)krow * (unsigned)MN + 16u * (unsigned)u : kOob;
    left = ok ? p.K - krow : 0;
  };
  auto dma_setup = [&](const Geo& g, const Tile& T, int kt, bool live, unsigned stage) {
    Dma d;
    const unsigned kk = (unsigned)(kt * kBK) + g.kchunk;
    const unsigned voff = kk < (unsigned)p.Kbytes ? g.row_k + kk : kOob;
    if constexpr (kAMaj) {
      mj_setup(g, p.A, p.M, T.m0, T.l, kt, live, d.ra, d.voff_a, d.left_a);
    } else {
      d.ra = make_rsrc(p.A + ((int64_t)T.l * p.M + T.m0) * p.Kbytes,
                       live ? (unsigned)T.mvalid * (unsigned)p.Kbytes : 0u);
      d.voff_a = voff;
      d.left_a = 0;
    }
    if constexpr (kBMaj) {
      mj_setup(g, p.B, p.N, T.n0, T.l, kt, live, d.rb, d.voff_b, d.left_b);
    } else {
      d.rb = make_rsrc(p.B + ((int64_t)T.l * p.N + T.n0) * p.Kbytes,
                       live ? (unsigned)T.nvalid * (unsigned)p.Kbytes : 0u);
      d.voff_b = voff;
      d.left_b = 0;
    }
    const int mn0 = sf_is_b ? T.n0 : T.m0;
    const int mnb = sf_is_b ? p.MNbB : p.MNbA;
    const int g0 = mn0 >> 7;
    const unsigned nrec =
        ((int)live & (int)sf_wave) ? (unsigned)min(Y::kGroups, mnb - g0) * (unsigned)p.Kg * 512u : 0u;
    d.rs = make_rsrc((sf_is_b ? p.SFB : p.SFA) + ((int64_t)T.l * mnb + g0) * p.Kg * 512, nrec);
    const int kg = NSF * kt + g.sf_j;
    d.sf_voff = kg < p.Kg ? (unsigned)(g.sf_rg * p.Kg + kg) * 512u + g.sf_lane : kOob;
    d.dst = stage;
    return d;
  };
  // A/B DMA instruction q of this wave: q < kDmaA -> A group wave + 4q, else
  // B group wave + 4(q - kDmaA)
  const unsigned grp_stride = 32u * (unsigned)p.Kbytes;
  auto dma_ab = [&](const Dma& d, int q) {
    const bool qb = q >= Y::kDmaA;
    const int qq = qb ? q - Y::kDmaA : q;
    const bool mj = qb ? kBMaj : kAMaj;
    unsigned voff;
    if (mj) {
      const unsigned mn = (unsigned)(qb ? p.N : p.M);
      voff = qq * kMjRowsPerQ < (qb ? d.left_b : d.left_a)
                 ? (qb ? d.voff_b : d.voff_a) + (unsigned)(qq * kMjRowsPerQ) * mn
                 : kOob;
    } else {
      voff = (qb ? d.voff_b : d.voff_a) + (unsigned)qq * grp_stride;
    }
    const unsigned dst = d.dst + (qb ? (unsigned)Y::kOffB : 0u) + (unsigned)(dw + 4 * qq) * 1024u;
    dma16_at(qb ? d.rb : d.ra, voff, dst);
  };
  // waves 2 and 3 (the only ones that use it) each own a kilobyte
  const unsigned sf_dummy = lds0 + (unsigned)Y::kOffDummy + (unsigned)(dw & 1) * 1024u;
  auto dma_sf = [&](const Dma& d) {
    const unsigned dst = d.dst + (sf_is_b ? (unsigned)Y::kOffSFB : (unsigned)Y::kOffSFA) +
                         (NSF == 1 ? 0u : (unsigned)(dw >> 1) * 1024u);
    dma16_at(d.rs, d.sf_voff, sf_wave ? dst : sf_dummy);
  };

  v16f acc[kTM][kTN];  // written by each tile's first step before any read
  constexpr int kNStores = kTM * kTN * 4;  // C store instructions per lane per tile (at least)
  static_assert(kNStores <= 64, "vmcnt counts to 63");
  const v16f zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  unsigned lmax = 0u;

  // --- C stores -----------------------------------------------------------------
  // n-major C: lane (r, h) of block (i, j) holds C row m = 128*wm + 32i + r
  // and, for q = 0..3, the 4 columns n = kWN*wn + 32j + 8q + 4h + (0..3).
  // m-major C (CT = 3, the MFMA operands swapped): the lane holds row
  // n = kWN*wn + 32j + r of the (L, N, M) layout and the 4 columns
  // m = 128*wm + 32i + 8q + 4h + (0..3).  Either way a "row" runs along the
  // layout's outer dimension and a "column" along its contiguous one.  Rows
  // past the tile's valid rows land past the resource (num_records = valid
  // rows * row length * element size); columns past the matrix get an offset
  // past it as well.  Every store folds its values into the lane's amax.
  constexpr bool kMM = kCMajorM<CT>;
  struct StoreCtx {
    __amdgpu_buffer_rsrc_t rc;
    unsigned c_bytes;
    int rvalid, cvalid, c0, stride;  // valid rows, valid columns, first column, row length
  };
  auto store_ctx = [&](const Tile& T) {
    StoreCtx x;
    x.stride = kMM ? p.M : p.N;
    x.rvalid = kMM ? T.nvalid : T.mvalid;
    x.cvalid = kMM ? T.mvalid : T.nvalid;
    x.c0 = kMM ? T.m0 : T.n0;
    const int64_t row0 = kMM ? (int64_t)T.l * p.N + T.n0 : (int64_t)T.l * p.M + T.m0;
    x.c_bytes = (unsigned)x.rvalid * (unsigned)x.stride * (unsigned)kEs;
    x.rc = make_rsrc(reinterpret_cast<uint8_t*>(p.C) + row0 * x.stride * kEs, x.c_bytes);
    return x;
  };
  // Every block of `acc` at tile end.  A block goes through the
  // wave's LDS area: lane (r, h) writes its row r, columns 8q + 4h straight
  // from the accumulation registers; lane L then reads row 8k + L/8, columns
  // 4(L%8) .. +4, so each of the block's 4 stores covers 8 rows x 128
  // contiguous bytes (whole cache lines; 64 bytes with a 16-bit C) instead
  // of 32 rows x 2 x 16 bytes.
  // Rows of 36 floats keep both passes free of bank conflicts.  The wave's LDS
  // operations execute in order, so block b+1 is written and read back while
  // block b's stores go out (its reads precede those writes), with no barrier.
  // 128x128 tiles (small problems, whose C mostly leaves L2 in the write-back
  // at the kernel's end) store non-temporally: 4% on 2048^3; on 256x256 tiles
  // it changed nothing measurable
  constexpr int kCPolicy = BT == 128 ? 2 : 0;
  auto store_all = [&](const StoreCtx& x) __attribute__((always_inline)) {
    const int ln = lane_opaque();
    uint8_t* epi = lds + Y::kOffEpi + wave * (32 * Y::kEpiRow * 4);
    const int wr_off = ((ln & 31) * Y::kEpiRow + 4 * (ln >> 5)) * 4;        // + 32 q bytes
    const int rd_row = ln >> 3, rd_col = 4 * (ln & 7);
    const int rd_off = (rd_row * Y::kEpiRow + rd_col) * 4;                  // + 8 k rows
    const int row_base = kMM ? kWN * wn : kWM * wm;                          // the wave's first tile row
    const int col_base = (kMM ? kWM * wm : kWN * wn) + rd_col;               // tile column of the lane's run
    const unsigned vrow0 =
        ((unsigned)(row_base + rd_row) * (unsigned)x.stride + (unsigned)(x.c0 + col_base)) * (unsigned)kEs;
    auto put = [&](int i, int j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v4f v;
        v[0] = acc[i][j][4 * q];
        v[1] = acc[i][j][4 * q + 1];
        v[2] = acc[i][j][4 * q + 2];
        v[3] = acc[i][j][4 * q + 3];
        *reinterpret_cast<v4f*>(epi + wr_off + 32 * q) = v;
      }
    };
    auto get = [&](v4f (&out)[4]) {
#pragma unroll
      for (int k = 0; k < 4; ++k) out[k] = *reinterpret_cast<const v4f*>(epi + rd_off + k * 8 * Y::kEpiRow * 4);
    };
    auto emit = [&](const v4f (&v)[4], int i, int j) {
      const int rb = kMM ? j : i, cb = kMM ? i : j;  // the block's row and column block
      const bool cok = col_base + 32 * cb < x.cvalid;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int row = row_base + 32 * rb + 8 * k + rd_row;
        const bool ok = cok & (row < x.rvalid);
        const unsigned off =
            vrow0 + (unsigned)(32 * rb + 8 * k) * (unsigned)x.stride * (unsigned)kEs + (unsigned)(32 * cb * kEs);
        store_c4<CT, kCPolicy>(v[k], x.rc, ok ? (int)off : (int)x.c_bytes, 0);
        const unsigned m4 = max(max(__float_as_uint(v[k][0]) & 0x7FFFFFFFu, __float_as_uint(v[k][1]) & 0x7FFFFFFFu),
                                max(__float_as_uint(v[k][2]) & 0x7FFFFFFFu, __float_as_uint(v[k][3]) & 0x7FFFFFFFu));
        lmax = max(lmax, m4 & (0u - (unsigned)ok));
      }
    };
    v4f cur[4], nxt[4];
    put(0, 0);
    get(cur);
#pragma unroll
    for (int b = 0; b < kTM * kTN; ++b) {
      const int i = b / kTN, j = b % kTN;
      if (b + 1 < kTM * kTN) {
        put((b + 1) / kTN, (b + 1) % kTN);
        get(nxt);
      }
      emit(cur, i, j);
      if (b + 1 < kTM * kTN) {
#pragma unroll
        for (int k = 0; k < 4; ++k) cur[k] = nxt[k];
      }
    }
  };
  // --- projection epilogue (CT == 4) --------------------------------------------
  // ("GEMM + RoPE + MXFP8 Projection (SM100)", sections "Overview", "Shapes"
  // and "Equations".)  In place of storing C, the tile's float32
  // accumulators, viewed per head of head_dim features, get RoPE on each
  // head's trailing qk_rope features -- pairs (y[2i], y[2i+1]) in, rotated
  // first members to position i and second members to R + i out (R =
  // qk_rope / 2), with the token's bf16 cos / sin rows, each product and sum
  // rounded on its own -- and then leave as E4M3 codes twice: blocks of 32
  // features of a token (row codes, scales (M, N/32)) and blocks of 32 tokens
  // of a feature (column codes, scales (M/32, N)); the block exponent is the
  // smallest e with 448 * 2^e >= the block's largest magnitude and codes
  // round to nearest even (the MX quantiser's rule).  Each wave works
  // through its 128 x 128 block 32 tokens at a time in its quarter of the
  // LDS stage the tile's last step freed (rows of 132 floats; the last 4 of
  // row g hold the column exponents of columns 4g..4g+3).  The host
  // guarantees M % 32 == 0, N % 128 == 0, head_dim % 32 == 0, qk_rope a
  // multiple of 16 up to 64, and that no head's rotary features cross a
  // 128-column boundary, so 32-token and 32-feature blocks and rotary
  // segments all lie inside one wave's block.
  auto store_proj = [&](const Tile& T, uint8_t* scratch) __attribute__((always_inline)) {
    constexpr int P = 132;
    float* z = reinterpret_cast<float*>(scratch) + wave * 32 * P;
    const int ln = lane_opaque();
    const int r = ln & 31, h = ln >> 5;
    const int N = p.N, D = p.head_dim, QR = p.qk_rope, R = QR >> 1;
    const int c0 = T.n0 + kWN * wn;  // the wave's first column
    // the wave's rotary segment [seg, seg + QR), relative to c0, if any: the
    // rotary part of the head holding column c0, or of the next head when
    // that one ends before c0
    int seg = (c0 / D) * D + D - QR - c0;
    if (seg + QR <= 0) seg += D;
    const bool rot = QR > 0 && seg < kWN;
    // RoPE lanes: lane pair (2t, 2t+1) takes token t of the block-row, R/2
    // pairs each; the bf16 cos / sin words of the next block-row are loaded
    // while this one is quantised
    const int t = ln >> 1;
    const int pp = (ln & 1) * (R >> 1);  // this lane's first pair
    uint2 tc1[4], tc2[4], ts1[4], ts2[4];
    auto load_tables = [&](int i) {
      const int64_t tok = (int64_t)T.m0 + kWM * wm + 32 * i + t;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (4 * u < (R >> 1)) {
          const uint16_t* cs = p.rope_cos + tok * QR + pp + 4 * u;
          const uint16_t* sn = p.rope_sin + tok * QR + pp + 4 * u;
          tc1[u] = *reinterpret_cast<const uint2*>(cs);
          tc2[u] = *reinterpret_cast<const uint2*>(cs + R);
          ts1[u] = *reinterpret_cast<const uint2*>(sn);
          ts2[u] = *reinterpret_cast<const uint2*>(sn + R);
        }
      }
    };
    if (rot && c0 < N && kWM * wm < T.mvalid) load_tables(0);
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int row0 = kWM * wm + 32 * i;  // the block-row's first tile row
      if (row0 >= T.mvalid || c0 >= N) continue;
      const int64_t tok0 = (int64_t)T.m0 + row0;
      // 1. accumulators to LDS, lane (r, h): row r, columns 32j + 8q + 4h
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v4f v;
          v[0] = acc[i][j][4 * q];
          v[1] = acc[i][j][4 * q + 1];
          v[2] = acc[i][j][4 * q + 2];
          v[3] = acc[i][j][4 * q + 3];
          *reinterpret_cast<v4f*>(z + r * P + 32 * j + 8 * q + 4 * h) = v;
        }
      // 2. RoPE; every read of the segment precedes every write (the wave's
      // LDS operations run in order)
      if (rot) {
#pragma clang fp contract(off)
        float a[16], b[16], c1[16], s1[16], c2[16], s2[16];
        auto lo = [](unsigned w) { return __uint_as_float(w << 16); };
        auto hi = [](unsigned w) { return __uint_as_float(w & 0xFFFF0000u); };
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (4 * u < (R >> 1)) {
            const float* zr = z + t * P + seg + 2 * pp + 8 * u;
            const v4f x0 = *reinterpret_cast<const v4f*>(zr);
            const v4f x1 = *reinterpret_cast<const v4f*>(zr + 4);
            a[4 * u] = x0[0], b[4 * u] = x0[1], a[4 * u + 1] = x0[2], b[4 * u + 1] = x0[3];
            a[4 * u + 2] = x1[0], b[4 * u + 2] = x1[1], a[4 * u + 3] = x1[2], b[4 * u + 3] = x1[3];
            c1[4 * u] = lo(tc1[u].x), c1[4 * u + 1] = hi(tc1[u].x), c1[4 * u + 2] = lo(tc1[u].y), c1[4 * u + 3] = hi(tc1[u].y);
            c2[4 * u] = lo(tc2[u].x), c2[4 * u + 1] = hi(tc2[u].x), c2[4 * u + 2] = lo(tc2[u].y), c2[4 * u + 3] = hi(tc2[u].y);
            s1[4 * u] = lo(ts1[u].x), s1[4 * u + 1] = hi(ts1[u].x), s1[4 * u + 2] = lo(ts1[u].y), s1[4 * u + 3] = hi(ts1[u].y);
            s2[4 * u] = lo(ts2[u].x), s2[4 * u + 1] = hi(ts2[u].x), s2[4 * u + 2] = lo(ts2[u].y), s2[4 * u + 3] = hi(ts2[u].y);
          }
        }
        if (i + 1 < kTM && row0 + 32 < T.mvalid) load_tables(i + 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (4 * u < (R >> 1)) {
            v4f f, g;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int x = 4 * u + e;
              const float ac = a[x] * c1[x], bs = b[x] * s1[x], bc = b[x] * c2[x], as = a[x] * s2[x];
              f[e] = ac - bs;
              g[e] = bc + as;
            }
            *reinterpret_cast<v4f*>(z + t * P + seg + pp + 4 * u) = f;
            *reinterpret_cast<v4f*>(z + t * P + seg + R + pp + 4 * u) = g;
          }
        }
      }
      // 3. column blocks: lane (cg, h) takes columns 4cg..4cg+3 over rows
      // 16h..16h+15; the halves meet by an xor shuffle over 32 lanes
      {
        v4f m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const v4f v = *reinterpret_cast<const v4f*>(z + (16 * h + rr) * P + 4 * r);
#pragma unroll
          for (int e = 0; e < 4; ++e) m[e] = fmaxf(m[e], fabsf(v[e]));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = fmaxf(m[e], __shfl_xor(m[e], 32));
        v4u ec;
#pragma unroll
        for (int e = 0; e < 4; ++e) ec[e] = (unsigned)quant::block_exponent<0>(m[e]);
        if (h == 0) {
          *reinterpret_cast<v4u*>(z + r * P + 128) = ec;
          const unsigned sb = ((ec[0] + 127u) & 0xFFu) | (((ec[1] + 127u) & 0xFFu) << 8) |
                              (((ec[2] + 127u) & 0xFFu) << 16) | (((ec[3] + 127u) & 0xFFu) << 24);
          *reinterpret_cast<unsigned*>(p.col_scales + (tok0 >> 5) * N + c0 + 4 * r) = sb;
        }
      }
      // 4. both directions' codes: lane takes the 16 columns 16q .. 16q+15
      // (q = ln % 8) of rows (ln / 8) + 8k, so that each direction's codes of
      // a row leave as one 16-byte store and 8 lanes write a whole 128-byte
      // line; a row block (32 columns) is a lane pair, whose maximum one DPP
      // swap finds, and the row's 4 block scales gather in its lane q = 0
      const int q = ln & 7;
      v4u ecol[4];  // column exponents of columns 16q + 4j .. 16q + 4j + 3
#pragma unroll
      for (int j = 0; j < 4; ++j) ecol[j] = *reinterpret_cast<const v4u*>(z + (4 * q + j) * P + 128);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rr = (ln >> 3) + 8 * k;
        const int64_t tok = tok0 + rr;
        v4f v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const v4f*>(z + rr * P + 16 * q + 4 * j);
        float bm = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bm = fmaxf(bm, fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3]))));
        bm = fmaxf(bm, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bm), 0xB1, 0xF, 0xF, false)));
        const int er = quant::block_exponent<0>(bm);
        v4u rc, cc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rc[j] = quant::codes4_e4m3_exp(v[j][0], v[j][1], v[j][2], v[j][3], er);
          cc[j] = quant::codes4<0>(ldexpf(v[j][0], -(int)ecol[j][0]), ldexpf(v[j][1], -(int)ecol[j][1]),
                                   ldexpf(v[j][2], -(int)ecol[j][2]), ldexpf(v[j][3], -(int)ecol[j][3]));
        }
        const int64_t o = tok * N + c0 + 16 * q;
        *reinterpret_cast<v4u*>(p.row_codes + o) = rc;
        *reinterpret_cast<v4u*>(p.col_codes + o) = cc;
        const unsigned sbyte = (unsigned)(er + 127) & 0xFFu;
        const int base = ln & ~7;
        const unsigned rs = sbyte | ((unsigned)__shfl((int)sbyte, base + 2) << 8) |
                            ((unsigned)__shfl((int)sbyte, base + 4) << 16) | ((unsigned)__shfl((int)sbyte, base + 6) << 24);
        if (q == 0) *reinterpret_cast<unsigned*>(p.row_scales + tok * (N >> 5) + (c0 >> 5)) = rs;
      }
    }
  };

  Tile cur = {0, 0, 0, 0, 0};
  int after_dma = 0;             // FP8 datapath: store instructions queued after the last DMA
  int s = 0;                     // global step index: selects the ring stage
  if (my_tiles > 0) {
    cur = make_tile<kBM, kBN>(p, t0);
    if (NW == 4 || producer) {
      const Dma d0 = dma_setup(geo(lane), cur, 0, true, lds0);
      dma_sf(d0);
#pragma unroll
      for (int q = 0; q < Y::kDma; ++q) dma_ab(d0, q);
    }
  }

  // FP8 datapath: one K step of tile `cur`; queues the DMA of the next step
  // (this tile's next K step or the next tile's first, `nt`).  On a tile's first step
  // (FIRST) the first MFMA of every accumulator takes a zero C operand instead
  // of the register, so the accumulators never need clearing and stay in the
  // matrix-core registers from tile to tile.
  auto step = [&](auto first, int kt, const Tile& nt, bool has_next) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first)::value;
    // this wave's DMA for step s is complete (only stores may have been
    // queued after it); the barrier extends that to every wave and frees the
    // other stage
    if (after_dma == 0) wait_vm<0>();
    else wait_vm<kNStores - 1>();
    after_dma = 0;
    barrier();
    const Geo g = kHoistGeo ? g_lane : geo(lane_opaque());
    const uint8_t* st = lds + (s & 1) * Y::kStage;
    // fragment row i (32-row steps keep f, so only the chunk is swizzled)
    auto a_frag = [&](int i, int c) { return lds16(st + g.a_off + ((c ^ g.xr) << 4) + 4096 * i); };
    auto b_frag = [&](int i, int c) { return lds16(st + g.b_off + ((c ^ g.xr) << 4) + 4096 * i); };

    const bool last_k = kt + 1 == p.ksteps;
    const Dma d = dma_setup(g, nt, last_k ? 0 : kt + 1, has_next, lds0 + (unsigned)(((s & 1) ^ 1) * Y::kStage));
    dma_sf(d);
    // SF dwords of this step: NSF atoms x kTM (kTN) fragment rows per operand.
    // A rows kWM*wm + 32i + r: atom group (kWM*wm)/128, dword
    // ((kWM*wm)/32)%4 + i; B rows kWN*wn + 32i + r likewise.
    unsigned sa[NSF][kTM], sb[NSF][kTN];
    const int arg = (kWM * wm) >> 7, adw = ((kWM * wm) >> 5) & 3;
    const int brg = (kWN * wn) >> 7, bdw = ((kWN * wn) >> 5) & 3;
#pragma unroll
    for (int j = 0; j < NSF; ++j) {
      const int ga = NSF * kt + j;
#pragma unroll
      for (int i = 0; i < kTM; ++i)
        sa[j][i] = sf_tail(lds4(st + Y::kOffSFA + (arg * NSF + j) * 512 + 16 * g.r + 4 * (adw + i)), ga, p.Kb);
#pragma unroll
      for (int i = 0; i < kTN; ++i)
        sb[j][i] = sf_tail(lds4(st + Y::kOffSFB + (brg * NSF + j) * 512 + 16 * g.r + 4 * (bdw + i)), ga, p.Kb);
    }

    // FP8 datapath (bf16 uses step_bf16 below)
#pragma unroll
    for (int S = 0; S < 2; ++S) {
      v8i af[kTM], bf[kTN];
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const uint4 lo = a_frag(i, 4 * S + g.h);
        const uint4 hi = a_frag(i, 4 * S + 2 + g.h);
        af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int i = 0; i < kTN; ++i) {
        const uint4 lo = b_frag(i, 4 * S + g.h);
        const uint4 hi = b_frag(i, 4 * S + 2 + g.h);
        bf[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int q = 0; q < Y::kDma / 2; ++q) dma_ab(d, (Y::kDma / 2) * S + q);
      if constexpr (SF == 32) {
        // lane r supplies block 2S (K [0,32) of the slice), lane r+32 block 2S+1
        const int sh = 8 * (2 * S + g.h);
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int jj = 0; jj < kTN; ++jj)
            acc[i][jj] = mfma_f8<0, FA, FB>(bf[jj], af[i], (kFirst && S == 0) ? zero16 : acc[i][jj],
                                            sb[0][jj] >> sh, sa[0][i] >> sh);
      } else {
        // 16-element blocks (atom S): the scale slot of K [0,32) gets block 0
        // (MFMA 1, odd-block A lanes zeroed) or block 1 (MFMA 2, even-block
        // A lanes zeroed); that of K [32,64) blocks 2 / 3
        const v8i zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
          const v8i a_even = g.h ? zero : af[i];
          const v8i a_odd = g.h ? af[i] : zero;
          const unsigned sai = sa[S][i] >> (16 * g.h);
#pragma unroll
          for (int jj = 0; jj < kTN; ++jj) {
            const unsigned sbj = sb[S][jj] >> (16 * g.h);
            acc[i][jj] = mfma_f8<0, FA, FB>(bf[jj], a_even, (kFirst && S == 0) ? zero16 : acc[i][jj], sbj, sai);
            acc[i][jj] = mfma_f8<1, FA, FB>(bf[jj], a_odd, acc[i][jj], sbj, sai);
          }
        }
      }
    }
    ++s;
  };

  // --- bf16 datapath: steps pipelined across step boundaries -----------------
  // Global step s reads ring stage s & 1; a step is S slices of 16 K (S = 8
  // for the 8-bit formats, 16 for FP4), four 32-byte chunks per row.  The next
  // step's scale dwords and first chunk are read, and its first MFMA slice
  // converted, while the current step's last slice runs, so a step issues
  // MFMAs from its first cycle.  A wave reads a stage for the last time in the
  // first slice of chunk 3, and that read has completed by the end of slice
  // S-3 (chunk 3's first conversion happens there); by then the scales of
  // chunk 3 are taken from the scale dwords as well.  One barrier per step,
  // B' (after slice S-3, right after the slice's MFMAs are queued, so its
  // wait overlaps them; the reads it releases then have two slices before
  // their first use).  Past B':
  //   * every wave's DMA of step s+1 has landed (each wave first waits for
  //     its own), so stage (s+1) & 1 may be read;
  //   * every wave is done with stage s & 1, so DMA into it may start.
  // A step queues the DMA of step s+1 over its slices 1..3 (into the stage
  // freed at the previous B'; spread so that the texture unit's queue does
  // not back up into instruction issue).  A tile's last step also queues the
  // DMA of the next tile's step 1 right after its B' (over slices S-2 and
  // S-1), ahead of the tile's C stores; that tile's first step then queues no
  // DMA, and its B' waits for all but 63 vector-memory operations (the 64
  // stores of each lane retire after that DMA, in issue order), so the stores
  // keep draining under its MFMAs; only the step after it waits for them.
  unsigned sa[NSF][kTM], sb[NSF][kTN];  // scale dwords of the current step
  uint4 ra[2][kTM], rb[2][kTN];         // raw 16-byte fragments, by chunk parity
  v8bf ab[2][kTM], bb[2][kTN];          // converted operands, by slice parity
  float fa[kTM], fb[kTN];               // scale operands of the chunk being converted
  const int arg = (kWM * wm) >> 7, adw = ((kWM * wm) >> 5) & 3;
  const int brg = (kWN * wn) >> 7, bdw = ((kWN * wn) >> 5) & 3;
  // SF dwords of step kt from stage st: NSF atoms x kTM (kTN) fragment rows
  // per operand.  A rows kWM*wm + 32i + r: atom group (kWM*wm)/128, dword
  // ((kWM*wm)/32)%4 + i; B rows kWN*wn + 32i + r likewise.
  auto load_sf = [&](const Geo& g, const uint8_t* st, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NSF; ++j) {
      const int ga = NSF * kt + j;
#pragma unroll
      for (int i = 0; i < kTM; ++i)
        sa[j][i] = sf_tail(lds4(st + Y::kOffSFA + (arg * NSF + j) * 512 + 16 * g.r + 4 * (adw + i)), ga, p.Kb);
#pragma unroll
      for (int i = 0; i < kTN; ++i)
        sb[j][i] = sf_tail(lds4(st + Y::kOffSFB + (brg * NSF + j) * 512 + 16 * g.r + 4 * (bdw + i)), ga, p.Kb);
    }
  };
  // chunk c's fragments (32-row steps keep f, so only the chunk is swizzled).
  // An m-major operand's lane (r, h) takes the same K elements of its row with
  // two transposing reads, K 32c + 16h + 8t + (0..7) for t = 0, 1: lane
  // i = r % 16 of its group of 16 addresses K row 32c + 16h + 8t + i/2 at
  // column 16 (r / 16) + 8 (i % 2) of the fragment's 32.
  auto mj_frag = [&](const Geo& g, const uint8_t* tile, int row0, int c) __attribute__((always_inline)) {
    const int i16 = g.r & 15;
    const int sw = BT == 256 ? (g.r & 14) : ((g.r >> 1) & 6);
    const int unit = ((row0 >> 4) ^ sw) | (g.r >> 4);
    const uint8_t* q = tile + (16 * g.h + (i16 >> 1) + 32 * c) * BT + 8 * (g.r & 1) + 16 * unit;
    const uint2 lo = lds_tr8(q), hi = lds_tr8(q + 8 * BT);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };
  auto load_raw = [&](const Geo& g, const uint8_t* st, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      if constexpr (kAMaj) ra[c & 1][i] = mj_frag(g, st, kWM * wm + 32 * i, c);
      else ra[c & 1][i] = lds16(st + g.a_off + (((2 * c + g.h) ^ g.xr) << 4) + 4096 * i);
    }
#pragma unroll
    for (int i = 0; i < kTN; ++i) {
      if constexpr (kBMaj) rb[c & 1][i] = mj_frag(g, st + Y::kOffB, kWN * wn + 32 * i, c);
      else rb[c & 1][i] = lds16(st + g.b_off + (((2 * c + g.h) ^ g.xr) << 4) + 4096 * i);
    }
  };
  // chunk c's scale: one atom per step (8-bit, sf=32) -> block c (byte c);
  // two atoms (8-bit with sf=16, or FP4 with sf=32, whose 16-byte chunk holds
  // 32 elements) -> block 2c+h, byte 2(c&1)+h of atom c>>1; four atoms (FP4
  // with sf=16: a lane's 32 elements are two blocks, dwords 0-1 and 2-3) ->
  // block 4c+2h+u for half u, byte 2h+u of atom c
  auto scales = [&](const Geo& g, int c, int u) __attribute__((always_inline)) {
    const int j = NSF == 1 ? 0 : NSF == 4 ? c : (c >> 1);
    const unsigned k = NSF == 1 ? (unsigned)c
                                : NSF == 4 ? (unsigned)(2 * g.h + u) : (unsigned)(2 * (c & 1) + g.h);
#pragma unroll
    for (int i = 0; i < kTM; ++i) fa[i] = e8m0_byte_operand(sa[j][i], k);
#pragma unroll
    for (int i = 0; i < kTN; ++i) fb[i] = e8m0_byte_operand(sb[j][i], k);
  };
  // 8-bit: slice n = chunk n/2, bytes 0..7 (even n) or 8..15 (odd n) of each
  // fragment.  FP4: slice n = chunk n/4, dword n%4 (eight elements) of each
  // fragment.  Either way A and B take the same K elements in the same order.
  auto pick = [](const uint4& v, int t) { return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w; };
  auto convert = [&](int n) __attribute__((always_inline)) {
    if constexpr (kFp4) {
      const int c = n >> 2, t = n & 3;
#pragma unroll
      for (int i = 0; i < kTM; ++i) ab[n & 1][i] = cvt8_fp4(pick(ra[c & 1][i], t), fa[i]);
#pragma unroll
      for (int i = 0; i < kTN; ++i) bb[n & 1][i] = cvt8_fp4(pick(rb[c & 1][i], t), fb[i]);
    } else {
      const int c = n >> 1, t = n & 1;
#pragma unroll
      for (int i = 0; i < kTM; ++i)
        ab[n & 1][i] = cvt8<FA>(t ? ra[c & 1][i].z : ra[c & 1][i].x, t ? ra[c & 1][i].w : ra[c & 1][i].y, fa[i]);
#pragma unroll
      for (int i = 0; i < kTN; ++i)
        bb[n & 1][i] = cvt8<FB>(t ? rb[c & 1][i].z : rb[c & 1][i].x, t ? rb[c & 1][i].w : rb[c & 1][i].y, fb[i]);
    }
  };
  // DMA target: a tile, its K step, and whether it exists
  struct Tgt {
    Tile t;
    int kt;
    bool live;
  };
  // steps 0 and 1 go into the two stages at once; step 0's inputs are read
  // after both have landed everywhere
  // (the projection epilogue queues step 1 from step 0 instead)
  auto prime = [&](const Tgt& n1) __attribute__((always_inline)) {
    const Geo g = kHoistGeo ? g_lane : geo(lane_opaque());
    if constexpr (CT != 4) {
      const Dma d1 = dma_setup(g, n1.t, n1.kt, n1.live, lds0 + (unsigned)Y::kStage);
      dma_sf(d1);
#pragma unroll
      for (int q = 0; q < Y::kDma; ++q) dma_ab(d1, q);
    }
    wait_vm<0>();
    barrier();
    load_sf(g, lds, 0);
    load_raw(g, lds, 0);
    scales(g, 0, 0);
    convert(0);
  };
  // One K step of tile `cur`.  FIRST: the tile's first step (its first MFMA
  // per accumulator takes a zero C operand, and its B' waits past the
  // previous tile's C stores).  nkt: the K step of step s+1 (for the scale
  // tail read at B').  EARLY (n2): the DMA of step s+2 goes out after B'.
  // LATE (n1): the DMA of step s+1 goes out over slices 1..3.
  auto step_bf16 = [&](auto first, auto late, auto early, int nkt, const Tgt& n1, const Tgt& n2)
                       __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first)::value;
    constexpr bool kLate = decltype(late)::value;
    constexpr bool kEarly = decltype(early)::value;
    const Geo g = kHoistGeo ? g_lane : geo(lane_opaque());
    const uint8_t* stn = lds + ((s & 1) ^ 1) * Y::kStage;
    const uint8_t* st = lds + (s & 1) * Y::kStage;
    // slices of 16 K per step: 8 (8-bit) or 16 (FP4); kSpc per 32-byte chunk
    constexpr int kSlices = kFp4 ? 16 : 8;
    constexpr int kSpc = kSlices / 4;
    constexpr int kPer2 = Y::kDma / 2;        // early DMA: per slice of S-2, S-1
    constexpr int kPer1 = (Y::kDma + 2) / 3;  // late DMA: per slice of 1..3
    Dma d1, d2;
#pragma unroll
    for (int n = 0; n < kSlices; ++n) {
      // chunk c+1 is read during chunk c's first slice, a slice before its
      // first conversion; chunk 0 of the next step after B'
      if (n % kSpc == 0 && n / kSpc < 3) load_raw(g, st, n / kSpc + 1);
      if constexpr (kLate) {
        if (n == 1) {
          d1 = dma_setup(g, n1.t, n1.kt, n1.live, lds0 + (unsigned)(((s & 1) ^ 1) * Y::kStage));
          dma_sf(d1);
        }
        if (n >= 1 && n <= 3) {
#pragma unroll
          for (int q = 0; q < kPer1; ++q)
            if ((n - 1) * kPer1 + q < Y::kDma) dma_ab(d1, (n - 1) * kPer1 + q);
        }
      }
      if constexpr (kEarly) {
        if (n >= kSlices - 2) {
#pragma unroll
          for (int q = 0; q < kPer2; ++q) dma_ab(d2, (n - (kSlices - 2)) * kPer2 + q);
        }
      }
      if (n < kSlices - 1) {
        if ((n + 1) % kSpc == 0) scales(g, (n + 1) / kSpc, 0);
        if constexpr (NSF == 4) {
          if ((n + 1) % kSpc == 2) scales(g, (n + 1) / kSpc, 1);
        }
        convert(n + 1);
      } else {
        // the next step's first slice (its inputs were read after B')
        scales(g, 0, 0);
        convert(0);
      }
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int jj = 0; jj < kTN; ++jj)
          acc[i][jj] = kMM ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab[n & 1][i], bb[n & 1][jj],
                                                                     (kFirst && n == 0) ? zero16 : acc[i][jj], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_32x32x16_bf16(bb[n & 1][jj], ab[n & 1][i],
                                                                     (kFirst && n == 0) ? zero16 : acc[i][jj], 0, 0, 0);
      // interleave: each MFMA followed by up to kValu VALU ops (3 for 16
      // MFMAs per slice, 6 for 4: the conversions per MFMA double when the
      // wave tile halves); the chunk's fragment reads go out one after each
      // of the first MFMAs
      constexpr int kValu = BT == 256 ? 3 : 6;
#pragma unroll
      for (int k = 0; k < kTM * kTN; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
        if (k < kTM + kTN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
      __builtin_amdgcn_sched_barrier(0);
      if (n == kSlices - 3) {
        // this wave's DMA of step s+1 has landed; on a tile's first step the
        // previous tile's 64 C stores per lane, queued after that DMA, may
        // still be in flight
        if constexpr (kFirst && !kLate) wait_vm<kNStores - 1>();
        else wait_vm<0>();
        barrier();  // B'
        load_sf(g, stn, nkt);
        load_raw(g, stn, 0);
        if constexpr (kEarly) {
          d2 = dma_setup(g, n2.t, n2.kt, n2.live, lds0 + (unsigned)((s & 1) * Y::kStage));
          dma_sf(d2);
        }
      }
    }
    ++s;
  };

  // --- bf16 datapath on a ring of kStages > 2 stages (128x128 tiles) ---------
  // Global step s reads stage s % kStages.  Step s queues, over its slices
  // 1..3, the DMA of step s + kStages - 1 (the stream runs on across tiles)
  // into stage (s - 1) % kStages, which every wave finished reading before
  // B' of step s - 1.  B' of step s waits for this wave's DMA of step s + 1
  // and leaves the DMAs of the kStages - 2 later steps in flight; on a tile's
  // first kStages - 2 steps ("hold") the previous tile's C stores may stay in
  // flight as well, since the DMA waited for went out before that tile's
  // epilogue.  Past the end of the work the DMAs go through empty resources,
  // so every step queues the same instructions and the counts hold.  With 8
  // waves the same DMA, stage for stage, comes from the DMA waves (produce,
  // below), which do the waiting, and the computing waves only meet them at
  // the barriers.
  constexpr int kDmaPerStep = Y::kDma + 1;
  int di = 0, dkt = 0;  // the step whose DMA goes out next: the workgroup's tile di, K step dkt
  Tile dtile = cur;
  auto next_target = [&]() {
    const Tgt t = {dtile, dkt, di < my_tiles};
    if (++dkt == p.ksteps) {
      dkt = 0;
      ++di;
      if (di < my_tiles) dtile = make_tile<kBM, kBN>(p, t0 + di * G);
    }
    return t;
  };
  auto stage_at = [&](int step) { return (unsigned)(step & (kStages - 1)) * (unsigned)Y::kStage; };
  // steps 1 .. kStages - 2 join step 0 (queued above) before anything is read
  auto prime_ring = [&]() __attribute__((always_inline)) {
    const Geo g = g_lane;
    if constexpr (NW == 4) {
      (void)next_target();  // step 0
#pragma unroll
      for (int j = 1; j + 1 < kStages; ++j) {
        const Tgt tg = next_target();
        const Dma d = dma_setup(g, tg.t, tg.kt, tg.live, lds0 + stage_at(j));
        dma_sf(d);
#pragma unroll
        for (int q = 0; q < Y::kDma; ++q) dma_ab(d, q);
      }
      wait_vm<0>();
    }
    barrier();
    load_sf(g, lds, 0);
    load_raw(g, lds, 0);
    if constexpr (!kFp4) load_raw(g, lds, 1);
    scales(g, 0, 0);
    convert(0);
  };
  // One K step on the ring.  FIRST: the tile's first step (zero C operand on
  // each accumulator's first MFMA); HOLD: B' lets the previous tile's stores
  // stay in flight; nkt: the K step of step s+1 (scale tail at B'); tg: the
  // step this one queues the DMA of.
  auto step_ring = [&](auto first, auto hold, int nkt, const Tgt& tg) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first)::value;
    constexpr bool kHold = decltype(hold)::value;
    static_assert((kStages & (kStages - 1)) == 0 && kStages > 2, "ring of a power-of-two number of stages");
    constexpr int kWaitSteady = (kStages - 2) * kDmaPerStep;
    constexpr int kWait = kHold ? kWaitSteady + kNStores : kWaitSteady;
    static_assert(kWait <= 63, "vmcnt counts to 63");
    const Geo g = g_lane;
    const uint8_t* st = lds + stage_at(s);
    const uint8_t* stn = lds + stage_at(s + 1);
    constexpr int kSlices = kFp4 ? 16 : 8;
    constexpr int kSpc = kSlices / 4;
    constexpr int kPer1 = (Y::kDma + 2) / 3;  // DMA instructions per slice of 1..3
    Dma d1;
#pragma unroll
    for (int n = 0; n < kSlices; ++n) {
      // fragment reads two slices ahead of their first conversion (a slice
      // of this tile is only 4 MFMAs): 8-bit chunks 2 and 3 in slices 1 and
      // 3, chunk 1 of the next step in slice S-1 (after B'); FP4 chunks span
      // four slices, so one chunk ahead is three slices
      if constexpr (kFp4) {
        if (n % kSpc == 0 && n / kSpc < 3) load_raw(g, st, n / kSpc + 1);
      } else {
        if (n == 1 || n == 3) load_raw(g, st, (n + 3) / 2);
      }
      if constexpr (NW == 4) {
        if (n == 1) {
          d1 = dma_setup(g, tg.t, tg.kt, tg.live, lds0 + stage_at(s + kStages - 1));
          dma_sf(d1);
        }
        if (n >= 1 && n <= 3) {
#pragma unroll
          for (int q = 0; q < kPer1; ++q)
            if ((n - 1) * kPer1 + q < Y::kDma) dma_ab(d1, (n - 1) * kPer1 + q);
        }
      }
      if (n < kSlices - 1) {
        if ((n + 1) % kSpc == 0) scales(g, (n + 1) / kSpc, 0);
        if constexpr (NSF == 4) {
          if ((n + 1) % kSpc == 2) scales(g, (n + 1) / kSpc, 1);
        }
        convert(n + 1);
      } else {
        scales(g, 0, 0);
        convert(0);
      }
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int jj = 0; jj < kTN; ++jj)
          acc[i][jj] = kMM ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab[n & 1][i], bb[n & 1][jj],
                                                                     (kFirst && n == 0) ? zero16 : acc[i][jj], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_32x32x16_bf16(bb[n & 1][jj], ab[n & 1][i],
                                                                     (kFirst && n == 0) ? zero16 : acc[i][jj], 0, 0, 0);
      constexpr int kValu = BT == 256 ? 3 : 6;
#pragma unroll
      for (int k = 0; k < kTM * kTN; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
        if (k < kTM + kTN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
      __builtin_amdgcn_sched_barrier(0);
      if (n == kSlices - 3) {
        // (8 waves: the DMA waves have waited for step s+1's DMA before it)
        if constexpr (NW == 4) wait_vm<kWait>();
        barrier();  // B'
        load_sf(g, stn, nkt);
        load_raw(g, stn, 0);
      }
      if constexpr (!kFp4) {
        if (n == kSlices - 2) load_raw(g, stn, 1);
      }
    }
    ++s;
  };

  // 8 waves: the DMA waves' whole life.  Steps 0 .. kStages - 2 go out
  // before the prime's barrier; then, between B' of step s - 1 and B' of step
  // s, the DMA of step s + kStages - 1 into the stage every computing wave
  // finished reading before B' of step s - 1, and a wait for their own DMA of
  // step s + 1 (the DMA of the two later steps stays in flight) ahead of B'
  // of step s.  That is the computing waves' barrier sequence: the prime's,
  // then one B' per step.  Past the work the DMA goes through empty
  // resources.
  auto produce = [&]() __attribute__((always_inline)) {
    if (my_tiles == 0) return;
    {
      const Geo g = g_lane;
      (void)next_target();  // step 0 (queued above)
#pragma unroll
      for (int j = 1; j + 1 < kStages; ++j) {
        const Tgt tg = next_target();
        const Dma d = dma_setup(g, tg.t, tg.kt, tg.live, lds0 + stage_at(j));
        dma_sf(d);
#pragma unroll
        for (int q = 0; q < Y::kDma; ++q) dma_ab(d, q);
      }
    }
    wait_vm<0>();
    barrier();
    const int64_t steps = (int64_t)my_tiles * p.ksteps;
    for (int64_t t = 0; t < steps; ++t) {
      const Geo g = g_lane;
      const Tgt tg = next_target();
      const Dma d = dma_setup(g, tg.t, tg.kt, tg.live, lds0 + stage_at((int)(t & (kStages - 1)) + kStages - 1));
      dma_sf(d);
#pragma unroll
      for (int q = 0; q < Y::kDma; ++q) dma_ab(d, q);
      wait_vm<(kStages - 2) * kDmaPerStep>();
      barrier();
    }
  };
  // the computing waves' DMA target of a step (8 waves: none, the DMA waves
  // queue it)
  auto ring_target = [&]() {
    if constexpr (NW == 4) return next_target();
    else return Tgt{cur, 0, false};
  };

  const std::true_type yes;
  const std::false_type no;
  if constexpr (MODE == kModeBf16 && kStages > 2) {
    if (producer) {
      produce();
    } else {
      if (my_tiles > 0) prime_ring();
      for (int i = 0; i < my_tiles; ++i) {
        const bool more = i + 1 < my_tiles;
        const Tile nxt = more ? make_tile<kBM, kBN>(p, t0 + (i + 1) * G) : cur;
        const int ks = p.ksteps;
        auto nk = [&](int kt) { return kt + 1 < ks ? kt + 1 : 0; };
        step_ring(yes, yes, nk(0), ring_target());
        int kt = 1;
#pragma unroll
        for (int h = 1; h + 2 < kStages; ++h)
          if (kt < ks) {
            step_ring(no, yes, nk(kt), ring_target());
            ++kt;
          }
        for (; kt < ks; ++kt) step_ring(no, no, nk(kt), ring_target());
        store_all(store_ctx(cur));
        cur = nxt;
      }
    }
  } else {
  if constexpr (MODE == kModeBf16) {
    if (my_tiles > 0) {
      if (p.ksteps > 1) prime(Tgt{cur, 1, true});
      else prime(Tgt{my_tiles > 1 ? make_tile<kBM, kBN>(p, t0 + G) : cur, 0, my_tiles > 1});
    }
  }
  for (int i = 0; i < my_tiles; ++i) {
    const bool more = i + 1 < my_tiles;
    const Tile nxt = more ? make_tile<kBM, kBN>(p, t0 + (i + 1) * G) : cur;
    if constexpr (MODE == kModeBf16 && CT == 4) {
      // the projection epilogue uses the stage the tile's last step freed,
      // so no DMA goes into it ahead: every step queues the next step's DMA
      const Tgt none = {cur, 0, false};
      if (p.ksteps == 1) {
        step_bf16(yes, yes, no, 0, Tgt{nxt, 0, more}, none);
      } else {
        step_bf16(yes, yes, no, 1, Tgt{cur, 1, true}, none);
        for (int kt = 1; kt + 1 < p.ksteps; ++kt) step_bf16(no, yes, no, kt + 1, Tgt{cur, kt + 1, true}, none);
        step_bf16(no, yes, no, 0, Tgt{nxt, 0, more}, none);
      }
    } else if constexpr (MODE == kModeBf16) {
      const Tgt none = {cur, 0, false};
      if (p.ksteps == 1) {
        const bool more2 = i + 2 < my_tiles;
        const Tgt n2 = {more2 ? make_tile<kBM, kBN>(p, t0 + (i + 2) * G) : cur, 0, more2};
        step_bf16(yes, no, yes, 0, none, n2);
      } else {
        // the tile's first step issues no DMA (its step 1 went out after
        // the previous tile's last B'); middle steps the DMA of step s+1;
        // the last step also that of the next tile's step 1, after B'
        step_bf16(yes, no, no, 1, none, none);
        for (int kt = 1; kt + 1 < p.ksteps; ++kt) step_bf16(no, yes, no, kt + 1, Tgt{cur, kt + 1, true}, none);
        step_bf16(no, yes, yes, 0, Tgt{nxt, 0, more}, Tgt{nxt, 1, more});
      }
    } else {
      if (p.ksteps == 1) {
        step(yes, 0, nxt, more);
      } else {
        step(yes, 0, cur, true);
        for (int kt = 1; kt + 1 < p.ksteps; ++kt) step(no, kt, cur, true);
        step(no, p.ksteps - 1, nxt, more);
      }
    }
    if constexpr (CT == 4) {
      store_proj(cur, lds + ((s - 1) & 1) * Y::kStage);
      barrier();  // every wave is done with that stage before the next step's DMA enters it
    } else {
      store_all(store_ctx(cur));
    }
    after_dma = 1;  // FP8 datapath: kNStores stores follow the DMA; waiting for all but one covers it
    cur = nxt;
  }
  }
  // no DMA may still be writing this workgroup's LDS when it exits
  wait_vm<0>();

  if constexpr (CT != 4) {  // the projection epilogue has no Amax (and no Amax pointer)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lmax = max(lmax, (unsigned)__shfl_xor((int)lmax, off));
    barrier();  // every wave is past its epilogue's LDS reads
    unsigned* red = reinterpret_cast<unsigned*>(lds + Y::kOffEpi);
    if (lane == 0 && wave < 4) red[wave] = lmax;
    barrier();
    if (wave == 0 && lane == 0) {
      const unsigned m = max(max(red[0], red[1]), max(red[2], red[3]));
      // The load is coherent at device scope, so it returns the value stored
      // before this launch (the clear, or the caller's value when
      // accumulating) or a later one from this launch; Amax only grows, so a
      // maximum at or below it changes nothing. A zero maximum reads nothing.
      if (m != 0u && m > __hip_atomic_load(p.amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        atomicMax(p.amax_bits, m);
    }
  }
}

}  // namespace big
}  // namespace mxg
