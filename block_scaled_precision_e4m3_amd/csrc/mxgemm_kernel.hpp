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
//   products are exact and whose partial sums stay within fp32 rounding.
//   This meets a 1e-5 * sum|A_hat||B_hat| error bound for any data.
// * kModeFp8.  The FP8 codes go straight into gfx950's scaled MFMA
//   (v_mfma_scale_f32_32x32x64_f8f6f4), which applies the E8M0 scales itself
//   at twice the bf16 rate.  Measured on MI355X, that instruction aligns the
//   products of each 8-element K group to the largest one and drops bits
//   more than 13 binary places below it, so terms far smaller than their
//   neighbours are truncated; on heavy-tailed data the result can miss the
//   bound above.  Opt-in only.
//
// Operand layouts (lane l, row r = l % 32, half h = l / 32):
//   32x32x64 f8f6f4: bytes 0..15 of a lane hold K [16h, 16h+16) of a 64-K
//     slice and bytes 16..31 hold K [32+16h, +16); lane r's scale covers
//     K [0,32) of row r and lane r+32's covers K [32,64).
//   32x32x16 bf16: 8 elements per lane; any assignment of (h, element) to K
//     works as long as A and B use the same one, because the scale is folded
//     into each element.  Lane half h takes the contiguous K range
//     [32h, 32h+32) of a 64-K slice and MFMA q (q = 0..3) its bytes
//     [8q, 8q+8).
//   Output (both): lane l, element e holds D[8(e/4) + 4h + e%4][r] for
//     (src0 row, src1 col).  B is src0 and A is src1, so a lane owns one
//     output row m and 4-element runs of n: 16-byte stores into n-major C.
//
// Workgroup: 256 threads = 4 waves in 2x2 on a 128x128 tile (each wave
// 64x64 = 2x2 MFMA blocks); two workgroups share a CU.  The K loop advances
// 128 bytes per step through a 2-stage LDS ring; a stage holds the A tile,
// the B tile (rows of 128 bytes, i.e. whole cache lines) and the E8M0 atoms
// of those rows for the step, all moved by direct global->LDS DMA
// (buffer_load_dwordx4 ... lds).  A wave's DMA instruction fills 1 KB = 8
// rows; the 16-byte chunk c of row r sits at chunk c ^ (r & 7), so the
// 16-byte fragment reads of 8 consecutive rows hit distinct banks.  Rows past
// M (N) and K chunks past K are fetched through an out-of-range buffer offset,
// which reads as zero.
//
// Steps form one stream over all tiles a workgroup owns: during step s the
// DMA for step s+1 (possibly the next tile's first) is in flight.  A tile's
// accumulators move to a second register set when it ends, and its C stores
// are issued a few per step during the next tile, each batch right after
// that step's DMA.  The vector-memory counter retires in issue order, so a
// wave waiting for step s+1's DMA never waits for stores issued after it:
// the stores drain under the next tile's math.  Each wave waits with an exact
// vmcnt, then one barrier per step.
//
// Scale factors: a stage holds the 512-byte atoms (l, row/128, g) of the
// tile's rows for the step's atoms g along K (one per step when sf=32, two
// when sf=16).  A lane's dword for a row is bytes
// [16*(row%32) + 4*((row/32)%4), +4) of its atom: the 4 K-blocks of that
// atom for that row.  Bytes of K-blocks past ceil(K/sf) are replaced by 0x7F
// (1.0), so padding bytes (which may be anything, NaN included) never meet
// data; rows past M (N) only feed outputs that are never stored.
//
// Scheduling: persistent; workgroup w takes tiles w, w+G, ...; tiles are
// ordered batch-major and, inside a batch, in groups of kGroupM tile rows
// walked column-major; with G a multiple of 8 the workgroup index is
// remapped so each XCD (workgroups are dispatched round-robin over the 8
// XCDs) works on a contiguous run of tiles.
//
// Amax: each lane keeps max(bits(|c|)) over the outputs it stores, as an
// unsigned integer (the order of non-negative IEEE floats, NaN above +inf),
// reduced across the wave with xor-shuffles, then one atomic max per wave.
#pragma once

#include "mxgemm_common.hpp"

namespace mxg {

constexpr int kThreads = 256;
constexpr int kBM = 128, kBN = 128;  // workgroup tile
constexpr int kBK = 128;             // K bytes per pipeline step

// LDS stage: A tile, B tile, then the SF atoms of A and of B (up to two
// atoms each: sf=16 needs two per 128-K step)
constexpr int kOffB = kBM * kBK;
constexpr int kOffSFA = kOffB + kBN * kBK;
constexpr int kOffSFB = kOffSFA + 1024;
constexpr int kStage = kOffSFB + 1024;  // 33 KB
constexpr int kStages = 2;

// per wave and step: 4 DMA instructions for A, 4 for B, 1 for the SF atoms
constexpr int kOps = kBM * kBK / 1024 / 4 + kBN * kBK / 1024 / 4 + 1;
// C stores (16-byte) per lane per tile, and how many go out per step
constexpr int kTM = 2, kTN = 2;  // MFMA blocks per wave
constexpr int kNStores = kTM * kTN * 4;
constexpr int kStoresPerStep = 2;
constexpr int kStoreSteps = kNStores / kStoresPerStep;

// --- fragments -----------------------------------------------------------------

// Byte offset of 16-byte chunk c of the 128-byte LDS row `row`.
__device__ __forceinline__ int chunk_addr(int row, int c) { return row * kBK + ((c ^ (row & 7)) << 4); }

__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int c0, int c1) {
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + chunk_addr(row, c0));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + chunk_addr(row, c1));
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// SF dword of tile-local row `row` from atom j of a stage's atom area.
__device__ __forceinline__ unsigned read_sf(const uint8_t* atoms, int j, int row) {
  return *reinterpret_cast<const unsigned*>(atoms + (j << 9) + 16 * (row & 31) + 4 * ((row >> 5) & 3));
}

// Replace the bytes of K-blocks at or past Kb of atom g by 0x7F.
__device__ __forceinline__ unsigned fix_tail(unsigned d, int g, int Kb) {
  const int valid = Kb - 4 * g;
  if (valid >= 4) return d;
  const unsigned keep = valid <= 0 ? 0u : (1u << (8 * valid)) - 1u;
  return (d & keep) | (0x7F7F7F7Fu & ~keep);
}

// One 64-K slice S (0 or 1) of a 128-K step for one wave.  `sfa`/`sfb` hold
// the K-tail-fixed SF dwords of the slice's atom; `blk` is the slice's first
// K-block inside that atom (sf=32: 2S; sf=16: 0, one atom per slice).
template <int MODE, int S, int SF, int FA, int FB>
__device__ __forceinline__ void compute_slice(v16f (&acc)[kTM][kTN], const uint8_t* tA, const uint8_t* tB,
                                              int arow0, int brow0, int lane, const unsigned (&sfa)[kTM],
                                              const unsigned (&sfb)[kTN]) {
  constexpr int blk = (SF == 32) ? 2 * S : 0;
  const int r = lane & 31;
  const int h = lane >> 5;
  if constexpr (MODE == kModeFp8) {
    v8i af[kTM], bf[kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i) af[i] = read_frag(tA, arow0 + 32 * i + r, 4 * S + h, 4 * S + h + 2);
#pragma unroll
    for (int j = 0; j < kTN; ++j) bf[j] = read_frag(tB, brow0 + 32 * j + r, 4 * S + h, 4 * S + h + 2);
    if constexpr (SF == 32) {
      // lane r supplies block blk (K [0,32) of the slice), lane r+32 block blk+1
      const int sh = 8 * (blk + h);
      unsigned sa[kTM], sb[kTN];
#pragma unroll
      for (int i = 0; i < kTM; ++i) sa[i] = sfa[i] >> sh;
#pragma unroll
      for (int j = 0; j < kTN; ++j) sb[j] = sfb[j] >> sh;
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = mfma_f8<0, FA, FB>(bf[j], af[i], acc[i][j], sb[j], sa[i]);
    } else {
      // 16-element blocks: the lane's bytes 0..15 are block h and bytes
      // 16..31 block h+2, which cannot share a scale.  MFMA 1 keeps only
      // lanes h=0 of A (blocks 0, 2: scale bytes 0, 2 = byte 0 of the dword
      // shifted by 16h), MFMA 2 only lanes h=1 (blocks 1, 3: byte 1).  A zero
      // A element times a finite B element adds exactly 0.
      const v8i zero = {0, 0, 0, 0, 0, 0, 0, 0};
      unsigned sa[kTM], sb[kTN];
#pragma unroll
      for (int i = 0; i < kTM; ++i) sa[i] = sfa[i] >> (16 * h);
#pragma unroll
      for (int j = 0; j < kTN; ++j) sb[j] = sfb[j] >> (16 * h);
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const v8i a_even = h ? zero : af[i];
        const v8i a_odd = h ? af[i] : zero;
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
          acc[i][j] = mfma_f8<0, FA, FB>(bf[j], a_even, acc[i][j], sb[j], sa[i]);
          acc[i][j] = mfma_f8<1, FA, FB>(bf[j], a_odd, acc[i][j], sb[j], sa[i]);
        }
      }
    }
  } else {
    v8i af[kTM], bf[kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i) af[i] = read_frag(tA, arow0 + 32 * i + r, 4 * S + 2 * h, 4 * S + 2 * h + 1);
#pragma unroll
    for (int j = 0; j < kTN; ++j) bf[j] = read_frag(tB, brow0 + 32 * j + r, 4 * S + 2 * h, 4 * S + 2 * h + 1);
    // scales: sf=32 -> the lane's 32 K are block blk+h; sf=16 -> blocks 2h
    // (bytes 0..15) and 2h+1 (bytes 16..31) of the slice's atom
    float sa0[kTM], sa1[kTM], sb0[kTN], sb1[kTN];
    const unsigned k0 = (SF == 32) ? (unsigned)(blk + h) : 2u * (unsigned)h;  // byte of the first block
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      sa0[i] = e8m0_byte_operand(sfa[i], k0);
      sa1[i] = (SF == 32) ? sa0[i] : e8m0_byte_operand(sfa[i], k0 + 1);
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      sb0[j] = e8m0_byte_operand(sfb[j], k0);
      sb1[j] = (SF == 32) ? sb0[j] : e8m0_byte_operand(sfb[j], k0 + 1);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v8bf ab[kTM], bb[kTN];
#pragma unroll
      for (int i = 0; i < kTM; ++i) ab[i] = cvt8<FA>(af[i][2 * q], af[i][2 * q + 1], q < 2 ? sa0[i] : sa1[i]);
#pragma unroll
      for (int j = 0; j < kTN; ++j) bb[j] = cvt8<FB>(bf[j][2 * q], bf[j][2 * q + 1], q < 2 ? sb0[j] : sb1[j]);
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bb[j], ab[i], acc[i][j], 0, 0, 0);
    }
  }
}

// --- the kernel --------------------------------------------------------------

template <int SF, int FA, int FB, int MODE, int CT>
__global__ __launch_bounds__(kThreads, 2) void mxgemm_amax_kernel(Params p) {
  constexpr int kEs = kCBytes<CT>;           // bytes per C element
  constexpr int WM = kBM / 2, WN = kBN / 2;  // wave tile
  constexpr int NSF = (SF == 32) ? 1 : 2;    // atoms per step
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31;
  const int h = lane >> 5;

  // DMA lane geometry (fixed per lane): row inside an 8-row group and the
  // logical K chunk that lands in this lane's swizzled slot
  const int dma_row = lane >> 3;
  const int dma_chunk = (lane & 7) ^ dma_row;
  // SF DMA: waves 0,1 fetch the A atoms, waves 2,3 the B atoms, each half of
  // them (NSF atoms of 512 bytes per operand) with its first NSF*16 lanes
  const bool sf_is_a = wave < 2;
  const int sf_half = wave & 1;
  const int sf_lanes = NSF * 16;
  const int sf_byte = sf_half * (NSF * 256) + 16 * lane;  // byte inside the operand's atom area

  unsigned lmax = 0u;

  const int G = (int)gridDim.x;
  const int t0 = first_tile(p);
  const int my_tiles = t0 < p.num_tiles ? (p.num_tiles - 1 - t0) / G + 1 : 0;
  const int total = my_tiles * p.ksteps;

  // queue the DMA of step kt of tile T into stage `st` (exactly kOps
  // instructions per wave)
  auto issue_step = [&](const Tile& T, int kt, uint8_t* st) {
    const unsigned kk = (unsigned)(kt * kBK + (dma_chunk << 4));
    {
      const unsigned oob = (unsigned)T.mvalid * (unsigned)p.K;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.A + ((int64_t)T.l * p.M + T.m0) * p.K, oob);
#pragma unroll
      for (int q = 0; q < kBM / 32; ++q) {
        const int grp = wave + 4 * q;  // 8-row group
        const int row = grp * 8 + dma_row;
        const unsigned voff = (row < T.mvalid && kk < (unsigned)p.K) ? (unsigned)row * (unsigned)p.K + kk : oob;
        dma16(rs, voff, st + grp * 1024);
      }
    }
    {
      const unsigned oob = (unsigned)T.nvalid * (unsigned)p.K;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.B + ((int64_t)T.l * p.N + T.n0) * p.K, oob);
#pragma unroll
      for (int q = 0; q < kBN / 32; ++q) {
        const int grp = wave + 4 * q;
        const int row = grp * 8 + dma_row;
        const unsigned voff = (row < T.nvalid && kk < (unsigned)p.K) ? (unsigned)row * (unsigned)p.K + kk : oob;
        dma16(rs, voff, st + kOffB + grp * 1024);
      }
    }
    {
      // atoms NSF*kt + j (j < NSF) of this tile's single 128-row group; the
      // branch is wave-uniform, one instruction per wave either way
      const int g = NSF * kt + (sf_byte >> 9);
      const unsigned nrec = (unsigned)p.Kg * 512u;
      const unsigned voff = g < p.Kg ? (unsigned)g * 512u + (unsigned)(sf_byte & 511) : nrec;
      uint8_t* dst = st + (sf_is_a ? kOffSFA : kOffSFB) + sf_half * (NSF * 256);
      if (sf_is_a) {
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(p.SFA + ((int64_t)T.l * p.MNbA + (T.m0 >> 7)) * p.Kg * 512, nrec);
        if (lane < sf_lanes) dma16(rs, voff, dst);
      } else {
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(p.SFB + ((int64_t)T.l * p.MNbB + (T.n0 >> 7)) * p.Kg * 512, nrec);
        if (lane < sf_lanes) dma16(rs, voff, dst);
      }
    }
  };

  v16f acc[kTM][kTN], prev[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = prev[i][j][e] = 0.f;

  // store batch B (kStoresPerStep stores) of the previous tile's C from
  // `prev` (B is a compile-time constant so the accumulators are indexed
  // statically); out-of-range lanes get an offset past the buffer resource,
  // which stores nothing, so every lane issues exactly kStoresPerStep stores
  auto store_batch = [&](const Tile& P, auto Bc) {
    constexpr int b = decltype(Bc)::value;
    const unsigned c_bytes = (unsigned)P.mvalid * (unsigned)p.N * (unsigned)kEs;
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(reinterpret_cast<uint8_t*>(p.C) + ((int64_t)P.l * p.M + P.m0) * p.N * kEs, c_bytes);
    const unsigned vbase =
        ((unsigned)(wm * WM + r) * (unsigned)p.N + (unsigned)(P.n0 + wn * WN + 4 * h)) * (unsigned)kEs;
#pragma unroll
    for (int u = 0; u < kStoresPerStep; ++u) {
      const int idx = b * kStoresPerStep + u;  // 0 .. kNStores-1
      const int i = idx / (kTN * 4), j = (idx / 4) % kTN, q = idx % 4;
      const bool ok = (wm * WM + 32 * i + r < P.mvalid) && (wn * WN + 32 * j + 8 * q + 4 * h < P.nvalid);
      v4f v;
      v[0] = prev[i][j][4 * q];
      v[1] = prev[i][j][4 * q + 1];
      v[2] = prev[i][j][4 * q + 2];
      v[3] = prev[i][j][4 * q + 3];
      store_c4<CT>(v, rc, ok ? (int)(vbase + (32 * j + 8 * q) * kEs) : (int)c_bytes, ok ? 32 * i * p.N * kEs : 0);
      const unsigned m4 = max(max(__float_as_uint(v[0]) & 0x7FFFFFFFu, __float_as_uint(v[1]) & 0x7FFFFFFFu),
                              max(__float_as_uint(v[2]) & 0x7FFFFFFFu, __float_as_uint(v[3]) & 0x7FFFFFFFu));
      lmax = ok ? max(lmax, m4) : lmax;
    }
  };
  static_assert(kStoreSteps == 8, "store dispatch below is written for 8 batches");
  auto store_one = [&](const Tile& P, int b) {
    switch (b) {
      case 0: store_batch(P, std::integral_constant<int, 0>{}); break;
      case 1: store_batch(P, std::integral_constant<int, 1>{}); break;
      case 2: store_batch(P, std::integral_constant<int, 2>{}); break;
      case 3: store_batch(P, std::integral_constant<int, 3>{}); break;
      case 4: store_batch(P, std::integral_constant<int, 4>{}); break;
      case 5: store_batch(P, std::integral_constant<int, 5>{}); break;
      case 6: store_batch(P, std::integral_constant<int, 6>{}); break;
      default: store_batch(P, std::integral_constant<int, 7>{}); break;
    }
  };
  // the store batches b0.. of the previous tile still to go
  auto store_rest = [&](const Tile& P, int b0) {
    for (int b = b0; b < kStoreSteps; ++b) store_one(P, b);
  };

  Tile cur = {0, 0, 0, 0, 0}, nxt = {0, 0, 0, 0, 0}, prv = {0, 0, 0, 0, 0};
  int tcur = t0;
  int kt = 0;
  bool have_prev = false;      // `prev` holds a tile whose stores are not all issued
  int stores_done = 0;         // store batches of `prev` issued so far
  int after_dma = 0;           // store instructions issued after the last DMA

  if (total > 0) {
    cur = make_tile<kBM, kBN>(p, tcur);
    issue_step(cur, 0, lds);
  } else if (p.ksteps == 0) {
    // K == 0: every C of this workgroup is an empty sum
    for (int i = 0; i < my_tiles; ++i) store_rest(make_tile<kBM, kBN>(p, t0 + i * G), 0);
  }

  for (int s = 0; s < total; ++s) {
    // step s's DMA has landed for this wave (only store instructions may
    // have been issued after it); the barrier makes that true for all waves
    // and frees the other stage, read during step s-1
    if (after_dma == 0) wait_vm<0>();
    else if (after_dma == kStoresPerStep) wait_vm<kStoresPerStep>();
    else wait_vm<0>();
    barrier();
    uint8_t* st = lds + (int)(s & 1) * kStage;

    // queue step s+1 (this tile's next step or the next tile's first)
    after_dma = 0;
    if (s + 1 < total) {
      if (kt + 1 < p.ksteps) {
        issue_step(cur, kt + 1, lds + (int)((s + 1) & 1) * kStage);
      } else {
        nxt = make_tile<kBM, kBN>(p, tcur + G);
        issue_step(nxt, 0, lds + (int)((s + 1) & 1) * kStage);
      }
    }
    // a few of the previous tile's C stores, queued after the DMA
    if (have_prev && stores_done < kStoreSteps) {
      store_one(prv, stores_done);
      ++stores_done;
      after_dma = kStoresPerStep;
      if (stores_done == kStoreSteps) have_prev = false;
    }

    // this step's math: SF dwords, then two 64-K slices
    {
      unsigned sfa0[kTM], sfb0[kTN], sfa1[kTM], sfb1[kTN];
      const int g0 = NSF * kt;
#pragma unroll
      for (int i = 0; i < kTM; ++i) sfa0[i] = fix_tail(read_sf(st + kOffSFA, 0, wm * WM + 32 * i + r), g0, p.Kb);
#pragma unroll
      for (int j = 0; j < kTN; ++j) sfb0[j] = fix_tail(read_sf(st + kOffSFB, 0, wn * WN + 32 * j + r), g0, p.Kb);
      if constexpr (SF == 16) {
#pragma unroll
        for (int i = 0; i < kTM; ++i)
          sfa1[i] = fix_tail(read_sf(st + kOffSFA, 1, wm * WM + 32 * i + r), g0 + 1, p.Kb);
#pragma unroll
        for (int j = 0; j < kTN; ++j)
          sfb1[j] = fix_tail(read_sf(st + kOffSFB, 1, wn * WN + 32 * j + r), g0 + 1, p.Kb);
      } else {
#pragma unroll
        for (int i = 0; i < kTM; ++i) sfa1[i] = sfa0[i];
#pragma unroll
        for (int j = 0; j < kTN; ++j) sfb1[j] = sfb0[j];
      }
      compute_slice<MODE, 0, SF, FA, FB>(acc, st, st + kOffB, wm * WM, wn * WN, lane, sfa0, sfb0);
      compute_slice<MODE, 1, SF, FA, FB>(acc, st, st + kOffB, wm * WM, wn * WN, lane, sfa1, sfb1);
    }

    if (++kt == p.ksteps) {
      // tile done: finish the previous tile's stores if K was too short to
      // spread them, then this tile's accumulators become `prev`
      if (have_prev) {
        store_rest(prv, stores_done);
        after_dma = -1;  // an unusual count: the next wait drains everything
      }
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
          prev[i][j] = acc[i][j];
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
        }
      prv = cur;
      have_prev = true;
      stores_done = 0;
      cur = nxt;
      tcur += G;
      kt = 0;
    }
  }
  // the last tile's stores (and any the loop did not reach)
  if (have_prev) store_rest(prv, stores_done);

#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lmax = max(lmax, (unsigned)__shfl_xor((int)lmax, off));
  if (lane == 0 && lmax != 0u) atomicMax(p.amax_bits, lmax);
}

}  // namespace mxg
