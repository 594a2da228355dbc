// Large-tile variant of the block-scaled FP8 GEMM + amax kernel for gfx950.
//
// Same operation, operand layouts, scale handling and amax as the 128x128
// kernel in mxgemm_kernel.hpp ("GEMM + Amax (SM100)", sections "Equations"
// and "Shapes"); what changes is the shape of the work:
//
// * One workgroup per CU (the LDS ring takes 132-136 KB of the 160 KB) owns a
//   256x256 C tile; its 4 waves, one per SIMD, each hold a 128x128 block in
//   4x4 MFMA accumulators (256 registers).  Per 128-K step a CU then moves
//   66-68 KB from L2 for 8.4 M multiply-adds, half the bytes per flop of two
//   128x128 workgroups, and each converted fragment feeds 4 MFMAs instead of 2.
// * The K loop is one straight block per step: the step's 16-17 DMA
//   instructions for the next stage are spread between its MFMAs (4 after each
//   32-K chunk's fragment reads), so the memory pipe sees a steady stream
//   instead of a burst, and the single wave per SIMD keeps the matrix core fed
//   by issuing conversions, LDS reads and DMA in the shadow of its MFMAs.
// * A tile's C is stored at its end straight from the accumulators (64
//   16-byte stores per lane), then the next tile starts; the stores drain
//   under the next tile's first step.
//
// bf16 datapath, per 32-K chunk c of a step: lane (r, h) reads the 16 bytes
// K [32c + 16h, +16) of its row for each of its 4 A and 4 B fragments; bytes
// 0..7 feed MFMA slice 0 and bytes 8..15 slice 1 (any K assignment is valid
// when A and B share it, since the scale is folded into every element).  The
// chunk lies in one K-block for sf=32 (block c) and for sf=16 (block 2c + h).
// FP8 datapath, per 64-K slice S: bytes 0..15 of a lane are K [16h, +16) and
// bytes 16..31 are K [32 + 16h, +16) of the slice, as the scaled MFMA needs.
#pragma once

#include "mxgemm_common.hpp"

namespace mxg {
namespace big {

constexpr int kThreads = 256;
constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kTM = 4, kTN = 4;  // 32x32 MFMA blocks per wave: a 128x128 wave tile
constexpr int kNStores = kTM * kTN * 4;

template <int SF>
struct Layout {
  static constexpr int NSF = SF == 32 ? 1 : 2;      // atoms per 128-row group per step
  static constexpr int kSF = 2 * NSF * 512;         // atom bytes per operand per stage
  static constexpr int kOffB = kBM * kBK;           // A tile: 256 rows x 128 bytes
  static constexpr int kOffSFA = kOffB + kBN * kBK;  // B tile
  static constexpr int kOffSFB = kOffSFA + kSF;
  static constexpr int kStage = kOffSFB + kSF;       // 66 KB (sf=32) or 68 KB (sf=16)
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

template <int SF, int FA, int FB, int MODE>
__global__ __launch_bounds__(kThreads, 1) void mxgemm_amax_big_kernel(Params p) {
  using Y = Layout<SF>;
  constexpr int NSF = Y::NSF;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * Y::kStage];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int G = (int)gridDim.x;
  const int t0 = first_tile(p);
  const int my_tiles = t0 < p.num_tiles ? (p.num_tiles - 1 - t0) / G + 1 : 0;
  const int total = my_tiles * p.ksteps;
  const unsigned lds0 = lds_addr(lds);

  // Per-lane geometry.  It is recomputed every step from an opaque copy of the
  // lane id: values the compiler sees as loop-invariant get hoisted out of the
  // K loop and then spilled, and a spill reload inside the loop makes it wait
  // for every DMA in flight.
  struct Geo {
    int r, h;           // fragment row (lane % 32) and lane half
    int xr;             // r & 7: the swizzle of every fragment row of this lane
    int a_off, b_off;   // LDS offset of the lane's first A / B fragment row
    unsigned row_k;     // DMA: byte offset of the lane's row in its first 8-row group
    unsigned kchunk;    // DMA: the lane's 16-byte K chunk inside a 128-byte row
    unsigned sf_lane;   // SF DMA: the lane's 16 bytes inside an atom
    int sf_rg, sf_j;    // SF DMA: 128-row group and atom along K of the lane's load
  };
  auto geo = [&](int ln) {
    Geo g;
    g.r = ln & 31;
    g.h = ln >> 5;
    g.xr = ln & 7;
    g.a_off = (128 * wm + g.r) * kBK;
    g.b_off = Y::kOffB + (128 * wn + g.r) * kBK;
    const int dma_row = ln >> 3;
    g.row_k = (unsigned)(wave * 8 + dma_row) * (unsigned)p.K;
    g.kchunk = (unsigned)(((ln & 7) ^ dma_row) << 4);
    g.sf_lane = 16u * (unsigned)(ln & 31);
    g.sf_rg = NSF == 1 ? (ln >> 5) : (wave >> 1);
    g.sf_j = NSF == 1 ? 0 : (ln >> 5);
    return g;
  };
  auto lane_opaque = [&]() {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return ln;
  };

  // --- DMA of one stage ------------------------------------------------------
  // A/B: wave w fills the 8-row groups w, w+4, ..., w+28 of each tile, one
  // instruction (1 KB) per group.  A lane's offset is row*K + k; rows past the
  // tile's valid rows fall past the resource (num_records = valid rows * K)
  // and K chunks past K get an offset of 2^31 or more: both read as zero.
  // A and B rows use the same offsets, only the resources differ.
  // SF: sf=32 -> waves 0 and 1 load the A and B atoms of both 128-row groups
  // (lanes 0-31 group 0, 32-63 group 1); sf=16 -> waves 0,1 (A,B) load row
  // group 0's two atoms, waves 2,3 row group 1's.
  constexpr unsigned kOob = 0x80000000u;
  const bool sf_wave = NSF == 2 || wave < 2;
  const bool sf_is_b = (wave & 1) != 0;
  struct Dma {
    __amdgpu_buffer_rsrc_t ra, rb, rs;
    unsigned voff;     // lane's offset in row group 0 of the step (or >= 2^31)
    unsigned sf_voff;  // lane's SF offset
    unsigned dst;      // LDS address of the stage
  };
  auto dma_setup = [&](const Geo& g, const Tile& T, int kt, bool live, unsigned stage) {
    Dma d;
    d.ra = make_rsrc(p.A + ((int64_t)T.l * p.M + T.m0) * p.K, live ? (unsigned)T.mvalid * (unsigned)p.K : 0u);
    d.rb = make_rsrc(p.B + ((int64_t)T.l * p.N + T.n0) * p.K, live ? (unsigned)T.nvalid * (unsigned)p.K : 0u);
    const unsigned kk = (unsigned)(kt * kBK) + g.kchunk;
    d.voff = kk < (unsigned)p.K ? g.row_k + kk : kOob;
    const int mn0 = sf_is_b ? T.n0 : T.m0;
    const int mnb = sf_is_b ? p.MNbB : p.MNbA;
    const int g0 = mn0 >> 7;
    const unsigned nrec = live ? (unsigned)min(2, mnb - g0) * (unsigned)p.Kg * 512u : 0u;
    d.rs = make_rsrc((sf_is_b ? p.SFB : p.SFA) + ((int64_t)T.l * mnb + g0) * p.Kg * 512, nrec);
    const int kg = NSF * kt + g.sf_j;
    d.sf_voff = kg < p.Kg ? (unsigned)(g.sf_rg * p.Kg + kg) * 512u + g.sf_lane : kOob;
    d.dst = stage;
    return d;
  };
  // A/B DMA instruction q (0..15) of this wave: q < 8 -> A group wave + 4q
  const unsigned grp_stride = 32u * (unsigned)p.K;
  auto dma_ab = [&](const Dma& d, int q) {
    const unsigned voff = d.voff + (unsigned)(q & 7) * grp_stride;
    const unsigned dst = d.dst + (q >= 8 ? (unsigned)Y::kOffB : 0u) + (unsigned)(wave + 4 * (q & 7)) * 1024u;
    dma16_at(q >= 8 ? d.rb : d.ra, voff, dst);
  };
  auto dma_sf = [&](const Dma& d) {
    if (sf_wave)
      dma16_at(d.rs, d.sf_voff,
               d.dst + (sf_is_b ? (unsigned)Y::kOffSFB : (unsigned)Y::kOffSFA) +
                   (NSF == 1 ? 0u : (unsigned)(wave >> 1) * 1024u));
  };

  v16f acc[kTM][kTN];  // written by each tile's first step before any read
  const v16f zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  unsigned lmax = 0u;

  Tile cur = {0, 0, 0, 0, 0};
  bool stores_pending = false;
  int s = 0;  // global step index: selects the ring stage
  if (total > 0) {
    cur = make_tile<kBM, kBN>(p, t0);
    const Dma d0 = dma_setup(geo(lane), cur, 0, true, lds0);
    dma_sf(d0);
#pragma unroll
    for (int q = 0; q < 16; ++q) dma_ab(d0, q);
  }

  // One K step of tile `cur`; queues the DMA of the next step (this tile's
  // next K step or the next tile's first, `nt`).  On a tile's first step
  // (FIRST) the first MFMA of every accumulator takes a zero C operand instead
  // of the register, so the accumulators never need clearing and stay in the
  // matrix-core registers from tile to tile.
  auto step = [&](auto first, int kt, const Tile& nt, bool has_next) {
    constexpr bool kFirst = decltype(first)::value;
    // this wave's DMA for step s is complete (stores queued after it may not
    // be); the barrier extends that to every wave and frees the other stage
    if (stores_pending) wait_vm<63>();
    else wait_vm<0>();
    stores_pending = false;
    barrier();
    const Geo g = geo(lane_opaque());
    const uint8_t* st = lds + (s & 1) * Y::kStage;
    // fragment row i (32-row steps keep row & 7, so only the chunk is swizzled)
    auto a_frag = [&](int i, int c) { return lds16(st + g.a_off + ((c ^ g.xr) << 4) + 4096 * i); };
    auto b_frag = [&](int i, int c) { return lds16(st + g.b_off + ((c ^ g.xr) << 4) + 4096 * i); };

    const bool last_k = kt + 1 == p.ksteps;
    const Dma d = dma_setup(g, nt, last_k ? 0 : kt + 1, has_next, lds0 + (unsigned)(((s & 1) ^ 1) * Y::kStage));
    dma_sf(d);
    // SF dwords of this step: NSF atoms x 4 fragment rows per operand
    unsigned sa[NSF][kTM], sb[NSF][kTN];
#pragma unroll
    for (int j = 0; j < NSF; ++j) {
      const int ga = NSF * kt + j;
#pragma unroll
      for (int i = 0; i < kTM; ++i)
        sa[j][i] = sf_tail(lds4(st + Y::kOffSFA + (wm * NSF + j) * 512 + 16 * g.r + 4 * i), ga, p.Kb);
#pragma unroll
      for (int i = 0; i < kTN; ++i)
        sb[j][i] = sf_tail(lds4(st + Y::kOffSFB + (wn * NSF + j) * 512 + 16 * g.r + 4 * i), ga, p.Kb);
    }

    if constexpr (MODE == kModeBf16) {
      // software pipeline over the 4 chunks: chunk c+1's fragment reads are
      // queued before chunk c's conversions and MFMAs; scheduling barriers
      // keep the compiler from hoisting further ahead (register pressure)
      uint4 ar[kTM], br[kTN];
#pragma unroll
      for (int i = 0; i < kTM; ++i) ar[i] = a_frag(i, g.h);
#pragma unroll
      for (int i = 0; i < kTN; ++i) br[i] = b_frag(i, g.h);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint4 an[kTM], bn[kTN];
        if (c < 3) {
#pragma unroll
          for (int i = 0; i < kTM; ++i) an[i] = a_frag(i, 2 * (c + 1) + g.h);
#pragma unroll
          for (int i = 0; i < kTN; ++i) bn[i] = b_frag(i, 2 * (c + 1) + g.h);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) dma_ab(d, 4 * c + q);
        // the chunk's scale: sf=32 -> block c (byte c); sf=16 -> block 2c+h,
        // byte 2(c&1)+h of atom c>>1
        float fa[kTM], fb[kTN];
        const int j = SF == 32 ? 0 : (c >> 1);
        const int sh = SF == 32 ? 8 * c : 8 * (2 * (c & 1) + g.h);
#pragma unroll
        for (int i = 0; i < kTM; ++i) fa[i] = e8m0_to_f32((sa[j][i] >> sh) & 0xFFu);
#pragma unroll
        for (int i = 0; i < kTN; ++i) fb[i] = e8m0_to_f32((sb[j][i] >> sh) & 0xFFu);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          v8bf ab[kTM], bb[kTN];
#pragma unroll
          for (int i = 0; i < kTM; ++i) ab[i] = cvt8<FA>(t ? ar[i].z : ar[i].x, t ? ar[i].w : ar[i].y, fa[i]);
#pragma unroll
          for (int i = 0; i < kTN; ++i) bb[i] = cvt8<FB>(t ? br[i].z : br[i].x, t ? br[i].w : br[i].y, fb[i]);
#pragma unroll
          for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int jj = 0; jj < kTN; ++jj)
              acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  bb[jj], ab[i], (kFirst && c == 0 && t == 0) ? zero16 : acc[i][jj], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (c < 3) {
#pragma unroll
          for (int i = 0; i < kTM; ++i) ar[i] = an[i];
#pragma unroll
          for (int i = 0; i < kTN; ++i) br[i] = bn[i];
        }
      }
    } else {
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
        for (int q = 0; q < 8; ++q) dma_ab(d, 8 * S + q);
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
    }
    ++s;
  };

  // C stores and amax of tile `cur` from the accumulators
  auto epilogue = [&]() {
    // tile done: C stores (lane owns row m, 4-element runs of n) and amax,
    // one 32x32 block at a time (its 16 accumulators are stored and folded
    // into the amax before the next block is touched).  Rows past the
    // tile's valid rows land past the resource (num_records = valid rows *
    // N * 4); columns past N get an offset past it as well.
    const Geo ge = geo(lane_opaque());
    const unsigned c_bytes = (unsigned)cur.mvalid * (unsigned)p.N * 4u;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + ((int64_t)cur.l * p.M + cur.m0) * p.N, c_bytes);
    const int mrow = 128 * wm + ge.r;
    const int ncol = 128 * wn + 4 * ge.h;
    const unsigned vbase = ((unsigned)mrow * (unsigned)p.N + (unsigned)(cur.n0 + ncol)) * 4u;
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const unsigned vrow = vbase + (unsigned)(32 * i) * (unsigned)p.N * 4u;
      const bool rok = mrow + 32 * i < cur.mvalid;
#pragma unroll
      for (int jj = 0; jj < kTN; ++jj) {
        // pin the block in the accumulator registers until here, so its
        // copies out are made block by block rather than all at once
        asm volatile("" : "+a"(acc[i][jj])::"memory");
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool ok = rok & (ncol + 32 * jj + 8 * q < cur.nvalid);
          v4f v;
          v[0] = acc[i][jj][4 * q];
          v[1] = acc[i][jj][4 * q + 1];
          v[2] = acc[i][jj][4 * q + 2];
          v[3] = acc[i][jj][4 * q + 3];
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), rc,
                                                 ok ? (int)(vrow + (32 * jj + 8 * q) * 4) : (int)c_bytes, 0, 0);
          const unsigned m4 = max(max(__float_as_uint(v[0]) & 0x7FFFFFFFu, __float_as_uint(v[1]) & 0x7FFFFFFFu),
                                  max(__float_as_uint(v[2]) & 0x7FFFFFFFu, __float_as_uint(v[3]) & 0x7FFFFFFFu));
          lmax = max(lmax, m4 & (0u - (unsigned)ok));  // arithmetic mask: no branch
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    stores_pending = true;
  };

  for (int i = 0; i < my_tiles; ++i) {
    const int tn = t0 + (i + 1) * G;
    const bool more = i + 1 < my_tiles;
    const Tile nxt = more ? make_tile<kBM, kBN>(p, tn) : cur;
    if (p.ksteps == 1) {
      step(std::true_type{}, 0, nxt, more);
    } else {
      step(std::true_type{}, 0, cur, true);
      for (int kt = 1; kt + 1 < p.ksteps; ++kt) step(std::false_type{}, kt, cur, true);
      step(std::false_type{}, p.ksteps - 1, nxt, more);
    }
    epilogue();
    cur = nxt;
  }
  // no DMA may still be writing this workgroup's LDS when it exits
  wait_vm<0>();

#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lmax = max(lmax, (unsigned)__shfl_xor((int)lmax, off));
  if (lane == 0 && lmax != 0u) atomicMax(p.amax_bits, lmax);
}

}  // namespace big
}  // namespace mxg
