// Pieces shared by the block-scaled FP8 GEMM + amax kernels for gfx950:
// kernel parameters, tile scheduling, buffer resources and the global->LDS
// DMA, waits and barriers, E8M0 decoding, the scaled conversions and the
// scaled FP8 MFMA wrapper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mxg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int kGroupM = 8;           // tile rows per raster group
constexpr int kRsrcFlags = 0x00020000;

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
  int Kbytes;  // bytes of one A / B row: K, or K/2 for packed FP4 (E2M1)
  int Kb;      // ceil(K / sf): K-blocks
  int Kg;      // ceil(K / (4 sf)): atoms along K
  int MNbA;    // ceil(M / 128)
  int MNbB;    // ceil(N / 128)
  int tilesM, tilesN;
  int ksteps;  // ceil(K / 128)
  int num_tiles;   // L * tilesM * tilesN (the host keeps it below 2^31)
  int xcd_remap;  // 1 when gridDim.x is a multiple of 8
  // projection epilogue only (C type 4): per-head RoPE and dual-direction
  // MXFP8 of C in place of storing it
  const uint16_t* rope_cos;  // (M, qk_rope) bf16 bits
  const uint16_t* rope_sin;  // (M, qk_rope) bf16 bits
  uint8_t* row_codes;        // (M, N) E4M3, blocks of 32 along N
  uint8_t* row_scales;       // (M, N / 32) E8M0
  uint8_t* col_codes;        // (M, N) E4M3, blocks of 32 along M
  uint8_t* col_scales;       // (M / 32, N) E8M0
  int head_dim, qk_rope;
};

// --- tile scheduling ---------------------------------------------------------

// Tile t -> (batch, tile row, tile column): batch-major, then groups of
// kGroupM tile rows walked column-major inside a batch.
__device__ __forceinline__ void tile_coords(const Params& p, int t, int& l, int& tm, int& tn) {
  const int per_batch = p.tilesM * p.tilesN;
  l = t / per_batch;
  const int r = t - l * per_batch;
  const int group_size = kGroupM * p.tilesN;
  const int g = r / group_size;
  const int first_m = g * kGroupM;
  const int gm = min(p.tilesM - first_m, kGroupM);
  const int rg = r - g * group_size;
  tm = first_m + rg % gm;
  tn = rg / gm;
}

struct Tile {
  int l, m0, n0, mvalid, nvalid;
};

template <int BM, int BN>
__device__ __forceinline__ Tile make_tile(const Params& p, int t) {
  int l, tm, tn;
  tile_coords(p, t, l, tm, tn);
  Tile T;
  T.l = __builtin_amdgcn_readfirstlane(l);
  T.m0 = __builtin_amdgcn_readfirstlane(tm * BM);
  T.n0 = __builtin_amdgcn_readfirstlane(tn * BN);
  T.mvalid = min(p.M - T.m0, BM);
  T.nvalid = min(p.N - T.n0, BN);
  return T;
}

// First tile of workgroup b in a grid of G: when G is a multiple of 8 the
// index is remapped so that the workgroups of one XCD (dispatched
// round-robin over the 8 XCDs) take a contiguous run of tiles.
__device__ __forceinline__ int first_tile(const Params& p) {
  const int G = (int)gridDim.x;
  const int b = (int)blockIdx.x;
  return p.xcd_remap ? (b & 7) * (G >> 3) + (b >> 3) : b;
}

// --- memory helpers ------------------------------------------------------------

// Buffer resource over [base, base + bytes) built from values forced into
// scalar registers (the DMA asm needs its resource in SGPRs; a value the
// compiler could not prove wave-uniform would otherwise land in VGPRs).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  void* ptr = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ptr, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcFlags);
}

// One 16-byte-per-lane buffer load into LDS at (m0 + 16 * lane).  Issued as
// inline assembly on purpose: the compiler cannot prove that a DMA into one
// ring stage does not alias the ds_reads of another, and for the builtin it
// inserts "s_waitcnt vmcnt(0)" before those reads, which drains the whole
// prefetch ring every step.  Ordering is kept by explicit per-wave vmcnt
// waits instead.
//
// Wait states.  A vector-memory instruction that reads an SGPR written by a
// VALU instruction (here v_readfirstlane, which forces the buffer resource
// and the LDS address into SGPRs) must come at least 5 wait states after it;
// the hardware does not interlock that dependence.  The compiler's hazard
// pass does not look inside inline assembly for it, so the 5 wait states
// are part of the assembly itself: s_mov to m0 (1) and s_nop 3 (4), which
// also covers the one wait state between writing m0 and the LDS DMA that
// reads it.  With fewer, whether the load sees the new or the stale
// resource depends on how the wave's instructions happen to be issued, so a
// DMA can fetch rows of the wrong operand or tile now and then.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, unsigned voff, const uint8_t* lds_dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(__attribute__((address_space(3))) const uint8_t*)lds_dst);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
               "s"(m0)
               : "memory", "m0");
}

// The same with the LDS destination given as a 32-bit LDS address (m0 value).
__device__ __forceinline__ void dma16_at(__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned lds_addr) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
               "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// 32-bit LDS address of a __shared__ object.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(__attribute__((address_space(3))) const uint8_t*)p;
}

// s_waitcnt with vmcnt = N (N <= 63), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that does not wait for vector memory.  __syncthreads()
// also waits for every outstanding vector-memory operation, which would drain
// the DMA ring and the C stores; here each wave has already waited for the
// DMA it needs.  What the barrier does enforce:
//  * every LDS read this wave issued before it has returned (lgkmcnt(0)), so
//    a DMA that another wave queues into that stage after the barrier cannot
//    overwrite data this wave has yet to read.  The compiler places its own
//    lgkmcnt waits just before the first use of a read, and an MFMA or
//    conversion that uses it may be scheduled past s_barrier (the barrier
//    orders memory instructions only);
//  * no memory access is moved across it by the compiler (the empty asm
//    statements clobber memory; s_barrier alone is not a memory operation
//    to the optimiser).
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left alone
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// E8M0 scale bytes as the f32 scale operand of the scaled conversions
// v_cvt_scalef32_pk_bf16_{fp8,bf8}.  Those instructions read only the
// exponent field (bits 23..30) of their scale and give it E8M0 meaning:
// exponent e scales by 2^(e-127), exponent 0 by 2^-127 and exponent 255 makes
// every result NaN (measured on MI355X for all 256 bytes).  The sign and
// mantissa bits are ignored: results are bitwise equal for every exponent,
// 40 sign/mantissa patterns, all 256 codes, both halves, E4M3 and E5M2.  So
// byte k (0..3) of a dword w becomes the operand by rotating w until bits
// 8k..8k+7 sit on the exponent field; the neighbouring bytes left in the
// other bits do no harm.  One v_alignbit, with a shift that may differ per
// lane.
__device__ __forceinline__ float e8m0_byte_operand(unsigned w, unsigned k) {
  return __uint_as_float(__builtin_amdgcn_alignbit(w, w, (8u * k + 9u) & 31u));
}

template <int OPSEL, int FA, int FB>
__device__ __forceinline__ v16f mfma_f8(const v8i& b, const v8i& a, const v16f& c, unsigned sb, unsigned sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, FB, FA, OPSEL, (int)sb, OPSEL, (int)sa);
}

// Two FP8 codes (bytes 0,1 or 2,3 of `w`) -> two bf16 times `scale`, as one
// dword (the pair is bit-cast whole; element-wise extraction of the v2bf16
// result was seen to duplicate the low half).
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

// C element type and layout, a kernel template parameter CT: 0 float32,
// 1 bfloat16, 2 float16, all n-major (L, M, N); 3 float32 m-major (L, N, M);
// 4: no C -- the projection epilogue (RoPE and dual-direction MXFP8 codes of
// the float32 accumulators).  The accumulators are float32 either way; a 16-bit C
// receives them rounded to nearest even (v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32), and the amax is taken over the float32 values.
template <int CT>
constexpr int kCBytes = (CT == 0 || CT == 3) ? 4 : 2;
template <int CT>
constexpr bool kCMajorM = CT == 3;

// Four consecutive outputs of one C row, given in float32, stored as C's
// element type at byte offset voff + soff of resource rc, with cache policy
// bits CP (2: non-temporal).
template <int CT, int CP = 0>
__device__ __forceinline__ void store_c4(const v4f& v, __amdgpu_buffer_rsrc_t rc, int voff, int soff) {
  if constexpr (CT == 0 || CT == 3)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), rc, voff, soff, CP);
  else if constexpr (CT == 1)
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, __builtin_convertvector(v, v4bf)), rc, voff, soff,
                                          CP);
  else
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, __builtin_convertvector(v, v4h)), rc, voff, soff, CP);
}

// Eight packed E2M1 elements (one dword, element 2i in the low nibble of byte
// i) to bf16 with the scale folded in: v_cvt_scalef32_pk_bf16_fp4 takes byte
// `sel` and puts its low nibble in the first bf16 of the pair (checked on
// MI355X for all 256 bytes and every byte select, scales 2^0, 2^-3, 2^5).
__device__ __forceinline__ v8bf cvt8_fp4(unsigned w, float scale) {
  v4u u;
  u[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  u[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  u[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  u[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return __builtin_bit_cast(v8bf, u);
}

}  // namespace mxg
