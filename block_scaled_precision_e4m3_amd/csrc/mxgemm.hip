// C-ABI entry points of the block-scaled FP8 GEMM + amax library (include/mxgemm.h).
//
// Host side: argument validation (reported before anything is queued, the
// error convention of "Grouped GEMM (SM100 BF16)", section "Scheduling,
// caching, and errors"), the per-shape tile choice, and the launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <stdlib.h>
#include <string.h>

#include "../../include/mxgemm.h"
#include "mx_quantize.hpp"
#include "sf_repack.hpp"
#include "codes_transpose.hpp"
#include "proj_rope.hpp"
#include "gemm_launch.hpp"

namespace mxg {

// The workspace of mxgemm_projection_mxfp8_noalloc: one array per device,
// reserved with the library's code object.  Host code never uses its name as
// an address (that is a host-side stand-in); the device address comes from
// hipGetSymbolAddress, once per device (scratch_address below).
static __device__ __align__(256) uint8_t scratch[MXGEMM_NOALLOC_SCRATCH_BYTES];

// Clears the Amax bits (queued before a GEMM that does not accumulate).
__global__ void amax_reset_kernel(unsigned* amax_bits) {
  if (threadIdx.x == 0) *amax_bits = 0u;
}

// C of an empty sum (K == 0): `n8` 8-byte words of zeros (every C type and
// layout is all-zero bytes), grid-strided.
__global__ void c_zero_kernel(uint2* c, int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) c[i] = make_uint2(0u, 0u);
}

}  // namespace mxg

namespace {

constexpr int kMaxDevices = 64;


struct DeviceInfo {
  int checked = 0;   // 0 unknown, 1 gfx950, -1 other
  int cus = 0;
};

DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mutex;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool fits_i32(int64_t v) { return v >= 0 && v <= 0x7FFFFFFFLL; }

// Pure size/format validation shared by every entry point.
int check_sizes(int64_t M, int64_t N, int64_t K, int64_t L, int sf, int a_fmt, int b_fmt) {
  if (M < 0 || N < 0 || K < 0 || L < 0) return MXG_ERR_SHAPE;
  if (sf != 16 && sf != 32) return MXG_ERR_SFVEC;
  const auto known = [](int f) { return f == MXG_FMT_E4M3 || f == MXG_FMT_E5M2 || f == MXG_FMT_E2M1; };
  if (!known(a_fmt) || !known(b_fmt)) return MXG_ERR_FMT;
  const bool fp4 = a_fmt == MXG_FMT_E2M1;
  if (fp4 != (b_fmt == MXG_FMT_E2M1)) return MXG_ERR_FMT;  // packed FP4 on both operands or neither
  // kernel indices are 32-bit per dimension, byte offsets 64-bit
  if (!fits_i32(M) || !fits_i32(N) || !fits_i32(K) || !fits_i32(L)) return MXG_ERR_SHAPE;
  const int64_t lim = INT64_MAX / 8;
  if (M && K && L && (M > lim / K || M * K > lim / L)) return MXG_ERR_SHAPE;
  if (N && K && L && (N > lim / K || N * K > lim / L)) return MXG_ERR_SHAPE;
  if (M && N && L && (M > lim / N || M * N > lim / (4 * L))) return MXG_ERR_SHAPE;
  // one tile's rows (up to 256) of A, B or C must be addressable with 32-bit
  // buffer offsets
  if (K > (1LL << 23) || N > (1LL << 22) - 4) return MXG_ERR_SHAPE;
  // tile and tile-step counts are 32-bit in the kernels
  if (L * cdiv(M, 128) * cdiv(N, 128) * (cdiv(K, 128) + 1) > 0x7FFFFFFFLL) return MXG_ERR_SHAPE;
  if (K % 16 != 0) return MXG_ERR_ALIGN;
  if (fp4 && K % 32 != 0) return MXG_ERR_ALIGN;             // packed rows of 16-byte multiples
  if (N % 4 != 0) return MXG_ERR_ALIGN;
  return MXG_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Current device must be gfx950; returns its CU count through *cus.
int device_check(int* dev_out, int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXG_ERR_DEVICE;
  DeviceInfo& d = g_dev[dev];
  if (d.checked == 0) {
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (d.checked == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXG_ERR_DEVICE;
      d.cus = prop.multiProcessorCount;
      d.checked = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
  }
  if (d.checked != 1) return MXG_ERR_DEVICE;
  *dev_out = dev;
  *cus = d.cus;
  return MXG_OK;
}

// Device address of `scratch` on device `dev` (current), looked up on the
// first call on that device and kept; nullptr if HIP cannot give it.
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

void* scratch_address(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(mxg::scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Device memory of `dev` (or managed memory) is accepted; host memory is not.
bool on_device(const void* p, int dev) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return false;
  return attr.device == dev;
}

// Tile shapes, one workgroup per CU either way (mxgemm_big.hpp): 256x256 (4
// waves of 128x128) or 128x128 (4 computing waves of 64x64 and 4 DMA waves).
// A 256x256 tile moves half the L2->LDS bytes per flop and converts half the
// operand bytes per MFMA, so it runs a tile's worth of flops faster; 128x128
// tiles spread a small problem over more CUs.  The choice compares the time
// of the rounds of tiles the CUs run, a 128x128 tile costing kSmallCost of a
// 256x256 tile's (which has four times its flops; measured on MI355X: 0.30
// on the 4000x7168x2048 and 8192x24576x1536 problems, each run both ways).
// kind 3 is the zero fill of K == 0.
struct Config {
  int kind;  // 0: 128x128 tiles, 1: 256x256 tiles, 3: K == 0
  int tile_m, tile_n, per_cu;
};
constexpr Config kT128 = {0, 128, 128, 1}, kT256 = {1, 256, 256, 1}, kZero = {3, 128, 128, 1};
constexpr double kSmallCost = 0.30;

Config choose(int64_t M, int64_t N, int64_t K, int64_t L, int cus) {
  if (K == 0) return kZero;
  const int64_t small = L * cdiv(M, 128) * cdiv(N, 128);
  const int64_t big = L * cdiv(M, 256) * cdiv(N, 256);
  const double t_big = (double)cdiv(big, cus), t_small = kSmallCost * (double)cdiv(small, cus);
  return t_big <= t_small ? kT256 : kT128;
}

// Workgroups for `tiles` tiles: one per tile up to the CUs' capacity; past it
// no more than the rounds of tiles need (in multiples of 8, whole XCDs), so
// that every workgroup runs the same number of tiles and the last round does
// not leave part of the chip idle while the rest runs it: the ragged
// 4000x7168x2048 problem (448 tiles of 256x256, 224 workgroups instead of
// 256) runs 7% faster on MI355X; a whole number of rounds is unchanged.
int64_t grid_for(int64_t tiles, int cus, int occ) {
  const int64_t g = (int64_t)cus * occ;
  if (tiles <= g) return tiles;
  const int64_t rounds = (tiles + g - 1) / g;
  const int64_t per_round = ((tiles + rounds - 1) / rounds + 7) / 8 * 8;
  return per_round < g ? per_round : g;
}

// --- MX block quantisation ------------------------------------------------------

// Size/format validation of mxgemm_mx_quantize (no HIP call).
int check_quantize(int64_t MN, int64_t K, int64_t L, int sf, int fmt) {
  if (MN < 0 || K < 0 || L < 0) return MXG_ERR_SHAPE;
  if (sf != 16 && sf != 32) return MXG_ERR_SFVEC;
  if (fmt != MXG_FMT_E4M3 && fmt != MXG_FMT_E5M2) return MXG_ERR_FMT;
  if (!fits_i32(MN) || !fits_i32(L)) return MXG_ERR_SHAPE;
  // an atom's 128 rows of float32 must be addressable with 32-bit buffer offsets
  if (K >= (1LL << 23)) return MXG_ERR_SHAPE;
  if (MN && K && L && (MN * K > (INT64_MAX / 8) / L)) return MXG_ERR_SHAPE;
  if (L * cdiv(MN, 128) * cdiv(K, 4 * sf) > 0x7FFFFFFFLL) return MXG_ERR_SHAPE;
  if (K % 16 != 0) return MXG_ERR_ALIGN;
  return MXG_OK;
}

template <int SF>
hipError_t launch_quantize(const mxg::quant::QParams& p, int fmt, int64_t grid, hipStream_t s) {
  const dim3 g((unsigned)grid), b(mxg::quant::kThreads);
  if (fmt == MXG_FMT_E4M3)
    hipLaunchKernelGGL((mxg::quant::mx_quantize_kernel<SF, 0>), g, b, 0, s, p);
  else
    hipLaunchKernelGGL((mxg::quant::mx_quantize_kernel<SF, 1>), g, b, 0, s, p);
  return hipGetLastError();
}

// --- validated, configured GEMM launch (shared by mxgemm_amax_ex and plans) ---

constexpr uint32_t kPlanMagic = 0x4D584731u;  // "MXG1"

struct Prepared {
  uint32_t magic;
  int dev;                  // plans: the device the plan was made for
  mxg::Params p{};          // sizes and tiling; pointers filled at launch
  int sf, fa, fb, kind, ct;
  int mj;                   // bit 0: m-major A, bit 1: n-major B
  unsigned flags;
  int64_t grid;
  bool fp8, accumulate, need_c, need_a;
};

// Validates sizes, formats and flags and fills everything that does not depend on
// the device; with query_device, also the device and the tiling (configure()).
int prepare(Prepared* pr, int64_t M, int64_t N, int64_t K, int64_t L, int sf_vec_size, int a_fmt, int b_fmt,
            unsigned flags, bool query_device);

void configure(Prepared* pr, int cus) {
  mxg::Params& p = pr->p;
  const int64_t M = p.M, N = p.N, K = p.K, L = p.L;
  const bool fp4 = pr->fa == MXG_FMT_E2M1;
  Config cfg = choose(M, N, K, L, cus);
  if (K > 0 && (pr->flags & MXG_FLAG_TILE_128)) cfg = kT128;
  if (K > 0 && (pr->flags & MXG_FLAG_TILE_256)) cfg = kT256;
  if (K > 0 && fp4 && pr->sf == 16) cfg = kT128;  // four scale atoms per step fit the 128x128 tile's LDS only
  pr->kind = cfg.kind;
  p.tilesM = (int)cdiv(M, cfg.tile_m);
  p.tilesN = (int)cdiv(N, cfg.tile_n);
  p.ksteps = (int)cdiv(K, fp4 ? 256 : 128);  // 128 bytes of every row per step
  p.num_tiles = (int)(L * p.tilesM * p.tilesN);
  pr->grid = grid_for(p.num_tiles, cus, cfg.per_cu);
  if (cfg.kind == 3) {
    // zero fill: 8-byte words of C, 256 threads per workgroup, up to 4 workgroups per CU
    const int64_t words = L * M * N * (pr->ct == 1 || pr->ct == 2 ? 2 : 4) / 8;
    pr->grid = std::max<int64_t>(1, std::min<int64_t>(cdiv(words, 256), 4LL * cus));
  }
  p.xcd_remap = (pr->grid % 8 == 0) ? 1 : 0;
}

int prepare(Prepared* pr, int64_t M, int64_t N, int64_t K, int64_t L, int sf_vec_size, int a_fmt, int b_fmt,
            unsigned flags, bool query_device) {
  int st = check_sizes(M, N, K, L, sf_vec_size, a_fmt, b_fmt);
  if (st != MXG_OK) return st;
  const unsigned tile_flags = flags & (MXG_FLAG_TILE_128 | MXG_FLAG_TILE_256);
  const unsigned c_flags = flags & (MXG_FLAG_C_BF16 | MXG_FLAG_C_F16);
  if (flags & ~(unsigned)(MXG_FLAG_AMAX_ACCUMULATE | MXG_FLAG_FP8_MFMA | MXG_FLAG_TILE_128 | MXG_FLAG_TILE_256 |
                          MXG_FLAG_C_BF16 | MXG_FLAG_C_F16 | MXG_FLAG_C_MMAJOR | MXG_FLAG_A_MMAJOR |
                          MXG_FLAG_B_NMAJOR))
    return MXG_ERR_FLAGS;
  // m-major A / n-major B: 8-bit codes, bf16 datapath, float32 n-major C;
  // contiguous dimension in whole 16-byte chunks; one batch below 2^31 bytes
  const int mj = ((flags & MXG_FLAG_A_MMAJOR) ? 1 : 0) | ((flags & MXG_FLAG_B_NMAJOR) ? 2 : 0);
  if (mj && (a_fmt == MXG_FMT_E2M1 ||
             (flags & (MXG_FLAG_FP8_MFMA | MXG_FLAG_C_BF16 | MXG_FLAG_C_F16 | MXG_FLAG_C_MMAJOR))))
    return MXG_ERR_FLAGS;
  if (((mj & 1) && M * K >= (1LL << 31)) || ((mj & 2) && N * K >= (1LL << 31))) return MXG_ERR_SHAPE;
  if (((mj & 1) && M % 16 != 0) || ((mj & 2) && N % 16 != 0)) return MXG_ERR_ALIGN;
  const bool c_mmajor = (flags & MXG_FLAG_C_MMAJOR) != 0;
  // m-major C: the bf16 datapath with a float32 C
  if (c_mmajor && (flags & (MXG_FLAG_FP8_MFMA | MXG_FLAG_C_BF16 | MXG_FLAG_C_F16))) return MXG_ERR_FLAGS;
  if (tile_flags & (tile_flags - 1)) return MXG_ERR_FLAGS;  // more than one tile flag
  if (c_flags & (c_flags - 1)) return MXG_ERR_FLAGS;        // both 16-bit C types
  if (c_flags && (flags & MXG_FLAG_FP8_MFMA)) return MXG_ERR_FLAGS;  // 16-bit C: bf16 datapath only
  if (a_fmt == MXG_FMT_E2M1 && (flags & MXG_FLAG_FP8_MFMA)) return MXG_ERR_FLAGS;  // FP4: bf16 datapath
  if (a_fmt == MXG_FMT_E2M1 && sf_vec_size == 16 && (flags & MXG_FLAG_TILE_256)) return MXG_ERR_FLAGS;
  // m-major C: rows of C run along M, so M takes N's place in the 32-bit
  // per-tile store offsets (256 rows * M * 4 bytes)
  if (c_mmajor && M > (1LL << 22) - 4) return MXG_ERR_SHAPE;
  if (c_mmajor && M % 4 != 0) return MXG_ERR_ALIGN;  // 16-byte runs along M
  memset(pr, 0, sizeof(*pr));
  pr->magic = kPlanMagic;
  pr->flags = flags;
  pr->sf = sf_vec_size;
  pr->fa = a_fmt;
  pr->fb = b_fmt;
  pr->fp8 = (flags & MXG_FLAG_FP8_MFMA) != 0;
  pr->accumulate = (flags & MXG_FLAG_AMAX_ACCUMULATE) != 0;
  pr->ct = (flags & MXG_FLAG_C_BF16) ? 1 : (flags & MXG_FLAG_C_F16) ? 2 : c_mmajor ? 3 : 0;
  pr->mj = mj;
  // A, B and the scales are read only when there is a non-empty C and a non-empty K
  pr->need_c = M > 0 && N > 0 && L > 0;
  pr->need_a = pr->need_c && K > 0;
  mxg::Params& p = pr->p;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.L = (int)L;
  p.Kbytes = (int)(a_fmt == MXG_FMT_E2M1 ? K / 2 : K);
  p.Kb = (int)cdiv(K, sf_vec_size);
  p.Kg = (int)cdiv(K, 4 * sf_vec_size);
  p.MNbA = (int)cdiv(M, 128);
  p.MNbB = (int)cdiv(N, 128);
  if (query_device) {
    int cus = 0;
    st = device_check(&pr->dev, &cus);
    if (st != MXG_OK) return st;
    configure(pr, cus);
  }
  return MXG_OK;
}

// Null and alignment checks of the operands a prepared launch reads and writes.
int check_ptrs(const Prepared& pr, const void* A, const void* B, const void* SFA, const void* SFB, const void* C,
               const void* Amax) {
  if (!Amax || (pr.need_a && (!A || !SFA || !B || !SFB)) || (pr.need_c && !C)) return MXG_ERR_NULL;
  if (!aligned16(Amax) || (pr.need_a && (!aligned16(A) || !aligned16(SFA) || !aligned16(B) || !aligned16(SFB))) ||
      (pr.need_c && !aligned16(C)))
    return MXG_ERR_ALIGN;
  return MXG_OK;
}

int launch_prepared(const Prepared& pr, const void* A, const void* B, const uint8_t* SFA, const uint8_t* SFB,
                    float* C, float* Amax, hipStream_t s) {
  if (!pr.accumulate) {
    hipLaunchKernelGGL(mxg::amax_reset_kernel, dim3(1), dim3(64), 0, s, reinterpret_cast<unsigned*>(Amax));
    if (hipGetLastError() != hipSuccess) return MXG_ERR_LAUNCH;
  }
  if (!pr.need_c) return MXG_OK;
  mxg::Params p = pr.p;
  p.A = static_cast<const uint8_t*>(A);
  p.B = static_cast<const uint8_t*>(B);
  p.SFA = SFA;
  p.SFB = SFB;
  p.C = C;
  p.amax_bits = reinterpret_cast<unsigned*>(Amax);
  const int sf = pr.sf, fa = pr.fa, fb = pr.fb;
  const int64_t grid = pr.grid;
  hipError_t e;
  if (pr.kind == 3) {
    const int64_t words = (int64_t)p.L * p.M * p.N * (pr.ct == 1 || pr.ct == 2 ? 2 : 4) / 8;
    hipLaunchKernelGGL(mxg::c_zero_kernel, dim3((unsigned)grid), dim3(256), 0, s, reinterpret_cast<uint2*>(C), words);
    e = hipGetLastError();
  } else if (pr.mj) {
    e = pr.kind == 1 ? mxg::launch_bf16_mj_t256(p, sf, fa, fb, pr.mj, grid, s)
                     : mxg::launch_bf16_mj_t128(p, sf, fa, fb, pr.mj, grid, s);
  } else if (pr.fp8) {
    e = mxg::launch_fp8(p, sf, fa, fb, pr.kind == 1 ? 256 : 128, grid, s);
  } else if (pr.ct == 1 || pr.ct == 2) {
    e = pr.kind == 1 ? mxg::launch_bf16_c16_t256(p, sf, fa, fb, pr.ct, grid, s)
                     : mxg::launch_bf16_c16_t128(p, sf, fa, fb, pr.ct, grid, s);
  } else {
    e = pr.kind == 1 ? mxg::launch_bf16_f32_t256(p, sf, fa, fb, pr.ct, grid, s)
                     : mxg::launch_bf16_f32_t128(p, sf, fa, fb, pr.ct, grid, s);
  }
  return e == hipSuccess ? MXG_OK : MXG_ERR_LAUNCH;
}

// --- the projection: GEMM with the RoPE + dual-direction MXFP8 epilogue -------

// Size and format rules of the fused projection (no HIP call).
int check_projection(int64_t tokens, int64_t H, int64_t D, int64_t QR, int64_t K, int sf, int fa, int fb) {
  if (tokens < 0 || H < 0 || D <= 0 || QR < 0 || K <= 0) return MXG_ERR_SHAPE;
  if (sf != 16 && sf != 32) return MXG_ERR_SFVEC;
  if ((fa != MXG_FMT_E4M3 && fa != MXG_FMT_E5M2) || (fb != MXG_FMT_E4M3 && fb != MXG_FMT_E5M2)) return MXG_ERR_FMT;
  if (!fits_i32(tokens) || !fits_i32(H) || !fits_i32(D) || !fits_i32(H * D)) return MXG_ERR_SHAPE;
  const int64_t N = H * D;
  const int st = check_sizes(tokens, N, K, 1, sf, fa, fb);
  if (st != MXG_OK) return st;
  // a head spans at least one 128-column wave block, blocks of 32 features
  // never cross heads, the rotary part is a multiple of 16 features up to 64
  if (D % 32 != 0 || D < 128 || QR % 16 != 0 || QR > 64 || N % 128 != 0) return MXG_ERR_SHAPE;
  // no head's rotary features cross a 128-column boundary (the pattern
  // repeats every 128 heads at most)
  for (int64_t h = 0; QR > 0 && h < std::min<int64_t>(H, 128); ++h) {
    const int64_t a = h * D + D - QR;
    if (a / 128 != (a + QR - 1) / 128) return MXG_ERR_SHAPE;
  }
  if (tokens % 32 != 0) return MXG_ERR_ALIGN;  // column blocks of 32 tokens
  return MXG_OK;
}

bool aligned16_all(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned16(p)) return false;
  return true;
}

// The fused kernel on atom-layout scales; sizes already validated.
int launch_projection(const void* A, const void* B, const uint8_t* SFA, const uint8_t* SFB, const uint16_t* cs,
                      const uint16_t* sn, uint8_t* rc, uint8_t* rsc, uint8_t* cc, uint8_t* csc, int64_t tokens,
                      int64_t H, int64_t D, int64_t QR, int64_t K, int sf, int fa, int fb, int cus, hipStream_t s) {
  mxg::Params p{};  // every pointer the launch does not set stays null
  memset(&p, 0, sizeof(p));
  p.A = static_cast<const uint8_t*>(A);
  p.B = static_cast<const uint8_t*>(B);
  p.SFA = SFA;
  p.SFB = SFB;
  p.M = (int)tokens;
  p.N = (int)(H * D);
  p.K = (int)K;
  p.L = 1;
  p.Kbytes = (int)K;
  p.Kb = (int)cdiv(K, sf);
  p.Kg = (int)cdiv(K, 4 * sf);
  p.MNbA = (int)cdiv(tokens, 128);
  p.MNbB = (int)cdiv(H * D, 128);
  p.tilesM = (int)cdiv(tokens, 256);
  p.tilesN = (int)cdiv(H * D, 256);
  p.ksteps = (int)cdiv(K, 128);
  p.num_tiles = p.tilesM * p.tilesN;
  const int64_t grid = grid_for(p.num_tiles, cus, 1);
  p.xcd_remap = grid % 8 == 0 ? 1 : 0;
  p.rope_cos = cs;
  p.rope_sin = sn;
  p.row_codes = rc;
  p.row_scales = rsc;
  p.col_codes = cc;
  p.col_scales = csc;
  p.head_dim = (int)D;
  p.qk_rope = (int)QR;
  return mxg::launch_proj_t256(p, sf, fa, fb, grid, s) == hipSuccess ? MXG_OK : MXG_ERR_LAUNCH;
}

// Row-wise E8M0 scales into atoms (the kernel of mxgemm_sf_rowwise_to_atoms);
// sizes already validated.
hipError_t launch_rowwise(const uint8_t* rowwise, uint8_t* SF, int64_t MN, int64_t K, int64_t L, int sf, int cus,
                          hipStream_t s) {
  mxg::repack::RParams p;
  p.R = rowwise;
  p.SF = SF;
  p.MN = (int)MN;
  p.Kb = (int)cdiv(K, sf);
  p.MNb = (int)cdiv(MN, 128);
  p.Kg = (int)cdiv(K, 4 * sf);
  p.num_atoms = (int)(L * p.MNb * p.Kg);
  const int64_t grid = std::min<int64_t>(p.num_atoms, 16LL * cus);
  hipLaunchKernelGGL(mxg::repack::rowwise_to_atoms_kernel, dim3((unsigned)grid), dim3(mxg::repack::kThreads), 0, s, p);
  return hipGetLastError();
}

// Workspace of the full projection: x's atoms, then w's, each 256-byte aligned.
size_t projection_ws_a(int64_t tokens, int64_t K, int sf) {
  return (size_t)((512 * cdiv(tokens, 128) * cdiv(K, 4 * sf) + 255) / 256 * 256);
}
size_t projection_ws_bytes(int64_t tokens, int64_t N, int64_t K, int sf) {
  return projection_ws_a(tokens, K, sf) + (size_t)(512 * cdiv(N, 128) * cdiv(K, 4 * sf));
}

// The page's projection on row-wise scales: both repacks into `ws`, then the
// fused kernel.  Everything validated by the caller.
int run_projection(const void* x, const void* w, const uint8_t* xs, const uint8_t* wsc, const uint16_t* cs,
                   const uint16_t* sn, uint8_t* rc, uint8_t* rsc, uint8_t* cc, uint8_t* csc, int64_t tokens, int64_t H,
                   int64_t D, int64_t QR, int64_t K, uint8_t* ws, int cus, hipStream_t s) {
  constexpr int sf = 32;
  uint8_t* sfa = ws;
  uint8_t* sfb = ws + projection_ws_a(tokens, K, sf);
  if (launch_rowwise(xs, sfa, tokens, K, 1, sf, cus, s) != hipSuccess) return MXG_ERR_LAUNCH;
  if (launch_rowwise(wsc, sfb, H * D, K, 1, sf, cus, s) != hipSuccess) return MXG_ERR_LAUNCH;
  return launch_projection(x, w, sfa, sfb, cs, sn, rc, rsc, cc, csc, tokens, H, D, QR, K, sf, MXG_FMT_E4M3,
                           MXG_FMT_E4M3, cus, s);
}

}  // namespace

extern "C" {

int mxgemm_check_support(int64_t M, int64_t N, int64_t K, int64_t L, int sf_vec_size, int a_fmt, int b_fmt) {
  return check_sizes(M, N, K, L, sf_vec_size, a_fmt, b_fmt);
}

size_t mxgemm_sf_bytes(int64_t MN, int64_t K, int64_t L, int sf_vec_size) {
  if (MN < 0 || K < 0 || L < 0 || (sf_vec_size != 16 && sf_vec_size != 32)) return 0;
  return (size_t)(512 * L * cdiv(MN, 128) * cdiv(K, 4 * sf_vec_size));
}

int mxgemm_launch_config(int64_t M, int64_t N, int64_t K, int64_t L, int sf_vec_size, int* tile_m, int* tile_n,
                         int64_t* grid) {
  int st = check_sizes(M, N, K, L, sf_vec_size, MXG_FMT_E4M3, MXG_FMT_E4M3);
  if (st != MXG_OK) return st;
  int cus = 256;
  if (grid) {
    int dev = 0;
    st = device_check(&dev, &cus);
    if (st != MXG_OK) return st;
  }
  const Config cfg = choose(M, N, K, L, cus);
  if (tile_m) *tile_m = cfg.tile_m;
  if (tile_n) *tile_n = cfg.tile_n;
  if (grid) {
    const int64_t tiles = L * cdiv(M, cfg.tile_m) * cdiv(N, cfg.tile_n);
    *grid = grid_for(tiles, cus, cfg.per_cu);
  }
  return MXG_OK;
}

int mxgemm_amax_reset(float* Amax, void* stream) {
  if (!Amax) return MXG_ERR_NULL;
  if (!aligned16(Amax)) return MXG_ERR_ALIGN;
  int dev = 0, cus = 0;
  int st = device_check(&dev, &cus);
  if (st != MXG_OK) return st;
  if (!on_device(Amax, dev)) return MXG_ERR_DEVICE;
  hipLaunchKernelGGL(mxg::amax_reset_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     reinterpret_cast<unsigned*>(Amax));
  return hipGetLastError() == hipSuccess ? MXG_OK : MXG_ERR_LAUNCH;
}

int mxgemm_amax_ex(const void* A, const void* B, const uint8_t* SFA, const uint8_t* SFB, float* C, float* Amax,
                   int64_t M, int64_t N, int64_t K, int64_t L, int sf_vec_size, int a_fmt, int b_fmt,
                   unsigned flags, void* stream) {
  Prepared pr;
  int st = prepare(&pr, M, N, K, L, sf_vec_size, a_fmt, b_fmt, flags, /*query_device=*/false);
  if (st != MXG_OK) return st;
  st = check_ptrs(pr, A, B, SFA, SFB, C, Amax);
  if (st != MXG_OK) return st;
  int dev = 0, cus = 0;
  st = device_check(&dev, &cus);
  if (st != MXG_OK) return st;
  if (!on_device(Amax, dev) || (pr.need_a && (!on_device(A, dev) || !on_device(SFA, dev) || !on_device(B, dev) ||
                                               !on_device(SFB, dev))) ||
      (pr.need_c && !on_device(C, dev)))
    return MXG_ERR_DEVICE;
  configure(&pr, cus);
  return launch_prepared(pr, A, B, SFA, SFB, C, Amax, (hipStream_t)stream);
}

int mxgemm_plan_init(mxgemm_plan* plan, int64_t M, int64_t N, int64_t K, int64_t L, int sf_vec_size, int a_fmt,
                     int b_fmt, unsigned flags) {
  if (!plan) return MXG_ERR_NULL;
  static_assert(sizeof(Prepared) <= sizeof(mxgemm_plan), "mxgemm_plan too small for the prepared launch");
  memset(plan, 0, sizeof(*plan));
  Prepared pr;
  int st = prepare(&pr, M, N, K, L, sf_vec_size, a_fmt, b_fmt, flags, /*query_device=*/true);
  if (st != MXG_OK) return st;
  memcpy(plan, &pr, sizeof(pr));
  return MXG_OK;
}

int mxgemm_plan_execute(const mxgemm_plan* plan, const void* A, const void* B, const uint8_t* SFA,
                        const uint8_t* SFB, float* C, float* Amax, void* stream) {
  if (!plan) return MXG_ERR_NULL;
  Prepared pr;
  memcpy(&pr, plan, sizeof(pr));
  if (pr.magic != kPlanMagic) return MXG_ERR_NULL;  // never initialised (or not by mxgemm_plan_init)
  int st = check_ptrs(pr, A, B, SFA, SFB, C, Amax);
  if (st != MXG_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != pr.dev) return MXG_ERR_DEVICE;
  return launch_prepared(pr, A, B, SFA, SFB, C, Amax, (hipStream_t)stream);
}

int mxgemm_mx_quantize(const float* X, void* Q, uint8_t* SF, int64_t MN, int64_t K, int64_t L, int sf_vec_size,
                       int fmt, void* stream) {
  int st = check_quantize(MN, K, L, sf_vec_size, fmt);
  if (st != MXG_OK) return st;
  if (MN == 0 || K == 0 || L == 0) return MXG_OK;  // nothing to read or write
  if (!X || !Q || !SF) return MXG_ERR_NULL;
  if (!aligned16(X) || !aligned16(Q) || !aligned16(SF)) return MXG_ERR_ALIGN;
  int dev = 0, cus = 0;
  st = device_check(&dev, &cus);
  if (st != MXG_OK) return st;
  if (!on_device(X, dev) || !on_device(Q, dev) || !on_device(SF, dev)) return MXG_ERR_DEVICE;

  mxg::quant::QParams p;
  p.X = X;
  p.Q = static_cast<uint8_t*>(Q);
  p.SF = SF;
  p.MN = (int)MN;
  p.K = (int)K;
  p.MNb = (int)cdiv(MN, 128);
  p.Kg = (int)cdiv(K, 4 * sf_vec_size);
  p.num_atoms = (int)(L * p.MNb * p.Kg);
  // 256-thread workgroups, up to 8 per CU resident; each loops over atoms
  const int64_t grid = std::min<int64_t>(p.num_atoms, 8LL * cus);
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = sf_vec_size == 32 ? launch_quantize<32>(p, fmt, grid, s) : launch_quantize<16>(p, fmt, grid, s);
  return e == hipSuccess ? MXG_OK : MXG_ERR_LAUNCH;
}

int mxgemm_sf_rowwise_to_atoms(const uint8_t* rowwise, uint8_t* SF, int64_t MN, int64_t K, int64_t L,
                               int sf_vec_size, void* stream) {
  if (MN < 0 || K < 0 || L < 0) return MXG_ERR_SHAPE;
  if (sf_vec_size != 16 && sf_vec_size != 32) return MXG_ERR_SFVEC;
  if (!fits_i32(MN) || !fits_i32(K) || !fits_i32(L)) return MXG_ERR_SHAPE;
  if (L * cdiv(MN, 128) * cdiv(K, 4 * sf_vec_size) > 0x7FFFFFFFLL) return MXG_ERR_SHAPE;
  if (MN == 0 || K == 0 || L == 0) return MXG_OK;
  if (!rowwise || !SF) return MXG_ERR_NULL;
  if (!aligned16(SF)) return MXG_ERR_ALIGN;
  int dev = 0, cus = 0;
  int st = device_check(&dev, &cus);
  if (st != MXG_OK) return st;
  if (!on_device(rowwise, dev) || !on_device(SF, dev)) return MXG_ERR_DEVICE;
  return launch_rowwise(rowwise, SF, MN, K, L, sf_vec_size, cus, (hipStream_t)stream) == hipSuccess ? MXG_OK
                                                                                                 : MXG_ERR_LAUNCH;
}

int mxgemm_codes_to_kmajor(const void* src, void* dst, int64_t MN, int64_t K, int64_t L, void* stream) {
  if (MN < 0 || K < 0 || L < 0) return MXG_ERR_SHAPE;
  if (!fits_i32(MN) || !fits_i32(K) || !fits_i32(L)) return MXG_ERR_SHAPE;
  if (L * cdiv(MN, 64) * cdiv(K, 64) > 0x7FFFFFFFLL) return MXG_ERR_SHAPE;
  if (MN % 16 != 0 || K % 16 != 0) return MXG_ERR_ALIGN;
  if (MN == 0 || K == 0 || L == 0) return MXG_OK;
  if (!src || !dst) return MXG_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return MXG_ERR_ALIGN;
  int dev = 0, cus = 0;
  int st = device_check(&dev, &cus);
  if (st != MXG_OK) return st;
  if (!on_device(src, dev) || !on_device(dst, dev)) return MXG_ERR_DEVICE;
  mxg::transpose::TParams p;
  p.S = static_cast<const uint8_t*>(src);
  p.D = static_cast<uint8_t*>(dst);
  p.MN = (int)MN;
  p.K = (int)K;
  p.tiles_mn = (int)cdiv(MN, mxg::transpose::kTile);
  p.tiles_k = (int)cdiv(K, mxg::transpose::kTile);
  p.num_tiles = (int)(L * p.tiles_mn * p.tiles_k);
  const int64_t grid = std::min<int64_t>(p.num_tiles, 16LL * cus);
  hipLaunchKernelGGL(mxg::transpose::codes_to_kmajor_kernel, dim3((unsigned)grid), dim3(mxg::transpose::kThreads), 0,
                     (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? MXG_OK : MXG_ERR_LAUNCH;
}

int mxgemm_proj_rope_mxfp8(const float* Y, const uint16_t* cos_bf16, const uint16_t* sin_bf16, uint8_t* row_codes,
                           uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, int64_t tokens,
                           int64_t num_heads, int64_t head_dim, int64_t qk_rope, void* stream) {
  if (tokens < 0 || num_heads < 0 || head_dim <= 0 || qk_rope < 0) return MXG_ERR_SHAPE;
  if (head_dim % 32 != 0 || head_dim > mxg::rope::kMaxD || qk_rope % 2 != 0 || qk_rope > head_dim ||
      qk_rope > mxg::rope::kMaxQR)
    return MXG_ERR_SHAPE;
  if (!fits_i32(tokens) || !fits_i32(num_heads) || !fits_i32(num_heads * head_dim) ||
      tokens * num_heads > (INT64_MAX / 8) / head_dim)
    return MXG_ERR_SHAPE;
  if (tokens % 32 != 0) return MXG_ERR_ALIGN;  // column blocks of 32 tokens
  if ((tokens / 32) * num_heads > 0x7FFFFFFFLL) return MXG_ERR_SHAPE;
  if (tokens == 0 || num_heads == 0) return MXG_OK;
  if (!Y || !row_codes || !row_scales || !col_codes || !col_scales || (qk_rope > 0 && (!cos_bf16 || !sin_bf16)))
    return MXG_ERR_NULL;
  if (!aligned16(Y) || !aligned16(row_codes) || !aligned16(col_codes) ||
      (qk_rope > 0 && (!aligned16(cos_bf16) || !aligned16(sin_bf16))))
    return MXG_ERR_ALIGN;
  int dev = 0, cus = 0;
  int st = device_check(&dev, &cus);
  if (st != MXG_OK) return st;
  if (!on_device(Y, dev) || !on_device(row_codes, dev) || !on_device(row_scales, dev) || !on_device(col_codes, dev) ||
      !on_device(col_scales, dev) || (qk_rope > 0 && (!on_device(cos_bf16, dev) || !on_device(sin_bf16, dev))))
    return MXG_ERR_DEVICE;
  mxg::rope::RParams p;
  p.Y = Y;
  p.cs = cos_bf16;
  p.sn = sin_bf16;
  p.row_codes = row_codes;
  p.row_scales = row_scales;
  p.col_codes = col_codes;
  p.col_scales = col_scales;
  p.H = (int)num_heads;
  p.D = (int)head_dim;
  p.QR = (int)qk_rope;
  p.num_tiles = (int)((tokens / 32) * num_heads);
  // runs of consecutive heads per workgroup (a run never crosses a block of
  // 32 tokens: its length divides num_heads), as long as that still leaves
  // 8 workgroups per CU
  p.per_wg = 1;
  for (int run : {16, 4})
    if (p.H % run == 0 && p.num_tiles >= 8LL * run * cus) {
      p.per_wg = run;
      break;
    }
  const int64_t grid = cdiv(p.num_tiles, p.per_wg);
  const unsigned lds = (unsigned)mxg::rope::lds_bytes(p.D, p.QR, p.per_wg);
  if (p.D == 192 && p.QR == 64)  // the projection page's head: constant index arithmetic
    hipLaunchKernelGGL((mxg::rope::proj_rope_mxfp8_kernel<192, 64>), dim3((unsigned)grid), dim3(mxg::rope::kThreads),
                       lds, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL((mxg::rope::proj_rope_mxfp8_kernel<0, 0>), dim3((unsigned)grid), dim3(mxg::rope::kThreads),
                       lds, (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? MXG_OK : MXG_ERR_LAUNCH;
}

int mxgemm_gemm_rope_mxfp8(const void* A, const void* B, const uint8_t* SFA, const uint8_t* SFB,
                           const uint16_t* cos_bf16, const uint16_t* sin_bf16, uint8_t* row_codes,
                           uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, int64_t tokens,
                           int64_t num_heads, int64_t head_dim, int64_t qk_rope, int64_t K, int sf_vec_size, int a_fmt,
                           int b_fmt, void* stream) {
  int st = check_projection(tokens, num_heads, head_dim, qk_rope, K, sf_vec_size, a_fmt, b_fmt);
  if (st != MXG_OK) return st;
  if (tokens == 0 || num_heads == 0) return MXG_OK;
  if (!A || !B || !SFA || !SFB || !row_codes || !row_scales || !col_codes || !col_scales ||
      (qk_rope > 0 && (!cos_bf16 || !sin_bf16)))
    return MXG_ERR_NULL;
  if (!aligned16_all({A, B, SFA, SFB, row_codes, row_scales, col_codes, col_scales}) ||
      (qk_rope > 0 && !aligned16_all({cos_bf16, sin_bf16})))
    return MXG_ERR_ALIGN;
  int dev = 0, cus = 0;
  st = device_check(&dev, &cus);
  if (st != MXG_OK) return st;
  for (const void* q : {A, B, (const void*)SFA, (const void*)SFB, (const void*)row_codes, (const void*)row_scales,
                        (const void*)col_codes, (const void*)col_scales})
    if (!on_device(q, dev)) return MXG_ERR_DEVICE;
  if (qk_rope > 0 && (!on_device(cos_bf16, dev) || !on_device(sin_bf16, dev))) return MXG_ERR_DEVICE;
  return launch_projection(A, B, SFA, SFB, cos_bf16, sin_bf16, row_codes, row_scales, col_codes, col_scales, tokens,
                           num_heads, head_dim, qk_rope, K, sf_vec_size, a_fmt, b_fmt, cus, (hipStream_t)stream);
}

size_t mxgemm_projection_workspace_bytes(int64_t tokens, int64_t num_heads, int64_t head_dim, int64_t K) {
  if (tokens < 0 || num_heads < 0 || head_dim < 0 || K < 0) return 0;
  return projection_ws_bytes(tokens, num_heads * head_dim, K, 32);
}

int mxgemm_projection_mxfp8(const void* x, const void* w, const uint8_t* x_scale, const uint8_t* w_scale,
                            const uint16_t* cos_bf16, const uint16_t* sin_bf16, uint8_t* row_codes,
                            uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, int64_t tokens,
                            int64_t num_heads, int64_t head_dim, int64_t qk_rope, int64_t K, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int st = check_projection(tokens, num_heads, head_dim, qk_rope, K, 32, MXG_FMT_E4M3, MXG_FMT_E4M3);
  if (st != MXG_OK) return st;
  if (tokens == 0 || num_heads == 0) return MXG_OK;
  if (!x || !w || !x_scale || !w_scale || !row_codes || !row_scales || !col_codes || !col_scales || !workspace ||
      (qk_rope > 0 && (!cos_bf16 || !sin_bf16)))
    return MXG_ERR_NULL;
  if (workspace_bytes < projection_ws_bytes(tokens, num_heads * head_dim, K, 32)) return MXG_ERR_SHAPE;
  if (!aligned16_all({x, w, row_codes, row_scales, col_codes, col_scales}) || (reinterpret_cast<uintptr_t>(workspace) & 255) ||
      (qk_rope > 0 && !aligned16_all({cos_bf16, sin_bf16})))
    return MXG_ERR_ALIGN;
  int dev = 0, cus = 0;
  st = device_check(&dev, &cus);
  if (st != MXG_OK) return st;
  for (const void* q : {x, w, (const void*)x_scale, (const void*)w_scale, (const void*)row_codes,
                        (const void*)row_scales, (const void*)col_codes, (const void*)col_scales, (const void*)workspace})
    if (!on_device(q, dev)) return MXG_ERR_DEVICE;
  if (qk_rope > 0 && (!on_device(cos_bf16, dev) || !on_device(sin_bf16, dev))) return MXG_ERR_DEVICE;
  return run_projection(x, w, x_scale, w_scale, cos_bf16, sin_bf16, row_codes, row_scales, col_codes, col_scales,
                        tokens, num_heads, head_dim, qk_rope, K, static_cast<uint8_t*>(workspace), cus,
                        (hipStream_t)stream);
}

int mxgemm_projection_mxfp8_noalloc(const void* x, const void* w, const uint8_t* x_scale, const uint8_t* w_scale,
                                    const uint16_t* cos_bf16, const uint16_t* sin_bf16, uint8_t* row_codes,
                                    uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, int64_t tokens,
                                    int64_t num_heads, int64_t head_dim, int64_t qk_rope, int64_t K, void* stream) {
  int st = check_projection(tokens, num_heads, head_dim, qk_rope, K, 32, MXG_FMT_E4M3, MXG_FMT_E4M3);
  if (st != MXG_OK) return st;
  if (projection_ws_bytes(tokens, num_heads * head_dim, K, 32) > (size_t)MXGEMM_NOALLOC_SCRATCH_BYTES)
    return MXG_ERR_SCRATCH;
  if (tokens == 0 || num_heads == 0) return MXG_OK;
  if (!x || !w || !x_scale || !w_scale || !row_codes || !row_scales || !col_codes || !col_scales ||
      (qk_rope > 0 && (!cos_bf16 || !sin_bf16)))
    return MXG_ERR_NULL;
  if (!aligned16_all({x, w, row_codes, row_scales, col_codes, col_scales}) ||
      (qk_rope > 0 && !aligned16_all({cos_bf16, sin_bf16})))
    return MXG_ERR_ALIGN;
  int dev = 0, cus = 0;
  st = device_check(&dev, &cus);
  if (st != MXG_OK) return st;
  for (const void* q : {x, w, (const void*)x_scale, (const void*)w_scale, (const void*)row_codes,
                        (const void*)row_scales, (const void*)col_codes, (const void*)col_scales})
    if (!on_device(q, dev)) return MXG_ERR_DEVICE;
  if (qk_rope > 0 && (!on_device(cos_bf16, dev) || !on_device(sin_bf16, dev))) return MXG_ERR_DEVICE;
  uint8_t* ws = static_cast<uint8_t*>(scratch_address(dev));
  if (!ws) return MXG_ERR_DEVICE;
  return run_projection(x, w, x_scale, w_scale, cos_bf16, sin_bf16, row_codes, row_scales, col_codes, col_scales,
                        tokens, num_heads, head_dim, qk_rope, K, ws, cus, (hipStream_t)stream);
}

int mxgemm_amax(const void* A, const void* B, const uint8_t* SFA, const uint8_t* SFB, float* C, float* Amax,
                int64_t M, int64_t N, int64_t K, int64_t L, int sf_vec_size, int a_fmt, int b_fmt, void* stream) {
  return mxgemm_amax_ex(A, B, SFA, SFB, C, Amax, M, N, K, L, sf_vec_size, a_fmt, b_fmt, 0u, stream);
}

const char* mxgemm_strerror(int status) {
  switch (status) {
    case MXG_OK: return "success";
    case MXG_ERR_NULL: return "a required pointer is NULL";
    case MXG_ERR_SHAPE: return "invalid size (negative, or offsets overflow)";
    case MXG_ERR_ALIGN: return "misaligned buffer (16 bytes), K not a multiple of 16, or N not a multiple of 4";
    case MXG_ERR_SFVEC: return "sf_vec_size must be 16 or 32";
    case MXG_ERR_FMT: return "element format must be MXG_FMT_E4M3 or MXG_FMT_E5M2 (or MXG_FMT_E2M1 for both A and B)";
    case MXG_ERR_DEVICE: return "current device is not gfx950, or a buffer is not memory of the current device";
    case MXG_ERR_LAUNCH: return "HIP kernel launch failed";
    case MXG_ERR_FLAGS: return "unknown flag bit";
    case MXG_ERR_SCRATCH: return "the problem needs more scratch than the library's fixed scratch array holds";
    default: return "unknown status";
  }
}

}  // extern "C"
