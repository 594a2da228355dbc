/*
 * mxgemm.h -- C ABI of the block-scaled FP8 GEMM with a fused global-amax
 * epilogue, for AMD Instinct MI355X (gfx950).
 *
 * Operation ("GEMM + Amax (SM100)", section "Equations"):
 *
 *   A_hat[m,k,l] = dec(A[m,k,l]) * 2^(SFA(m, k/sf, l) - 127)
 *   B_hat[n,k,l] = dec(B[n,k,l]) * 2^(SFB(n, k/sf, l) - 127)
 *   C[m,n,l]     = sum_k A_hat[m,k,l] * B_hat[n,k,l]      (FP32 accumulation)
 *   Amax         = max_{m,n,l} |C[m,n,l]|
 *
 * with sf = sf_vec_size in {16, 32} consecutive K elements per E8M0 scale.
 *
 * Memory layout (section "Parameters", input/output tensors; all buffers are
 * device memory owned by the caller, contiguous, byte offsets 64-bit):
 *   A    : (L, M, K) element codes, one byte each ("k-major" A, strides
 *          (K, 1, M*K) in the page's (M, K, L) notation).
 *   B    : (L, N, K) element codes ("k-major" B).
 *   SFA  : E8M0 scale bytes in the physical atom layout
 *          (L, ceil(M/128), ceil(K/(4*sf)), 32, 4, 4) -- the C-contiguous
 *          allocation whose permutation (3,4,1,5,2,0) is the logical
 *          (32, 4, ceil(M/128), 4, ceil(K/(4*sf)), L) of section "Shapes"
 *          (section "Using JAX arrays").  Row mn = i0 + 32*i1 + 128*i2 and
 *          K-block kb = i3 + 4*i4 of logical index (i0,i1,i2,i3,i4,l), i.e.
 *          byte 16*(mn%32) + 4*((mn/32)%4) + kb%4 of 512-byte atom
 *          (l*ceil(M/128) + mn/128)*ceil(K/(4*sf)) + kb/4.
 *          Padding bytes (rows >= M, K-blocks >= ceil(K/sf)) are never used
 *          and may hold anything.
 *   SFB  : the same for B with N in place of M.
 *   C    : (L, M, N) float32 ("n-major" C, the page's default c_major="n").
 *   Amax : one float32 (the page's (1,1,1) tensor).
 *
 * Element formats: MXG_FMT_E4M3 (float8_e4m3fn) and MXG_FMT_E5M2
 * (float8_e5m2).  A and B may use different formats and FP8 may be used
 * with sf = 16; both go beyond the page's support list (section "Support
 * surface and constraints", Dtypes) and follow the format-agnostic equations.
 *
 * Errors: every entry point returns MXG_OK (0) or a negative status, and an
 * invalid argument is reported before any work is queued on the stream
 * (the error convention of "Grouped GEMM (SM100 BF16)", section
 * "Scheduling, caching, and errors").  MXG_ERR_LAUNCH reports a HIP error
 * from the launch itself.
 *
 * Streams: `stream` is a hipStream_t passed as void*; NULL is the null
 * stream (the page's eager default, section "Using JAX arrays").  Calls are
 * asynchronous; inputs must stay alive and unmodified, and outputs unread,
 * until the stream has reached the call.
 *
 * The library allocates no device memory (inputs, outputs and the stream
 * are the caller's) and keeps no pointer after a call returns.
 */
#ifndef MXGEMM_H
#define MXGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element formats of A and B */
enum {
  MXG_FMT_E4M3 = 0, /* float8_e4m3fn: bias 7, no inf, NaN = 0x7F/0xFF, max 448 */
  MXG_FMT_E5M2 = 1, /* float8_e5m2:   bias 15, inf = 0x7C/0xFC, max 57344      */
  MXG_FMT_E2M1 = 2  /* float4_e2m1fn_x2: packed FP4, two elements per byte,
                       element 2k in the low nibble; bias 1, no inf/NaN, max 6.
                       A is then (L, M, K/2) bytes and B (L, N, K/2).  Both
                       operands must be E2M1, K % 32 == 0, and the default
                       (bf16) datapath; sf_vec_size 32 or 16 (the pages
                       exclude 16 only for 8-bit A/B, "Support surface and
                       constraints", dtypes); at 16 the kernel runs 128x128
                       tiles (the scale atoms of a 256x256 tile's step do
                       not fit beside it in LDS), and MXG_FLAG_TILE_256 is
                       MXG_ERR_FLAGS.  The pages list the packed container
                       ("Parameters", A dtype) but not which nibble comes
                       first: low first is the reading. */
};

/* status codes */
enum {
  MXG_OK = 0,
  MXG_ERR_NULL = -1,   /* a required pointer is NULL                          */
  MXG_ERR_SHAPE = -2,  /* a negative size, or a size whose offsets overflow   */
  MXG_ERR_ALIGN = -3,  /* A/B/C/Amax not 16-byte aligned, K % 16, N % 4       */
  MXG_ERR_SFVEC = -4,  /* sf_vec_size not 16 or 32                            */
  MXG_ERR_FMT = -5,    /* element format unknown, or E2M1 on one operand only */
  MXG_ERR_DEVICE = -6, /* current device is not gfx950, or a pointer is not
                          device memory of the current device                 */
  MXG_ERR_LAUNCH = -7, /* HIP reported an error when launching                */
  MXG_ERR_FLAGS = -8,  /* unknown bit in `flags`                              */
  MXG_ERR_SCRATCH = -9 /* the problem needs more scratch than the library's
                          fixed scratch array holds (the _noalloc entry)      */
};

/* flags of mxgemm_amax_ex */
enum {
  /* Do not clear Amax first: Amax := max(Amax, max|C|).  The caller keeps
     Amax a non-negative float (or NaN); lets several GEMMs share one Amax. */
  MXG_FLAG_AMAX_ACCUMULATE = 1u,
  /* Feed the FP8 codes straight to gfx950's scaled FP8 MFMA (twice the
     matrix rate of the default path).  That instruction keeps only the top
     ~13 bits, relative to the largest product, of each 8-element partial
     dot product, so small products next to large ones are truncated and
     the result can miss a 1e-5 * sum|A_hat*B_hat| error bound on
     heavy-tailed data.  The default path dequantises each element exactly
     to bf16 (scale folded in) and accumulates in fp32 on the bf16 MFMA. */
  MXG_FLAG_FP8_MFMA = 2u,
  /* Force the tile size instead of the automatic choice (for tests and
     tuning).  TILE_128: 128x128 tiles; TILE_256: 256x256 tiles; one
     workgroup per CU either way, of 4 computing waves (128x128 tiles on the
     default path, FP4 at sf = 16 aside: and 4 more that only stream the
     operands into LDS).  Both sizes compute every output the same way, so
     results agree bit for bit.  Ignored when K == 0.  Setting both is an
     error. */
  MXG_FLAG_TILE_128 = 4u,
  MXG_FLAG_TILE_256 = 8u,
  /* A 16-bit C ("GEMM + Amax (SM100)", section "Parameters": the C tensor
     may be float16 or bfloat16 as well as float32): C then holds (L, M, N)
     bfloat16 (C_BF16) or float16 (C_F16) elements, each the float32
     accumulator rounded to nearest even (float16 overflows to +-inf).  Amax
     is still taken over the float32 accumulators (the pages do not say which;
     the fused epilogue sees those).  The C pointer keeps its float* type in
     the signature and must still be 16-byte aligned.  Not with
     MXG_FLAG_FP8_MFMA; setting both C flags is an error. */
  MXG_FLAG_C_BF16 = 32u,
  MXG_FLAG_C_F16 = 64u,
  /* m-major C ("GEMM + Amax (SM100)", section "Parameters": C of shape
     (M, N, L) with strides (1, M, M*N), the wrapper's c_major="m"): C then
     holds (L, N, M) float32 elements, M contiguous.  The contiguous dimension
     must be 16-byte aligned, so M % 4 == 0 as well (MXG_ERR_ALIGN otherwise).
     The default datapath with a float32 C only: not with MXG_FLAG_FP8_MFMA
     or MXG_FLAG_C_BF16 / _F16 (MXG_ERR_FLAGS). */
  MXG_FLAG_C_MMAJOR = 128u,
  /* m-major A and n-major B ("GEMM + Amax (SM100)", section "Parameters":
     A of shape (M, K, L) with strides (1, M, M*K), B (N, K, L) with strides
     (1, N, N*K)): A then holds (L, K, M) codes, M contiguous (A_MMAJOR), B
     (L, K, N) codes, N contiguous (B_NMAJOR); either or both.  The kernel
     stages such a tile as K rows in LDS and reads it with gfx950's
     transposing LDS load, so no copy is made; results are bitwise those of
     the k-major operands.  8-bit formats, the default datapath and a
     float32 n-major C only (MXG_ERR_FLAGS otherwise); the contiguous
     dimension must be a multiple of 16 (MXG_ERR_ALIGN) and one batch of the
     operand (M*K or N*K bytes) below 2^31 (MXG_ERR_SHAPE). */
  MXG_FLAG_A_MMAJOR = 256u,
  MXG_FLAG_B_NMAJOR = 512u
};

/*
 * mxgemm_amax -- C = A_hat . B_hat^T per batch and Amax = max |C|.
 *
 *   A, B       device pointers to the element codes (layouts above).
 *   SFA, SFB   device pointers to the physical SF atom buffers,
 *              mxgemm_sf_bytes(M or N, K, L, sf_vec_size) bytes each.
 *   C          device pointer, L*M*N float32, fully overwritten.
 *   Amax       device pointer to one float32; set to max|C| (0 when
 *              M*N*L == 0; NaN if any C is NaN).
 *   M, N, K, L sizes, each >= 0.  K == 0 gives C == 0.
 *   sf_vec_size 16 or 32.
 *   a_fmt, b_fmt MXG_FMT_E4M3, MXG_FMT_E5M2, or MXG_FMT_E2M1 for both.
 *   stream     hipStream_t (NULL = null stream).
 *
 * Requirements: A, B, C, Amax, SFA, SFB 16-byte aligned; K % 16 == 0 (16-byte
 * rows of A/B) and K <= 2^23; N % 4 == 0 (16-byte rows of C) and N < 2^22 -- the page's "16-byte aligned along
 * the contiguous dimension" (section "Support surface and constraints",
 * Layouts and strides).  Current device must be gfx950 and own every pointer.
 *
 * Queues a one-wave kernel that clears Amax, then the GEMM kernel.
 */
int mxgemm_amax(const void* A, const void* B, const uint8_t* SFA, const uint8_t* SFB,
                float* C, float* Amax, int64_t M, int64_t N, int64_t K, int64_t L,
                int sf_vec_size, int a_fmt, int b_fmt, void* stream);

/*
 * mxgemm_amax_ex -- mxgemm_amax with flags.  flags == 0 is exactly
 * mxgemm_amax; MXG_FLAG_AMAX_ACCUMULATE skips the clearing kernel and
 * max-reduces into the existing Amax (queues the GEMM kernel only);
 * MXG_FLAG_FP8_MFMA selects the reduced-precision FP8 matrix path;
 * MXG_FLAG_TILE_128 / _256 force a tile configuration; MXG_FLAG_C_BF16 /
 * _F16 store a 16-bit C; MXG_FLAG_C_MMAJOR stores C m-major, (L, N, M)
 * float32 with M contiguous, which needs M % 4 == 0 (MXG_ERR_ALIGN) and
 * M < 2^22 (MXG_ERR_SHAPE; M takes N's place in the per-tile offsets).
 * Returns MXG_ERR_FLAGS for unknown bits, more than one tile flag, both C
 * flags, a C flag with MXG_FLAG_FP8_MFMA, or MXG_FLAG_C_MMAJOR with a flag it
 * excludes.
 *
 * Accuracy of the default path.  Every dequantised element is exact when its
 * value fits bf16: for every code when the scale byte lies in 3..246 (E4M3)
 * or 10..239 (E5M2); outside those bytes, codes whose value still fits bf16
 * stay exact and the others round to bf16.  Products are exact; the K sum is
 * an fp32 accumulation, one rounded add per 16 K, so its error grows with K:
 * at most about (K/16 + 1) * 2^-24 * S, S = sum_k |A_hat||B_hat|, reached
 * only when all products share a sign; mixed signs grow like sqrt(K).  The
 * bound is within 1e-5 * S for K <= 2048 whatever the data; beyond that,
 * same-sign data can exceed it (measured ratios are in the GPU tests).
 */
int mxgemm_amax_ex(const void* A, const void* B, const uint8_t* SFA, const uint8_t* SFB,
                   float* C, float* Amax, int64_t M, int64_t N, int64_t K, int64_t L,
                   int sf_vec_size, int a_fmt, int b_fmt, unsigned flags, void* stream);

/*
 * mxgemm_amax_reset -- queue the one-wave kernel that sets *Amax = 0.0f.
 * mxgemm_amax == mxgemm_amax_reset + mxgemm_amax_ex(MXG_FLAG_AMAX_ACCUMULATE).
 */
int mxgemm_amax_reset(float* Amax, void* stream);

/*
 * mxgemm_check_support -- host-only check of a problem description, the
 * counterpart of the page's check_support() (section "API Usage", class
 * API).  Returns MXG_OK or the status mxgemm_amax would return for these
 * sizes/formats (pointers and device are not checked).  No HIP call.
 */
int mxgemm_check_support(int64_t M, int64_t N, int64_t K, int64_t L, int sf_vec_size,
                         int a_fmt, int b_fmt);

/*
 * mxgemm_sf_bytes -- size of one physical SF buffer:
 * 512 * L * ceil(MN/128) * ceil(K/(4*sf_vec_size)); 0 for invalid input.
 * No HIP call.
 */
size_t mxgemm_sf_bytes(int64_t MN, int64_t K, int64_t L, int sf_vec_size);

/*
 * mxgemm_launch_config -- the tile shape and grid the GEMM kernel would use
 * for this problem with 8-bit operands (for reporting and tests; packed FP4
 * at sf_vec_size 16 always runs 128x128 tiles).  Writes tile_m, tile_n and
 * the number of workgroups (the tile count when the tiles fit the compute
 * units; otherwise the tiles of one of the rounds a full grid would need,
 * rounded up to a multiple of 8 and capped at the compute units, so every
 * workgroup runs the same number of tiles give or take one); any output
 * pointer may be NULL.  Returns a
 * status like mxgemm_check_support.  Queries the current device's compute
 * unit count (HIP call) only when `grid` is requested.
 */
int mxgemm_launch_config(int64_t M, int64_t N, int64_t K, int64_t L, int sf_vec_size,
                         int* tile_m, int* tile_n, int64_t* grid);

/*
 * Plans ("GEMM + Amax (SM100)", sections on the class API: check_support,
 * compile, then execute per call, and its note on per-launch CPU cost).
 * mxgemm_plan_init validates sizes, formats and flags once (the checks of
 * mxgemm_check_support plus the flag rules of mxgemm_amax_ex), queries the
 * current device and fixes the tile configuration.  mxgemm_plan_execute then
 * runs mxgemm_amax_ex with those sizes and flags on the given buffers,
 * checking only null pointers, 16-byte alignment and that the current device
 * is the plan's; it does not ask HIP where each pointer lives, so the caller
 * guarantees the buffers are device memory of that device (as the pages'
 * execute takes tensors already placed for the compiled kernel).
 *
 * mxgemm_plan is plain caller-owned memory (no allocation, nothing to free);
 * a plan may be copied and used from several threads and streams.  Results
 * are identical to mxgemm_amax_ex with the same arguments.  Errors:
 * init returns mxgemm_amax_ex's validation statuses (and MXG_ERR_DEVICE
 * without a gfx950 device); execute returns MXG_ERR_NULL (also for a plan
 * never initialised), MXG_ERR_ALIGN, MXG_ERR_DEVICE (another current
 * device) or MXG_ERR_LAUNCH.
 */
typedef struct mxgemm_plan {
  uint64_t opaque[32];
} mxgemm_plan;

int mxgemm_plan_init(mxgemm_plan* plan, int64_t M, int64_t N, int64_t K, int64_t L, int sf_vec_size,
                     int a_fmt, int b_fmt, unsigned flags);
int mxgemm_plan_execute(const mxgemm_plan* plan, const void* A, const void* B, const uint8_t* SFA,
                        const uint8_t* SFB, float* C, float* Amax, void* stream);

/*
 * mxgemm_mx_quantize -- MX block quantisation of float32 data into the
 * GEMM's input form: element codes plus E8M0 block scales in the physical
 * atom layout ("GEMM + RoPE + MXFP8 Projection (SM100)", section
 * "Equations": MXFP8 quantisation with an E8M0 scale per block of 32 and
 * E4M3 data; E5M2 and blocks of 16 follow the same rule).
 *
 *   X   : (L, MN, K) float32, K contiguous (an A or B operand before
 *         quantisation).
 *   Q   : (L, MN, K) element codes, one byte each (the layout of A / B).
 *   SF  : mxgemm_sf_bytes(MN, K, L, sf_vec_size) bytes, the physical atom
 *         layout described above for SFA / SFB.  Every byte is written:
 *         padding entries (rows >= MN, K-blocks >= ceil(K/sf)) get 127.
 *   fmt : MXG_FMT_E4M3 (FMAX = 448) or MXG_FMT_E5M2 (FMAX = 57344).
 *
 * Per row and block of sf_vec_size consecutive K elements (the last block
 * may be partial): bm = max |x|; e = the smallest integer with
 * FMAX * 2^e >= bm, clamped to [-127, 127], and e = 0 when bm = 0; scale
 * byte = e + 127; code = x * 2^-e rounded to the nearest code, ties to even
 * (nothing saturates: |x * 2^-e| <= FMAX).  The pages give no formula for
 * the scale; this rule is the one the GEMM's test inputs are made with (a
 * scale of 2^ceil(log2(blockmax / FMAX))).  Results for non-finite inputs
 * are unspecified.
 *
 * Errors (before any work): MXG_ERR_SHAPE (a negative size, K >= 2^23 or
 * too many atoms), MXG_ERR_SFVEC, MXG_ERR_FMT, MXG_ERR_ALIGN (K % 16 or a
 * pointer not 16-byte aligned), MXG_ERR_NULL, MXG_ERR_DEVICE.  MN, K or
 * L == 0 queues nothing and returns MXG_OK.  Q and SF must not overlap X.
 */
int mxgemm_mx_quantize(const float* X, void* Q, uint8_t* SF, int64_t MN, int64_t K, int64_t L,
                       int sf_vec_size, int fmt, void* stream);

/*
 * mxgemm_sf_rowwise_to_atoms -- row-wise E8M0 block scales into the
 * physical atom layout that mxgemm_amax reads (for operands quantised with
 * row-wise scales: "GEMM + RoPE + MXFP8 Projection (SM100)", section
 * "Shapes", x_scale (tokens, Q_LORA/32) and w_scale (rows, Q_LORA/32)).
 *
 *   rowwise : (L, MN, ceil(K/sf)) bytes, contiguous; byte (l, row, kb) is
 *             the scale of row `row`, K elements [kb*sf, (kb+1)*sf).
 *   SF      : mxgemm_sf_bytes(MN, K, L, sf_vec_size) bytes, 16-byte aligned;
 *             every byte is written, padding entries (rows >= MN, K-blocks
 *             >= ceil(K/sf)) get 127.
 *
 * Errors (before any work): MXG_ERR_SHAPE, MXG_ERR_SFVEC, MXG_ERR_NULL,
 * MXG_ERR_ALIGN (SF), MXG_ERR_DEVICE.  MN, K or L == 0 queues nothing.
 */
int mxgemm_sf_rowwise_to_atoms(const uint8_t* rowwise, uint8_t* SF, int64_t MN, int64_t K, int64_t L,
                               int sf_vec_size, void* stream);

/*
 * mxgemm_gemm_rope_mxfp8 -- the projection of "GEMM + RoPE + MXFP8
 * Projection (SM100)" (sections "Overview", "Shapes", "Equations") in one
 * kernel: Y = A B^T as in mxgemm_amax (L = 1; A (tokens, K) and B (N, K)
 * codes, N = num_heads * head_dim, SF atoms as there), and in place of
 * storing Y, per head: RoPE on the trailing qk_rope features (the rule of
 * mxgemm_proj_rope_mxfp8 below) and E4M3 codes with E8M0 scales in both
 * block directions, exactly what mxgemm_proj_rope_mxfp8 makes of the
 * float32 Y that mxgemm_amax (with 256x256 tiles) computes for these
 * operands.  No Y and no Amax is written.
 *   cos_bf16, sin_bf16 : (tokens, qk_rope) bf16 bits.
 *   row_codes (tokens, N) bytes, row_scales (tokens, N / 32),
 *   col_codes (tokens, N), col_scales (tokens / 32, N): caller-owned outputs.
 * Requirements: K > 0 and the GEMM's rules on K; tokens % 32 == 0
 * (MXG_ERR_ALIGN); head_dim a multiple of 32, at least 128; qk_rope a
 * multiple of 16, at most 64; N % 128 == 0; no head's rotary features
 * crossing a multiple of 128 columns (else MXG_ERR_SHAPE); a_fmt, b_fmt
 * E4M3 or E5M2; sf_vec_size 16 or 32; every pointer 16-byte aligned.
 * Asynchronous on `stream`; errors before any work; tokens or num_heads == 0
 * queues nothing.
 */
int mxgemm_gemm_rope_mxfp8(const void* A, const void* B, const uint8_t* SFA, const uint8_t* SFB,
                           const uint16_t* cos_bf16, const uint16_t* sin_bf16, uint8_t* row_codes,
                           uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, int64_t tokens,
                           int64_t num_heads, int64_t head_dim, int64_t qk_rope, int64_t K, int sf_vec_size, int a_fmt,
                           int b_fmt, void* stream);

/*
 * mxgemm_projection_workspace_bytes -- bytes of workspace that
 * mxgemm_projection_mxfp8 needs: the atom-layout scales of x and w
 * (mxgemm_sf_bytes of each, the first rounded up to 256).
 */
size_t mxgemm_projection_workspace_bytes(int64_t tokens, int64_t num_heads, int64_t head_dim, int64_t K);

/*
 * mxgemm_projection_mxfp8 -- the projection page's MXFP8-input path as the
 * page passes it: x (tokens, K) and w (num_heads * head_dim, K) E4M3 codes
 * with row-wise E8M0 scales x_scale (tokens, ceil(K/32)) and w_scale
 * (num_heads * head_dim, ceil(K/32)) ("Shapes": blocks of 32 along Q_LORA).
 * The scales are rewritten into the atom layout in `workspace` (device
 * memory of at least mxgemm_projection_workspace_bytes, 256-byte aligned,
 * caller-owned, overwritten), then mxgemm_gemm_rope_mxfp8 runs with
 * sf_vec_size 32.  Rules, outputs and errors as there; a short workspace is
 * MXG_ERR_SHAPE.  Three kernels on `stream`.
 */
int mxgemm_projection_mxfp8(const void* x, const void* w, const uint8_t* x_scale, const uint8_t* w_scale,
                            const uint16_t* cos_bf16, const uint16_t* sin_bf16, uint8_t* row_codes,
                            uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, int64_t tokens,
                            int64_t num_heads, int64_t head_dim, int64_t qk_rope, int64_t K, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * mxgemm_projection_mxfp8_noalloc -- mxgemm_projection_mxfp8 for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid it): the same operation, arguments and
 * results, with the workspace taken from a fixed array inside the library
 * (MXGEMM_NOALLOC_SCRATCH_BYTES per device, reserved when the library is
 * loaded and held until the process ends) instead of a caller buffer.  It
 * calls no allocator.  A problem whose workspace
 * (mxgemm_projection_workspace_bytes) exceeds the array is rejected with
 * MXG_ERR_SCRATCH before any work.  Every call on one device shares that
 * device's array: calls that may overlap on one device (other streams,
 * other threads) race and must be serialised by the caller.  The array's
 * contents are overwritten in full by each call before they are read.
 */
#define MXGEMM_NOALLOC_SCRATCH_BYTES (8u << 20)
int mxgemm_projection_mxfp8_noalloc(const void* x, const void* w, const uint8_t* x_scale, const uint8_t* w_scale,
                                    const uint16_t* cos_bf16, const uint16_t* sin_bf16, uint8_t* row_codes,
                                    uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, int64_t tokens,
                                    int64_t num_heads, int64_t head_dim, int64_t qk_rope, int64_t K, void* stream);

/*
 * mxgemm_codes_to_kmajor -- m-major (or n-major) 8-bit element codes into the
 * k-major rows mxgemm_amax reads ("GEMM + Amax (SM100)", section
 * "Parameters": A of shape (M, K, L) may have strides (1, M, M*K), B of shape
 * (N, K, L) strides (1, N, N*K); packed FP4 operands must be k-major).
 *
 *   src : (L, K, MN) bytes, MN contiguous -- byte (mn, k, l) at
 *         mn + MN*k + MN*K*l; 16-byte aligned.
 *   dst : (L, MN, K) bytes, K contiguous -- the A or B argument of
 *         mxgemm_amax; 16-byte aligned, caller-owned, not overlapping src.
 *   MN  : M for A, N for B.
 *
 * Asynchronous on `stream`; the library allocates nothing.  Errors (before
 * any work): MXG_ERR_SHAPE, MXG_ERR_ALIGN (MN % 16 or K % 16 -- the 16-byte
 * alignment of both contiguous dimensions -- or a pointer), MXG_ERR_NULL,
 * MXG_ERR_DEVICE.  MN, K or L == 0 queues nothing and returns MXG_OK.
 */
int mxgemm_codes_to_kmajor(const void* src, void* dst, int64_t MN, int64_t K, int64_t L, void* stream);

/*
 * mxgemm_proj_rope_mxfp8 -- the projection's per-head RoPE and dual-direction
 * MXFP8 quantisation ("GEMM + RoPE + MXFP8 Projection (SM100)", sections
 * "Overview", "Shapes" and "Equations"), applied to the float32 output Y of
 * mxgemm_amax (M = tokens, N = num_heads * head_dim).
 *
 *   Y          : (tokens, num_heads * head_dim) float32, 16-byte aligned.
 *   cos_bf16,
 *   sin_bf16   : (tokens, qk_rope) bfloat16 bit patterns, 16-byte aligned.
 *   row_codes  : (tokens, num_heads, head_dim) E4M3 codes, blocks of 32 along
 *                head_dim; row_scales: (tokens, num_heads, head_dim / 32)
 *                E8M0 bytes.
 *   col_codes  : (tokens, num_heads, head_dim) E4M3 codes, blocks of 32 along
 *                tokens; col_scales: (tokens / 32, num_heads, head_dim) E8M0.
 *
 * RoPE acts on the last qk_rope features of each head, interleaved in and
 * halves out: with (a_i, b_i) = (y[2i], y[2i+1]) of that part and
 * R = qk_rope / 2, out[i] = a_i cos[i] - b_i sin[i] and
 * out[R+i] = b_i cos[R+i] + a_i sin[R+i], in float32 with each product and
 * the sum rounded on its own.  Block scale 2^e with e the smallest integer
 * giving 448 * 2^e >= the block's largest magnitude (0 for an all-zero
 * block), codes rounded to nearest, ties to even (the rule of
 * mxgemm_mx_quantize).
 *
 * Asynchronous on `stream`; all buffers caller-owned device memory, outputs
 * not overlapping the inputs.  Errors (before any work): MXG_ERR_SHAPE
 * (head_dim not a multiple of 32 or above 256, qk_rope odd or above
 * head_dim or 128, sizes too large), MXG_ERR_ALIGN (tokens % 32, or Y, the
 * code buffers, cos or sin not 16-byte aligned), MXG_ERR_NULL,
 * MXG_ERR_DEVICE.  tokens or
 * num_heads == 0 queues nothing and returns MXG_OK.
 */
int mxgemm_proj_rope_mxfp8(const float* Y, const uint16_t* cos_bf16, const uint16_t* sin_bf16, uint8_t* row_codes,
                           uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, int64_t tokens,
                           int64_t num_heads, int64_t head_dim, int64_t qk_rope, void* stream);

/* mxgemm_strerror -- static text for a status code. No HIP call. */
const char* mxgemm_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* MXGEMM_H */
