/*
 * mxgemm_probe.h -- measurement probes of the MI355X (gfx950) hardware under
 * the block-scaled GEMM: matrix-core rate and clock, the global->LDS operand
 * path, and HBM streaming bandwidth.  They compute nothing of the GEMM; the
 * benchmark times them (HIP events around one launch) to state the ceilings
 * the GEMM's roofline figures are read against.  All pointers are device
 * memory of the current device, owned by the caller; every call queues one
 * kernel on `stream` (NULL = null stream) and returns 0, or a negative value
 * for invalid arguments (before any work) or a failed launch (-7).
 */
#ifndef MXGEMM_PROBE_H
#define MXGEMM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mxprobe_mfma -- `workgroups` workgroups of 4 waves; each wave issues
 * `iters` rounds of 8 independent MFMAs: kind 0 v_mfma_f32_32x32x16_bf16
 * (32768 flops each), kind 1 v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 with
 * unit scales (131072 flops each).  spans: 2 * workgroups uint64, written
 * per workgroup: shader-clock cycles, then 100 MHz real-time ticks, of the
 * timed loop (so the clock the loop ran at is cycles / ticks * 100 MHz).
 */
int mxprobe_mfma(int kind, int workgroups, int iters, unsigned long long* spans, void* stream);

/*
 * mxprobe_copy_lds -- the GEMM's operand staging without the math:
 * `workgroups` workgroups of 4 waves run `steps` steps; in each, every wave
 * moves `per_step` (1..16) blocks of 1 KB (16 bytes per lane) from the
 * source region into a two-stage LDS ring with buffer_load_dwordx4 ... lds
 * (vgpr == 0) or into registers (vgpr != 0), waits for them, and meets the
 * other waves at a barrier.  Blocks walk the region (wrapping), so a region
 * of a few MB stays in L2.  row_stride == 0: a block is 1 KB of contiguous
 * bytes; otherwise 8 rows of 128 bytes, row_stride bytes apart (>= 128, a
 * multiple of 16), the shape of the GEMM's operand DMA with row_stride = K.
 * src_bytes: a multiple of 1 KB, 64 KB .. 2 GB, holding at least 64 blocks.
 * sink: one uint32 that keeps register loads live (written only by chance).
 */
int mxprobe_copy_lds(const void* src, uint64_t src_bytes, int workgroups, int steps, int per_step, int vgpr,
                     unsigned row_stride, unsigned* sink, void* stream);

/*
 * mxprobe_hbm -- write != 0: store `bytes` (a multiple of 16) of a counter
 * pattern over buf; write == 0: read them with 16-byte loads, folded into
 * one value per thread (sink, written only by chance).  Grid-strided over
 * `workgroups` workgroups of 256 threads.
 */
int mxprobe_hbm(int write, void* buf, uint64_t bytes, int workgroups, unsigned* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXGEMM_PROBE_H */
