/*
 * qgemm_probe.h - measurement yardsticks
 *
 * Not part of any GEMM: the benchmark times these beside the GEMMs of qgemm.h
 * to give their bandwidth, MFMA rate and launch cost a practical ceiling on
 * this chip. The read kernels read a device buffer once with 16-byte loads and
 * write nothing (`sink`, one device u32, is written only if the XOR of all data
 * a workgroup read equals one fixed value). Conventions (device pointers, host
 * checks before any launch, asynchronous on `stream`, status codes) are those
 * of qgemm.h.
 */
#ifndef QGEMM_PROBE_H
#define QGEMM_PROBE_H

#include "qgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * qg_read_contiguous - `workgroups` workgroups each stream one contiguous chunk
 * of the `bytes`-byte buffer at `src` (ceil(bytes / 16 / workgroups) 16-byte
 * chunks each; the last one may be short).
 *   src 16-byte aligned and bytes a multiple of 16 (QG_ERR_ALIGN);
 *   workgroups > 0 (QG_ERR_INVALID_ARG); bytes == 0 is a no-op.
 */
qg_status qg_read_contiguous(const void* src, uint64_t bytes, int32_t workgroups, uint32_t* sink,
                             hipStream_t stream);

/*
 * qg_read_strips - the buffer is `rows` rows of `row_bytes` bytes; workgroup s
 * reads bytes [s * strip_bytes, (s + 1) * strip_bytes) of every row, rows in
 * order (row_bytes / strip_bytes workgroups). This is the access pattern of a
 * kernel that gives each workgroup a column strip of a [K/8, N] packed weight
 * matrix and all of K. With a strip count that is a multiple of eight, each
 * of the eight XCDs reads a contiguous run of strips (as qgemm_w4's decode
 * kernel does).
 *   src 16-byte aligned, row_bytes and strip_bytes multiples of 16
 *   (QG_ERR_ALIGN); strip_bytes divides row_bytes (QG_ERR_SHAPE).
 */
qg_status qg_read_strips(const void* src, int64_t rows, int64_t row_bytes, int32_t strip_bytes, uint32_t* sink,
                         hipStream_t stream);

/*
 * qg_mfma_loop - an MFMA issue loop: `workgroups` workgroups of 512 threads
 * (eight waves; two per SIMD when there is one workgroup per CU), every wave
 * issuing `iters` rounds of eight MFMAs over four accumulators and nothing
 * else, with operands that change from one MFMA to the next (pseudo-random
 * finite values). kind 0: v_mfma_f32_32x32x16_f16, 1: v_mfma_f32_32x32x16_bf16
 * (32768 FLOPs each), 2: v_mfma_scale_f32_16x16x128_f8f6f4 on e4m3 operands
 * with unit scales (65536 FLOPs). FLOPs per launch = workgroups * 8 * iters *
 * 8 * (FLOPs per MFMA).
 *   clocks  DEVICE u64[2 * workgroups], written: for workgroup w, [2w] = shader
 *           clock cycles (s_memtime) and [2w + 1] = 100 MHz reference ticks
 *           (s_memrealtime) counted by wave 0 across its loop, so the clock
 *           held under the load is 100 MHz * [2w] / [2w + 1].
 *   sink    DEVICE u32, written only if the accumulators sum to FLT_MAX.
 *   QG_ERR_NULL for a NULL pointer; QG_ERR_INVALID_ARG for kind outside 0..2,
 *   iters <= 0 or workgroups <= 0.
 */
qg_status qg_mfma_loop(int32_t kind, int32_t iters, int32_t workgroups, unsigned long long* clocks, uint32_t* sink,
                       hipStream_t stream);

/*
 * qg_empty_launch - launch a kernel that does nothing with `workgroups`
 * workgroups of `threads` threads: its duration is the floor under any kernel
 * of that launch shape.
 *   QG_ERR_INVALID_ARG for workgroups <= 0 or threads outside 1..1024.
 */
qg_status qg_empty_launch(int32_t workgroups, int32_t threads, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif  // QGEMM_PROBE_H
