/*
 * qgemm_probe.h - read-only HBM streaming kernels (measurement yardsticks)
 *
 * Not part of any GEMM: the benchmark times these beside the memory-bound
 * GEMMs of qgemm.h to give their bandwidth a practical ceiling on this chip.
 * Each reads a device buffer once with 16-byte loads and writes nothing
 * (`sink`, one device u32, is written only if the XOR of all data a workgroup
 * read equals one fixed value). Conventions (device pointers, host checks
 * before any launch, asynchronous on `stream`, status codes) are those of
 * qgemm.h.
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

#ifdef __cplusplus
}
#endif

#endif  // QGEMM_PROBE_H
