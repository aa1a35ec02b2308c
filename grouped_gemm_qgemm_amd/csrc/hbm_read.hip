// Read-only HBM streaming kernels: yardsticks for the memory-bound GEMMs, not
// part of any GEMM. They read a buffer once with 16-byte loads, issuing every
// load of a thread before using any of them, and store nothing unless the XOR
// of everything a workgroup read equals a fixed value (which keeps the loads
// from being removed).
//   * contiguous: each workgroup streams one contiguous chunk of the buffer;
//   * strips: the buffer is `rows` rows of `row_bytes`, and each workgroup
//     reads one `strip_bytes`-wide column strip of every row, which is how a
//     kernel that gives each workgroup a column strip and all of K must read a
//     [K/8, N] packed weight matrix. When the strip count is a multiple of
//     eight, each XCD takes a contiguous run of strips (workgroup b reads strip
//     (b % 8) * strips / 8 + b / 8), as the decode GEMM does, so neighbouring
//     strips that share a cache line are read through the same L2.
#include "qgemm_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;                              // loads in flight per thread per round
constexpr uint32_t kNever = 0x9E3779B9u;                // the sink is written only on this XOR

__global__ __launch_bounds__(kThreads) void read_contiguous_kernel(const u32x4_t* __restrict__ src,
                                                                  uint64_t chunks, uint64_t per_wg,
                                                                  uint32_t* __restrict__ sink) {
  const uint64_t begin = (uint64_t)blockIdx.x * per_wg;
  const uint64_t end = begin + per_wg < chunks ? begin + per_wg : chunks;
  uint32_t acc = 0;
  for (uint64_t i0 = begin + threadIdx.x; i0 < end; i0 += (uint64_t)kThreads * kUnroll) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t i = i0 + (uint64_t)u * kThreads;
      v[u] = i < end ? src[i] : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == kNever) sink[0] = acc;
}

// one workgroup per strip; threads take (row, 16-byte chunk) pairs in row order;
// xcd_run > 0: strips per XCD (workgroup b takes strip (b % 8) * xcd_run + b / 8)
__global__ __launch_bounds__(kThreads) void read_strips_kernel(const unsigned char* __restrict__ src, int64_t rows,
                                                              int64_t row_bytes, int32_t strip_chunks, int32_t xcd_run,
                                                              uint32_t* __restrict__ sink) {
  const int64_t strip = xcd_run > 0 ? (int64_t)(blockIdx.x & 7) * xcd_run + (blockIdx.x >> 3) : (int64_t)blockIdx.x;
  const int64_t col0 = strip * strip_chunks * 16;
  const int64_t total = rows * strip_chunks;
  uint32_t acc = 0;
  for (int64_t i0 = threadIdx.x; i0 < total; i0 += (int64_t)kThreads * kUnroll) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * kThreads;
      const int64_t r = i / strip_chunks, c = i % strip_chunks;
      v[u] = i < total ? *reinterpret_cast<const u32x4_t*>(src + r * row_bytes + col0 + c * 16)
                       : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == kNever) sink[0] = acc;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

qg_status qg_read_contiguous(const void* src, uint64_t bytes, int32_t workgroups, uint32_t* sink,
                             hipStream_t stream) {
  if (!sink || (bytes && !src)) return QG_ERR_NULL;
  if (!aligned16(src) || bytes % 16 != 0) return QG_ERR_ALIGN;
  if (workgroups <= 0) return QG_ERR_INVALID_ARG;
  if (bytes == 0) return QG_OK;
  const uint64_t chunks = bytes / 16;
  const uint64_t per_wg = (chunks + workgroups - 1) / workgroups;
  hipLaunchKernelGGL(read_contiguous_kernel, dim3(workgroups), dim3(kThreads), 0, stream,
                     static_cast<const u32x4_t*>(src), chunks, per_wg, sink);
  return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

qg_status qg_read_strips(const void* src, int64_t rows, int64_t row_bytes, int32_t strip_bytes, uint32_t* sink,
                         hipStream_t stream) {
  if (!sink || (rows && row_bytes && !src)) return QG_ERR_NULL;
  if (rows < 0 || row_bytes < 0 || strip_bytes <= 0) return QG_ERR_INVALID_ARG;
  if (!aligned16(src) || row_bytes % 16 != 0 || strip_bytes % 16 != 0) return QG_ERR_ALIGN;
  if (row_bytes % strip_bytes != 0) return QG_ERR_SHAPE;
  if (rows == 0 || row_bytes == 0) return QG_OK;
  const int64_t strips = row_bytes / strip_bytes;
  if (strips > INT32_MAX) return QG_ERR_UNSUPPORTED;
  const int32_t xcd_run = strips % 8 == 0 ? (int32_t)(strips / 8) : 0;
  hipLaunchKernelGGL(read_strips_kernel, dim3((unsigned)strips), dim3(kThreads), 0, stream,
                     static_cast<const unsigned char*>(src), rows, row_bytes, strip_bytes / 16, xcd_run, sink);
  return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

}  // extern "C"
