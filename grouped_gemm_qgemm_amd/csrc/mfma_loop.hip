// Compute-side yardsticks, not part of any GEMM:
//   * an MFMA issue loop: one workgroup of eight waves (two per SIMD) per CU,
//     every wave issuing nothing but MFMAs of one kind over four accumulators,
//     with operands that change from one MFMA to the next (four A and four B
//     fragments of pseudo-random finite values, rotated), so the matrix cores
//     run as busy as a GEMM can keep them and draw comparable power. Lane 0 of
//     wave 0 records the shader clock count (s_memtime) and the 100 MHz
//     reference count (s_memrealtime) around the loop, which gives the clock
//     the chip holds under that load;
//   * an empty kernel of a chosen launch shape: the duration of a launch that
//     does no work, the floor under any kernel of that shape.
#include "qgemm_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kLoopThreads = 512;
constexpr uint32_t kNever = 0x7F7FFFFFu;   // the sink is written only for this float sum (FLT_MAX)

// 32-bit mix (an xorshift-multiply finaliser): operand bits from (block, lane, index)
__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// four 32-bit words of finite values of the kind: fp16 / bf16 magnitudes below 2,
// e4m3 bytes with exponent field at most 14 (never the NaN code)
template <int KIND>
__device__ __forceinline__ u32x4_t operand(uint32_t seed) {
  constexpr uint32_t mask = KIND == 0 ? 0xBBFFBBFFu : KIND == 1 ? 0xBF7FBF7Fu : 0xF7F7F7F7u;
  u32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = mix(seed * 4u + i) & mask;
  return v;
}

// KIND 0: v_mfma_f32_32x32x16_f16, 1: v_mfma_f32_32x32x16_bf16,
// 2: v_mfma_scale_f32_16x16x128_f8f6f4 with e4m3 operands and unit scales
template <int KIND>
__global__ __launch_bounds__(kLoopThreads) void mfma_loop_kernel(int iters, unsigned long long* __restrict__ clocks,
                                                                uint32_t* __restrict__ sink) {
  const uint32_t base = (blockIdx.x * kLoopThreads + threadIdx.x) * 8u;
  u32x4_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = operand<KIND>(base + i);
    b[i] = operand<KIND>(base + 4 + i);
  }
  constexpr int ACC = KIND == 2 ? 4 : 16;
  typedef float acc_t __attribute__((ext_vector_type(ACC)));
  acc_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < ACC; ++e) acc[j][e] = 0.f;

  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4_t x = a[j], y = b[(j + r) & 3];
        if constexpr (KIND == 0) {
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, x),
                                                          __builtin_bit_cast(f16x8_t, y), acc[j], 0, 0, 0);
        } else if constexpr (KIND == 1) {
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x),
                                                           __builtin_bit_cast(bf16x8_t, y), acc[j], 0, 0, 0);
        } else {
          const u32x4_t x2 = a[(j + 1) & 3], y2 = b[(j + r + 1) & 3];
          const i32x8_t av = {(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)x2[0], (int)x2[1], (int)x2[2], (int)x2[3]};
          const i32x8_t bv = {(int)y[0], (int)y[1], (int)y[2], (int)y[3], (int)y2[0], (int)y2[1], (int)y2[2], (int)y2[3]};
          acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[j], 0, 0, 0, 127, 0, 127);
        }
      }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();

  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < ACC; ++e) s += acc[j][e];
  if (__builtin_bit_cast(uint32_t, s) == kNever) sink[0] = kNever;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

__global__ __launch_bounds__(1024) void empty_kernel() {}

}  // namespace

extern "C" {

qg_status qg_mfma_loop(int32_t kind, int32_t iters, int32_t workgroups, unsigned long long* clocks, uint32_t* sink,
                       hipStream_t stream) {
  if (!clocks || !sink) return QG_ERR_NULL;
  if (kind < 0 || kind > 2 || iters <= 0 || workgroups <= 0) return QG_ERR_INVALID_ARG;
  const dim3 grid((unsigned)workgroups), block(kLoopThreads);
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_loop_kernel<0>, grid, block, 0, stream, iters, clocks, sink); break;
    case 1: hipLaunchKernelGGL(mfma_loop_kernel<1>, grid, block, 0, stream, iters, clocks, sink); break;
    default: hipLaunchKernelGGL(mfma_loop_kernel<2>, grid, block, 0, stream, iters, clocks, sink); break;
  }
  return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

qg_status qg_empty_launch(int32_t workgroups, int32_t threads, hipStream_t stream) {
  if (workgroups <= 0 || threads <= 0 || threads > 1024) return QG_ERR_INVALID_ARG;
  hipLaunchKernelGGL(empty_kernel, dim3((unsigned)workgroups), dim3((unsigned)threads), 0, stream);
  return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

}  // extern "C"
