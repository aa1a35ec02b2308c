// Device-side building blocks shared by the gfx950 kernels: vector types,
// MFMA wrappers, 4-bit dequantization and fp8 decoding in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// v_mfma_f32_16x16x32_f16: D[16x16] += A[16x32] . B[32x16].
// Lane l supplies A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16]; it holds
// D[4*(l/16) + i][l%16] for i = 0..3. Any permutation of the 8 K slots is fine as
// long as A and B use the same one.
__device__ __forceinline__ float4_t mfma16x16x32_f16(u32x4_t a, u32x4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float4_t mfma16x16x32_bf16(u32x4_t a, u32x4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_{f16,bf16}: D[32x32] += A[32x16] . B[16x32]. Lane l
// supplies A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32]; it holds
// D[8*(i/4) + 4*(l/32) + i%4][l%32] for i = 0..15. On gfx950 this shape runs
// at twice the sustained rate of the 16x16x32 one.
__device__ __forceinline__ float16_t mfma32x32x16_f16(u32x4_t a, u32x4_t b, float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float16_t mfma32x32x16_bf16(u32x4_t a, u32x4_t b, float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Raw buffer access: a 128-bit descriptor (base, size in bytes) in SGPRs, a
// per-lane byte offset in one VGPR and a uniform byte offset in an SGPR, so a
// loop of loads that advance together costs no per-load 64-bit address math.
// Reads at or past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

__device__ __forceinline__ uint64_t buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// Locates work tile t of a routed (grouped) GEMM. Group g < num_active with
// ids[g] >= 0 and rows = a_off[g+1] - a_off[g] > 0 owns ceil(rows / bm) * tiles_n
// consecutive tiles, in group order. The calling wave scans 64 groups at a
// time (one group per lane, prefix sum by shuffles, ballot for the owner);
// every lane gets the same result: the group (-1 past the last tile) and the
// tile's index within it.
struct TileLoc {
  int g, local;
};

__device__ __forceinline__ TileLoc locate_tile(int t, const uint32_t* __restrict__ a_off,
                                               const int32_t* __restrict__ ids, int num_active, int bm,
                                               int tiles_n) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int g0 = 0; g0 < num_active; g0 += 64) {
    const int g = g0 + lane;
    int cnt = 0;
    if (g < num_active) {
      const int rows = (int)(a_off[g + 1] - a_off[g]);
      cnt = (ids[g] >= 0 && rows > 0) ? ((rows + bm - 1) / bm) * tiles_n : 0;
    }
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const unsigned long long hit = __ballot(t < base + incl);
    if (hit) {
      const int first = __ffsll((long long)hit) - 1;
      const int excl = __shfl(incl - cnt, first);
      // the same in every lane: readfirstlane lets the compiler keep it in SGPRs
      return TileLoc{__builtin_amdgcn_readfirstlane(g0 + first), __builtin_amdgcn_readfirstlane(t - base - excl)};
    }
    base += __shfl(incl, 63);
  }
  return TileLoc{-1, 0};
}

// Total work tiles of a routed GEMM (see locate_tile), by the same wave scan.
__device__ __forceinline__ int count_tiles(const uint32_t* __restrict__ a_off, const int32_t* __restrict__ ids,
                                           int num_active, int bm, int tiles_n) {
  const int lane = threadIdx.x & 63;
  int total = 0;
  for (int g0 = 0; g0 < num_active; g0 += 64) {
    const int g = g0 + lane;
    int cnt = 0;
    if (g < num_active) {
      const int rows = (int)(a_off[g + 1] - a_off[g]);
      cnt = (ids[g] >= 0 && rows > 0) ? ((rows + bm - 1) / bm) * tiles_n : 0;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) cnt += __shfl_xor(cnt, d);
    total += cnt;
  }
  return __builtin_amdgcn_readfirstlane(total);   // the same in every lane
}

// (a & m) | b. Written in C (no inline assembly): the compiler's hazard checks
// do not cover instructions hidden in inline assembly, and a VGPR write issued
// right after an MFMA that reads the same register as an operand must be
// spaced by the compiler.
// x in a VGPR, opaque to constant folding: the empty asm statement emits no
// instruction. v_and_or_b32 takes no literal operand on gfx950, so a mask the
// compiler can see as a constant turns each fused mask-and-bias into two
// instructions (v_and_b32 and v_or_b32 with literals).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t x) {
  asm("" : "=v"(x) : "0"(x));
  return x;
}

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t b) {
  return (a & m) | b;
}

// One 32-bit word of eight 4-bit codes (code i in bits 4i..4i+3) -> eight fp16
// weights (q - 8), exact, as four packed half pairs in the K-slot order
// (0,4), (1,5), (2,6), (3,7). OR-ing a code into the low mantissa bits of
// 1024.0 (0x6400) gives 1024 + q exactly; subtracting 1032 leaves q - 8.
// The mask and bias are fused (v_and_or_b32); `m` must hold 0x000F000F (in a
// VGPR) and `bias` 0x64006400.
__device__ __forceinline__ u32x4_t dequant_w4_word_fused(uint32_t w, uint32_t m, uint32_t bias) {
  const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const uint32_t p0 = and_or(w, m, bias);
  const uint32_t p1 = and_or(w >> 4, m, bias);
  const uint32_t p2 = and_or(w >> 8, m, bias);
  const uint32_t p3 = and_or(w >> 12, m, bias);
  u32x4_t r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p0) - off);
  r.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p1) - off);
  r.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p2) - off);
  r.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p3) - off);
  return r;
}

// One 32-bit word of eight 4-bit codes -> eight fp16 weights (q - 8), exact, as
// four packed half pairs in natural K order (0,1), (2,3), (4,5), (6,7): byte i of
// the word (codes 2i, 2i + 1) and byte i of the word shifted right by 4 (code
// 2i + 1 in its low nibble) are placed in the two halves by one byte permute,
// then masked into the mantissa of 1024.0 as in dequant_w4_word_fused. Two more
// instructions per word than that K-slot order, so activations can enter LDS as
// they are in memory. `m` must hold 0x000F000F (in a VGPR), `bias` 0x64006400
// (fp16) or 0x43004300 (bf16: 128 + q, no subtraction).
template <bool SUB1032>
__device__ __forceinline__ u32x4_t unpack_w4_word_natural(uint32_t w, uint32_t m, uint32_t bias) {
  const uint32_t x = w >> 4;
  const uint32_t p0 = and_or(__builtin_amdgcn_perm(x, w, 0x0C040C00u), m, bias);
  const uint32_t p1 = and_or(__builtin_amdgcn_perm(x, w, 0x0C050C01u), m, bias);
  const uint32_t p2 = and_or(__builtin_amdgcn_perm(x, w, 0x0C060C02u), m, bias);
  const uint32_t p3 = and_or(__builtin_amdgcn_perm(x, w, 0x0C070C03u), m, bias);
  if constexpr (!SUB1032) return u32x4_t{p0, p1, p2, p3};
  const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  u32x4_t r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p0) - off);
  r.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p1) - off);
  r.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p2) - off);
  r.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p3) - off);
  return r;
}

// global_load_lds, written out so that the compiler neither waits on these
// loads before unrelated LDS reads nor keeps per-lane 64-bit addresses: the
// wave's 64 lanes each fetch 16 (or 4) bytes at sbase + voff and the data
// lands at LDS byte lds + 16 * lane (4 * lane). Completion is tracked by the
// caller with explicit vmcnt waits, so the kernels that use these issue no
// other vector-memory loads in their main loops. M0 is listed as clobbered
// and the compiler warns that it does not preserve reserved registers around
// inline asm; in these kernels nothing but these loads reads M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
// the same with 4 bytes per lane, for the lanes where `on` holds
__device__ __forceinline__ void dma4_lanes(const void* sbase, uint32_t voff, uint32_t lds, bool on) {
  if (on)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
// 2 bytes per lane; lane l's value lands in the 4-byte LDS word at lds + 4 l
__device__ __forceinline__ void dma2(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ushort %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Eight consecutive fp16 values (a0..a7 in four registers) reordered to the
// K-slot order used by dequant_w4_word_fused: (a0,a4), (a1,a5), (a2,a6), (a3,a7).
__device__ __forceinline__ u32x4_t permute_k_0415(u32x4_t v) {
  u32x4_t r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return r;
}

// Packed fp16 multiply of a register pair by s. Vector lanes are always read
// into scalars first: bit-casting an element of a vector that is being
// reassigned in place (v.y = bit_cast(..., v.y) ...) is miscompiled by this
// toolchain (later lanes pick up the already updated first lane).
__device__ __forceinline__ uint32_t hmul2(uint32_t a, half2_t s) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) * s);
}

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f2h_rn(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> a bf16 pair (lo, hi), round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f2bf2_rn(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f2bf_rn(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <bool BF>
__device__ __forceinline__ float bits2f(uint32_t b) {
  return BF ? bf2f((uint16_t)b) : h2f((uint16_t)b);
}

// x * sigmoid(x) = x / (1 + e^-x); v_exp_f32 and v_rcp_f32 (about 1 ulp each).
// For x below about -88, e^-x is +inf and the result is -0.
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

}  // namespace qg
