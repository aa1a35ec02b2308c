// Internal launcher interface between the C ABI layer (capi.cpp) and the
// kernels. Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// Fixed epilogue of the GEMMs, applied in fp32 before the output rounding.
// EPI_BIAS: y += bias[n] (the grouped GEMMs: the row of the group's expert,
// bias [E, N]); EPI_SILU_GATE: columns come in (gate, up) pairs and
// z[m][j] = silu(y[m][2j]) * y[m][2j+1] (output N / 2 wide); EPI_RESIDUAL:
// z += residual[m][j] (residual shaped like the output). Bias and residual have
// the output type.
enum { EPI_BIAS = 1, EPI_RESIDUAL = 2, EPI_SILU_GATE = 4 };
struct Epilogue {
  const uint16_t* bias = nullptr;      // [N]
  const uint16_t* residual = nullptr;  // [M, N_out]
  int flags = 0;
};

struct W4Args {
  uint16_t* C;          // f16 or bf16 [M, N]
  const uint16_t* A;    // f16 or bf16 [M, K]
  const uint32_t* B;    // u32 [K/8, N]
  const uint16_t* S;    // f16 or bf16 [K/group_size, N]
  int64_t M, N, K;
  int group_size;
  int bf16;             // A, S and C are bf16
  Epilogue epi;       // C is [M, N / 2] with EPI_SILU_GATE
  int nk = 0;         // B is [N, K/8] and S is [N, K/group_size] (no epilogue)
};

struct W4GroupedArgs {
  uint16_t* C;                // f16 or bf16 [T, N]
  const uint16_t* A;          // f16 or bf16 [T, K]
  const uint32_t* a_offsets;  // [G+1]
  const uint32_t* B;          // u32 [E, K/8, N]
  const uint16_t* S;          // f16 or bf16 [E, K/group_size, N]
  const int32_t* expert_ids;  // [G]
  int64_t T, N, K, E;
  int group_size;
  int num_active;
  Epilogue epi;               // C is [T, N / 2] with EPI_SILU_GATE; bias [E, N]
  int bf16 = 0;               // A, S, C (and bias, residual) are bf16
};

// Planes of A for the grouped GEMM (fused LoRA QKV): output columns [0, pb1),
// [pb1, pb2) and [pb2, N) read their activation rows from planes 0, 1 and 2 of
// A, plane p starting at row p * plane_rows. Without planes pb1 = pb2 = N.
struct Planes {
  int pb1, pb2;
  int plane_rows;
};

struct GroupedArgs {
  uint16_t* C;              // bf16 [T, N]
  const uint16_t* A;        // bf16 [T, K]
  const uint32_t* a_offsets;  // [G+1]
  const uint16_t* B;        // bf16 [E, N, K] (transpose_b) or [E, K, N]
  const int32_t* expert_ids;  // [G]
  int64_t T, N, K, E;
  int num_active;
  int max_rows_hint;
  int num_cus;
  int transpose_b;
  Epilogue epi;             // C is [T, N / 2] with EPI_SILU_GATE; bias [E, N]
  Planes planes;
};

struct KProjArgs {
  const uint16_t* hidden;        // bf16 [T, Kh]
  const uint32_t* row_offsets;   // [B+1]
  const uint8_t* weight;         // e4m3 [Kh, N]
  const float* input_scale;      // [T, Kh/128]
  const float* weight_scale;     // [Kh/128, N/128]
  void* blocks;                  // bf16 or e4m3 [L, 2, P, S, Hkv, D]
  const uint32_t* cache_lengths; // [B]
  const uint32_t* page_table;    // [B, max_pages]
  int64_t T, Kh, N, batch, max_pages;
  int64_t num_layers, num_pages, page_size;
  uint32_t layer_idx;
  int num_cus;
  int64_t n_plane = 0;           // columns per cache plane (Hkv * D); N / n_plane planes from plane 0
  int fp8 = 0;                   // e4m3 cache with f32 scales
  float* kv_scales = nullptr;    // fp8: [L, 2, P, S, Hkv, D / qgran]
  int qgran = 0;                 // fp8: head-dim elements per scale (32, 64, 128)
  int hidden_fp8 = 0;            // hidden is e4m3 [T, Kh] (then `hidden` points at bytes)
};

// Decode-shaped W4A16 (M <= 16).
hipError_t launch_w4_decode(const W4Args& p, hipStream_t stream);

// Prefill-shaped W4A16 (M > 16); num_cus picks the launch shape.
hipError_t launch_w4_prefill(const W4Args& p, int num_cus, hipStream_t stream);

hipError_t launch_grouped_bf16(const GroupedArgs& p, hipStream_t stream);

// Grouped W4A16 (int4 experts, fp16 or bf16 activations).
hipError_t launch_w4_grouped(const W4GroupedArgs& p, hipStream_t stream);

hipError_t launch_kproj_fp8(const KProjArgs& p, hipStream_t stream);

}  // namespace qg
