/*
 * qgemm.h - C ABI of the MI355X (gfx950) dequant-in-kernel GEMM library.
 *
 * Four operations, each a GEMM whose B operand holds low-precision weights
 * that the kernel dequantizes on the fly:
 *
 *   qgemm_w4                     4-bit group-quantized weights, fp16 activations
 *                                (Modular MAX page "multistage_gemm_q")
 *   grouped_gemm                 per-expert bf16 GEMM routed by row offsets
 *                                (Modular MAX page "grouped_matmul_sm100_persistent")
 *   k_matmul_ragged_paged_scale  block-scaled fp8 weights, ragged rows, output
 *                                written into a paged KV cache (bf16 or fp8 with
 *                                scales)
 *                                (Modular MAX page "k_matmul_ragged_paged_scale")
 *   kv_matmul_ragged_paged_scale the same for keys and values at once
 *   grouped_gemm_w4              the routing of grouped_gemm over experts stored in
 *                                qgemm_w4's packed 4-bit format
 *
 * Conventions shared by every entry point
 *   - Tensor data pointers are DEVICE pointers unless a comment says "host".
 *     Every tensor is dense, row-major (last dimension contiguous), and its base
 *     address must be 16-byte aligned.
 *   - The caller allocates and owns every buffer. The library never allocates or
 *     frees device memory and keeps no pointer after the call returns.
 *   - All argument checks run on the host before anything is enqueued. On any
 *     error nothing is launched and every output is left untouched; the return
 *     value says what was wrong (qg_status_string gives a message).
 *   - Work is enqueued on `stream` and the call returns without synchronizing.
 *     Empty problems (a zero-sized M, T, N or no active group) are a successful
 *     no-op that enqueues nothing. A zero reduction depth (K = 0, or Kh = 0 for
 *     the projections), whose result would be the epilogue of an all-zero
 *     product, returns QG_ERR_UNSUPPORTED.
 *   - Outputs must not alias inputs. Calls on different streams may run
 *     concurrently; the library holds no mutable global state besides a cache of
 *     device properties.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QG_OK = 0,
  QG_ERR_NULL = 1,         /* a required pointer is NULL                          */
  QG_ERR_RANK = 2,         /* a tensor has the wrong number of dimensions         */
  QG_ERR_DTYPE = 3,        /* a tensor has the wrong element type                 */
  QG_ERR_SHAPE = 4,        /* dimensions disagree with each other                 */
  QG_ERR_ALIGN = 5,        /* base pointer or a row length breaks 16-byte alignment */
  QG_ERR_UNSUPPORTED = 6,  /* a valid configuration this build does not implement */
  QG_ERR_INVALID_ARG = 7,  /* a scalar argument is out of range                   */
  QG_ERR_LAUNCH = 8        /* the HIP runtime reported an error at launch         */
} qg_status;

typedef enum {
  QG_F16 = 0,       /* IEEE binary16                               */
  QG_BF16 = 1,      /* bfloat16                                    */
  QG_F32 = 2,       /* IEEE binary32                               */
  QG_FP8_E4M3 = 3,  /* OCP FP8 E4M3 ("fn": max 448, no infinities) */
  QG_U32 = 4,
  QG_I32 = 5
} qg_dtype;

#define QG_MAX_RANK 6

/* A dense row-major tensor: `rank` dimensions in shape[0..rank-1]. */
typedef struct {
  void* data;
  qg_dtype dtype;
  int32_t rank;
  int64_t shape[QG_MAX_RANK];
} qg_tensor;

/*
 * qgemm_w4 - C = A . dequant(B)   (W4A16 group-quantized GEMM)
 *
 * Follows "multistage_gemm_q": group_size K elements share one scale
 * (Parameters: group_size); pack_factor 4-bit codes sit in one uint32
 * (Parameters: pack_factor); tensors that are not rank-2 are an error (Raises).
 * Code layout and zero point, which the page leaves open, are fixed here:
 * word B[kp][n] holds the codes of K rows 8*kp + i (i = 0..7) in bits
 * 4i..4i+3, and code q stands for the weight (q - 8) * scales[k / group_size][n].
 *
 *   c        f16 or bf16 [M, N]              output, written entirely
 *   a        f16 or bf16 [M, K]              activations
 *   b_packed u32 [K / pack_factor, N]        packed 4-bit weight codes
 *   scales   f16 or bf16 [K / group_size, N] one scale per group per column
 *   group_size   a power of two in 32 .. 256 that divides K
 *                (QG_ERR_SHAPE when it does not divide K, QG_ERR_UNSUPPORTED
 *                for other values)
 *   pack_factor  must be 8                   (QG_ERR_UNSUPPORTED otherwise)
 *
 * a, scales and c share one type, fp16 or bf16 (the page's a_type and c_type
 * parameters; QG_ERR_DTYPE when they differ). Accumulation is fp32; the result
 * is rounded to the output type (nearest-even). N must be a multiple of 8 and K a
 * multiple of group_size (QG_ERR_ALIGN / QG_ERR_SHAPE). M <= 16 runs the
 * skinny-M (decode) kernel, larger M the MFMA-tiled (prefill) kernel. With bf16
 * both keep (q - 8) exact and scale each group's fp32 partial once; with fp16
 * the decode kernel does the same and the prefill kernel rounds each weight
 * (q - 8) * scale to fp16 before its MFMAs. For M > 16, K >= 2^24 or N >= 2^27
 * returns QG_ERR_UNSUPPORTED (32-bit offsets within a tile's rows).
 */
qg_status qgemm_w4(const qg_tensor* c, const qg_tensor* a, const qg_tensor* b_packed,
                   const qg_tensor* scales, int32_t group_size, int32_t pack_factor,
                   hipStream_t stream);

/*
 * qgemm_w4_nk - qgemm_w4 with the weights stored the other way round
 *
 * The page's configuration type carries a transpose_b flag (its signature's
 * MatmulConfig[a_type, b_type, c_type, True]); this is that layout: each output
 * column's codes and scales are contiguous.
 *
 *   b_packed  u32 [N, K / pack_factor]   word (n, kp): codes of K rows 8 kp + i in
 *                                        bits 4i .. 4i + 3
 *   scales    f16 or bf16 [N, K / group_size]
 *
 * Every other argument, type, check and result as qgemm_w4 (the same values:
 * b_packed and scales are the transposes of qgemm_w4's). M > 16 returns
 * results bit-identical to qgemm_w4 on the transposed operands.
 */
qg_status qgemm_w4_nk(const qg_tensor* c, const qg_tensor* a, const qg_tensor* b_packed,
                      const qg_tensor* scales, int32_t group_size, int32_t pack_factor,
                      hipStream_t stream);

/*
 * qgemm_w4_epilogue - qgemm_w4 with a fixed epilogue
 *
 * Stands in for the page's elementwise_lambda_fn parameter (Parameters: a
 * device function run on each output element), which a C ABI cannot carry:
 * a bitwise OR of the operations below, applied to the fp32 product Y =
 * A . dequant(B) ([M, N]) before the single rounding to the output type.
 *
 *   QG_EPI_BIAS       Y[m][n] += bias[n]                    bias [N]
 *   QG_EPI_SILU_GATE  columns come in (gate, up) pairs:     c [M, N / 2]
 *                     Z[m][j] = silu(Y[m][2j]) * Y[m][2j+1], silu(x) = x / (1 + e^-x)
 *                     (without it Z = Y, c [M, N])
 *   QG_EPI_RESIDUAL   Z[m][j] += residual[m][j]             residual shaped like c
 *
 * bias and residual have the activations' type (fp16 or bf16) and may be NULL
 * when their operation is not requested (QG_ERR_NULL otherwise). Other flag bits
 * are QG_ERR_INVALID_ARG; with QG_EPI_SILU_GATE, N must be a multiple of 16
 * (QG_ERR_ALIGN). With QG_EPI_SILU_GATE every kernel keeps the weights
 * (q - 8) * scale exact (fp32 group partials scaled once), fp16 prefill
 * included, since the gate would magnify a rounding of the weights. Everything
 * else as qgemm_w4; epilogue 0 is qgemm_w4.
 */
#define QG_EPI_BIAS 1
#define QG_EPI_RESIDUAL 2
#define QG_EPI_SILU_GATE 4
qg_status qgemm_w4_epilogue(const qg_tensor* c, const qg_tensor* a, const qg_tensor* b_packed,
                            const qg_tensor* scales, int32_t group_size, int32_t pack_factor,
                            int32_t epilogue, const qg_tensor* bias, const qg_tensor* residual,
                            hipStream_t stream);

/*
 * grouped_gemm - per-group GEMM over routed rows (MoE expert GEMM)
 *
 * Follows "grouped_matmul_sm100_persistent" (Args): a_offsets is a prefix sum of
 * the groups' row counts; expert_ids gives each group's expert, and a group
 * whose id is negative is not computed; expert_usage_stats[1] is the active
 * count; transpose_b (Parameters) says each expert matrix is stored [N, K];
 * a_plane_splits (Parameters) gives the planes of A of a fused LoRA QKV product.
 *
 *   c          bf16 [T, N]   output; for g < num_active with expert_ids[g] >= 0,
 *                            rows a_offsets[g] .. a_offsets[g+1]-1 are set to
 *                            A[rows] . B[expert_ids[g]]^T (transpose_b != 0) or
 *                            A[rows] . B[expert_ids[g]] (transpose_b == 0); all
 *                            other rows keep their prior content
 *   a          bf16 [T, K], or [3 T, K] with planes (below)
 *   a_offsets  u32  [G + 1]  non-decreasing, a_offsets[num_active] <= T
 *   b          bf16 [E, N, K] when transpose_b != 0, else [E, K, N]
 *   expert_ids i32  [G]      each < E, or negative to skip
 *   expert_usage_stats_host  HOST u32[2]: [1] = num_active (<= G) groups to
 *                            process; [0] = largest rows-per-group (a hint only)
 *   a_plane_splits_host      HOST i32[2] (s0, s1), or NULL for (0, 0). (0, 0):
 *                            no planes. Otherwise a holds three planes of T rows
 *                            (the LoRA shrink outputs of q, k, v) and output
 *                            columns [0, s0), [s0, s0 + s1), [s0 + s1, N) read
 *                            their rows from planes 0, 1, 2: row r of plane p is
 *                            a row p T + r. s0, s1 >= 0, s0 + s1 <= N
 *                            (QG_ERR_SHAPE) and multiples of 8 (QG_ERR_ALIGN).
 *
 * K and N must be multiples of 8 (QG_ERR_ALIGN). Accumulation is fp32; results are
 * rounded to bf16 (nearest-even). The device-side tables are not re-validated:
 * offsets past T, or expert ids >= E, are undefined behaviour. An expert
 * matrix of more than 2^32 - 1 bytes returns QG_ERR_UNSUPPORTED.
 */
qg_status grouped_gemm(const qg_tensor* c, const qg_tensor* a, const qg_tensor* a_offsets,
                       const qg_tensor* b, const qg_tensor* expert_ids,
                       const uint32_t* expert_usage_stats_host, int32_t transpose_b,
                       const int32_t* a_plane_splits_host, hipStream_t stream);

/*
 * grouped_gemm_epilogue - grouped_gemm with a fixed epilogue
 *
 * Stands in for the grouped page's elementwise_lambda_fn parameter (a device
 * function on the stored C fragments): the steps of qgemm_w4_epilogue applied to
 * each processed row's fp32 product before its rounding, with
 *
 *   bias      bf16 [E, N]      QG_EPI_BIAS: the row of the group's expert is added
 *   residual  bf16 [T, N_out]  QG_EPI_RESIDUAL: added last (row of the token)
 *   c         bf16 [T, N_out]  N_out = N / 2 with QG_EPI_SILU_GATE (N % 16 == 0,
 *                              else QG_ERR_ALIGN), N otherwise
 *
 * Rows of skipped or unprocessed groups keep their prior content. Everything else
 * (planes included) as grouped_gemm; epilogue 0 is grouped_gemm.
 */
qg_status grouped_gemm_epilogue(const qg_tensor* c, const qg_tensor* a, const qg_tensor* a_offsets,
                                const qg_tensor* b, const qg_tensor* expert_ids,
                                const uint32_t* expert_usage_stats_host, int32_t transpose_b,
                                const int32_t* a_plane_splits_host, int32_t epilogue,
                                const qg_tensor* bias, const qg_tensor* residual, hipStream_t stream);

/*
 * grouped_gemm_w4 - per-group W4A16 GEMM over routed rows (MoE with 4-bit experts)
 *
 * The routing of "grouped_matmul_sm100_persistent" (Args: a_offsets, expert_ids
 * with negative entries skipping the group, expert_usage_stats[1] = active count)
 * over experts stored in the format of "multistage_gemm_q" (Parameters:
 * pack_factor = 8 codes per uint32, group_size K elements per scale). Neither page
 * defines the combination; this is the plain joint reading: for g < num_active
 * with e = expert_ids[g] >= 0, rows a_offsets[g] .. a_offsets[g+1]-1 of c are set to
 * round(A[rows] . W_e) with W_e[k][n] = (q - 8) * scales[e][k / group_size][n],
 * q = code k % 8 of b_packed[e][k / 8][n] (bits 4(k%8) .. 4(k%8)+3). All other
 * rows of c keep their prior content.
 *
 *   c          f16 or bf16 [T, N]
 *   a          f16 or bf16 [T, K]
 *   a_offsets  u32 [G + 1]   non-decreasing, a_offsets[num_active] <= T
 *   b_packed   u32 [E, K / 8, N]
 *   scales     f16 or bf16 [E, K / group_size, N]
 *   expert_ids i32 [G]       each < E, or negative to skip
 *   expert_usage_stats_host  HOST u32[2]: [1] = num_active (<= G); [0] a hint only
 *   group_size multiple of 32 and a power of two, at most 256, dividing K
 *   pack_factor must be 8
 *
 * a, scales and c share one type (the W4 page's a_type and c_type; QG_ERR_DTYPE
 * when they differ). N must be a multiple of 8 (QG_ERR_ALIGN). Accumulation is
 * fp32; results are rounded to the output type (nearest-even). In both types
 * the codes enter the MFMAs exactly and each group's fp32 partial is scaled
 * once (no weight is rounded).
 * The device-side tables are not re-validated: offsets past T, or expert ids
 * >= E, are undefined behaviour.
 */
qg_status grouped_gemm_w4(const qg_tensor* c, const qg_tensor* a, const qg_tensor* a_offsets,
                          const qg_tensor* b_packed, const qg_tensor* scales, const qg_tensor* expert_ids,
                          const uint32_t* expert_usage_stats_host, int32_t group_size,
                          int32_t pack_factor, hipStream_t stream);

/*
 * grouped_gemm_w4_epilogue - grouped_gemm_w4 with the fixed epilogue of
 * grouped_gemm_epilogue (bias [E, N], residual [T, N_out], c [T, N_out], all of
 * the activation type). Everything else as grouped_gemm_w4; epilogue 0 is
 * grouped_gemm_w4.
 */
qg_status grouped_gemm_w4_epilogue(const qg_tensor* c, const qg_tensor* a, const qg_tensor* a_offsets,
                                   const qg_tensor* b_packed, const qg_tensor* scales,
                                   const qg_tensor* expert_ids, const uint32_t* expert_usage_stats_host,
                                   int32_t group_size, int32_t pack_factor, int32_t epilogue,
                                   const qg_tensor* bias, const qg_tensor* residual, hipStream_t stream);

/*
 * A paged KV cache collection (keys and values of every layer).
 *
 * The K-projection page's kv_collection parameter carries a scale type and a
 * quantization granularity (PagedKVCacheCollection[scale_dtype_,
 * quantization_granularity_]), so the cache may hold quantized values:
 *   - blocks bf16: plain values; `scales` and `quantization_granularity` are
 *     ignored (scales may be an empty descriptor).
 *   - blocks fp8 e4m3: every run of G = quantization_granularity head-dim
 *     elements of one (layer, plane, page, slot, kv head) has one f32 scale s in
 *     `scales`; the stored code q stands for q * s. A writer sets
 *     s = amax / 448 (amax: the largest |x| of the run, in fp32) and
 *     q = e4m3(x / s) rounded to nearest even (q = 0 when amax = 0); G is 32, 64
 *     or 128 and divides D.
 */
typedef struct {
  qg_tensor blocks;                /* bf16 or fp8 e4m3 [L, 2, P, S, Hkv, D]: layer, K/V plane
                                      (0 = keys), physical page, slot in page, kv head, head dim */
  const uint32_t* cache_lengths;   /* device u32 [B]: tokens already cached per sequence  */
  const uint32_t* page_table;      /* device u32 [B, max_pages_per_seq]: physical page ids */
  int64_t max_pages_per_seq;
  qg_tensor scales;                /* fp8 cache: f32 [L, 2, P, S, Hkv, D / G]               */
  int64_t quantization_granularity; /* fp8 cache: G                                          */
} qg_paged_kv;

/*
 * k_matmul_ragged_paged_scale - K = (hidden * input_scale) . (weight * weight_scale),
 * written into the key plane of layer `layer_idx` of a paged KV cache.
 *
 * Follows "k_matmul_ragged_paged_scale" (Args): hidden_state is
 * (sum(seq_lens), num_heads*head_size); input_row_offsets (batch+1) marks where
 * each sequence starts; weight is (num_heads*head_size, num_kv_heads*head_size);
 * input_scale / weight_scale multiply the input / the weight; the layer's cache is
 * chosen by layer_idx (Parameters: scales_granularity_mnk gives the scale blocks).
 *
 *   hidden            bf16 or fp8 e4m3 [T, Kh] (the page's dtype parameter; e4m3 runs
 *                     both MFMA operands in e4m3)
 *   input_row_offsets u32  [B + 1]   offs[0] = 0, non-decreasing, offs[B] = T
 *   weight            fp8 e4m3 [Kh, N], N = Hkv * D
 *   input_scale       f32  [T, Kh / 128]
 *   weight_scale      f32  [Kh / 128, N / 128]
 *   scales_granularity_mnk  HOST int32[3], must be {1, 128, 128}
 *   kv                paged cache; token j of sequence b goes to position
 *                     p = cache_lengths[b] + j: page page_table[b][p / S], slot p % S
 *   layer_idx         < L (QG_ERR_INVALID_ARG otherwise)
 *
 * Only the addressed (page, slot) rows of plane 0 of layer layer_idx are written
 * (with an fp8 cache, also their scales); every other byte of the cache is left
 * as it was, and cache_lengths is not updated. Kh and N must be multiples of 128
 * (QG_ERR_SHAPE). Accumulation is fp32; results are rounded to bf16
 * (nearest-even), or quantized as described at qg_paged_kv. Offsets, cache
 * lengths and page ids are not re-validated on the device: a position past
 * max_pages_per_seq * S or a page id >= P is undefined behaviour, as is two
 * tokens addressing one slot. An fp8 cache with a granularity other than 32, 64
 * or 128, or one that does not divide D, is QG_ERR_UNSUPPORTED; a scales tensor
 * of the wrong shape is QG_ERR_SHAPE.
 */
qg_status k_matmul_ragged_paged_scale(const qg_tensor* hidden, const qg_tensor* input_row_offsets,
                                      const qg_tensor* weight, const qg_tensor* input_scale,
                                      const qg_tensor* weight_scale,
                                      const int32_t* scales_granularity_mnk,
                                      const qg_paged_kv* kv, uint32_t layer_idx,
                                      hipStream_t stream);

/*
 * kv_matmul_ragged_paged_scale - the key and the value projections of the same
 * tokens in one call, written into planes 0 (keys) and 1 (values) of layer
 * `layer_idx`.
 *
 * The K-projection page's kv_collection holds keys and values; this is its
 * computation with the value weights appended: weight = [W_k | W_v], so
 *
 *   weight        fp8 e4m3 [Kh, 2N], N = Hkv * D: columns 0..N-1 give keys,
 *                 N..2N-1 values
 *   weight_scale  f32 [Kh / 128, 2N / 128]
 *
 * and every other argument, check and rule is as k_matmul_ragged_paged_scale's
 * (bf16 or fp8 cache).
 */
qg_status kv_matmul_ragged_paged_scale(const qg_tensor* hidden, const qg_tensor* input_row_offsets,
                                       const qg_tensor* weight, const qg_tensor* input_scale,
                                       const qg_tensor* weight_scale,
                                       const int32_t* scales_granularity_mnk,
                                       const qg_paged_kv* kv, uint32_t layer_idx,
                                       hipStream_t stream);

/* Static, never-NULL text for a status code. */
const char* qg_status_string(qg_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t qg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
