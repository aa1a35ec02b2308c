// C ABI entry points: host-side argument checks, launch-shape choice and
// launch. Every check runs before the first HIP call, so a rejected call
// enqueues nothing and touches no output.
#include <mutex>

#include <hip/hip_runtime.h>

#include "qgemm.h"
#include "launch.h"

namespace {

constexpr int kMaxDevices = 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

qg_status check_tensor(const qg_tensor* t, int rank, qg_dtype dt) {
  if (!t) return QG_ERR_NULL;
  if (t->rank != rank) return QG_ERR_RANK;
  if (t->dtype != dt) return QG_ERR_DTYPE;
  int64_t n = 1;
  for (int i = 0; i < rank; ++i) {
    if (t->shape[i] < 0) return QG_ERR_SHAPE;
    n *= t->shape[i];
  }
  if (n > 0) {
    if (!t->data) return QG_ERR_NULL;
    if (!aligned16(t->data)) return QG_ERR_ALIGN;
  }
  return QG_OK;
}

int device_cus() {
  static int cache[kMaxDevices] = {0};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

qg_status launch_status(hipError_t e) {
  if (e == hipErrorNotSupported) return QG_ERR_UNSUPPORTED;
  return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

}  // namespace

extern "C" {

const char* qg_status_string(qg_status s) {
  switch (s) {
    case QG_OK: return "ok";
    case QG_ERR_NULL: return "a required pointer is NULL";
    case QG_ERR_RANK: return "a tensor has the wrong rank";
    case QG_ERR_DTYPE: return "a tensor has the wrong dtype";
    case QG_ERR_SHAPE: return "tensor shapes are inconsistent";
    case QG_ERR_ALIGN: return "a base pointer or row length is not 16-byte aligned";
    case QG_ERR_UNSUPPORTED: return "configuration not supported by this build";
    case QG_ERR_INVALID_ARG: return "a scalar argument is out of range";
    case QG_ERR_LAUNCH: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t qg_version(void) { return 100; }

// Epilogue operands of a product Y [M, N] (gated output [M, N / 2]): bias has
// the output type and shape [N] (E == 0) or one row per expert [E, N]; residual
// is shaped like the output.
static qg_status check_epilogue(int32_t epilogue, const qg_tensor* bias, const qg_tensor* residual, qg_dtype act,
                                int64_t E, int64_t M, int64_t N, qg::Epilogue* out) {
  qg_status st;
  const int64_t N_out = (epilogue & QG_EPI_SILU_GATE) ? N / 2 : N;
  out->flags = epilogue;
  if (epilogue & QG_EPI_BIAS) {
    if (!bias) return QG_ERR_NULL;
    const int rank = E == 0 ? 1 : 2;
    if (bias->rank != rank) return QG_ERR_RANK;
    if ((st = check_tensor(bias, rank, act)) != QG_OK) return st;
    if (E == 0 ? bias->shape[0] != N : (bias->shape[0] != E || bias->shape[1] != N)) return QG_ERR_SHAPE;
    out->bias = static_cast<const uint16_t*>(bias->data);
  }
  if (epilogue & QG_EPI_RESIDUAL) {
    if (!residual) return QG_ERR_NULL;
    if (residual->rank != 2) return QG_ERR_RANK;
    if ((st = check_tensor(residual, 2, act)) != QG_OK) return st;
    if (residual->shape[0] != M || residual->shape[1] != N_out) return QG_ERR_SHAPE;
    out->residual = static_cast<const uint16_t*>(residual->data);
  }
  return QG_OK;
}

// nk: B is [N, K/8] and the scales [N, K/group_size] (no epilogue)
static qg_status qgemm_w4_impl(const qg_tensor* c, const qg_tensor* a, const qg_tensor* b_packed,
                               const qg_tensor* scales, int32_t group_size, int32_t pack_factor,
                               int32_t epilogue, const qg_tensor* bias, const qg_tensor* residual,
                               hipStream_t stream, bool nk = false) {
  if (!c || !a || !b_packed || !scales) return QG_ERR_NULL;
  // rank-2 requirement first: the page's only stated error condition
  if (c->rank != 2 || a->rank != 2 || b_packed->rank != 2 || scales->rank != 2) return QG_ERR_RANK;
  qg_status st;
  // activations, scales and output are all fp16 or all bf16 (the page's a_type
  // and c_type parameters)
  const qg_dtype act = a->dtype == QG_BF16 ? QG_BF16 : QG_F16;
  if ((st = check_tensor(c, 2, act)) != QG_OK) return st;
  if ((st = check_tensor(a, 2, act)) != QG_OK) return st;
  if ((st = check_tensor(b_packed, 2, QG_U32)) != QG_OK) return st;
  if ((st = check_tensor(scales, 2, act)) != QG_OK) return st;
  if (pack_factor != 8) return QG_ERR_UNSUPPORTED;
  if (group_size <= 0) return QG_ERR_INVALID_ARG;
  if (epilogue & ~(QG_EPI_BIAS | QG_EPI_RESIDUAL | QG_EPI_SILU_GATE)) return QG_ERR_INVALID_ARG;
  const int64_t M = a->shape[0], K = a->shape[1], N = b_packed->shape[nk ? 0 : 1];
  const bool gate = (epilogue & QG_EPI_SILU_GATE) != 0;
  if (gate && N % 16 != 0) return QG_ERR_ALIGN;   // (gate, up) pairs, and an 8-aligned output
  const int64_t N_out = gate ? N / 2 : N;
  if (c->shape[0] != M || c->shape[1] != N_out) return QG_ERR_SHAPE;
  if (K % group_size != 0) return QG_ERR_SHAPE;
  if (b_packed->shape[nk ? 1 : 0] * pack_factor != K) return QG_ERR_SHAPE;
  if (nk ? (scales->shape[0] != N || scales->shape[1] != K / group_size)
         : (scales->shape[0] != K / group_size || scales->shape[1] != N))
    return QG_ERR_SHAPE;
  if (group_size % 32 != 0 || group_size > 256 || (group_size & (group_size - 1)) != 0)
    return QG_ERR_UNSUPPORTED;
  if (N % 8 != 0) return QG_ERR_ALIGN;
  qg::Epilogue epi;
  if ((st = check_epilogue(epilogue, bias, residual, act, 0, M, N, &epi)) != QG_OK) return st;
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return QG_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return QG_OK;
  if (K == 0) return QG_ERR_UNSUPPORTED;  // would need a zero fill of C
  qg::W4Args p{static_cast<uint16_t*>(c->data), static_cast<const uint16_t*>(a->data),
               static_cast<const uint32_t*>(b_packed->data), static_cast<const uint16_t*>(scales->data),
               M, N, K, group_size, act == QG_BF16 ? 1 : 0, epi};
  p.nk = nk ? 1 : 0;
  if (M <= 16) return launch_status(qg::launch_w4_decode(p, stream));
  // the tiled kernel addresses 128 rows of A and eight packed rows of B (from a
  // stage's first packed row) with 32-bit buffer offsets
  if (K >= (1LL << 24) || N >= (1LL << 27)) return QG_ERR_UNSUPPORTED;
  return launch_status(qg::launch_w4_prefill(p, device_cus(), stream));
}

qg_status qgemm_w4_nk(const qg_tensor* c, const qg_tensor* a, const qg_tensor* b_packed,
                      const qg_tensor* scales, int32_t group_size, int32_t pack_factor,
                      hipStream_t stream) {
  return qgemm_w4_impl(c, a, b_packed, scales, group_size, pack_factor, 0, nullptr, nullptr, stream, true);
}

qg_status qgemm_w4(const qg_tensor* c, const qg_tensor* a, const qg_tensor* b_packed,
                   const qg_tensor* scales, int32_t group_size, int32_t pack_factor,
                   hipStream_t stream) {
  return qgemm_w4_impl(c, a, b_packed, scales, group_size, pack_factor, 0, nullptr, nullptr, stream);
}

qg_status qgemm_w4_epilogue(const qg_tensor* c, const qg_tensor* a, const qg_tensor* b_packed,
                            const qg_tensor* scales, int32_t group_size, int32_t pack_factor,
                            int32_t epilogue, const qg_tensor* bias, const qg_tensor* residual,
                            hipStream_t stream) {
  return qgemm_w4_impl(c, a, b_packed, scales, group_size, pack_factor, epilogue, bias, residual, stream);
}

static qg_status grouped_gemm_impl(const qg_tensor* c, const qg_tensor* a, const qg_tensor* a_offsets,
                                   const qg_tensor* b, const qg_tensor* expert_ids,
                                   const uint32_t* expert_usage_stats_host, int32_t transpose_b,
                                   const int32_t* a_plane_splits, int32_t epilogue, const qg_tensor* bias,
                                   const qg_tensor* residual, hipStream_t stream) {
  if (!c || !a || !a_offsets || !b || !expert_ids || !expert_usage_stats_host) return QG_ERR_NULL;
  if (c->rank != 2 || a->rank != 2 || a_offsets->rank != 1 || b->rank != 3 || expert_ids->rank != 1)
    return QG_ERR_RANK;
  qg_status st;
  if ((st = check_tensor(c, 2, QG_BF16)) != QG_OK) return st;
  if ((st = check_tensor(a, 2, QG_BF16)) != QG_OK) return st;
  if ((st = check_tensor(a_offsets, 1, QG_U32)) != QG_OK) return st;
  if ((st = check_tensor(b, 3, QG_BF16)) != QG_OK) return st;
  if ((st = check_tensor(expert_ids, 1, QG_I32)) != QG_OK) return st;
  const int64_t T = c->shape[0], K = a->shape[1];
  const int64_t E = b->shape[0];
  const int64_t N = transpose_b ? b->shape[1] : b->shape[2];
  const int64_t Kb = transpose_b ? b->shape[2] : b->shape[1];
  const int64_t G = expert_ids->shape[0];
  // planes of A (fused LoRA QKV): splits (s0, s1) != (0, 0) cut the columns into
  // [0, s0), [s0, s0 + s1), [s0 + s1, N), read from three planes of T rows of A
  const int64_t s0 = a_plane_splits ? a_plane_splits[0] : 0, s1 = a_plane_splits ? a_plane_splits[1] : 0;
  const bool planes = s0 != 0 || s1 != 0;
  if (s0 < 0 || s1 < 0 || s0 + s1 > N) return QG_ERR_SHAPE;
  if (s0 % 8 != 0 || s1 % 8 != 0) return QG_ERR_ALIGN;   // 8-aligned like N; gate pairs stay in one plane
  if (a->shape[0] != (planes ? 3 * T : T)) return QG_ERR_SHAPE;
  if (epilogue & ~(QG_EPI_BIAS | QG_EPI_RESIDUAL | QG_EPI_SILU_GATE)) return QG_ERR_INVALID_ARG;
  const bool gate = (epilogue & QG_EPI_SILU_GATE) != 0;
  if (gate && N % 16 != 0) return QG_ERR_ALIGN;   // (gate, up) pairs, and an 8-aligned output
  const int64_t N_out = gate ? N / 2 : N;
  if (c->shape[1] != N_out || Kb != K) return QG_ERR_SHAPE;
  if (a_offsets->shape[0] != G + 1) return QG_ERR_SHAPE;
  const uint32_t num_active = expert_usage_stats_host[1];
  if ((int64_t)num_active > G) return QG_ERR_INVALID_ARG;
  if (K % 8 != 0 || N % 8 != 0) return QG_ERR_ALIGN;
  qg::Epilogue epi;
  if ((st = check_epilogue(epilogue, bias, residual, QG_BF16, E, T, N, &epi)) != QG_OK) return st;
  if (3 * T > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return QG_ERR_UNSUPPORTED;
  if (N * K * 2 > 0xFFFFFFFFLL) return QG_ERR_UNSUPPORTED;   // 32-bit buffer offsets within an expert
  if (num_active == 0 || T == 0 || N == 0 || E == 0) return QG_OK;
  if (K == 0) return QG_ERR_UNSUPPORTED;
  qg::GroupedArgs p{static_cast<uint16_t*>(c->data), static_cast<const uint16_t*>(a->data),
                    static_cast<const uint32_t*>(a_offsets->data), static_cast<const uint16_t*>(b->data),
                    static_cast<const int32_t*>(expert_ids->data), T, N, K, E, (int)num_active,
                    (int)expert_usage_stats_host[0], device_cus(), transpose_b ? 1 : 0, epi};
  p.planes = planes ? qg::Planes{(int)s0, (int)(s0 + s1), (int)T} : qg::Planes{(int)N, (int)N, 0};
  return launch_status(qg::launch_grouped_bf16(p, stream));
}

qg_status grouped_gemm(const qg_tensor* c, const qg_tensor* a, const qg_tensor* a_offsets,
                       const qg_tensor* b, const qg_tensor* expert_ids,
                       const uint32_t* expert_usage_stats_host, int32_t transpose_b,
                       const int32_t* a_plane_splits_host, hipStream_t stream) {
  return grouped_gemm_impl(c, a, a_offsets, b, expert_ids, expert_usage_stats_host, transpose_b,
                           a_plane_splits_host, 0, nullptr, nullptr, stream);
}

qg_status grouped_gemm_epilogue(const qg_tensor* c, const qg_tensor* a, const qg_tensor* a_offsets,
                                const qg_tensor* b, const qg_tensor* expert_ids,
                                const uint32_t* expert_usage_stats_host, int32_t transpose_b,
                                const int32_t* a_plane_splits_host, int32_t epilogue, const qg_tensor* bias,
                                const qg_tensor* residual, hipStream_t stream) {
  return grouped_gemm_impl(c, a, a_offsets, b, expert_ids, expert_usage_stats_host, transpose_b,
                           a_plane_splits_host, epilogue, bias, residual, stream);
}

static qg_status grouped_gemm_w4_impl(const qg_tensor* c, const qg_tensor* a, const qg_tensor* a_offsets,
                                      const qg_tensor* b_packed, const qg_tensor* scales,
                                      const qg_tensor* expert_ids, const uint32_t* expert_usage_stats_host,
                                      int32_t group_size, int32_t pack_factor, int32_t epilogue,
                                      const qg_tensor* bias, const qg_tensor* residual, hipStream_t stream) {
  if (!c || !a || !a_offsets || !b_packed || !scales || !expert_ids || !expert_usage_stats_host)
    return QG_ERR_NULL;
  if (c->rank != 2 || a->rank != 2 || a_offsets->rank != 1 || b_packed->rank != 3 || scales->rank != 3 ||
      expert_ids->rank != 1)
    return QG_ERR_RANK;
  qg_status st;
  // a, scales and c (and bias, residual) share one type, fp16 or bf16
  const qg_dtype act = a->dtype == QG_BF16 ? QG_BF16 : QG_F16;
  if ((st = check_tensor(c, 2, act)) != QG_OK) return st;
  if ((st = check_tensor(a, 2, act)) != QG_OK) return st;
  if ((st = check_tensor(a_offsets, 1, QG_U32)) != QG_OK) return st;
  if ((st = check_tensor(b_packed, 3, QG_U32)) != QG_OK) return st;
  if ((st = check_tensor(scales, 3, act)) != QG_OK) return st;
  if ((st = check_tensor(expert_ids, 1, QG_I32)) != QG_OK) return st;
  if (pack_factor != 8) return QG_ERR_UNSUPPORTED;
  if (group_size <= 0) return QG_ERR_INVALID_ARG;
  if (epilogue & ~(QG_EPI_BIAS | QG_EPI_RESIDUAL | QG_EPI_SILU_GATE)) return QG_ERR_INVALID_ARG;
  const int64_t T = a->shape[0], K = a->shape[1], N = b_packed->shape[2];
  const int64_t E = b_packed->shape[0], G = expert_ids->shape[0];
  const bool gate = (epilogue & QG_EPI_SILU_GATE) != 0;
  if (gate && N % 16 != 0) return QG_ERR_ALIGN;   // (gate, up) pairs, and an 8-aligned output
  if (c->shape[0] != T || c->shape[1] != (gate ? N / 2 : N)) return QG_ERR_SHAPE;
  if (K % group_size != 0) return QG_ERR_SHAPE;
  if (b_packed->shape[1] * pack_factor != K) return QG_ERR_SHAPE;
  if (scales->shape[0] != E || scales->shape[1] != K / group_size || scales->shape[2] != N) return QG_ERR_SHAPE;
  if (a_offsets->shape[0] != G + 1) return QG_ERR_SHAPE;
  if (group_size % 32 != 0 || group_size > 256 || (group_size & (group_size - 1)) != 0)
    return QG_ERR_UNSUPPORTED;
  if (N % 8 != 0) return QG_ERR_ALIGN;
  const uint32_t num_active = expert_usage_stats_host[1];
  if ((int64_t)num_active > G) return QG_ERR_INVALID_ARG;
  qg::Epilogue epi;
  if ((st = check_epilogue(epilogue, bias, residual, act, E, T, N, &epi)) != QG_OK) return st;
  if (T > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2 || E > INT32_MAX / 2) return QG_ERR_UNSUPPORTED;
  // the tiled kernel addresses a tile's rows of A and eight packed rows of an
  // expert's B with 32-bit buffer offsets
  if (K >= (1LL << 24) || N >= (1LL << 27)) return QG_ERR_UNSUPPORTED;
  if (T == 0 || N == 0 || num_active == 0) return QG_OK;
  if (K == 0) return QG_ERR_UNSUPPORTED;  // would need a zero fill of the routed rows
  qg::W4GroupedArgs p{static_cast<uint16_t*>(c->data), static_cast<const uint16_t*>(a->data),
                      static_cast<const uint32_t*>(a_offsets->data), static_cast<const uint32_t*>(b_packed->data),
                      static_cast<const uint16_t*>(scales->data), static_cast<const int32_t*>(expert_ids->data),
                      T, N, K, E, group_size, (int)num_active, epi};
  p.bf16 = act == QG_BF16 ? 1 : 0;
  return launch_status(qg::launch_w4_grouped(p, stream));
}

qg_status grouped_gemm_w4(const qg_tensor* c, const qg_tensor* a, const qg_tensor* a_offsets,
                          const qg_tensor* b_packed, const qg_tensor* scales, const qg_tensor* expert_ids,
                          const uint32_t* expert_usage_stats_host, int32_t group_size, int32_t pack_factor,
                          hipStream_t stream) {
  return grouped_gemm_w4_impl(c, a, a_offsets, b_packed, scales, expert_ids, expert_usage_stats_host, group_size,
                              pack_factor, 0, nullptr, nullptr, stream);
}

qg_status grouped_gemm_w4_epilogue(const qg_tensor* c, const qg_tensor* a, const qg_tensor* a_offsets,
                                   const qg_tensor* b_packed, const qg_tensor* scales,
                                   const qg_tensor* expert_ids, const uint32_t* expert_usage_stats_host,
                                   int32_t group_size, int32_t pack_factor, int32_t epilogue,
                                   const qg_tensor* bias, const qg_tensor* residual, hipStream_t stream) {
  return grouped_gemm_w4_impl(c, a, a_offsets, b_packed, scales, expert_ids, expert_usage_stats_host, group_size,
                              pack_factor, epilogue, bias, residual, stream);
}

// planes: 1 (keys only) or 2 (weight columns = [W_k | W_v])
static qg_status kv_proj_impl(const qg_tensor* hidden, const qg_tensor* input_row_offsets,
                              const qg_tensor* weight, const qg_tensor* input_scale,
                              const qg_tensor* weight_scale, const int32_t* scales_granularity_mnk,
                              const qg_paged_kv* kv, uint32_t layer_idx, int planes, hipStream_t stream) {
  if (!hidden || !input_row_offsets || !weight || !input_scale || !weight_scale ||
      !scales_granularity_mnk || !kv)
    return QG_ERR_NULL;
  if (hidden->rank != 2 || input_row_offsets->rank != 1 || weight->rank != 2 || input_scale->rank != 2 ||
      weight_scale->rank != 2 || kv->blocks.rank != 6)
    return QG_ERR_RANK;
  qg_status st;
  const bool hidden_fp8 = hidden->dtype == QG_FP8_E4M3;   // the page's dtype parameter: bf16 or e4m3
  if ((st = check_tensor(hidden, 2, hidden_fp8 ? QG_FP8_E4M3 : QG_BF16)) != QG_OK) return st;
  if ((st = check_tensor(input_row_offsets, 1, QG_U32)) != QG_OK) return st;
  if ((st = check_tensor(weight, 2, QG_FP8_E4M3)) != QG_OK) return st;
  if ((st = check_tensor(input_scale, 2, QG_F32)) != QG_OK) return st;
  if ((st = check_tensor(weight_scale, 2, QG_F32)) != QG_OK) return st;
  const bool fp8 = kv->blocks.dtype == QG_FP8_E4M3;   // quantized cache
  if ((st = check_tensor(&kv->blocks, 6, fp8 ? QG_FP8_E4M3 : QG_BF16)) != QG_OK) return st;
  if (scales_granularity_mnk[0] != 1 || scales_granularity_mnk[1] != 128 || scales_granularity_mnk[2] != 128)
    return QG_ERR_UNSUPPORTED;
  const int64_t T = hidden->shape[0], Kh = hidden->shape[1];
  const int64_t N = weight->shape[1];
  const int64_t B = input_row_offsets->shape[0] - 1;
  const int64_t* bs = kv->blocks.shape;
  const int64_t L = bs[0], P = bs[2], S = bs[3], Hkv = bs[4], D = bs[5];
  if (B < 0) return QG_ERR_SHAPE;
  if (weight->shape[0] != Kh) return QG_ERR_SHAPE;
  if (Kh % 128 != 0 || N % 128 != 0) return QG_ERR_SHAPE;
  if (input_scale->shape[0] != T || input_scale->shape[1] != Kh / 128) return QG_ERR_SHAPE;
  if (weight_scale->shape[0] != Kh / 128 || weight_scale->shape[1] != N / 128) return QG_ERR_SHAPE;
  if (bs[1] != 2 || Hkv * D * planes != N) return QG_ERR_SHAPE;
  if (planes > 1 && (Hkv * D) % 128 != 0) return QG_ERR_SHAPE;   // each 128-column tile in one plane
  int64_t G = 0;
  if (fp8) {
    G = kv->quantization_granularity;
    if (G != 32 && G != 64 && G != 128) return QG_ERR_UNSUPPORTED;
    if (D % G != 0) return QG_ERR_UNSUPPORTED;
    if (kv->scales.rank != 6) return QG_ERR_RANK;
    if ((st = check_tensor(&kv->scales, 6, QG_F32)) != QG_OK) return st;
    const int64_t* ss = kv->scales.shape;
    if (ss[0] != L || ss[1] != 2 || ss[2] != P || ss[3] != S || ss[4] != Hkv || ss[5] != D / G) return QG_ERR_SHAPE;
  }
  if ((int64_t)layer_idx >= L) return QG_ERR_INVALID_ARG;
  if (kv->max_pages_per_seq <= 0 && T > 0) return QG_ERR_INVALID_ARG;
  if (B > 0 && T > 0 && (!kv->cache_lengths || !kv->page_table)) return QG_ERR_NULL;
  if (T > INT32_MAX / 2 || Kh > INT32_MAX / 2 || N > INT32_MAX / 2) return QG_ERR_UNSUPPORTED;
  if (T == 0 || B == 0 || N == 0) return QG_OK;
  if (Kh == 0) return QG_ERR_UNSUPPORTED;
  qg::KProjArgs p{static_cast<const uint16_t*>(hidden->data),
                  static_cast<const uint32_t*>(input_row_offsets->data),
                  static_cast<const uint8_t*>(weight->data),
                  static_cast<const float*>(input_scale->data),
                  static_cast<const float*>(weight_scale->data),
                  kv->blocks.data,
                  kv->cache_lengths, kv->page_table,
                  T, Kh, N, B, kv->max_pages_per_seq, L, P, S, layer_idx, device_cus()};
  p.n_plane = Hkv * D;
  p.fp8 = fp8 ? 1 : 0;
  p.kv_scales = fp8 ? static_cast<float*>(kv->scales.data) : nullptr;
  p.qgran = (int)G;
  p.hidden_fp8 = hidden_fp8 ? 1 : 0;
  return launch_status(qg::launch_kproj_fp8(p, stream));
}

qg_status k_matmul_ragged_paged_scale(const qg_tensor* hidden, const qg_tensor* input_row_offsets,
                                      const qg_tensor* weight, const qg_tensor* input_scale,
                                      const qg_tensor* weight_scale,
                                      const int32_t* scales_granularity_mnk,
                                      const qg_paged_kv* kv, uint32_t layer_idx,
                                      hipStream_t stream) {
  return kv_proj_impl(hidden, input_row_offsets, weight, input_scale, weight_scale, scales_granularity_mnk, kv,
                      layer_idx, 1, stream);
}

qg_status kv_matmul_ragged_paged_scale(const qg_tensor* hidden, const qg_tensor* input_row_offsets,
                                       const qg_tensor* weight, const qg_tensor* input_scale,
                                       const qg_tensor* weight_scale,
                                       const int32_t* scales_granularity_mnk,
                                       const qg_paged_kv* kv, uint32_t layer_idx,
                                       hipStream_t stream) {
  return kv_proj_impl(hidden, input_row_offsets, weight, input_scale, weight_scale, scales_granularity_mnk, kv,
                      layer_idx, 2, stream);
}

}  // extern "C"
