// MFMA-tiled W4A16 GEMM for M > 16 (the prefill-shaped case of the group-
// quantized GEMM on the Modular page "multistage_gemm_q"; Parameters:
// group_size, pack_factor; its Description's multi-stage shared-memory
// pipeline becomes an LDS double buffer here).
//
// Workgroup tile BM x BN, K advanced BK = 64 at a time:
//   * A (fp16) and the packed B words of the next K tile are fetched from HBM
//     into registers while the current tile is multiplied out of LDS, then
//     written to the other LDS buffer (one barrier per K tile).
//   * A rows sit in LDS with an XOR swizzle on their 16-byte chunks so the
//     MFMA operand reads of 16 consecutive rows hit distinct banks; the eight
//     fp16 values of each chunk are stored in the K-slot order (0,4,1,5,2,6,3,7)
//     that the in-register 4-bit unpack produces for B.
//   * Each wave reads 16 bytes of packed B per lane per 32-deep K step: four
//     words = four MFMA column tiles (lane j of tile t is column 4j + t), so its
//     fp16 results for one row come out as four adjacent columns.
//   * Dequantization happens once per wave per word, in VGPRs: nibble -> fp16
//     (q - 8) exactly, then one packed multiply by the column's group scale.
//   * 16x16x32 fp16 MFMA, fp32 accumulation, fp16 round-to-nearest-even store.
//   * Workgroup ids are remapped so each XCD works on a contiguous run of tiles,
//     M-fastest, sharing B panels (and A panels) in its own L2.
#include "device_common.h"
#include "launch.h"

namespace qg {

namespace {

constexpr int BK = 64;            // K per LDS stage (two 32-deep MFMA steps)
constexpr int CHUNKS = BK / 8;    // 16-byte chunks per A row in LDS

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }
// transposed fp16 B rows: the 16 rows {4j + t} one fragment read touches get
// distinct chunk positions
__device__ __forceinline__ int swzb(int n, int chunk) { return chunk ^ ((n >> 2) & 7); }

}  // namespace

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M * WAVES_N * kWave) void w4_prefill_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ B,
    const uint16_t* __restrict__ S, int M, int N, int K, int group_size, int tiles_m, int tiles_n) {
  constexpr int NTHR = WAVES_M * WAVES_N * kWave;
  constexpr int TM = BM / WAVES_M;       // rows per wave
  constexpr int TN = BN / WAVES_N;       // columns per wave
  constexpr int MT = TM / 16;            // MFMA row tiles per wave
  constexpr int NB = TN / 64;            // 64-column blocks per wave (4 MFMA column tiles each)
  static_assert(TN % 64 == 0 && TM % 16 == 0, "wave tile");
  constexpr int A_CHUNKS = BM * CHUNKS;              // 16-byte chunks of A per stage
  constexpr int A_PER_T = A_CHUNKS / NTHR;
  static_assert(A_CHUNKS % NTHR == 0, "A chunks per thread");
  constexpr int B_CHUNKS = (BK / 8) * (BN / 4);      // 16-byte chunks of packed B per stage
  constexpr int B_PER_T = B_CHUNKS >= NTHR ? B_CHUNKS / NTHR : 1;
  static_assert(B_CHUNKS % NTHR == 0 || NTHR % B_CHUNKS == 0, "B chunks per thread");

  __shared__ __attribute__((aligned(16))) uint32_t lds_a[2][BM * BK / 2];     // fp16 pairs
  __shared__ __attribute__((aligned(16))) uint32_t lds_b[2][(BK / 8) * BN];   // packed words

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // XCD-aware tile order: block b runs on XCD b % 8; give each XCD a contiguous
  // range of the M-fastest linear tile order.
  const int tiles = tiles_m * tiles_n;
  const int per = (tiles + 7) >> 3;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= tiles) return;
  const int m0 = (lin % tiles_m) * BM;
  const int n0 = (lin / tiles_m) * BN;

  // ---- global -> register staging (addresses clamped into range) ----
  int a_row[A_PER_T], a_chunk[A_PER_T];
  const uint16_t* a_src[A_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int id = tid + i * NTHR;
    a_row[i] = id / CHUNKS;
    a_chunk[i] = id % CHUNKS;
    const int gr = min(m0 + a_row[i], M - 1);
    a_src[i] = A + (size_t)gr * K + a_chunk[i] * 8;
  }
  const bool b_loader = tid < B_CHUNKS;
  int b_kp[B_PER_T], b_c4[B_PER_T], b_col[B_PER_T];
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    const int id = (tid + i * NTHR) % B_CHUNKS;
    b_kp[i] = id / (BN / 4);
    b_c4[i] = id % (BN / 4);
    b_col[i] = min(n0 + 4 * b_c4[i], N - 4);
  }
  const int kp_total = K / 8;

  // this lane's scale columns: 4 adjacent columns per 64-column block
  int s_col[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) s_col[nb] = min(n0 + wn * TN + nb * 64 + 4 * (lane & 15), N - 4);

  u32x4_t ra[A_PER_T];
  u32x4_t rb[B_PER_T];

  auto load_stage = [&](int kt, u32x2_t (&sc)[2][NB]) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int kk = min(k0 + a_chunk[i] * 8, K - 8) - a_chunk[i] * 8;
      ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + kk);
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int kp = min(k0 / 8 + b_kp[i], kp_total - 1);
      rb[i] = *reinterpret_cast<const u32x4_t*>(B + (size_t)kp * N + b_col[i]);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int g = min(k0 + 32 * s, K - 1) / group_size;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sc[s][nb] = *reinterpret_cast<const u32x2_t*>(S + (size_t)g * N + s_col[nb]);
    }
  };

  auto store_stage = [&](int kt, int buf) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      u32x4_t v = permute_k_0415(ra[i]);
      if (k0 + a_chunk[i] * 8 >= K) v = u32x4_t{0u, 0u, 0u, 0u};  // K tail
      *reinterpret_cast<u32x4_t*>(&lds_a[buf][(a_row[i] * CHUNKS + swz(a_row[i], a_chunk[i])) * 4]) = v;
    }
    if (b_loader) {
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) *reinterpret_cast<u32x4_t*>(&lds_b[buf][b_kp[i] * BN + 4 * b_c4[i]]) = rb[i];
    }
  };

  float4_t acc[MT][NB * 4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NB * 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  u32x2_t sc_cur[2][NB], sc_nxt[2][NB];
  load_stage(0, sc_cur);
  store_stage(0, 0);
  __syncthreads();

  const int q = lane >> 4;      // K slot group within a 32-deep step
  const int r16 = lane & 15;    // row / column index within an MFMA tile

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) load_stage(kt + 1, sc_nxt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // B: 16 bytes per lane per 64-column block -> 4 column tiles
      u32x4_t bq[NB * 4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(
            &lds_b[cur][(s * 4 + q) * BN + wn * TN + nb * 64 + 4 * r16]);
        const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
        const uint32_t sp[2] = {sc_cur[s][nb].x, sc_cur[s][nb].y};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t sh = (sp[t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
          const half2_t s2 = __builtin_bit_cast(half2_t, sh | (sh << 16));
          const u32x4_t d = dequant_w4_word(words[t]);
          const uint32_t d0 = d.x, d1 = d.y, d2 = d.z, d3 = d.w;
          bq[nb * 4 + t] = u32x4_t{hmul2(d0, s2), hmul2(d1, s2), hmul2(d2, s2), hmul2(d3, s2)};
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = wm * TM + mt * 16 + r16;
        const u32x4_t av = *reinterpret_cast<const u32x4_t*>(
            &lds_a[cur][(row * CHUNKS + swz(row, s * 4 + q)) * 4]);
#pragma unroll
        for (int j = 0; j < NB * 4; ++j) acc[mt][j] = mfma16x16x32_f16(av, bq[j], acc[mt][j]);
      }
    }
    if (more) store_stage(kt + 1, cur ^ 1);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sc_cur[s][nb] = sc_nxt[s][nb];
  }

  // ---- epilogue: fp32 -> fp16 (RNE), four adjacent columns per 8-byte store ----
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + wm * TM + mt * 16 + q * 4 + i;
      if (row >= M) continue;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = n0 + wn * TN + nb * 64 + 4 * r16;
        if (col >= N) continue;
        const uint32_t lo = (uint32_t)f2h_rn(acc[mt][nb * 4 + 0][i]) | ((uint32_t)f2h_rn(acc[mt][nb * 4 + 1][i]) << 16);
        const uint32_t hi = (uint32_t)f2h_rn(acc[mt][nb * 4 + 2][i]) | ((uint32_t)f2h_rn(acc[mt][nb * 4 + 3][i]) << 16);
        *reinterpret_cast<u32x2_t*>(C + (size_t)row * N + col) = u32x2_t{lo, hi};
      }
    }
  }
}

// Second design: the workgroup dequantizes each packed word once (not once per
// wave) into an fp16 copy of the B tile in LDS, stored transposed ([n][k], k
// contiguous) so both MFMA operands are plain 16-byte LDS reads; 8 waves
// (2 per SIMD) overlap one wave's VALU work with the other's MFMAs; global
// loads run two K tiles ahead through a pair of register sets.
template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M * WAVES_N * kWave) void w4_prefill_lds_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ B,
    const uint16_t* __restrict__ S, int M, int N, int K, int group_size, int tiles_m, int tiles_n) {
  constexpr int NTHR = WAVES_M * WAVES_N * kWave;
  constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  constexpr int MT = TM / 16, NT = TN / 16;
  static_assert(TN % 64 == 0 && TM % 16 == 0, "wave tile");
  constexpr int A_PER_T = BM * CHUNKS / NTHR;               // 16-byte A chunks per thread per stage
  static_assert((BM * CHUNKS) % NTHR == 0, "A staging");
  constexpr int WORDS = (BK / 8) * BN;                      // packed words per stage
  constexpr int W_PER_T = WORDS / NTHR;                     // 1, 2 or 4 adjacent columns per thread
  static_assert(WORDS % NTHR == 0 && (W_PER_T == 1 || W_PER_T == 2 || W_PER_T == 4), "B staging");

  __shared__ __attribute__((aligned(16))) u32x4_t lds_a[2][BM * CHUNKS];
  __shared__ __attribute__((aligned(16))) u32x4_t lds_b[2][BN * CHUNKS];   // [n][k chunk]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int q = lane >> 4, r16 = lane & 15;

  const int tiles = tiles_m * tiles_n;
  const int per = (tiles + 7) >> 3;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= tiles) return;
  const int m0 = (lin % tiles_m) * BM;
  const int n0 = (lin / tiles_m) * BN;

  // A staging map
  int a_row[A_PER_T], a_ch[A_PER_T];
  uint32_t a_off[A_PER_T];
  const uint16_t* a_base = A;
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int id = tid + i * NTHR;
    a_row[i] = id / CHUNKS;
    a_ch[i] = id % CHUNKS;
    a_off[i] = (uint32_t)(min(m0 + a_row[i], M - 1) * K + a_ch[i] * 8);
  }
  // B staging map: packed row kp of the stage, W_PER_T adjacent columns
  constexpr int CPT = BN / W_PER_T;   // threads per packed row
  const int b_kp = tid / CPT;
  const int b_c = (tid % CPT) * W_PER_T;
  const int b_col = min(n0 + b_c, N - W_PER_T);
  const int kp_total = K / 8;

  struct Regs {
    u32x4_t a[A_PER_T];
    uint32_t w[W_PER_T];
    uint32_t s[(W_PER_T + 1) / 2];
  };
  auto load_stage = [&](int kt, Regs& r) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int kk = min(k0 + a_ch[i] * 8, K - 8) - a_ch[i] * 8;
      r.a[i] = *reinterpret_cast<const u32x4_t*>(a_base + (a_off[i] + kk));
    }
    const int kp = min(k0 / 8 + b_kp, kp_total - 1);
    const uint32_t* bp = B + (size_t)kp * N + b_col;
    if constexpr (W_PER_T == 4) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(bp);
      r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else if constexpr (W_PER_T == 2) {
      const u32x2_t v = *reinterpret_cast<const u32x2_t*>(bp);
      r.w[0] = v.x; r.w[1] = v.y;
    } else {
      r.w[0] = *bp;
    }
    const int g = (kp * 8) / group_size;
    const uint16_t* sp = S + (size_t)g * N + b_col;
    if constexpr (W_PER_T == 4) {
      const u32x2_t v = *reinterpret_cast<const u32x2_t*>(sp);
      r.s[0] = v.x; r.s[1] = v.y;
    } else if constexpr (W_PER_T == 2) {
      r.s[0] = *reinterpret_cast<const uint32_t*>(sp);
    } else {
      r.s[0] = *sp;
    }
  };
  auto store_stage = [&](int kt, int buf, const Regs& r) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      u32x4_t v = permute_k_0415(r.a[i]);
      if (k0 + a_ch[i] * 8 >= K) v = u32x4_t{0u, 0u, 0u, 0u};   // K tail
      lds_a[buf][a_row[i] * CHUNKS + swz(a_row[i], a_ch[i])] = v;
    }
    const uint32_t vmask = in_vgpr(0x000F000Fu);
    const uint32_t bias = __builtin_amdgcn_readfirstlane(0x64006400u);
#pragma unroll
    for (int j = 0; j < W_PER_T; ++j) {
      const uint32_t sh = (r.s[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      const half2_t s2 = __builtin_bit_cast(half2_t, sh | (sh << 16));
      const u32x4_t d = dequant_w4_word_fused(r.w[j], vmask, bias);
      const uint32_t d0 = d.x, d1 = d.y, d2 = d.z, d3 = d.w;
      const int n = b_c + j;
      lds_b[buf][n * CHUNKS + swzb(n, b_kp)] = u32x4_t{hmul2(d0, s2), hmul2(d1, s2), hmul2(d2, s2), hmul2(d3, s2)};
    }
  };

  float4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4_t bf[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        // column tile t of the wave: lane j holds column 4j + (t & 3) of 64-column block t / 4
        const int n = wn * TN + (t >> 2) * 64 + 4 * r16 + (t & 3);
        bf[t] = lds_b[buf][n * CHUNKS + swzb(n, s * 4 + q)];
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = wm * TM + mt * 16 + r16;
        const u32x4_t av = lds_a[buf][row * CHUNKS + swz(row, s * 4 + q)];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[mt][t] = mfma16x16x32_f16(av, bf[t], acc[mt][t]);
      }
    }
  };

  const int nk = (K + BK - 1) / BK;
  Regs r0, r1;
  load_stage(0, r0);
  if (nk > 1) load_stage(1, r1);
  store_stage(0, 0, r0);
  __syncthreads();
  if (nk > 2) load_stage(2, r0);
  // iteration kt: compute stage kt; stage kt+1 (in the other register set) goes
  // to LDS; the freed set fetches stage kt+3. Unrolled by two so set indices are static.
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    compute(0);
    store_stage(kt + 1, 1, r1);
    __syncthreads();
    if (kt + 3 < nk) load_stage(kt + 3, r1);
    if (kt + 2 < nk) {
      compute(1);
      store_stage(kt + 2, 0, r0);
      __syncthreads();
      if (kt + 4 < nk) load_stage(kt + 4, r0);
    } else {
      compute(1);
      kt += 2;
      break;
    }
  }
  if (kt < nk) compute(kt & 1);

  // epilogue: four adjacent columns per 8-byte store
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + wm * TM + mt * 16 + q * 4 + i;
      if (row >= M) continue;
#pragma unroll
      for (int nb = 0; nb < NT / 4; ++nb) {
        const int col = n0 + wn * TN + nb * 64 + 4 * r16;
        if (col >= N) continue;
        const uint32_t lo = (uint32_t)f2h_rn(acc[mt][nb * 4 + 0][i]) | ((uint32_t)f2h_rn(acc[mt][nb * 4 + 1][i]) << 16);
        const uint32_t hi = (uint32_t)f2h_rn(acc[mt][nb * 4 + 2][i]) | ((uint32_t)f2h_rn(acc[mt][nb * 4 + 3][i]) << 16);
        *reinterpret_cast<u32x2_t*>(C + (size_t)row * N + col) = u32x2_t{lo, hi};
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_lds_tile(const W4Args& p, hipStream_t stream) {
  const int tm = (int)((p.M + BM - 1) / BM), tn = (int)((p.N + BN - 1) / BN);
  const int grid = ((tm * tn + 7) / 8) * 8;
  hipLaunchKernelGGL((w4_prefill_lds_kernel<BM, BN, WM, WN>), dim3(grid), dim3(WM * WN * kWave), 0, stream,
                     p.C, p.A, p.B, p.S, (int)p.M, (int)p.N, (int)p.K, p.group_size, tm, tn);
  return hipGetLastError();
}

// Third design (the default for large N): per-wave dequantization as in the
// first kernel, but sized so the unpack work is amortised over eight MFMA row
// tiles (wave tile 128 x 64, 2 x 2 waves, 256 x 128 workgroup tile), and lean
// enough (<= 256 registers, 72 KiB LDS) for two workgroups per CU, so one
// workgroup's VALU unpack overlaps the other's MFMAs. Unpack uses the fused
// mask/bias form; scale pairs are built with one byte permute; the K tail is
// handled only in the last stage; addresses are 32-bit offsets from
// wave-uniform bases.
template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M * WAVES_N * kWave, 2) void w4_prefill_v3_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ B,
    const uint16_t* __restrict__ S, int M, int N, int K, int group_size, int tiles_m, int tiles_n) {
  constexpr int NTHR = WAVES_M * WAVES_N * kWave;
  constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  constexpr int MT = TM / 16, NB = TN / 64;
  static_assert(TN % 64 == 0 && TM % 16 == 0, "wave tile");
  constexpr int A_PER_T = BM * CHUNKS / NTHR;
  static_assert((BM * CHUNKS) % NTHR == 0, "A staging");
  constexpr int B_CHUNKS = (BK / 8) * (BN / 4);
  constexpr int B_PER_T = B_CHUNKS / NTHR;   // 16-byte packed chunks per thread
  static_assert(B_CHUNKS % NTHR == 0, "B staging");

  __shared__ __attribute__((aligned(16))) u32x4_t lds_a[2][BM * CHUNKS];
  __shared__ __attribute__((aligned(16))) u32x4_t lds_b[2][(BK / 8) * BN / 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int q = lane >> 4, r16 = lane & 15;

  const int tiles = tiles_m * tiles_n;
  const int per = (tiles + 7) >> 3;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= tiles) return;
  const int m0 = (lin % tiles_m) * BM;
  const int n0 = (lin / tiles_m) * BN;

  // A staging: chunk id -> (row, chunk); 32-bit element offsets
  uint32_t a_off[A_PER_T];
  int a_lds[A_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int id = tid + i * NTHR;
    const int row = id / CHUNKS, ch = id % CHUNKS;
    a_off[i] = (uint32_t)(min(m0 + row, M - 1) * K + ch * 8);
    a_lds[i] = row * CHUNKS + swz(row, ch);
  }
  const int a_ch0 = tid % CHUNKS;   // the chunk index is the same for all of a thread's A chunks
  // B staging: 16-byte chunks (4 words, 4 adjacent columns of one packed row)
  uint32_t b_off[B_PER_T];
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    const int id = tid + i * NTHR;
    const int b_kp = id / (BN / 4), b_c4 = id % (BN / 4);
    b_off[i] = (uint32_t)(b_kp * N + min(n0 + 4 * b_c4, N - 4));
  }
  const int kp_total = K / 8;
  // this lane's 4 output columns per 64-column block (scale columns)
  uint32_t s_off[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) s_off[nb] = (uint32_t)min(n0 + wn * TN + nb * 64 + 4 * r16, N - 4);

  u32x4_t ra[A_PER_T];
  u32x4_t rb[B_PER_T];
  u32x2_t sc_nxt[2][NB], sc_cur[2][NB];
  auto load_stage = [&](int kt) {
    const int k0 = kt * BK;
    if (k0 + BK <= K) {
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(A + k0 + a_off[i]);
      const uint32_t* bbase = B + (size_t)(k0 / 8) * N;
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(bbase + b_off[i]);
    } else {
      // partial last stage (K % 64 == 32): per-chunk clamped addresses; A chunks
      // past K are zeroed when stored, so the clamped B rows never contribute
      const int k = min(k0 + a_ch0 * 8, K - 8) - a_ch0 * 8;
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(A + k + a_off[i]);
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) {
        const int b_kp = (tid + i * NTHR) / (BN / 4);
        const int kp = min(k0 / 8 + b_kp, kp_total - 1);
        rb[i] = *reinterpret_cast<const u32x4_t*>(B + (size_t)(kp - b_kp) * N + b_off[i]);
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint16_t* sbase = S + (size_t)(min(k0 + 32 * s, K - 1) / group_size) * N;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sc_nxt[s][nb] = *reinterpret_cast<const u32x2_t*>(sbase + s_off[nb]);
    }
  };
  auto store_stage = [&](int kt, int buf) {
    const int k0 = kt * BK;
    if (k0 + BK <= K) {
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) lds_a[buf][a_lds[i]] = permute_k_0415(ra[i]);
    } else {
      // partial last stage: chunks past K enter as zeros
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) {
        const bool past = k0 + a_ch0 * 8 >= K;
        lds_a[buf][a_lds[i]] = past ? u32x4_t{0u, 0u, 0u, 0u} : permute_k_0415(ra[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) lds_b[buf][tid + i * NTHR] = rb[i];
  };

  float4_t acc[MT][NB * 4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NB * 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t vmask = in_vgpr(0x000F000Fu);
  const uint32_t bias = __builtin_amdgcn_readfirstlane(0x64006400u);
  const int nk = (K + BK - 1) / BK;
  load_stage(0);
  store_stage(0, 0);
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sc_cur[s][nb] = sc_nxt[s][nb];
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) load_stage(kt + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4_t bq[NB * 4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        // packed row s*4+q of the stage, this lane's 4 adjacent columns
        const u32x4_t wv = lds_b[cur][(s * 4 + q) * (BN / 4) + (wn * TN + nb * 64) / 4 + r16];
        const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
        const uint32_t sp[2] = {sc_cur[s][nb].x, sc_cur[s][nb].y};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          // (s_t, s_t) from the packed scales with one byte permute
          const uint32_t pair = __builtin_amdgcn_perm(sp[t >> 1], sp[t >> 1], (t & 1) ? 0x03020302u : 0x01000100u);
          const half2_t s2 = __builtin_bit_cast(half2_t, pair);
          const u32x4_t d = dequant_w4_word_fused(w4[t], vmask, bias);
          const uint32_t d0 = d.x, d1 = d.y, d2 = d.z, d3 = d.w;
          bq[nb * 4 + t] = u32x4_t{hmul2(d0, s2), hmul2(d1, s2), hmul2(d2, s2), hmul2(d3, s2)};
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = wm * TM + mt * 16 + r16;
        const u32x4_t av = lds_a[cur][row * CHUNKS + swz(row, s * 4 + q)];
#pragma unroll
        for (int j = 0; j < NB * 4; ++j) acc[mt][j] = mfma16x16x32_f16(av, bq[j], acc[mt][j]);
      }
    }
    if (more) store_stage(kt + 1, cur ^ 1);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sc_cur[s][nb] = sc_nxt[s][nb];
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + wm * TM + mt * 16 + q * 4 + i;
      if (row >= M) continue;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = n0 + wn * TN + nb * 64 + 4 * r16;
        if (col >= N) continue;
        const uint32_t lo = (uint32_t)f2h_rn(acc[mt][nb * 4 + 0][i]) | ((uint32_t)f2h_rn(acc[mt][nb * 4 + 1][i]) << 16);
        const uint32_t hi = (uint32_t)f2h_rn(acc[mt][nb * 4 + 2][i]) | ((uint32_t)f2h_rn(acc[mt][nb * 4 + 3][i]) << 16);
        *reinterpret_cast<u32x2_t*>(C + (size_t)row * N + col) = u32x2_t{lo, hi};
      }
    }
  }
}

// Fourth design: the third design's staging with 32x32x16 MFMA tiles, which
// gfx950 runs at twice the rate of 16x16x32. A wave tile is TM x 64: TM / 32
// row tiles by two column tiles of 32, where column tile t holds the columns
// 2j + t (lane j of the tile), so one 8-byte read of packed B per lane per
// 16-deep K step yields both tiles' words and the results of a row come out as
// two adjacent columns. Per 16-deep step a wave unpacks two words per lane and
// issues 2 * TM / 32 MFMAs. Global loads run PD stages ahead of the multiply
// (PD register sets); a stage's loads are written to LDS at the end of the
// stage before it is multiplied, so with PD = 2 they have two stages to land.
// With KG = 2 the workgroup holds two groups of WAVES_M x WAVES_N waves that
// take the even and the odd K stages (each with its own LDS buffers) and sum
// their accumulators through LDS at the end: the same tile and the same unpack
// work per wave, twice the waves per SIMD to cover each other's waits (for
// shapes with about one tile per CU).
// LDS of one fourth-design tile: per K group, two stages of A chunks and of
// packed B (no B when each wave loads its own B words, BD).
template <int BM, int BN, int KG, bool BD = false>
struct W4TileLds {
  u32x4_t a[KG][2][BM * CHUNKS];
  u32x4_t b[KG][2][BD ? 1 : (BK / 8) * BN / 4];
};

// One BM x BN output tile of the fourth design: rows m0 .. m0+BM-1 (those < M)
// and columns n0 .. n0+BN-1 (those < N) of C = A . dequant(B, S).
// BF: activations, scales and output are bf16 (weights (q - 8) * s rounded to
// bf16 through fp32, bf16 MFMAs); otherwise fp16.
// NK: B stored [N, K/8] and scales [N, K/group_size]. The stage's B tile is
// then read as each column's eight words (two 16-byte loads per column) and
// written into the same [8][BN] LDS tile word by word, so the MFMA loop is
// unchanged; the lane's two scales are two 2-byte loads.
// BD: B does not pass through LDS. Each lane loads the packed words its MFMAs
// take (two adjacent columns of one packed row per 16-deep step: 8 bytes, 256
// contiguous bytes per half-wave) one stage ahead, like the scales. This pays
// when a wave's B columns are its own (WAVES_M == 1, as in the grouped tiles).
template <int BM, int BN, int WAVES_M, int WAVES_N, int PD, int KG, bool BF = false, bool NK = false,
          bool BD = false>
__device__ __forceinline__ void w4_mfma_tile(uint16_t* __restrict__ C, const uint16_t* __restrict__ A,
                                             const uint32_t* __restrict__ B, const uint16_t* __restrict__ S,
                                             int M, int N, int K, int group_size, int m0, int n0,
                                             W4TileLds<BM, BN, KG, BD>& lds, const Epilogue& ep) {
  constexpr int NTHR = WAVES_M * WAVES_N * kWave;   // threads of one K group
  constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  constexpr int MT = TM / 32;
  static_assert(TN == 64 && TM % 32 == 0, "wave tile");
  static_assert(PD >= 1 && PD <= 4, "prefetch distance");
  static_assert(KG == 1 || (KG == 2 && PD == 1 && MT % 2 == 0), "K groups");
  static_assert(!BD || (KG == 1 && !NK), "direct B: one K group, [K/8, N] layout");
  constexpr int NBD = BD ? BK / 16 : 1;      // direct B words per lane and stage
  constexpr int A_PER_T = BM * CHUNKS / NTHR;
  static_assert((BM * CHUNKS) % NTHR == 0, "A staging");
  constexpr int B_CHUNKS = (BK / 8) * (BN / 4);
  constexpr int B_PER_T = B_CHUNKS / NTHR;   // 16-byte packed chunks per thread
  static_assert(B_CHUNKS % NTHR == 0, "B staging");

  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = wave_all / (WAVES_M * WAVES_N);        // K group
  const int wave = wave_all % (WAVES_M * WAVES_N);      // wave within the group
  const int tid = threadIdx.x % NTHR;                  // thread within the group
  auto& lds_a = lds.a[kg];
  auto& lds_b = lds.b[kg];
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int h = lane >> 5, c32 = lane & 31;

  // Staging through raw buffer loads: descriptors over the tile's A rows, over
  // B from column n0 on and over the scales; per-lane byte offsets, the stage's
  // K offset is uniform (an SGPR). Reads past a descriptor's end return zeros,
  // which is what the packed rows past K of a partial last stage need.
  const int rows = min(BM, M - m0);
  const __amdgpu_buffer_rsrc_t a_src = buffer_rsrc(A + (size_t)m0 * K, (uint32_t)rows * K * 2);
  const __amdgpu_buffer_rsrc_t b_src =
      NK ? buffer_rsrc(B + (size_t)n0 * (K / 8), (uint32_t)((size_t)(N - n0) * (K / 8) * 4))
         : buffer_rsrc(B + n0, (uint32_t)((size_t)(K / 8) * N - n0) * 4);
  const __amdgpu_buffer_rsrc_t s_src = buffer_rsrc(S, (uint32_t)((size_t)(K / group_size) * N * 2));
  const int gshift = __builtin_ctz(group_size);
  uint32_t a_voff[A_PER_T];
  int a_lds[A_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int id = tid + i * NTHR;
    const int row = id / CHUNKS, ch = id % CHUNKS;
    a_voff[i] = (uint32_t)(min(row, rows - 1) * K + ch * 8) * 2;
    a_lds[i] = row * CHUNKS + swz(row, ch);
  }
  const int a_ch0 = tid % CHUNKS;   // the chunk index is the same for all of a thread's A chunks
  // B staging: 16-byte chunks (4 words, 4 adjacent columns of one packed row)
  uint32_t b_voff[B_PER_T];
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    const int id = tid + i * NTHR;
    if constexpr (NK) {   // column id % BN, words 4 (id / BN) .. + 3 of its stage
      const int half = id / BN, c = id % BN;
      b_voff[i] = (uint32_t)(min(c, N - n0 - 1) * (K / 8) + 4 * half) * 4;
    } else {
      const int b_kp = id / (BN / 4), b_c4 = id % (BN / 4);
      b_voff[i] = (uint32_t)(b_kp * N + min(n0 + 4 * b_c4, N - 4) - n0) * 4;
    }
  }
  // this lane's two output columns (scale columns)
  const uint32_t s_voff = (uint32_t)min(n0 + wn * TN + 2 * c32, N - 2) * 2;
  // direct B: packed row h of each 16-deep step, the same two columns (from n0)
  const uint32_t bd_voff = (uint32_t)(h * N + min(wn * TN + 2 * c32, N - n0 - 2)) * 4;

  // one stage of prefetched operands: A chunks, packed B chunks, the lane's scale pairs
  struct Regs {
    u32x4_t a[A_PER_T];
    u32x4_t b[BD ? 1 : B_PER_T];
    uint64_t bd[NBD];
    uint32_t sc[2];
  };
  // what the MFMA loop takes from a stage's registers: scale pairs, direct B words
  struct Cur {
    uint32_t sc[2];
    uint64_t bd[NBD];
  };
  auto cur_of = [](const Regs& r) {
    Cur c;
    c.sc[0] = r.sc[0];
    c.sc[1] = r.sc[1];
#pragma unroll
    for (int j = 0; j < NBD; ++j) c.bd[j] = BD ? r.bd[j] : 0ull;
    return c;
  };
  auto load_stage = [&](int kt, Regs& r) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) r.a[i] = buffer_load16(a_src, a_voff[i], (uint32_t)k0 * 2);
    if constexpr (BD) {
#pragma unroll
      for (int j = 0; j < NBD; ++j) r.bd[j] = buffer_load8(b_src, bd_voff, (uint32_t)(k0 / 8 + 2 * j) * N * 4);
    } else {
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i)
        r.b[i] = buffer_load16(b_src, b_voff[i], NK ? (uint32_t)(k0 / 8) * 4 : (uint32_t)(k0 / 8) * N * 4);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int g = min(k0 + 32 * s, K - 1) >> gshift;
      if constexpr (NK) {
        const int col0 = (int)(s_voff / 2);
        const uint16_t* sp = S + (size_t)col0 * (K >> gshift) + g;
        r.sc[s] = (uint32_t)sp[0] | ((uint32_t)sp[K >> gshift] << 16);
      } else {
        r.sc[s] = buffer_load4(s_src, s_voff, (uint32_t)g * N * 2);
      }
    }
    // partial last stage (K % 64 == 32): A chunks past K must enter as zeros.
    // The outer test is uniform, so full stages branch past the per-lane selects.
    if (__builtin_expect(k0 + BK > K, 0)) {
      if (k0 + a_ch0 * 8 >= K) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) r.a[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_stage = [&](int kt, int buf, const Regs& r) {
    (void)kt;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) lds_a[buf][a_lds[i]] = permute_k_0415(r.a[i]);
#pragma unroll
    for (int i = 0; i < (BD ? 0 : B_PER_T); ++i) {
      if constexpr (NK) {
        const int id = tid + i * NTHR, half = id / BN, c = id % BN;
        uint32_t* wb = reinterpret_cast<uint32_t*>(lds_b[buf]);
        wb[(4 * half + 0) * BN + c] = r.b[i].x;
        wb[(4 * half + 1) * BN + c] = r.b[i].y;
        wb[(4 * half + 2) * BN + c] = r.b[i].z;
        wb[(4 * half + 3) * BN + c] = r.b[i].w;
      } else {
        lds_b[buf][tid + i * NTHR] = r.b[i];
      }
    }
  };

  float16_t acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][t][e] = 0.f;

  const uint32_t vmask = in_vgpr(0x000F000Fu);
  const uint32_t bias = __builtin_amdgcn_readfirstlane(0x64006400u);
  // one stage out of LDS buffer `buf` with the stage's scale pairs (and direct B words)
  auto compute = [&](int buf, const Cur& cur) {
    const uint64_t* bw = reinterpret_cast<const uint64_t*>(lds_b[buf]);
#pragma unroll
    for (int j = 0; j < BK / 16; ++j) {
      // packed row 2j + h of the stage, columns 2*c32 and 2*c32 + 1 of the wave's 64
      const uint64_t w2 = BD ? cur.bd[BD ? j : 0] : bw[(2 * j + h) * (BN / 2) + wn * (TN / 2) + c32];
      const uint32_t sp = cur.sc[j >> 1];
      u32x4_t bq[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if constexpr (BF) {
          bq[t] = dequant_w4_word_bf16((uint32_t)(w2 >> (32 * t)), bf2f((uint16_t)(t ? sp >> 16 : sp & 0xFFFFu)));
        } else {
          const uint32_t pair = __builtin_amdgcn_perm(sp, sp, t ? 0x03020302u : 0x01000100u);
          const half2_t s2 = __builtin_bit_cast(half2_t, pair);
          const u32x4_t d = dequant_w4_word_fused((uint32_t)(w2 >> (32 * t)), vmask, bias);
          const uint32_t d0 = d.x, d1 = d.y, d2 = d.z, d3 = d.w;
          bq[t] = u32x4_t{hmul2(d0, s2), hmul2(d1, s2), hmul2(d2, s2), hmul2(d3, s2)};
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = wm * TM + mt * 32 + c32;
        const u32x4_t av = lds_a[buf][row * CHUNKS + swz(row, 2 * j + h)];
        if constexpr (BF) {
          acc[mt][0] = mfma32x32x16_bf16(av, bq[0], acc[mt][0]);
          acc[mt][1] = mfma32x32x16_bf16(av, bq[1], acc[mt][1]);
        } else {
          acc[mt][0] = mfma32x32x16_f16(av, bq[0], acc[mt][0]);
          acc[mt][1] = mfma32x32x16_f16(av, bq[1], acc[mt][1]);
        }
      }
    }
  };

  const int nk = (K + BK - 1) / BK;
  if constexpr (KG == 2) {
    // group kg takes stages kg, kg + 2, ...; both groups run the same number of
    // iterations so every wave reaches every barrier
    Regs r;
    Cur cur{};
    if (kg < nk) {
      load_stage(kg, r);
      store_stage(kg, 0, r);
      cur = cur_of(r);
    }
    __syncthreads();
    const int iters = (nk + 1) / 2;
    for (int j = 0; j < iters; ++j) {
      const int kt = kg + 2 * j;
      const bool more = kt + 2 < nk;
      if (more) load_stage(kt + 2, r);
      __builtin_amdgcn_sched_barrier(0);
      if (kt < nk) compute(j & 1, cur);
      if (more) store_stage(kt + 2, (j + 1) & 1, r);
      __syncthreads();
      if (more) cur = cur_of(r);
    }
    // group 1 hands its partial sums to group 0 through the (now free) stage
    // buffers, two row tiles at a time; lane-major so the accesses are
    // conflict-free
    float* red = reinterpret_cast<float*>(&lds);
    static_assert(sizeof(W4TileLds<BM, BN, KG>) >= 64 * NTHR * sizeof(float), "reduction space");
#pragma unroll
    for (int p = 0; p < MT / 2; ++p) {
      if (kg == 1) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) red[((m * 2 + t) * 16 + i) * NTHR + tid] = acc[2 * p + m][t][i];
      }
      __syncthreads();
      if (kg == 0) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[2 * p + m][t][i] += red[((m * 2 + t) * 16 + i) * NTHR + tid];
      }
      __syncthreads();
    }
    if (kg == 1) return;
  } else if constexpr (PD == 1) {
    Regs r;
    load_stage(0, r);
    store_stage(0, 0, r);
    Cur cur = cur_of(r);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) load_stage(kt + 1, r);
      __builtin_amdgcn_sched_barrier(0);
      compute(kt & 1, cur);
      if (more) store_stage(kt + 1, (kt + 1) & 1, r);
      __syncthreads();
      cur = cur_of(r);
    }
  } else if constexpr (PD == 2) {
    // Stage kt + 1 waits in one register set while stage kt + 2 loads into the
    // other; unrolled by two so the sets are static. Set u holds stages of
    // parity u. Loads retire in issue order, so waiting for the older set never
    // waits for the newer one.
    Regs r0, r1;
    load_stage(0, r0);
    if (nk > 1) load_stage(1, r1);
    store_stage(0, 0, r0);
    Cur cur = cur_of(r0);
    __syncthreads();
    int kt = 0;
    // Loads past the last stage re-read it (their copies are never stored), so
    // every iteration issues the same loads and the compiler's in-order load
    // counting waits only for the older register set.
    for (; kt + 1 < nk; kt += 2) {
      // even stage kt: buffer 0; stage kt + 1 is in r1
      load_stage(min(kt + 2, nk - 1), r0);
      __builtin_amdgcn_sched_barrier(0);
      compute(0, cur);
      store_stage(kt + 1, 1, r1);
      __syncthreads();
      cur = cur_of(r1);
      // odd stage kt + 1: buffer 1; stage kt + 2 (if any) is in r0
      load_stage(min(kt + 3, nk - 1), r1);
      __builtin_amdgcn_sched_barrier(0);
      compute(1, cur);
      if (kt + 2 < nk) {
        store_stage(kt + 2, 0, r0);
        cur = cur_of(r0);
      }
      __syncthreads();
    }
    if (kt < nk) compute(0, cur);   // nk odd: the last stage sits in buffer 0
  } else {
    // PD register sets, unrolled by PD so each set is static: stage i + PD is
    // requested into the set that held stage i (already in LDS) while stage i is
    // multiplied, and stage i + 1, requested PD - 1 stages earlier, is stored
    // after it. Loads past the last stage re-read it and are never stored.
    Regs r[PD];
#pragma unroll
    for (int p = 0; p < PD; ++p) load_stage(min(p, nk - 1), r[p]);
    store_stage(0, 0, r[0]);
    Cur cur = cur_of(r[0]);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += PD) {
#pragma unroll
      for (int p = 0; p < PD; ++p) {
        const int i = kt + p;
        load_stage(min(i + PD, nk - 1), r[p]);
        __builtin_amdgcn_sched_barrier(0);
        if (i < nk) compute(i & 1, cur);
        if (i + 1 < nk) {
          store_stage(i + 1, (i + 1) & 1, r[(p + 1) % PD]);
          cur = cur_of(r[(p + 1) % PD]);
        }
        __syncthreads();
      }
    }
  }

  // epilogue: two adjacent columns per 4-byte store (or one gated output)
  const int col = n0 + wn * TN + 2 * c32;
  if (col >= N) return;
  if (ep.flags == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = m0 + wm * TM + mt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (row < M)
          *reinterpret_cast<uint32_t*>(C + (size_t)row * N + col) =
              BF ? f2bf2_rn(acc[mt][0][i], acc[mt][1][i])
                 : (uint32_t)f2h_rn(acc[mt][0][i]) | ((uint32_t)f2h_rn(acc[mt][1][i]) << 16);
      }
    }
    return;
  }
  // Fixed epilogue. Every bias and residual value this lane needs is loaded
  // before its first store: the compiler cannot tell that C does not alias
  // them, and would otherwise wait for each load after the previous store.
  const bool gate = (ep.flags & 4) != 0;
  const int NO = gate ? N / 2 : N;                  // output width
  const int oc = gate ? col / 2 : col;              // this lane's output column
  uint32_t bias2 = 0;
  if (ep.flags & 1) bias2 = *reinterpret_cast<const uint32_t*>(ep.bias + col);
  uint32_t res[MT][16];
  if (ep.flags & 2) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = min(m0 + wm * TM + mt * 32 + 8 * (i >> 2) + 4 * h + (i & 3), M - 1);
        const uint16_t* r = ep.residual + (size_t)row * NO + oc;
        res[mt][i] = gate ? (uint32_t)*r : *reinterpret_cast<const uint32_t*>(r);
      }
    }
  }
  const float b0 = (ep.flags & 1) ? bits2f<BF>(bias2 & 0xFFFFu) : 0.f;
  const float b1 = (ep.flags & 1) ? bits2f<BF>(bias2 >> 16) : 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = m0 + wm * TM + mt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
      if (row >= M) continue;
      float y0 = acc[mt][0][i] + b0, y1 = acc[mt][1][i] + b1;
      if (gate) {
        float z = silu(y0) * y1;
        if (ep.flags & 2) z += bits2f<BF>(res[mt][i]);
        C[(size_t)row * NO + oc] = BF ? f2bf_rn(z) : f2h_rn(z);
      } else {
        if (ep.flags & 2) {
          y0 += bits2f<BF>(res[mt][i] & 0xFFFFu);
          y1 += bits2f<BF>(res[mt][i] >> 16);
        }
        *reinterpret_cast<uint32_t*>(C + (size_t)row * NO + oc) =
            BF ? f2bf2_rn(y0, y1) : (uint32_t)f2h_rn(y0) | ((uint32_t)f2h_rn(y1) << 16);
      }
    }
  }
}

// Dense fourth-design kernel: one tile per workgroup, tile order within each
// XCD's run: 0 = M fastest, 1 = N fastest, else groups of `order` row panels
// swept across N.
template <int BM, int BN, int WAVES_M, int WAVES_N, int MINB, int PD, int KG, bool BF, bool NK = false>
__global__ __launch_bounds__(WAVES_M * WAVES_N * kWave * KG, MINB) void w4_prefill_v4_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ B,
    const uint16_t* __restrict__ S, int M, int N, int K, int group_size, int tiles_m, int tiles_n, int order,
    Epilogue ep) {
  __shared__ W4TileLds<BM, BN, KG> lds;
  const int tiles = tiles_m * tiles_n;
  const int per = (tiles + 7) >> 3;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= tiles) return;
  int tm, tn;
  if (order == 0) {
    tm = lin % tiles_m;
    tn = lin / tiles_m;
  } else if (order == 1) {
    tm = lin / tiles_n;
    tn = lin % tiles_n;
  } else {
    const int span = order * tiles_n;
    const int first = (lin / span) * order;
    const int gm = min(tiles_m - first, order);
    const int r = lin % span;
    tm = first + r % gm;
    tn = r / gm;
  }
  w4_mfma_tile<BM, BN, WAVES_M, WAVES_N, PD, KG, BF, NK>(C, A, B, S, M, N, K, group_size, tm * BM, tn * BN, lds,
                                                         ep);
}

// Grouped (MoE) W4A16 GEMM on the same tiles: group g (expert ids[g] >= 0,
// rows a_off[g] .. a_off[g+1]-1) is cut into ceil(rows / BM) row chunks times
// ceil(N / BN) column tiles; tiles are numbered group by group and each XCD
// takes a contiguous run, so a group's column tiles share that XCD's L2 for its
// activation rows. Expert e's packed words and scales are b[e] ([K/8, N]) and
// s[e] ([K/group_size, N]). Rows of skipped groups are never written. The grid
// holds an upper bound on the tile count (only the device knows the group
// sizes); the real count is split evenly over the eight XCDs, at most
// ceil(count / 8) <= grid / 8 tiles each, and workgroups past their XCD's run exit.
template <int BM, int BN, int WAVES_M, int WAVES_N, int MINB, int KG, int PD, bool BD>
__global__ __launch_bounds__(WAVES_M * WAVES_N * kWave * KG, MINB) void w4_grouped_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ a_off,
    const uint32_t* __restrict__ B, const uint16_t* __restrict__ S, const int32_t* __restrict__ ids, int N, int K,
    int group_size, int num_active, int tiles_n, Epilogue ep) {
  __shared__ W4TileLds<BM, BN, KG, BD> lds;
  // The tile's coordinates are the same in every lane; readfirstlane makes that
  // visible to the compiler, so the buffer descriptors built from them stay in
  // SGPRs (otherwise every buffer load becomes a loop over distinct values).
  const int total = __builtin_amdgcn_readfirstlane(count_tiles(a_off, ids, num_active, BM, tiles_n));
  const int xcd = blockIdx.x & 7;
  const int t = (int)(((long long)total * xcd) >> 3) + (int)(blockIdx.x >> 3);
  if (t >= (int)(((long long)total * (xcd + 1)) >> 3)) return;
  const TileLoc loc = locate_tile(t, a_off, ids, num_active, BM, tiles_n);
  const int g = __builtin_amdgcn_readfirstlane(loc.g);
  if (g < 0) return;
  const int local = __builtin_amdgcn_readfirstlane(loc.local);
  const int chunk = local / tiles_n, nt = local - chunk * tiles_n;
  const int e = __builtin_amdgcn_readfirstlane(ids[g]);
  const int r_begin = __builtin_amdgcn_readfirstlane((int)a_off[g] + chunk * BM);
  const int rows = __builtin_amdgcn_readfirstlane(min(BM, (int)a_off[g + 1] - r_begin));
  const size_t wpe = (size_t)(K / 8) * N, spe = (size_t)(K / group_size) * N;   // per-expert sizes
  // the fixed epilogue sees the group's rows as a matrix of their own: C and the
  // residual from row r_begin (N / 2 wide with the gate), the expert's bias row
  const int NO = (ep.flags & EPI_SILU_GATE) ? N / 2 : N;
  Epilogue ept = ep;
  if (ep.flags & EPI_BIAS) ept.bias = ep.bias + (size_t)e * N;
  if (ep.flags & EPI_RESIDUAL) ept.residual = ep.residual + (size_t)r_begin * NO;
  w4_mfma_tile<BM, BN, WAVES_M, WAVES_N, PD, KG, false, false, BD>(C + (size_t)r_begin * NO,
                                                                   A + (size_t)r_begin * K, B + e * wpe,
                                                                   S + e * spe, rows, N, K, group_size, 0,
                                                                   nt * BN, lds, ept);
}

template <int BM, int BN, int WM, int WN, int MINB, int KG, int PD = 1, bool BD = false>
static hipError_t launch_grouped_tile(const W4GroupedArgs& p, hipStream_t stream) {
  if (p.K / 8 * p.N * 4 > 0xFFFFFFFFLL) return hipErrorNotSupported;
  const int tiles_n = (int)((p.N + BN - 1) / BN);
  // every group has at most ceil(rows / BM) <= rows / BM + 1 row chunks
  const long long bound = ((p.T + BM - 1) / BM + p.num_active) * (long long)tiles_n;
  if (bound > INT32_MAX / 2) return hipErrorNotSupported;
  const int grid = (int)((bound + 7) / 8 * 8);
  hipLaunchKernelGGL((w4_grouped_kernel<BM, BN, WM, WN, MINB, KG, PD, BD>), dim3(grid), dim3(WM * WN * kWave * KG), 0,
                     stream, p.C, p.A, p.a_offsets, p.B, p.S, p.expert_ids, (int)p.N, (int)p.K, p.group_size,
                     p.num_active, tiles_n, p.epi);
  return hipGetLastError();
}

hipError_t launch_w4_grouped(const W4GroupedArgs& p, int variant, hipStream_t stream) {
  switch (variant) {
    case 0: return launch_grouped_tile<128, 256, 1, 4, 1, 2>(p, stream);
    case 1: return launch_grouped_tile<128, 256, 1, 4, 2, 1>(p, stream);
    case 2: return launch_grouped_tile<64, 256, 1, 4, 2, 1>(p, stream);
    case 3: return launch_grouped_tile<64, 256, 1, 4, 1, 2>(p, stream);
    case 4: return launch_grouped_tile<64, 256, 1, 4, 3, 1>(p, stream);
    case 5: return launch_grouped_tile<32, 256, 1, 4, 4, 1>(p, stream);
    case 6: return launch_grouped_tile<64, 128, 1, 2, 4, 1>(p, stream);
    // two stages of prefetch in registers
    case 7: return launch_grouped_tile<64, 256, 1, 4, 2, 1, 2>(p, stream);
    case 8: return launch_grouped_tile<64, 256, 1, 4, 3, 1, 2>(p, stream);
    case 9: return launch_grouped_tile<32, 256, 1, 4, 4, 1, 2>(p, stream);
    case 10: return launch_grouped_tile<64, 128, 1, 2, 4, 1, 2>(p, stream);
    case 11: return launch_grouped_tile<128, 256, 1, 4, 2, 1, 2>(p, stream);
    // three or four stages of prefetch in registers
    case 12: return launch_grouped_tile<64, 256, 1, 4, 3, 1, 3>(p, stream);
    case 13: return launch_grouped_tile<64, 256, 1, 4, 2, 1, 3>(p, stream);
    case 14: return launch_grouped_tile<64, 256, 1, 4, 2, 1, 4>(p, stream);
    case 15: return launch_grouped_tile<32, 256, 1, 4, 4, 1, 3>(p, stream);
    // B words loaded straight into each wave's registers (no LDS for B)
    case 16: return launch_grouped_tile<64, 256, 1, 4, 3, 1, 2, true>(p, stream);
    case 17: return launch_grouped_tile<64, 256, 1, 4, 3, 1, 1, true>(p, stream);
    case 18: return launch_grouped_tile<64, 256, 1, 4, 2, 1, 3, true>(p, stream);
    case 19: return launch_grouped_tile<32, 256, 1, 4, 4, 1, 2, true>(p, stream);
    // taller row chunks (one per group of up to 96 or 128 rows): each weight
    // is unpacked once per group, narrower column tiles keep the tile count up
    case 20: return launch_grouped_tile<96, 128, 1, 2, 4, 1, 2, true>(p, stream);
    case 21: return launch_grouped_tile<96, 256, 1, 4, 2, 1, 2, true>(p, stream);
    case 22: return launch_grouped_tile<128, 128, 1, 2, 3, 1, 2, true>(p, stream);
    case 23: return launch_grouped_tile<64, 128, 1, 2, 2, 1, 2, true>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_v3_tile(const W4Args& p, hipStream_t stream) {
  const int tm = (int)((p.M + BM - 1) / BM), tn = (int)((p.N + BN - 1) / BN);
  const int grid = ((tm * tn + 7) / 8) * 8;
  hipLaunchKernelGGL((w4_prefill_v3_kernel<BM, BN, WM, WN>), dim3(grid), dim3(WM * WN * kWave), 0, stream,
                     p.C, p.A, p.B, p.S, (int)p.M, (int)p.N, (int)p.K, p.group_size, tm, tn);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int MINB, int PD, int KG = 1>
static hipError_t launch_v4_tile(const W4Args& p, hipStream_t stream, int order = 0) {
  // byte offsets into B and the scales are 32-bit buffer offsets
  if (p.K / 8 * p.N * 4 > 0xFFFFFFFFLL || p.K / p.group_size * p.N * 2 > 0xFFFFFFFFLL) return hipErrorNotSupported;
  const int tm = (int)((p.M + BM - 1) / BM), tn = (int)((p.N + BN - 1) / BN);
  const int grid = ((tm * tn + 7) / 8) * 8;
#define QG_V4_LAUNCH(BFV, NKV)                                                                                  \
  hipLaunchKernelGGL((w4_prefill_v4_kernel<BM, BN, WM, WN, MINB, PD, KG, BFV, NKV>), dim3(grid),              \
                     dim3(WM * WN * kWave * KG), 0, stream, p.C, p.A, p.B, p.S, (int)p.M, (int)p.N, (int)p.K,     \
                     p.group_size, tm, tn, order, p.epi)
  if (p.nk) {   // [N, K/8] weights: the default launch shapes only (15, 16)
    if constexpr (PD == 1 && BM == 128 && BN == 256 && MINB == 2 && KG == 1) {
      if (p.bf16) QG_V4_LAUNCH(true, true); else QG_V4_LAUNCH(false, true);
    } else if constexpr (PD == 1 && BM == 128 && BN == 256 && MINB == 1 && KG == 2) {
      if (p.bf16) QG_V4_LAUNCH(true, true); else QG_V4_LAUNCH(false, true);
    } else {
      return hipErrorNotSupported;
    }
  } else if (p.bf16) {
    QG_V4_LAUNCH(true, false);
  } else {
    QG_V4_LAUNCH(false, false);
  }
#undef QG_V4_LAUNCH
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_tile(const W4Args& p, hipStream_t stream) {
  const int tm = (int)((p.M + BM - 1) / BM), tn = (int)((p.N + BN - 1) / BN);
  const int tiles = tm * tn;
  const int grid = ((tiles + 7) / 8) * 8;
  hipLaunchKernelGGL((w4_prefill_kernel<BM, BN, WM, WN>), dim3(grid), dim3(WM * WN * kWave), 0, stream,
                     p.C, p.A, p.B, p.S, (int)p.M, (int)p.N, (int)p.K, p.group_size, tm, tn);
  return hipGetLastError();
}

// Variants: tile shapes (BM x BN, wave grid).
hipError_t launch_w4_prefill(const W4Args& p, int variant, hipStream_t stream) {
  if ((p.bf16 || p.epi.flags) && variant < 11) return hipErrorInvalidValue;   // bf16 and epilogues: fourth design
  switch (variant) {
    case 0: return launch_tile<256, 128, 2, 2>(p, stream);
    case 1: return launch_tile<128, 128, 2, 2>(p, stream);
    case 2: return launch_tile<128, 256, 2, 2>(p, stream);
    case 3: return launch_tile<64, 128, 1, 2>(p, stream);
    case 4: return launch_lds_tile<256, 128, 4, 2>(p, stream);
    case 5: return launch_lds_tile<128, 128, 2, 2>(p, stream);
    case 6: return launch_lds_tile<256, 128, 2, 2>(p, stream);
    case 7: return launch_lds_tile<128, 256, 2, 4>(p, stream);
    case 8: return launch_v3_tile<256, 128, 2, 2>(p, stream);
    case 9: return launch_v3_tile<128, 256, 1, 4>(p, stream);
    case 10: return launch_v3_tile<128, 128, 1, 2>(p, stream);
    // fourth design, 128 x 256 tiles; the last argument is the tile order
    case 11: return launch_v4_tile<128, 256, 1, 4, 2, 1>(p, stream, 0);
    case 12: return launch_v4_tile<128, 256, 1, 4, 2, 2>(p, stream, 8);
    case 13: return launch_v4_tile<128, 256, 1, 4, 2, 1>(p, stream, 1);
    case 14: return launch_v4_tile<128, 256, 1, 4, 2, 1>(p, stream, 4);
    case 15: return launch_v4_tile<128, 256, 1, 4, 2, 1>(p, stream, 8);
    // two K groups of four waves (128 x 64 wave tiles), one workgroup per CU
    case 16: return launch_v4_tile<128, 256, 1, 4, 1, 1, 2>(p, stream, 8);
    case 17: return launch_v4_tile<128, 256, 1, 4, 1, 1, 2>(p, stream, 0);
    // three stages in flight in registers
    case 18: return launch_v4_tile<128, 256, 1, 4, 2, 3>(p, stream, 8);
    case 19: return launch_v4_tile<128, 256, 1, 4, 1, 3>(p, stream, 8);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qg
