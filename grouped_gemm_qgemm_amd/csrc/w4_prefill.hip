// MFMA-tiled W4A16 GEMM for M > 16 (the prefill-shaped case of the group-
// quantized GEMM on the Modular page "multistage_gemm_q"; Parameters:
// group_size, pack_factor; its Description's multi-stage shared-memory
// pipeline becomes an LDS double buffer here), and the grouped (MoE) form of
// the same GEMM over the routing of the page "grouped_matmul_sm100_persistent"
// (Args: a_offsets, expert_ids, expert_usage_stats).
//
// One tile body (w4_mfma_tile) serves both kernels: a BM x BN output tile, K
// advanced BK = 64 at a time, A and the packed B words of the next stage
// fetched with raw buffer loads into registers while the current stage is
// multiplied out of LDS, 32x32x16 MFMAs with fp32 accumulation, and the
// 4-bit codes unpacked in VGPRs. Its comment below gives the details. When K
// is a multiple of 64 (whole stages), both kernels use a direct-to-LDS form of
// the tile (w4_tile_dma): every operand of a stage goes from global memory
// straight into LDS, three stages deep. Dense fp16 calls without the SiLU gate
// round each weight (q - 8) * scale to fp16; every other form (bf16, gated
// fp16, the grouped kernel in both types) keeps the codes exact and scales fp32
// group partials.
#include "device_common.h"
#include "launch.h"

#include <type_traits>
namespace qg {

namespace {

constexpr int BK = 64;            // K per LDS stage (two 32-deep MFMA steps)
constexpr int CHUNKS = BK / 8;    // 16-byte chunks per A row in LDS

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// The 32x32x16 MFMA of the operand type: bf16 (BF) or fp16.
template <bool BF>
__device__ __forceinline__ float16_t mfma32x32x16_t(u32x4_t a, u32x4_t b, float16_t c) {
  if constexpr (BF) return mfma32x32x16_bf16(a, b, c);
  else return mfma32x32x16_f16(a, b, c);
}

}  // namespace

// LDS of one tile: per K group, two stages of A chunks and of packed B (no B
// when each wave loads its own B words, BD).
template <int BM, int BN, int KG, bool BD = false>
struct W4TileLds {
  u32x4_t a[KG][2][BM * CHUNKS];
  u32x4_t b[KG][2][BD ? 1 : (BK / 8) * BN / 4];
};

// Store of a wave's TM x 64 tile (rows r0 .., columns c0 + 2 c32, + 1 per lane
// half h) from the 32x32 MFMA accumulators, with the fixed epilogue: two
// adjacent columns per 4-byte store (or one gated output).
template <int MT, bool BF>
__device__ __forceinline__ void w4_tile_store(const float16_t (&acc)[MT][2], uint16_t* __restrict__ C, int M, int N,
                                              int r0, int c0, int h, int c32, const Epilogue& ep) {
  const int col = c0 + 2 * c32;
  if (col >= N) return;
  if (ep.flags == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = r0 + mt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
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
        const int row = min(r0 + mt * 32 + 8 * (i >> 2) + 4 * h + (i & 3), M - 1);
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
      const int row = r0 + mt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
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

// One BM x BN output tile: rows m0 .. m0+BM-1 (those < M) and columns
// n0 .. n0+BN-1 (those < N) of C = A . dequant(B, S).
//
// A wave tile is TM x 64: TM / 32 row tiles by two column tiles of 32, where
// column tile t holds the columns 2j + t (lane j of the tile), so one 8-byte
// read of packed B per lane per 16-deep K step yields both tiles' words and
// the results of a row come out as two adjacent columns.
//   * Staging: A, the packed B words and the lane's scale pairs of stage
//     kt + PD are fetched with raw buffer loads (descriptors in SGPRs, per-lane
//     byte offsets) while stage kt is multiplied; a stage is written to LDS
//     right before it is needed. The B and scale descriptors are rebuilt at
//     each stage's first packed row, so a packed B of any size is addressed
//     with 32-bit offsets. Reads past a descriptor's end return zeros.
//   * A rows sit in LDS in memory order with an XOR swizzle on their 16-byte
//     chunks; the weights are unpacked in natural K order
//     (unpack_w4_word_natural), as in the direct-to-LDS tile, so every path
//     feeds the MFMAs the same operands slot for slot.
//   * fp16: each word unpacks to (q - 8) exactly (code OR-ed into the mantissa
//     of 1024.0, minus 1032), then one packed multiply by the column's group
//     scale rounds each weight to fp16 before the MFMA.
//   * bf16 (BF): the weights stay exact. A code enters the bf16 MFMA as
//     128 + q (0x4300 | q per half), one more MFMA per row tile against a
//     constant -136 operand adds -136 * (sum of the row's activations), and the
//     fp32 partial of each quantization group is scaled once by the group's
//     scale when the group ends (deferred scaling).
//   * exact fp16 (XH, for gated outputs): the bf16 form's tiles and group
//     partials with the exact fp16 codes q - 8 and no correction MFMA.
//   * KG = 2: two groups of WAVES_M x WAVES_N waves take the even and the odd
//     K stages (each with its own LDS buffers) and sum their accumulators
//     through LDS at the end (for shapes with about one tile per CU).
//   * NK: B stored [N, K/8] and scales [N, K/group_size]. The stage's B tile
//     is read as each column's eight words (two 16-byte loads per column) and
//     written into the same [8][BN] LDS tile word by word, so the MFMA loop is
//     unchanged; the lane's two scales are two 2-byte loads.
//   * BD: B does not pass through LDS. Each lane loads the packed words its
//     MFMAs take with the stage; this pays when a wave's B columns are its own
//     (WAVES_M == 1). [K/8, N]: 8 bytes (two columns) per packed row, 256
//     contiguous bytes per half-wave. [N, K/8]: one 16-byte load per column
//     (the lane's four words of the stage). On the fp16 path lane half h then
//     takes K rows 32h + 8j .. + 7 at 16-deep step j (A fragments read to
//     match), so a lane's words of a column are contiguous; the bf16 path keeps
//     rows 16j + 8h .. + 7, which keeps every step inside one quantization
//     group for the group partials.
template <int BM, int BN, int WAVES_M, int WAVES_N, int PD, int KG, bool BF = false, bool NK = false,
          bool BD = false, bool XH = false>
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
  static_assert(!BD || (KG == 1 && !(NK && BF)), "direct B: one K group");
  constexpr bool GP = BF || XH;   // exact codes and group partials (bf16, or fp16 with XH)
  static_assert(!GP || KG == 1, "group partials: a quantization group's stages stay in one K group");
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
  // (the host limits K so that BM rows of A stay below 4 GiB)
  const __amdgpu_buffer_rsrc_t a_src = buffer_rsrc(A + (size_t)m0 * K, (uint32_t)rows * K * 2);
  const int gshift = __builtin_ctz(group_size);
  // a descriptor's size: bytes from its base to the end of the tensor, capped
  // at 2^32 - 1 (a capped descriptor lies wholly inside the tensor)
  auto cap32 = [](size_t bytes) { return (uint32_t)(bytes > 0xFFFFFFFFull ? 0xFFFFFFFFull : bytes); };
  // [N, K/8]: one descriptor from column n0 on (the stage's K offset goes in soffset)
  const __amdgpu_buffer_rsrc_t bnk_src =
      buffer_rsrc(B + (size_t)n0 * (K / 8), cap32((size_t)(N - n0) * (K / 8) * 4));
  // [K/8, N]: packed row k0 / 8 from column n0 on, and the scales from row k0 >> gshift
  auto b_stage = [&](int k0) {
    const size_t at = (size_t)(k0 / 8) * N + n0;
    return buffer_rsrc(B + at, cap32(((size_t)(K / 8) * N - at) * 4));
  };
  auto s_stage = [&](int g0) {
    const size_t at = (size_t)g0 * N;
    return buffer_rsrc(S + at, cap32(((size_t)(K >> gshift) * N - at) * 2));
  };
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
      b_voff[i] = (uint32_t)(b_kp * N + min(n0 + 4 * b_c4, N - 4) - n0) * 4;   // from the stage's base
    }
  }
  // this lane's two output columns (scale columns)
  const uint32_t s_voff = (uint32_t)min(n0 + wn * TN + 2 * c32, N - 2) * 2;
  // direct B: packed rows of the stage, the same two columns (from n0). The fp16
  // path takes rows 4h .. 4h + 3 in the lane half h (K rows 32h + 8j .. + 7 at
  // step j); the bf16 path, whose group partials need each step inside one
  // quantization group, takes row 2j + h at step j.
  constexpr bool KH = BD && !GP;   // the lane half's K rows are contiguous in the stage
  const uint32_t bd_voff = (uint32_t)((KH ? 4 * h : h) * N + min(wn * TN + 2 * c32, N - n0 - 2)) * 4;
  // direct B, [N, K/8]: words 4h .. 4h + 3 of the stage of the lane's two columns
  const int bdn_col = min(wn * TN + 2 * c32, N - n0 - 2);
  const uint32_t bdn_voff0 = (uint32_t)(bdn_col * (K / 8) + 4 * h) * 4;
  const uint32_t bdn_voff1 = (uint32_t)((bdn_col + 1) * (K / 8) + 4 * h) * 4;

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
    const __amdgpu_buffer_rsrc_t b_src = NK ? bnk_src : b_stage(k0);
    if constexpr (BD && NK) {
      // one 16-byte load per column: the lane's four words of the stage
      const u32x4_t w0 = buffer_load16(b_src, bdn_voff0, (uint32_t)(k0 / 8) * 4);
      const u32x4_t w1 = buffer_load16(b_src, bdn_voff1, (uint32_t)(k0 / 8) * 4);
      r.bd[0] = (uint64_t)w0.x | ((uint64_t)w1.x << 32);
      r.bd[1] = (uint64_t)w0.y | ((uint64_t)w1.y << 32);
      r.bd[2] = (uint64_t)w0.z | ((uint64_t)w1.z << 32);
      r.bd[3] = (uint64_t)w0.w | ((uint64_t)w1.w << 32);
    } else if constexpr (BD) {
#pragma unroll
      for (int j = 0; j < NBD; ++j) r.bd[j] = buffer_load8(b_src, bd_voff, (uint32_t)(KH ? j : 2 * j) * N * 4);
    } else {
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) r.b[i] = buffer_load16(b_src, b_voff[i], NK ? (uint32_t)(k0 / 8) * 4 : 0u);
    }
    const int g0 = min(k0, K - 1) >> gshift;
    const __amdgpu_buffer_rsrc_t s_src = s_stage(NK ? 0 : g0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int g = min(k0 + 32 * s, K - 1) >> gshift;
      if constexpr (NK) {
        const int col0 = (int)(s_voff / 2);
        const uint16_t* sp = S + (size_t)col0 * (K >> gshift) + g;
        r.sc[s] = (uint32_t)sp[0] | ((uint32_t)sp[K >> gshift] << 16);
      } else {
        r.sc[s] = buffer_load4(s_src, s_voff, (uint32_t)(g - g0) * N * 2);
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
    for (int i = 0; i < A_PER_T; ++i) lds_a[buf][a_lds[i]] = r.a[i];
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
  const uint32_t bias = __builtin_amdgcn_readfirstlane(BF ? 0x43004300u : 0x64006400u);
  // bf16: per row tile, the group partials of both column tiles and the
  // row-sum correction -136 * sum(a) (the same for every column)
  constexpr int MP = GP ? MT : 1;
  float16_t part[MP][2], corr[MP];
  auto clear_partials = [&]() {
#pragma unroll
    for (int i = 0; i < MP; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) part[i][0][e] = part[i][1][e] = corr[i][e] = 0.f;
  };
  if constexpr (GP) clear_partials();
  const uint32_t m136 = 0xC308C308u;   // bf16 pair (-136, -136)
  // one stage (K offset k0) out of LDS buffer `buf` with the stage's scale pairs
  // (and direct B words)
  auto compute = [&](int buf, const Cur& cur, int k0) {
    const uint64_t* bw = reinterpret_cast<const uint64_t*>(lds_b[buf]);
    // The stage's A fragments and packed B words are read out of LDS first, so
    // the MFMAs do not each wait for a read issued just before them; on the bf16
    // path (two row tiles per wave) the reads are pinned ahead of the math.
    u32x4_t afr[BK / 16][MT];
    uint64_t bwr[BK / 16];
#pragma unroll
    for (int j = 0; j < BK / 16; ++j) {
      // packed row 2j + h of the stage, columns 2*c32 and 2*c32 + 1 of the wave's 64
      bwr[j] = BD ? cur.bd[BD ? j : 0] : bw[(2 * j + h) * (BN / 2) + wn * (TN / 2) + c32];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = wm * TM + mt * 32 + c32;
        afr[j][mt] = lds_a[buf][row * CHUNKS + swz(row, KH ? 4 * h + j : 2 * j + h)];
      }
    }
    if constexpr (GP && MT <= 2) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < BK / 16; ++j) {
      const uint64_t w2 = bwr[j];
      const uint32_t sp = KH ? (h ? cur.sc[1] : cur.sc[0]) : cur.sc[j >> 1];
      u32x4_t bq[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t wd = (uint32_t)(w2 >> (32 * t));
        if constexpr (GP) {
          // 128 + q (bf16) or q - 8 (fp16) per half, exact
          bq[t] = unpack_w4_word_natural<!BF>(wd, vmask, bias);
        } else {
          const uint32_t pair = __builtin_amdgcn_perm(sp, sp, t ? 0x03020302u : 0x01000100u);
          const half2_t s2 = __builtin_bit_cast(half2_t, pair);
          const u32x4_t d = unpack_w4_word_natural<true>(wd, vmask, bias);
          const uint32_t d0 = d.x, d1 = d.y, d2 = d.z, d3 = d.w;
          bq[t] = u32x4_t{hmul2(d0, s2), hmul2(d1, s2), hmul2(d2, s2), hmul2(d3, s2)};
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4_t av = afr[j][mt];
        if constexpr (GP) {
          part[mt][0] = mfma32x32x16_t<BF>(av, bq[0], part[mt][0]);
          part[mt][1] = mfma32x32x16_t<BF>(av, bq[1], part[mt][1]);
          if constexpr (BF) corr[mt] = mfma32x32x16_bf16(av, u32x4_t{m136, m136, m136, m136}, corr[mt]);
        } else {
          acc[mt][0] = mfma32x32x16_f16(av, bq[0], acc[mt][0]);
          acc[mt][1] = mfma32x32x16_f16(av, bq[1], acc[mt][1]);
        }
      }
      if constexpr (GP) {
        // the quantization group ends with this 16-deep step: scale its partials
        // once (uniform test; steps past K hold zero activations)
        if (((k0 + 16 * (j + 1)) & (group_size - 1)) == 0) {
          const float s0 = bits2f<BF>(sp & 0xFFFFu), s1 = bits2f<BF>(sp >> 16);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              acc[mt][0][e] += s0 * (BF ? part[mt][0][e] + corr[mt][e] : part[mt][0][e]);
              acc[mt][1][e] += s1 * (BF ? part[mt][1][e] + corr[mt][e] : part[mt][1][e]);
            }
          clear_partials();
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
      if (kt < nk) compute(j & 1, cur, kt * BK);
      if (more) store_stage(kt + 2, (j + 1) & 1, r);
      __syncthreads();
      if (more) cur = cur_of(r);
    }
    // group 1 hands its partial sums to group 0 through the (now free) stage
    // buffers, two row tiles at a time; lane-major so the accesses are
    // conflict-free
    float* red = reinterpret_cast<float*>(&lds);
    static_assert(sizeof(W4TileLds<BM, BN, KG, BD>) >= 64 * NTHR * sizeof(float), "reduction space");
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
      compute(kt & 1, cur, kt * BK);
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
      compute(0, cur, kt * BK);
      store_stage(kt + 1, 1, r1);
      __syncthreads();
      cur = cur_of(r1);
      // odd stage kt + 1: buffer 1; stage kt + 2 (if any) is in r0
      load_stage(min(kt + 3, nk - 1), r1);
      __builtin_amdgcn_sched_barrier(0);
      compute(1, cur, (kt + 1) * BK);
      if (kt + 2 < nk) {
        store_stage(kt + 2, 0, r0);
        cur = cur_of(r0);
      }
      __syncthreads();
    }
    if (kt < nk) compute(0, cur, kt * BK);   // nk odd: the last stage sits in buffer 0
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
        if (i < nk) compute(i & 1, cur, i * BK);
        if (i + 1 < nk) {
          store_stage(i + 1, (i + 1) & 1, r[(p + 1) % PD]);
          cur = cur_of(r[(p + 1) % PD]);
        }
        __syncthreads();
      }
    }
  }

  w4_tile_store<MT, BF>(acc, C, M, N, m0 + wm * TM, n0 + wn * TN, h, c32, ep);
}

// Dense kernel: one tile per workgroup, tile order within each
// XCD's run: 0 = M fastest, 1 = N fastest, else groups of `order` row panels
// swept across N.
template <int BM, int BN, int WAVES_M, int WAVES_N, int MINB, int PD, int KG, bool BF, bool NK = false,
          bool BD = false, bool XH = false>
__global__ __launch_bounds__(WAVES_M * WAVES_N * kWave * KG, MINB) void w4_prefill_v4_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ B,
    const uint16_t* __restrict__ S, int M, int N, int K, int group_size, int tiles_m, int tiles_n, int order,
    Epilogue ep) {
  __shared__ W4TileLds<BM, BN, KG, BD> lds;
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
  w4_mfma_tile<BM, BN, WAVES_M, WAVES_N, PD, KG, BF, NK, BD, XH>(C, A, B, S, M, N, K, group_size, tm * BM,
                                                                 tn * BN, lds, ep);
}

// Direct-to-LDS form of the tile body for K a multiple of 64: a BM x 256 tile
// (BM = 128 or 64) per K group of 4 WAVES_M waves (TM x 64 wave tiles), fp16 or
// bf16 (BF: exact codes, group partials as in w4_mfma_tile) or fp16 with exact
// codes and group partials (XH), weights [K/8, N] or [N, K/8] (NK).
//   * Every stage's A rows (BM x 128 B), packed B words (8 KiB) and the scales
//     of its two 32-deep halves go from global memory straight into LDS with
//     global_load_lds (lane l of a 16-byte wave load fills bytes 16 l .. + 15 of
//     a 1 KiB block; the [N, K/gs] scales come with 2-byte loads, one scale per
//     4-byte LDS word), into NBUF stage buffers, so NBUF - 1 stages of loads are
//     in flight without registers; each wave waits with an explicit vmcnt for
//     all but its newest stage's loads and one barrier per stage publishes the
//     next stage and frees the oldest buffer.
//   * A stays in memory order (16-byte chunks XOR-swizzled by (row >> 1) & 7);
//     the weights are unpacked in natural K order (unpack_w4_word_natural).
//     [K/8, N]: B in LDS as [packed row][column]. [N, K/8]: as each column's
//     eight words, in 16-byte halves placed so that a read phase meets 16
//     different bank groups; a lane reads its columns' halves whole.
//   * KG = 2: two groups of four waves take the even and the odd stages, each
//     with its own buffers, and add their accumulators through LDS at the end.
template <int BM, int KG, int NBUF, bool NK = false>
struct W4DmaLds {
  u32x4_t a[KG][NBUF][BM * 8];     // [row][chunk], 128 B per row
  uint32_t b[KG][NBUF][8 * 256];   // [packed row][column]
  // [half][column pair]: the scales of two columns; [N, K/gs] scales: [half][column],
  // one scale in the low half of each word (a 2-byte LDS load fills 4 bytes per lane)
  uint32_t s[KG][NBUF][NK ? 2 * 256 : 2 * 128];
};

template <int BM, int KG, int NBUF, int WAVES_M = 1, bool BF = false, bool NK = false, bool PART = false,
          bool XH = false>
__device__ __forceinline__ void w4_tile_dma(uint16_t* __restrict__ C, const uint16_t* __restrict__ A,
                                            const uint32_t* __restrict__ B, const uint16_t* __restrict__ S, int M,
                                            int N, int K, int group_size, int m0, int n0,
                                            W4DmaLds<BM, KG, NBUF, NK>& lds, const Epilogue& ep) {
  constexpr int BN = 256, WAVES = 4 * WAVES_M, NTHR = WAVES * kWave;
  constexpr int TM = BM / WAVES_M, MT = TM / 32;
  constexpr int AW = BM / 8 / WAVES;   // A wave loads (1 KiB, eight rows) per stage and wave
  constexpr int BW = 8 / WAVES;        // B wave loads (1 KiB) per stage and wave
  constexpr int SW = NK ? 8 / WAVES : 0;   // [N, K/gs] scales: 2-byte wave loads (64 columns) per wave
  static_assert(BM % (8 * WAVES) == 0 && TM % 32 == 0 && BW >= 1, "tile shape");
  constexpr bool GP = BF || XH;   // exact codes and group partials (bf16, or fp16 with XH)
  static_assert(!GP || KG == 1, "group partials: a quantization group's stages stay in one K group");
  // lane half h takes K rows 32h + 8j .. + 7 at 16-deep step j with one fp16 K
  // group (as the register-staged tile with direct B does), else rows
  // 16j + 8h .. + 7 (as its staged-B and bf16 forms do: a bf16 step stays in one
  // quantization group), so both weight layouts give the same results bit for bit
  constexpr bool KH = KG == 1 && !GP;
  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = wave_all / WAVES;   // K group
  const int wave = wave_all % WAVES;
  const int wm = wave >> 2, wn = wave & 3;   // the wave's row block and 64-column strip
  const int tid = threadIdx.x % NTHR;
  const int h = lane >> 5, c32 = lane & 31;
  const int rows = min(BM, M - m0);
  const int gshift = __builtin_ctz(group_size);
  const int nk = K / BK;

  // wave loads of a stage (per K group): A blocks wave + WAVES i (rows 8a .. 8a + 7),
  // packed B rows wave + WAVES i, and (wave 0) the scale rows of the two halves
  uint32_t aoff[AW];
#pragma unroll
  for (int i = 0; i < AW; ++i) {
    const int row = 8 * (wave + WAVES * i) + (lane >> 3);
    const int ch = (lane & 7) ^ ((row >> 1) & 7);   // the chunk that swz puts at slot lane & 7
    aoff[i] = (uint32_t)min(row, rows - 1) * (uint32_t)K * 2u + ch * 16;
  }
  const int c4 = min(n0 + 4 * lane, N - 4) - n0;   // this lane's four columns of a packed row
  uint32_t boff[BW];
#pragma unroll
  for (int i = 0; i < BW; ++i) {
    if constexpr (NK) {
      // [N, K/8]: 16-byte slot s' of the stage's B area holds half s & 1 (words
      // 4 (s & 1) .. + 3) of column s >> 1, s = s' ^ ((s' >> 4) & 3), so that the
      // 16 lanes of a read phase, which read the same half of 16 even (or odd)
      // columns, meet 16 different bank groups
      const int sp = 64 * (wave + WAVES * i) + lane;
      const int sl = sp ^ ((sp >> 4) & 3);
      const int col = min(n0 + (sl >> 1), N - 1) - n0;
      boff[i] = ((uint32_t)col * (uint32_t)(K / 8) + 4 * (sl & 1)) * 4u;
    } else {
      boff[i] = (uint32_t)(wave + WAVES * i) * (uint32_t)N * 4u + c4 * 4;
    }
  }
  const int c8 = min(n0 + 8 * (lane & 31), N - 8) - n0;   // eight columns of a scale row
  // [N, K/gs] scales: wave load q (0..7) brings half q >> 2, columns 64 (q & 3) + lane
  uint32_t soffk[NK ? SW : 1];
#pragma unroll
  for (int i = 0; i < (NK ? SW : 1); ++i) {
    const int q = wave + WAVES * i;
    const int col = min(n0 + 64 * (q & 3) + lane, N - 1) - n0;
    soffk[i] = (uint32_t)col * (uint32_t)(K >> gshift) * 2u;
  }
  const int nw = AW + BW + (NK ? SW : (wave == 0));        // loads per stage of this wave
  auto lds_addr = [](const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
  };
  auto issue = [&](int kt, int buf) {
    const int k0 = kt * BK;
    const uint16_t* ab = A + (size_t)m0 * K + k0;
    const uint32_t* bb = NK ? B + (size_t)n0 * (K / 8) + k0 / 8 : B + (size_t)(k0 / 8) * N + n0;
#pragma unroll
    for (int i = 0; i < AW; ++i) dma16(ab, aoff[i], lds_addr(&lds.a[kg][buf][(wave + WAVES * i) * 64]));
#pragma unroll
    for (int i = 0; i < BW; ++i) dma16(bb, boff[i], lds_addr(&lds.b[kg][buf][(wave + WAVES * i) * 256]));
    if constexpr (NK) {
      const int g0 = k0 >> gshift;
      const int dg = ((k0 + 32) >> gshift) - g0;
      const uint16_t* sb = S + (size_t)n0 * (K >> gshift) + g0;
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        const int q = wave + WAVES * i;
        dma2(sb, soffk[i] + (uint32_t)((q >> 2) * dg) * 2u, lds_addr(&lds.s[kg][buf][256 * (q >> 2) + 64 * (q & 3)]));
      }
    } else if (wave == 0) {
      const int g0 = k0 >> gshift;
      const int dg = ((k0 + 32) >> gshift) - g0;   // 1 when the second half starts a new group
      const uint16_t* sb = S + (size_t)g0 * N + n0;
      const uint32_t soff = (uint32_t)((lane >> 5) * dg) * (uint32_t)N * 2u + c8 * 2;
      dma16(sb, soff, lds_addr(&lds.s[kg][buf][0]));
    }
  };
  auto wait_loads = [](int n) {   // at most n of this wave's loads in flight (n uniform)
    switch (n) {
      case 0: __builtin_amdgcn_s_waitcnt(0xF70); break;
      case 3: __builtin_amdgcn_s_waitcnt(0xF73); break;
      case 4: __builtin_amdgcn_s_waitcnt(0xF74); break;
      case 5: __builtin_amdgcn_s_waitcnt(0xF75); break;
      case 6: __builtin_amdgcn_s_waitcnt(0xF76); break;
      case 7: __builtin_amdgcn_s_waitcnt(0xF77); break;
      case 8: __builtin_amdgcn_s_waitcnt(0xF78); break;
      default: __builtin_amdgcn_s_waitcnt(0xF70); break;
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
  const uint32_t bias = __builtin_amdgcn_readfirstlane(BF ? 0x43004300u : 0x64006400u);
  // bf16: per row tile, the group partials of both column tiles and the
  // row-sum correction -136 * sum(a) (the same for every column)
  constexpr int MP = GP ? MT : 1;
  float16_t part[MP][2], corr[MP];
  auto clear_partials = [&]() {
#pragma unroll
    for (int i = 0; i < MP; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) part[i][0][e] = part[i][1][e] = corr[i][e] = 0.f;
  };
  if constexpr (GP) clear_partials();
  const uint32_t m136 = 0xC308C308u;   // bf16 pair (-136, -136)

  // PART (routed tiles): a wave whose column strip lies wholly past N does no
  // arithmetic, and one whose second row tile holds only padding rows skips that
  // tile's fragment reads and MFMAs (a uniform branch, no second instance of the
  // tile body); the loads and barriers stay the same.
  static_assert(!PART || KG == 1, "partial tiles: one K group");
  const bool strip_live = n0 + wn * 64 < N;   // uniform
  // routed tiles: row tiles past the first hold real rows only when the chunk
  // has more than 32 rows (uniform); a padding-only row tile is skipped
  const bool rows_hi = !PART || rows - wm * TM > 32;
  auto compute = [&](int buf, int k0) {
    const uint64_t* bw = reinterpret_cast<const uint64_t*>(lds.b[kg][buf]);
    u32x4_t afr[BK / 16][MT];
    uint64_t bwr[BK / 16];
    uint32_t spr[2];
    if constexpr (NK) {
      // the lane's two columns: words 4h .. 4h + 3 (KH), or all eight
      const u32x4_t* bq4 = reinterpret_cast<const u32x4_t*>(lds.b[kg][buf]);
      auto slot = [](int col, int half) { const int s = 2 * col + half; return s ^ ((s >> 4) & 3); };
      u32x4_t wv[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int col = wn * 64 + 2 * c32 + t;
        if constexpr (KH) {
          wv[t][0] = bq4[slot(col, h)];
        } else {
          wv[t][0] = bq4[slot(col, 0)];
          wv[t][1] = bq4[slot(col, 1)];
        }
      }
#pragma unroll
      for (int j = 0; j < BK / 16; ++j) {
        uint32_t w01[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if constexpr (KH) {
            w01[t] = wv[t][0][j];
          } else {   // word 2j + h
            const u32x4_t& v = wv[t][j >> 1];
            w01[t] = h ? v[2 * (j & 1) + 1] : v[2 * (j & 1)];
          }
        }
        bwr[j] = (uint64_t)w01[0] | ((uint64_t)w01[1] << 32);
      }
    } else {
#pragma unroll
      for (int j = 0; j < BK / 16; ++j) {
        const int kc = KH ? 4 * h + j : 2 * j + h;   // the lane half's 8-deep K chunk (packed row) at step j
        bwr[j] = bw[kc * (BN / 2) + wn * 32 + c32];   // columns 2 c32, 2 c32 + 1 of the strip
      }
    }
#pragma unroll
    for (int j = 0; j < BK / 16; ++j) {
      const int kc = KH ? 4 * h + j : 2 * j + h;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt > 0 && !rows_hi) continue;
        const int row = wm * TM + mt * 32 + c32;
        afr[j][mt] = lds.a[kg][buf][row * CHUNKS + swz(row, kc)];
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      if constexpr (NK) {   // the low halves of two column words
        const u32x2_t v = *reinterpret_cast<const u32x2_t*>(&lds.s[kg][buf][s2 * 256 + wn * 64 + 2 * c32]);
        spr[s2] = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
      } else {
        spr[s2] = lds.s[kg][buf][s2 * 128 + wn * 32 + c32];
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // every read of the stage ahead of its arithmetic
#pragma unroll
    for (int j = 0; j < BK / 16; ++j) {
      const uint64_t w2 = bwr[j];
      const uint32_t sp = KH ? spr[h] : spr[j >> 1];
      u32x4_t bq[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t wd = (uint32_t)(w2 >> (32 * t));
        if constexpr (GP) {
          bq[t] = unpack_w4_word_natural<!BF>(wd, vmask, bias);   // 128 + q (bf16) or q - 8 (fp16), exact
        } else {
          const uint32_t pair = __builtin_amdgcn_perm(sp, sp, t ? 0x03020302u : 0x01000100u);
          const half2_t s2 = __builtin_bit_cast(half2_t, pair);
          const u32x4_t d = unpack_w4_word_natural<true>(wd, vmask, bias);
          const uint32_t d0 = d.x, d1 = d.y, d2 = d.z, d3 = d.w;
          bq[t] = u32x4_t{hmul2(d0, s2), hmul2(d1, s2), hmul2(d2, s2), hmul2(d3, s2)};
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt > 0 && !rows_hi) continue;
        if constexpr (GP) {
          part[mt][0] = mfma32x32x16_t<BF>(afr[j][mt], bq[0], part[mt][0]);
          part[mt][1] = mfma32x32x16_t<BF>(afr[j][mt], bq[1], part[mt][1]);
          if constexpr (BF) corr[mt] = mfma32x32x16_bf16(afr[j][mt], u32x4_t{m136, m136, m136, m136}, corr[mt]);
        } else {
          acc[mt][0] = mfma32x32x16_f16(afr[j][mt], bq[0], acc[mt][0]);
          acc[mt][1] = mfma32x32x16_f16(afr[j][mt], bq[1], acc[mt][1]);
        }
      }
      if constexpr (GP) {
        // the quantization group ends with this 16-deep step: scale its partials
        // once (uniform test)
        if (((k0 + 16 * (j + 1)) & (group_size - 1)) == 0) {
          const float s0 = bits2f<BF>(sp & 0xFFFFu), s1 = bits2f<BF>(sp >> 16);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              acc[mt][0][e] += s0 * (BF ? part[mt][0][e] + corr[mt][e] : part[mt][0][e]);
              acc[mt][1][e] += s1 * (BF ? part[mt][1][e] + corr[mt][e] : part[mt][1][e]);
            }
          clear_partials();
        }
      }
    }
  };

  // group kg takes stages kg, kg + KG, ...; t counts its own stages. Both groups
  // run the same number of iterations so every wave reaches every barrier.
  const int iters = (nk + KG - 1) / KG;
  auto valid = [&](int t) { return kg + KG * t < nk; };
  // prologue: stages 0 .. NBUF - 2 in flight (with KG = 2 and one stage, group 1
  // has none), then stage 0 landed
  int pro_inflight = 0;
#pragma unroll
  for (int d = 0; d < NBUF - 1; ++d) {
    if (valid(d)) {
      issue(kg + KG * d, d);
      if (d > 0) pro_inflight += nw;
    }
  }
  wait_loads(pro_inflight);
  __syncthreads();
  auto stage = [&](int t, int buf) {
    const bool more = valid(t + NBUF - 1);
    if (more) issue(kg + KG * (t + NBUF - 1), (buf + NBUF - 1) % NBUF);
    if (valid(t) && (!PART || strip_live)) compute(buf, (kg + KG * t) * BK);
    // stage t + 1 must have landed; stages t + 2 .. t + NBUF - 1 may stay in flight
    int inflight = 0;
#pragma unroll
    for (int d = 2; d < NBUF; ++d) inflight += valid(t + d) ? nw : 0;
    wait_loads(inflight);
    __syncthreads();
  };
  int t0 = 0;
  for (; t0 + NBUF <= iters; t0 += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) stage(t0 + u, u);
  }
  for (; t0 < iters; ++t0) stage(t0, t0 % NBUF);

  if constexpr (KG == 2) {
    // group 1 hands its sums to group 0 through the (now free) stage buffers,
    // two row tiles at a time, lane-major so the accesses are conflict-free
    float* red = reinterpret_cast<float*>(&lds);
    static_assert(sizeof(W4DmaLds<BM, KG, NBUF, NK>) >= 64 * NTHR * sizeof(float), "reduction space");
    static_assert(KG == 1 || MT % 2 == 0, "row tile pairs");
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
  }
  w4_tile_store<MT, BF>(acc, C, M, N, m0 + wm * TM, n0 + wn * 64, h, c32, ep);
}

// Dense kernel of the direct-to-LDS tile body (tile order as in w4_prefill_v4_kernel).
template <int KG, int MINB, int NBUF, int WAVES_M = 1, bool BF = false, bool NK = false, bool XH = false>
__global__ __launch_bounds__(4 * WAVES_M * kWave * KG, MINB) void w4_prefill_dma_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ B,
    const uint16_t* __restrict__ S, int M, int N, int K, int group_size, int tiles_m, int tiles_n, int order,
    Epilogue ep) {
  __shared__ W4DmaLds<128, KG, NBUF, NK> lds;
  const int tiles = tiles_m * tiles_n;
  const int per = (tiles + 7) >> 3;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= tiles) return;
  const int span = order * tiles_n;
  const int first = (lin / span) * order;
  const int gm = min(tiles_m - first, order);
  const int r = lin % span;
  const int tm = first + r % gm, tn = r / gm;
  w4_tile_dma<128, KG, NBUF, WAVES_M, BF, NK, false, XH>(C, A, B, S, M, N, K, group_size, tm * 128, tn * 256,
                                                          lds, ep);
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
template <int BM, int BN, int WAVES_M, int WAVES_N, int MINB, int KG, int PD, bool BD, bool BF, bool DMA = false,
          bool XH = false>
__global__ __launch_bounds__(WAVES_M * WAVES_N * kWave * KG, MINB) void w4_grouped_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ a_off,
    const uint32_t* __restrict__ B, const uint16_t* __restrict__ S, const int32_t* __restrict__ ids, int N, int K,
    int group_size, int num_active, int tiles_n, Epilogue ep) {
  // the direct-to-LDS tile (fp16, K a multiple of 64) or the register-staged one
  __shared__ std::conditional_t<DMA, W4DmaLds<BM, 1, 3>, W4TileLds<BM, BN, KG, BD>> lds;
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
  if constexpr (DMA)
    w4_tile_dma<BM, 1, 3, 1, BF, false, true, XH>(C + (size_t)r_begin * NO, A + (size_t)r_begin * K, B + e * wpe,
                                              S + e * spe, rows, N, K, group_size, 0, nt * BN, lds, ept);
  else
    w4_mfma_tile<BM, BN, WAVES_M, WAVES_N, PD, KG, BF, false, BD, XH>(C + (size_t)r_begin * NO,
                                                                     A + (size_t)r_begin * K, B + e * wpe,
                                                                     S + e * spe, rows, N, K, group_size, 0,
                                                                     nt * BN, lds, ept);
}

// Grouped launch: 64-row chunks of a group by 256 columns, both types with
// exact weights: bf16 (128 + q codes, a group partial and a row-sum correction
// beside each accumulator) and fp16 (XH: exact (q - 8) codes and a group
// partial, no correction; within 3 % of rounding each weight to fp16 per
// launch), two workgroups per CU. K a multiple of 64: the direct-to-LDS tile
// (three stage buffers); otherwise the register-staged tile with B words loaded
// straight into the lanes' registers (one wave per column strip, so no B word
// is shared), one stage in flight.
template <int MINB, int PD, bool BF, bool DMA = false, bool XH = false>
static hipError_t launch_w4_grouped_t(const W4GroupedArgs& p, hipStream_t stream) {
  constexpr int BM = 64, BN = 256, WM = 1, WN = 4, KG = 1;
  constexpr bool BD = true;
  const int tiles_n = (int)((p.N + BN - 1) / BN);
  // every group has at most ceil(rows / BM) <= rows / BM + 1 row chunks
  const long long bound = ((p.T + BM - 1) / BM + p.num_active) * (long long)tiles_n;
  if (bound > INT32_MAX / 2) return hipErrorNotSupported;
  const int grid = (int)((bound + 7) / 8 * 8);
  hipLaunchKernelGGL((w4_grouped_kernel<BM, BN, WM, WN, MINB, KG, PD, BD, BF, DMA, XH>), dim3(grid),
                     dim3(WM * WN * kWave * KG), 0, stream, p.C, p.A, p.a_offsets, p.B, p.S, p.expert_ids, (int)p.N,
                     (int)p.K, p.group_size, p.num_active, tiles_n, p.epi);
  return hipGetLastError();
}

hipError_t launch_w4_grouped(const W4GroupedArgs& p, hipStream_t stream) {
  if (p.bf16) return p.K % BK == 0 ? launch_w4_grouped_t<2, 1, true, true>(p, stream)
                                   : launch_w4_grouped_t<2, 1, true>(p, stream);
  return p.K % BK == 0 ? launch_w4_grouped_t<2, 1, false, true, true>(p, stream)
                       : launch_w4_grouped_t<2, 1, false, false, true>(p, stream);
}

// Row panels per group of the dense tile order: each XCD takes a contiguous run
// of tiles in which groups of this many 128-row panels are swept across N. At
// M = 2048 an XCD's run then covers four A panels and eight (N = 4096) or about
// twenty (N = 11008) B panels, whose sum is smaller than with eight A panels.
constexpr int kPanelGroup = 4;

// Dense launch: 128 x 256 tiles in the order above. fp16: one K group of four 128 x 64 wave tiles, two workgroups per
// CU, or (at most one tile per CU) one workgroup of two K groups per CU. bf16:
// eight 64 x 64 wave tiles (two waves per column strip), one workgroup per CU:
// the exact-code path keeps a group partial and a row-sum correction beside
// each accumulator, which leaves no registers for a second workgroup. fp16 with
// the SiLU gate (XH): the same tiles with exact (q - 8) fp16 codes and fp32
// group partials (no correction), so that the gate does not magnify a rounding
// of the weights.
template <int WM, int MINB, int KG, bool BF, bool NK, bool XH = false>
static void launch_v4(const W4Args& p, hipStream_t stream, int tm, int tn) {
  // one K group of waves with a column strip each (fp16): B words go straight
  // into the lanes' registers, two stages ahead
  constexpr bool BD = (KG == 1 && !BF && !XH && WM == 1);
  constexpr int BM = 128, BN = 256, WN = 4, PD = BD ? 2 : 1;
  const int grid = ((tm * tn + 7) / 8) * 8;
  hipLaunchKernelGGL((w4_prefill_v4_kernel<BM, BN, WM, WN, MINB, PD, KG, BF, NK, BD, XH>), dim3(grid),
                     dim3(WM * WN * kWave * KG), 0, stream, p.C, p.A, p.B, p.S, (int)p.M, (int)p.N, (int)p.K,
                     p.group_size, tm, tn, kPanelGroup, p.epi);
}

hipError_t launch_w4_prefill(const W4Args& p, int num_cus, hipStream_t stream) {
  const int tm = (int)((p.M + 127) / 128), tn = (int)((p.N + 255) / 256);
  const bool one_pass = (long long)tm * tn <= num_cus;
  const int grid = ((tm * tn + 7) / 8) * 8;
  // whole 64-deep stages: the direct-to-LDS tile. fp16: two workgroups of four
  // 128 x 64 wave tiles per CU, or (at most one tile per CU) one workgroup of two
  // K groups; bf16: one workgroup of eight 64 x 64 wave tiles per CU.
  auto dma = [&](auto kernel, int waves) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(waves * kWave), 0, stream, p.C, p.A, p.B, p.S, (int)p.M, (int)p.N,
                       (int)p.K, p.group_size, tm, tn, kPanelGroup, p.epi);
  };
  // fp16 with the SiLU gate: exact weights as on the bf16 path (the [N, K/8]
  // layout has no epilogue)
  const bool xh = !p.bf16 && (p.epi.flags & EPI_SILU_GATE) != 0;
  if (p.K % BK == 0) {
    if (p.bf16) {
      if (p.nk) dma(w4_prefill_dma_kernel<1, 1, 3, 2, true, true>, 8);
      else dma(w4_prefill_dma_kernel<1, 1, 3, 2, true, false>, 8);
    } else if (xh) {
      dma(w4_prefill_dma_kernel<1, 1, 3, 2, false, false, true>, 8);
    } else if (one_pass) {
      if (p.nk) dma(w4_prefill_dma_kernel<2, 1, 3, 1, false, true>, 8);
      else dma(w4_prefill_dma_kernel<2, 1, 3, 1, false, false>, 8);
    } else {
      if (p.nk) dma(w4_prefill_dma_kernel<1, 2, 3, 1, false, true>, 4);
      else dma(w4_prefill_dma_kernel<1, 2, 3, 1, false, false>, 4);
    }
    return hipGetLastError();
  }
  // K = 32 mod 64: the register-staged tile (its partial last stage)
  if (p.bf16) {
    if (p.nk) launch_v4<2, 1, 1, true, true>(p, stream, tm, tn);
    else launch_v4<2, 1, 1, true, false>(p, stream, tm, tn);
  } else if (xh) {
    launch_v4<2, 1, 1, false, false, true>(p, stream, tm, tn);
  } else if (p.nk) {
    if (one_pass) launch_v4<1, 1, 2, false, true>(p, stream, tm, tn);
    else launch_v4<1, 2, 1, false, true>(p, stream, tm, tn);
  } else {
    if (one_pass) launch_v4<1, 1, 2, false, false>(p, stream, tm, tn);
    else launch_v4<1, 2, 1, false, false>(p, stream, tm, tn);
  }
  return hipGetLastError();
}

}  // namespace qg
