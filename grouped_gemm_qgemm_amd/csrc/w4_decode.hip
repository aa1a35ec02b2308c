// Skinny-M W4A16 GEMM (M <= 16): the decode-shaped case of the group-quantized
// GEMM described on the Modular page "multistage_gemm_q" (Parameters:
// group_size, pack_factor).
//
// The problem is bound by HBM reads of the packed weights, so the kernel is
// built around keeping as many of those reads in flight as possible:
//   * a workgroup owns a strip of 16*CPL output columns and all of K; its NW
//     waves split K by whole scale groups and each wave issues every weight load
//     of its share before doing any arithmetic;
//   * lane l reads CPL consecutive packed words of one K-row (4*CPL bytes), the
//     16 lanes of a quarter-wave read 64*CPL contiguous bytes, and the four
//     quarter-waves read four consecutive packed rows;
//   * each word is one lane's B operand of a 16x16x32 fp16 MFMA: its eight codes
//     are the eight K values that lane supplies for one column. The A rows are
//     padded to 16 with zeros (M <= 16 needs a single MFMA row tile);
//   * the MFMA sees (q - 8) exactly; the group scale is applied to the fp32
//     partial of each group (deferred scaling), one FMA per output per group;
//   * the waves' fp32 partials are summed through LDS in a fixed order, so the
//     result does not depend on timing; the sum is rounded to fp16 once.
#include "device_common.h"
#include "launch.h"

namespace qg {

// The activations are staged through LDS: each wave copies the A columns of
// its own K batch (MROWS >= M rows) into a private LDS slice with one coalesced
// 16-byte load per lane per row, reordering the K slots once on the way in;
// the MFMA A fragments are then read from LDS (rows >= M are never loaded).
//
// BF: bf16 activations, scales and output. A packed code q then enters the bf16
// MFMA as 128 + q (exact: the pair is 0x4300 | q in each half), and one more
// MFMA per step against a constant -136 matrix adds -136 * (sum of the row's
// activations), so each group's partial is exactly the sum of a * (q - 8) up
// to fp32 accumulation order.
//
// EPI: the fixed epilogue (a kernel of its own, w4_decode_lds_epi_kernel, so the
// plain kernel's arguments stay as small as before).
//
// NK: B stored [N, K/8] and scales [N, K/group_size] (each column's words and
// scales contiguous). Within a group, lane quarter q then takes the SPG
// consecutive words q * SPG .. q * SPG + SPG - 1 of its column (one 4 to
// 32-byte load) instead of every fourth word, and reads the matching
// activation chunks: the MFMA's K slots are a permutation of the group's K
// rows, the same for A and B, so each group's sum is unchanged.
template <int CPL, int NW, int SPG, int MROWS, int BSTEPS, bool BF, bool EPI, bool NK = false>
__device__ __forceinline__ void w4_decode_lds_body(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ B,
    const uint16_t* __restrict__ S, int M, int N, int K, int xcd_remap, const Epilogue& ep) {
  constexpr int SN = 16 * CPL;
  constexpr int STEPS = SPG > BSTEPS ? SPG : BSTEPS;   // K steps per batch
  constexpr int GB = STEPS / SPG;              // groups per batch
  static_assert(!NK || (GB >= 2 && GB % 2 == 0 && GB <= 16), "scale runs");
  constexpr int CH = STEPS * 4;                // 16-byte A chunks per row per batch
  constexpr int AIT = (MROWS * CH + kWave - 1) / kWave;   // A chunk loads per lane
  __shared__ u32x4_t a_lds[NW][MROWS * CH];
  __shared__ float red[NW][16][SN];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int quarter = lane >> 4;
  const int col16 = lane & 15;
  const uint32_t vmask = in_vgpr(0x000F000Fu);   // a VGPR operand for the fused unpack
  const uint32_t bias = __builtin_amdgcn_readfirstlane(BF ? 0x43004300u : 0x64006400u);
  const uint32_t m136 = 0xC308C308u;    // bf16 pair (-136, -136)

  int strip = blockIdx.x;
  if (xcd_remap) strip = (blockIdx.x & 7) * xcd_remap + (blockIdx.x >> 3);
  const int n0 = strip * SN;
  const int ncol_raw = n0 + CPL * col16;
  const bool col_ok = ncol_raw < N;
  const int ncol = col_ok ? ncol_raw : N - CPL;
  const int frag_row = col16 < MROWS ? col16 : MROWS - 1;   // rows >= M hold copies; never stored

  // Fixed epilogue operands of the column pairs (2c, 2c + 1) this thread finishes,
  // loaded now so their latency hides under the main loop.
  constexpr int PAIRS = 16 * SN / 2, PER = EPI ? (PAIRS + NW * kWave - 1) / (NW * kWave) : 1;
  const bool gate = EPI && (ep.flags & 4) != 0;
  const int NO = gate ? N / 2 : N;   // output width
  uint32_t bias2[PER], res[PER];
  if constexpr (EPI) {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int e = threadIdx.x + it * NW * kWave;
      const int row = e / (SN / 2), col = n0 + 2 * (e % (SN / 2));
      bias2[it] = 0;
      res[it] = 0;
      if (e < PAIRS && row < M && col < N) {
        if (ep.flags & 1) bias2[it] = *reinterpret_cast<const uint32_t*>(ep.bias + col);
        if (ep.flags & 2) {
          const uint16_t* r = ep.residual + (size_t)row * NO + (gate ? col / 2 : col);
          res[it] = gate ? (uint32_t)*r : *reinterpret_cast<const uint32_t*>(r);
        }
      }
    }
  }

  const int groups = K / (SPG * 32);
  const int g_begin = (wave * groups) / NW;
  const int g_end = ((wave + 1) * groups) / NW;

  float4_t acc[CPL];
#pragma unroll
  for (int t = 0; t < CPL; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int g0 = g_begin; g0 < g_end; g0 += GB) {
    const int kb0 = g0 * SPG * 32;
    // 1. this batch's activation columns (all rows < MROWS), coalesced; chunk ids
    //    past the slice repeat the last chunk (same data to the same place)
    u32x4_t av[AIT];
#pragma unroll
    for (int it = 0; it < AIT; ++it) {
      const int id = min(lane + it * kWave, MROWS * CH - 1);
      const int i = id / CH, c = id % CH;
      const int row = i < M ? i : M - 1;
      const int k = min(kb0 + c * 8, K - 8);
      av[it] = *reinterpret_cast<const u32x4_t*>(A + (size_t)row * K + k);
    }
    // 2. scales and packed weights of the batch
    uint32_t w[GB][SPG][CPL];
    uint16_t sc[GB][CPL];
    if constexpr (NK) {
      // [N, K/group_size] scales: the batch's GB scales of a column are
      // contiguous, so when the run is aligned and whole (a wave-uniform test)
      // it is one 4 to 32-byte load instead of GB scattered 2-byte loads
      const int groups_per_col = K / (SPG * 32);
      const bool run = groups_per_col % GB == 0 && g0 % GB == 0 && g0 + GB <= g_end;
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        const uint16_t* sp = S + (size_t)(ncol + t) * groups_per_col;
        if (run) {
          uint32_t words[GB / 2];
          if constexpr (GB == 2) {
            words[0] = *reinterpret_cast<const uint32_t*>(sp + g0);
          } else if constexpr (GB == 4) {
            const u32x2_t v = *reinterpret_cast<const u32x2_t*>(sp + g0);
            words[0] = v.x; words[1] = v.y;
          } else {
#pragma unroll
            for (int i = 0; i < GB / 8; ++i) {
              const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sp + g0 + 8 * i);
              words[4 * i] = v.x; words[4 * i + 1] = v.y; words[4 * i + 2] = v.z; words[4 * i + 3] = v.w;
            }
          }
#pragma unroll
          for (int j = 0; j < GB; ++j) sc[j][t] = (uint16_t)(words[j / 2] >> (16 * (j % 2)));
        } else {
#pragma unroll
          for (int j = 0; j < GB; ++j) sc[j][t] = sp[g0 + j < g_end ? g0 + j : g_end - 1];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int g = g0 + j < g_end ? g0 + j : g_end - 1;
      if constexpr (NK) {
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
          const uint32_t* bp = B + (size_t)(ncol + t) * (K / 8) + (g * SPG * 4 + quarter * SPG);
#pragma unroll
          for (int s4 = 0; s4 < SPG; s4 += 4) {
            if constexpr (SPG >= 4) {
              const u32x4_t v = *reinterpret_cast<const u32x4_t*>(bp + s4);
              w[j][s4][t] = v.x; w[j][s4 + 1][t] = v.y; w[j][s4 + 2][t] = v.z; w[j][s4 + 3][t] = v.w;
            } else if constexpr (SPG == 2) {
              const u32x2_t v = *reinterpret_cast<const u32x2_t*>(bp);
              w[j][0][t] = v.x; w[j][1][t] = v.y;
            } else {
              w[j][0][t] = *bp;
            }
          }
        }
        continue;
      }
      if constexpr (CPL == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(S + (size_t)g * N + ncol);
        sc[j][0] = v.x & 0xFFFF; sc[j][1] = v.x >> 16; sc[j][2] = v.y & 0xFFFF; sc[j][3] = v.y >> 16;
      } else if constexpr (CPL == 2) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(S + (size_t)g * N + ncol);
        sc[j][0] = v & 0xFFFF; sc[j][1] = v >> 16;
      } else {
        sc[j][0] = S[(size_t)g * N + ncol];
      }
#pragma unroll
      for (int s = 0; s < SPG; ++s) {
        const uint32_t* bp = B + (size_t)((g * SPG + s) * 4 + quarter) * N + ncol;
        if constexpr (CPL == 4) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(bp);
          w[j][s][0] = v.x; w[j][s][1] = v.y; w[j][s][2] = v.z; w[j][s][3] = v.w;
        } else if constexpr (CPL == 2) {
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(bp);
          w[j][s][0] = v.x; w[j][s][1] = v.y;
        } else {
          w[j][s][0] = *bp;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // 3. activations -> this wave's LDS slice, K slots reordered, chunks swizzled by row
#pragma unroll
    for (int it = 0; it < AIT; ++it) {
      const int id = min(lane + it * kWave, MROWS * CH - 1);
      const int i = id / CH, c = id % CH;
      a_lds[wave][i * CH + (c ^ (i & 15 & (CH - 1)))] = permute_k_0415(av[it]);
    }
    // 4. per group: MFMA chain on (q - 8), then one scaled FMA
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      float4_t part[CPL];
      float4_t corr = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < CPL; ++t) part[t] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < SPG; ++s) {
        // the 8-deep K chunk of this quarter at step s (see NK above)
        const int chunk = NK ? j * SPG * 4 + quarter * SPG + s : (j * SPG + s) * 4 + quarter;
        const u32x4_t a = a_lds[wave][frag_row * CH + (chunk ^ (frag_row & 15 & (CH - 1)))];
        if constexpr (BF) {
          corr = mfma16x16x32_bf16(a, u32x4_t{m136, m136, m136, m136}, corr);
#pragma unroll
          for (int t = 0; t < CPL; ++t) {
            const uint32_t wd = w[j][s][t];
            part[t] = mfma16x16x32_bf16(a, u32x4_t{and_or(wd, vmask, bias), and_or(wd >> 4, vmask, bias),
                                                  and_or(wd >> 8, vmask, bias), and_or(wd >> 12, vmask, bias)},
                                        part[t]);
          }
        } else {
#pragma unroll
          for (int t = 0; t < CPL; ++t)
            part[t] = mfma16x16x32_f16(a, dequant_w4_word_fused(w[j][s][t], vmask, bias), part[t]);
        }
      }
      const bool keep = col_ok && (g0 + j < g_end);
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        const float sv = keep ? (BF ? bf2f(sc[j][t]) : h2f(sc[j][t])) : 0.f;
        acc[t] += sv * (BF ? part[t] + corr : part[t]);
      }
    }
  }

#pragma unroll
  for (int t = 0; t < CPL; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][quarter * 4 + i][CPL * col16 + t] = acc[t][i];
  __syncthreads();
  if constexpr (!EPI) {
    for (int e = threadIdx.x; e < 16 * SN; e += NW * kWave) {
      const int row = e / SN, col = e % SN;
      float sum = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) sum += red[v][row][col];
      if (row < M && n0 + col < N) C[(size_t)row * N + n0 + col] = BF ? f2bf_rn(sum) : f2h_rn(sum);
    }
  } else {
    // fixed epilogue on column pairs (2c, 2c + 1) of the strip (n0 and N are even),
    // with the bias and residual loaded at the start
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int e = threadIdx.x + it * NW * kWave;
      const int row = e / (SN / 2), c = 2 * (e % (SN / 2)), col = n0 + c;
      if (e >= PAIRS || row >= M || col >= N) continue;
      float y0 = 0.f, y1 = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        y0 += red[v][row][c];
        y1 += red[v][row][c + 1];
      }
      if (ep.flags & 1) {
        y0 += bits2f<BF>(bias2[it] & 0xFFFFu);
        y1 += bits2f<BF>(bias2[it] >> 16);
      }
      if (gate) {
        float z = silu(y0) * y1;
        if (ep.flags & 2) z += bits2f<BF>(res[it]);
        C[(size_t)row * NO + col / 2] = BF ? f2bf_rn(z) : f2h_rn(z);
      } else {
        if (ep.flags & 2) {
          y0 += bits2f<BF>(res[it] & 0xFFFFu);
          y1 += bits2f<BF>(res[it] >> 16);
        }
        *reinterpret_cast<uint32_t*>(C + (size_t)row * NO + col) =
            BF ? f2bf2_rn(y0, y1) : (uint32_t)f2h_rn(y0) | ((uint32_t)f2h_rn(y1) << 16);
      }
    }
  }
}

template <int CPL, int NW, int SPG, int MROWS, int BSTEPS, bool BF>
__global__ __launch_bounds__(NW * kWave) void w4_decode_lds_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ B,
    const uint16_t* __restrict__ S, int M, int N, int K, int xcd_remap) {
  w4_decode_lds_body<CPL, NW, SPG, MROWS, BSTEPS, BF, false>(C, A, B, S, M, N, K, xcd_remap, Epilogue{});
}

template <int CPL, int NW, int SPG, int MROWS, int BSTEPS, bool BF>
__global__ __launch_bounds__(NW * kWave) void w4_decode_lds_nk_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ B,
    const uint16_t* __restrict__ S, int M, int N, int K, int xcd_remap) {
  w4_decode_lds_body<CPL, NW, SPG, MROWS, BSTEPS, BF, false, true>(C, A, B, S, M, N, K, xcd_remap, Epilogue{});
}

template <int CPL, int NW, int SPG, int MROWS, int BSTEPS, bool BF>
__global__ __launch_bounds__(NW * kWave) void w4_decode_lds_epi_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ B,
    const uint16_t* __restrict__ S, int M, int N, int K, int xcd_remap, Epilogue ep) {
  w4_decode_lds_body<CPL, NW, SPG, MROWS, BSTEPS, BF, true>(C, A, B, S, M, N, K, xcd_remap, ep);
}

template <int CPL, int NW, int SPG, int MROWS>
static hipError_t launch_lds_cfg(const W4Args& p, hipStream_t stream) {
  constexpr int SN = 16 * CPL;
  constexpr int BSTEPS = NW >= 16 ? 8 : 16;   // LDS: NW * MROWS * BSTEPS * 64 bytes
  const int strips = (int)((p.N + SN - 1) / SN);
  // strips per XCD when they divide evenly, else 0 (no remap); passing it keeps
  // the kernels off the hidden grid-size arguments, whose 256 extra kernarg bytes
  // cost launch time
  const int remap = (strips % 8 == 0) ? strips / 8 : 0;
  const dim3 grid(strips), block(NW * kWave);
  const int M = (int)p.M, N = (int)p.N, K = (int)p.K;
  if (p.nk) {                     // [N, K/8] weights (no epilogue)
    if (p.bf16)
      hipLaunchKernelGGL((w4_decode_lds_nk_kernel<CPL, NW, SPG, MROWS, BSTEPS, true>), grid, block, 0, stream,
                         p.C, p.A, p.B, p.S, M, N, K, remap);
    else
      hipLaunchKernelGGL((w4_decode_lds_nk_kernel<CPL, NW, SPG, MROWS, BSTEPS, false>), grid, block, 0, stream,
                         p.C, p.A, p.B, p.S, M, N, K, remap);
  } else if (p.epi.flags) {
    if (p.bf16)
      hipLaunchKernelGGL((w4_decode_lds_epi_kernel<CPL, NW, SPG, MROWS, BSTEPS, true>), grid, block, 0, stream,
                         p.C, p.A, p.B, p.S, M, N, K, remap, p.epi);
    else
      hipLaunchKernelGGL((w4_decode_lds_epi_kernel<CPL, NW, SPG, MROWS, BSTEPS, false>), grid, block, 0, stream,
                         p.C, p.A, p.B, p.S, M, N, K, remap, p.epi);
  } else if (p.bf16) {
    hipLaunchKernelGGL((w4_decode_lds_kernel<CPL, NW, SPG, MROWS, BSTEPS, true>), grid, block, 0, stream,
                       p.C, p.A, p.B, p.S, M, N, K, remap);
  } else {
    hipLaunchKernelGGL((w4_decode_lds_kernel<CPL, NW, SPG, MROWS, BSTEPS, false>), grid, block, 0, stream,
                       p.C, p.A, p.B, p.S, M, N, K, remap);
  }
  return hipGetLastError();
}

template <int CPL, int NW, int MROWS>
static hipError_t launch_lds_spg(const W4Args& p, hipStream_t stream) {
  switch (p.group_size) {
    case 32: return launch_lds_cfg<CPL, NW, 1, MROWS>(p, stream);
    case 64: return launch_lds_cfg<CPL, NW, 2, MROWS>(p, stream);
    case 128: return launch_lds_cfg<CPL, NW, 4, MROWS>(p, stream);
    case 256: return launch_lds_cfg<CPL, NW, 8, MROWS>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int CPL, int NW>
static hipError_t launch_lds(const W4Args& p, hipStream_t stream) {
  if (p.M <= 1) return launch_lds_spg<CPL, NW, 1>(p, stream);
  if (p.M <= 2) return launch_lds_spg<CPL, NW, 2>(p, stream);
  if (p.M <= 4) return launch_lds_spg<CPL, NW, 4>(p, stream);
  if (p.M <= 8) return launch_lds_spg<CPL, NW, 8>(p, stream);
  return launch_lds_spg<CPL, NW, 16>(p, stream);
}

// One 16-column strip per workgroup of eight waves.
hipError_t launch_w4_decode(const W4Args& p, hipStream_t stream) { return launch_lds<1, 8>(p, stream); }

}  // namespace qg
