// Persistent grouped (MoE) bf16 GEMM, after the Modular page
// "grouped_matmul_sm100_persistent" (Args: a_offsets prefix sum, expert_ids
// with negative entries skipped, expert_usage_stats[1] active count;
// Parameters: transpose_b).
//
// The problem is bound by reading each active expert's weights once, so the
// schedule is weight-stationary: a work tile is (group, block of up to 128 of
// its rows, 64 output columns); the workgroup streams that 64 x K slice of the
// expert's weights from HBM exactly once and multiplies every row of the block
// against it.
//   * Each of the four waves owns 16 columns. Its B operand for a 32-deep K step
//     is one 16-byte load per lane of B[e][n][k..k+7] (transpose_b layout puts K
//     contiguous), kept in registers and prefetched several K steps ahead, so
//     weights never pass through LDS.
//   * The rows' activations are shared by the four waves through a double-
//     buffered LDS stage, stored in MFMA fragment order (each 1 KiB fragment is
//     read back as lane * 16 bytes: no bank conflicts, no swizzle).
//   * 16x16x32 bf16 MFMA with fp32 accumulation; bf16 round-to-nearest-even.
//   * A persistent grid walks the tile list computed on the device from
//     a_offsets / expert_ids; each XCD takes a contiguous range of tiles so
//     the n-tiles of one group, which share its activation rows, meet in the
//     same L2. Rows of skipped or unlisted groups are never written.
#include "device_common.h"
#include "launch.h"

namespace qg {

namespace {

constexpr int GBM = 128;         // rows per work tile (8 MFMA row tiles)
constexpr int GMT = GBM / 16;
constexpr int GBN = 64;          // columns per work tile: 4 waves x 16
constexpr int GWAVES = 4;
constexpr int GTHR = GWAVES * kWave;
constexpr int GSTEPS = 2;        // 32-deep K steps per LDS stage (BK = 64)
constexpr int GP = 4;            // B prefetch distance, in stages

}  // namespace

__global__ __launch_bounds__(GTHR) void grouped_bf16_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ a_off,
    const uint16_t* __restrict__ B, const int32_t* __restrict__ ids, int N, int K, int num_active,
    int tiles_n) {
  // A stage: [GMT row tiles][GSTEPS steps][64 lanes][16 bytes]
  __shared__ __attribute__((aligned(16))) u32x4_t lds_a[2][GMT * GSTEPS * kWave];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q = lane >> 4;

  // ---- tile count (every workgroup walks the same small table) ----
  int total = 0;
  for (int g = 0; g < num_active; ++g) {
    const int rows = (int)(a_off[g + 1] - a_off[g]);
    if (ids[g] >= 0 && rows > 0) total += ((rows + GBM - 1) / GBM) * tiles_n;
  }
  const int xcd = blockIdx.x & 7;
  const int per_xcd = gridDim.x >> 3;
  const int lo = (int)(((long)total * xcd) >> 3), hi = (int)(((long)total * (xcd + 1)) >> 3);

  int g = 0, g_first = 0;  // group cursor and the first tile index of group g
  const int nst = (K + 32 * GSTEPS - 1) / (32 * GSTEPS);

  for (int t = lo + (int)(blockIdx.x >> 3); t < hi; t += per_xcd) {
    // advance the cursor to the group holding tile t
    int cnt;
    for (;;) {
      const int rows = (int)(a_off[g + 1] - a_off[g]);
      cnt = (ids[g] >= 0 && rows > 0) ? ((rows + GBM - 1) / GBM) * tiles_n : 0;
      if (t < g_first + cnt) break;
      g_first += cnt;
      ++g;
    }
    const int local = t - g_first;
    const int chunk = local / tiles_n, nt = local % tiles_n;
    const int e = ids[g];
    const int r_begin = (int)a_off[g] + chunk * GBM;
    const int rows = min(GBM, (int)a_off[g + 1] - r_begin);
    const int mt_n = (rows + 15) >> 4;
    const int r_last = r_begin + rows - 1;

    // B: this wave's 16 columns, this lane's column and K slot
    const int ncol = min(nt * GBN + wave * 16 + r16, N - 1);
    const uint16_t* bsrc = B + ((size_t)e * N + ncol) * K + q * 8;

    // A loaders: fragment f = (mt, s) is 64 lanes x 16 bytes
    auto load_a = [&](int st, u32x4_t (&ra)[GMT * GSTEPS / GWAVES]) {
#pragma unroll
      for (int i = 0; i < GMT * GSTEPS / GWAVES; ++i) {
        const int f = wave + i * GWAVES;          // wave-uniform fragment id
        const int mt = f / GSTEPS, s = f % GSTEPS;
        if (mt < mt_n) {
          const int row = min(r_begin + mt * 16 + r16, r_last);
          const int k = st * 32 * GSTEPS + s * 32 + q * 8;
          ra[i] = *reinterpret_cast<const u32x4_t*>(A + (size_t)row * K + min(k, K - 8));
          if (k >= K) ra[i] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    };
    auto store_a = [&](int buf, const u32x4_t (&ra)[GMT * GSTEPS / GWAVES]) {
#pragma unroll
      for (int i = 0; i < GMT * GSTEPS / GWAVES; ++i) {
        const int f = wave + i * GWAVES;
        if (f / GSTEPS < mt_n) lds_a[buf][f * kWave + lane] = ra[i];
      }
    };
    auto load_b = [&](int st, u32x4_t (&rb)[GSTEPS]) {
#pragma unroll
      for (int s = 0; s < GSTEPS; ++s) {
        const int k = min(st * 32 * GSTEPS + s * 32, K - 8 - q * 8);
        rb[s] = *reinterpret_cast<const u32x4_t*>(bsrc + k);
      }
    };

    float4_t acc[GMT];
#pragma unroll
    for (int i = 0; i < GMT; ++i) acc[i] = float4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t ring[GP][GSTEPS];
    u32x4_t ra[GMT * GSTEPS / GWAVES];
#pragma unroll
    for (int u = 0; u < GP; ++u) load_b(min(u, nst - 1), ring[u]);
    load_a(0, ra);
    __syncthreads();  // the previous tile's readers are done with both buffers
    store_a(0, ra);
    __syncthreads();

    for (int st0 = 0; st0 < nst; st0 += GP) {
#pragma unroll
      for (int u = 0; u < GP; ++u) {
        const int st = st0 + u;
        if (st < nst) {
          const bool more = st + 1 < nst;
          if (more) load_a(st + 1, ra);
          u32x4_t bq[GSTEPS];
#pragma unroll
          for (int s = 0; s < GSTEPS; ++s) bq[s] = ring[u][s];
          load_b(min(st + GP, nst - 1), ring[u]);   // refill this slot GP stages ahead
          __builtin_amdgcn_sched_barrier(0);
          const int buf = st & 1;
#pragma unroll
          for (int s = 0; s < GSTEPS; ++s) {
#pragma unroll
            for (int mt = 0; mt < GMT; ++mt) {
              if (mt < mt_n) {
                const u32x4_t av = lds_a[buf][(mt * GSTEPS + s) * kWave + lane];
                acc[mt] = mfma16x16x32_bf16(av, bq[s], acc[mt]);
              }
            }
          }
          if (more) store_a(buf ^ 1, ra);
          __syncthreads();
        }
      }
    }

    // ---- epilogue: bf16 RNE; rows past the block and columns past N are not written ----
    const int col = nt * GBN + wave * 16 + r16;
    if (col < N) {
#pragma unroll
      for (int mt = 0; mt < GMT; ++mt) {
        if (mt < mt_n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = mt * 16 + q * 4 + i;
            if (r < rows) C[(size_t)(r_begin + r) * N + col] = f2bf_rn(acc[mt][i]);
          }
        }
      }
    }
  }
}

hipError_t launch_grouped_bf16(const GroupedArgs& p, int variant, hipStream_t stream) {
  (void)variant;
  const int tiles_n = (int)((p.N + GBN - 1) / GBN);
  int grid = 2 * p.num_cus;
  grid = ((grid + 7) / 8) * 8;
  hipLaunchKernelGGL(grouped_bf16_kernel, dim3(grid), dim3(GTHR), 0, stream, p.C, p.A, p.a_offsets, p.B,
                     p.expert_ids, (int)p.N, (int)p.K, p.num_active, tiles_n);
  return hipGetLastError();
}

}  // namespace qg
