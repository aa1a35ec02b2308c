// Persistent grouped (MoE) bf16 GEMM, after the Modular page
// "grouped_matmul_sm100_persistent" (Args: a_offsets prefix sum, expert_ids
// with negative entries skipped, expert_usage_stats[1] active count;
// Parameters: transpose_b).
//
// The problem is bound by reading each active expert's weights once, so the
// schedule is weight-stationary: a work tile is (group, block of up to 128 of
// its rows, 16 * W output columns). A workgroup of W waves owns a tile and
// streams the tile's columns of the expert's weights from HBM exactly once
// while it multiplies every row of the block against them. All loads are raw
// buffer loads (descriptor in SGPRs, uniform per-step offset).
//   * Both weight layouts are staged through LDS, loaded as whole 128-byte
//     row segments: the vector memory path spends one request per cache line
//     an instruction touches, and a per-wave MFMA fragment can only cover half
//     a line of each of 16 weight rows ([E, N, K]: 64-deep steps, ds_read_b128
//     fragments; [E, K, N]: LDS transpose reads).
//   * The rows' activation fragments are loaded once per workgroup (split over
//     the waves, several steps ahead) and shared through an LDS ring in MFMA
//     fragment order (read back as lane * 16 bytes: no bank conflicts).
//   * The activation rows of a group are re-read by each of its column tiles;
//     the tiles of one group are adjacent in the tile order and every XCD takes
//     a contiguous range of it, so those re-reads hit that XCD's L2.
//   * 16x16x32 bf16 MFMA, fp32 accumulation, bf16 round-to-nearest-even.
//   * The tile list is derived on the device from a_offsets / expert_ids: each
//     wave scans the group table 64 groups at a time (one per lane) to count
//     the tiles and to find each tile's group. Rows of skipped or unlisted
//     groups are never written.
#include "device_common.h"
#include "launch.h"

namespace qg {

namespace {

constexpr int GMAXMT = 8;           // row tiles per work tile (128 rows)
constexpr int GBM = 16 * GMAXMT;

}  // namespace

// Column tile nt of a row chunk -> its plane, first column and column limit.
// The planes' column ranges are [0, pb1), [pb1, pb2) and [pb2, N), each cut
// into tiles of GBN columns; without planes pb1 = pb2 = N (one range). A plane
// p reads its activation rows from A + p * plane_rows * K.
struct PlaneTile {
  int plane, n0, n_lim;
};

__device__ __forceinline__ PlaneTile plane_tile(const Planes& pl, int nt, int N, int gbn) {
  const int t0 = (pl.pb1 + gbn - 1) / gbn, t1 = (pl.pb2 - pl.pb1 + gbn - 1) / gbn;
  if (nt < t0) return PlaneTile{0, nt * gbn, pl.pb1};
  if (nt < t0 + t1) return PlaneTile{1, pl.pb1 + (nt - t0) * gbn, pl.pb2};
  return PlaneTile{2, pl.pb2 + (nt - t0 - t1) * gbn, N};
}

// One work tile with MT row tiles over weights stored [E, K, N]. D = steps of
// prefetch (ring depth).
//
// Every thread issues, per 32-deep K step, one 16-byte load of the step's
// weight tile and every wave (MT / W, rounded up) of the tile's activation
// fragments. Loads run D steps ahead. At step s each wave copies its activation fragments of
// step s into the LDS ring, one barrier makes all of them visible, and each
// wave multiplies every row tile against its own weight fragment. Because a
// wave's loads are issued in step order and each step waits only for its own
// (oldest) loads, the hardware's in-order load counter never forces a wave to
// wait for a prefetch that lies further ahead.
//
// The workgroup loads the step's 32 x 16W weight tile cooperatively (one 16-byte chunk per thread, whole
// 32W-byte row segments), stores it into a second LDS ring and every wave reads
// its B fragment with two 16-bit LDS transpose reads: within each 16-lane
// group, element j of lane i comes from the 8 bytes named by lane 4j + i / 4, at
// element i % 4, so lane m naming K row 8q + 4h + m / 4, columns 4(m % 4) .. + 3
// of the wave's sixteen hands lane i column i at K rows 8q + 4h .. + 3.
template <int W>
struct WRing {
  static constexpr int ROW = 2 * W + 2;   // 16-byte chunks per K row (two spare: rows land on distinct banks)
  static constexpr int SLOT = 32 * ROW;
};

// Stores a wave's 16-column slice of a tile (lane: column n0 + 16 wave + r16,
// rows 16 mt + 4q + i of the group's chunk), plain or through the fixed
// epilogue: bias row of expert e, SiLU gate of column pairs (the odd column's
// value comes from the neighbouring lane, and the even lane stores
// silu(gate) * up at column col / 2 of the N / 2 wide output), residual.
// Residual values are loaded before the first store (the compiler cannot rule
// out that C aliases them).
// EPI false: the plain store only (the kernels without an epilogue are their
// own instantiations, so the epilogue code costs them nothing).
// Columns at or past n_lim (the end of the tile's plane, at most N) belong to
// another tile and are not stored.
template <int MT, bool EPI>
__device__ __forceinline__ void grouped_store(uint16_t* __restrict__ C, const float4_t (&acc)[MT], int N, int n_lim,
                                              int e, int r_begin, int rows, int col, int q, const Epilogue& ep) {
  if (!EPI || ep.flags == 0) {
    if (col < n_lim) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mt * 16 + q * 4 + i;
          if (r < rows) C[(size_t)(r_begin + r) * N + col] = f2bf_rn(acc[mt][i]);
        }
      }
    }
    return;
  }
  const bool gate = (ep.flags & EPI_SILU_GATE) != 0;
  const int NO = gate ? N / 2 : N;
  const int oc = gate ? col / 2 : col;
  const bool owner = col < n_lim && (!gate || (col & 1) == 0);   // lanes that store
  const float b = (ep.flags & EPI_BIAS) && col < n_lim ? bf2f(ep.bias[(size_t)e * N + col]) : 0.f;
  float res[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = mt * 16 + q * 4 + i;
      res[mt][i] = (ep.flags & EPI_RESIDUAL) && owner && r < rows ? bf2f(ep.residual[(size_t)(r_begin + r) * NO + oc])
                                                                 : 0.f;
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = mt * 16 + q * 4 + i;
      float y = acc[mt][i] + b;
      if (gate) {
        const float up = __shfl_xor(y, 1);   // every lane takes part
        y = silu(y) * up;
      }
      if (owner && r < rows) C[(size_t)(r_begin + r) * NO + oc] = f2bf_rn(y + res[mt][i]);
    }
  }
}

// P > 1: the loads of P consecutive steps are issued together (a weight row's
// P * 64 contiguous bytes requested back to back).
template <int W, int MT, int D, int P, bool EPI>
__device__ __forceinline__ void grouped_tile(uint16_t* __restrict__ C, const uint16_t* __restrict__ A,
                                             const uint16_t* __restrict__ B, u32x4_t* __restrict__ ring,
                                             u32x4_t* __restrict__ wring, int N, int K, int e, int r_begin,
                                             int rows, int n0, int n_lim, const Epilogue& ep) {
  constexpr int FPW = (MT + W - 1) / W;   // activation fragments per wave per step
  static_assert(FPW * W <= GMAXMT, "LDS slots for every loaded fragment");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int nfull = K >> 5;

  // buffer descriptors over this tile's activation rows and the expert's weights;
  // per-lane byte offsets, the step's K offset is uniform (an SGPR)
  const __amdgpu_buffer_rsrc_t a_src = buffer_rsrc(A + (size_t)r_begin * K, (uint32_t)rows * K * 2);
  const __amdgpu_buffer_rsrc_t b_src = buffer_rsrc(B + (size_t)e * N * K, (uint32_t)N * K * 2);
  // this thread's chunk of the step's weight tile (K rows past the expert's end
  // read as zeros)
  constexpr int WROW = WRing<W>::ROW;
  const int w_kr = threadIdx.x / (2 * W), w_c = threadIdx.x % (2 * W);
  const uint32_t wt_voff = (uint32_t)(w_kr * N + n0 + 8 * w_c) * 2;
  const int wt_lds = w_kr * WROW + w_c;
  // byte offsets of this lane's two transpose reads within a weight slot
  const int tr_off = (8 * q + (r16 >> 2)) * WROW * 16 + wave * 32 + 8 * (r16 & 3);
  // Wave w loads fragments w, w + W, ... Those past MT are not needed: their
  // offset lies past the descriptor, so the load returns zeros without a memory
  // request, and they land in LDS slots MT .. GMAXMT-1 that no MFMA reads.
  uint32_t a_voff[FPW];
  int a_frag[FPW];
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    a_frag[i] = wave + i * W;
    a_voff[i] = a_frag[i] < MT ? (uint32_t)(min(a_frag[i] * 16 + r16, rows - 1) * K + q * 8) * 2 : 0x80000000u;
  }
  const uint32_t b_voff = wt_voff;

  u32x4_t ra[D][FPW], rb[D];
  // whole step s: K elements 32s .. 32s + 31
  auto load_step = [&](int s, u32x4_t (&a)[FPW], u32x4_t& b) {
    const uint32_t soff = (uint32_t)s * 64;
    b = buffer_load16(b_src, b_voff, (uint32_t)s * 32 * N * 2);
#pragma unroll
    for (int i = 0; i < FPW; ++i) a[i] = buffer_load16(a_src, a_voff[i], soff);
  };
  // partial last step (K % 32 != 0): each lane's chunk start is clamped into its row
  auto load_tail = [&](u32x4_t (&a)[FPW], u32x4_t& b) {
    const uint32_t k2 = (uint32_t)max(0, min(nfull * 32, K - 8 - q * 8)) * 2;
    b = buffer_load16(b_src, b_voff, (uint32_t)nfull * 32 * N * 2);
#pragma unroll
    for (int i = 0; i < FPW; ++i) a[i] = buffer_load16(a_src, a_voff[i] + k2, 0);
  };

  float4_t acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = float4_t{0.f, 0.f, 0.f, 0.f};

  // one step through LDS slot `slot` (data already in registers). Two slots
  // suffice: the slot written at step s was last read at step s - 2, and every
  // wave has passed step s - 1's barrier, so it is done with those reads.
  auto step = [&](int slot, const u32x4_t (&a)[FPW], const u32x4_t& b) {
#pragma unroll
    for (int i = 0; i < FPW; ++i) ring[(slot * GMAXMT + a_frag[i]) * kWave + lane] = a[i];
    wring[slot * WRing<W>::SLOT + wt_lds] = b;
    __syncthreads();
    u32x4_t bf;
    {
      const unsigned char* base = reinterpret_cast<const unsigned char*>(wring + slot * WRing<W>::SLOT) + tr_off;
      typedef short s16x4_t __attribute__((ext_vector_type(4)));
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(__attribute__((address_space(3))) const unsigned char*)base);
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(__attribute__((address_space(3))) const unsigned char*)(base + 4 * WROW * 16));
      const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
      bf = u32x4_t{l2.x, l2.y, h2.x, h2.y};
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      acc[mt] = mfma16x16x32_bf16(ring[(slot * GMAXMT + mt) * kWave + lane], bf, acc[mt]);
  };

  __syncthreads();   // the previous tile's readers are done with the ring
#pragma unroll
  for (int u = 0; u < D; ++u) load_step(max(0, min(u, nfull - 1)), ra[u], rb[u]);

  int s0 = 0;
  for (; s0 + D <= nfull; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      step((s0 + u) & 1, ra[u], rb[u]);
      if ((u + 1) % P == 0) {
#pragma unroll
        for (int v = u + 1 - P; v <= u; ++v) load_step(min(s0 + v + D, nfull - 1), ra[v], rb[v]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // fewer than D whole steps left: register slots 0 .. nfull - s0 - 1 hold them
#pragma unroll
  for (int u = 0; u < D - 1; ++u)
    if (u < nfull - s0) step((s0 + u) & 1, ra[u], rb[u]);
  // partial last step (K % 32 != 0): activation chunks past K enter the MFMA
  // as zeros (weight rows past the expert's end read as zeros too)
  if (K & 31) {
    load_tail(ra[0], rb[0]);
    const bool past = nfull * 32 + q * 8 >= K;
#pragma unroll
    for (int i = 0; i < FPW; ++i) ra[0][i] = past ? u32x4_t{0u, 0u, 0u, 0u} : ra[0][i];
    step(nfull & 1, ra[0], rb[0]);
  }

  // ---- epilogue: bf16 RNE ----
  grouped_store<MT, EPI>(C, acc, N, n_lim, e, r_begin, rows, n0 + wave * 16 + r16, q, ep);
}

// Transposed weights ([E, N, K]) staged through LDS in 64-deep steps. A 16-byte
// load can only feed the MFMA lane that owns its column, so per-wave weight
// fragments touch each 128-byte line of a weight row half at a time; here the
// workgroup loads the step's 16W x 64 weight tile as whole 128-byte row
// segments (eight lanes per row, two chunks per thread), stores it into an LDS
// slot (16-byte chunks XOR-swizzled by row) and every wave reads its fragments
// back with 16-byte LDS reads. A step is two 32-deep MFMA sub-steps; the
// activation ring holds both. D steps are in flight.
template <int W, int MT, int D, bool EPI>
__device__ __forceinline__ void grouped_tile_wl(uint16_t* __restrict__ C, const uint16_t* __restrict__ A,
                                                const uint16_t* __restrict__ B, u32x4_t* __restrict__ ring,
                                                u32x4_t* __restrict__ wring, int N, int K, int e, int r_begin,
                                                int rows, int n0, int n_lim, const Epilogue& ep) {
  constexpr int FPW = (MT + W - 1) / W;
  static_assert(FPW * W <= GMAXMT, "LDS slots for every loaded fragment");
  constexpr int WSLOT = 16 * W * 8;   // 16-byte chunks of one weight step
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int ns = K >> 6;          // whole 64-deep steps
  const int ktail = K & 63;       // elements of the partial last step (a multiple of 8)

  const __amdgpu_buffer_rsrc_t a_src = buffer_rsrc(A + (size_t)r_begin * K, (uint32_t)rows * K * 2);
  const __amdgpu_buffer_rsrc_t b_src = buffer_rsrc(B + (size_t)e * N * K, (uint32_t)N * K * 2);
  uint32_t a_voff[FPW];
  int a_frag[FPW];
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    a_frag[i] = wave + i * W;
    a_voff[i] = a_frag[i] < MT ? (uint32_t)(min(a_frag[i] * 16 + r16, rows - 1) * K + q * 8) * 2 : 0x80000000u;
  }
  // weight chunks h = 0, 1 of this thread: row h * 8W + tid / 8, chunk tid % 8
  const int tid = threadIdx.x;
  const int w_c = tid & 7;
  uint32_t w_voff[2];
  int w_lds[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = h * 8 * W + (tid >> 3);
    w_voff[h] = (uint32_t)(min(n0 + r, N - 1) * K + 8 * w_c) * 2;
    w_lds[h] = r * 8 + (w_c ^ ((r >> 1) & 7));
  }
  // this lane's fragment rows in a weight slot
  const int f_row = wave * 16 + r16;

  u32x4_t ra[D][FPW][2], rb[D][2];
  auto load_step = [&](int s, u32x4_t (&a)[FPW][2], u32x4_t (&b)[2]) {
    const uint32_t soff = (uint32_t)s * 128;
#pragma unroll
    for (int h = 0; h < 2; ++h) b[h] = buffer_load16(b_src, w_voff[h], soff);
#pragma unroll
    for (int i = 0; i < FPW; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) a[i][j] = buffer_load16(a_src, a_voff[i] + 64 * j, soff);
  };

  float4_t acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = float4_t{0.f, 0.f, 0.f, 0.f};

  // slot `slot` of both rings; the slot written at step s was last read at
  // step s - 2, before every wave passed step s - 1's barrier
  auto step = [&](int slot, const u32x4_t (&a)[FPW][2], const u32x4_t (&b)[2]) {
#pragma unroll
    for (int i = 0; i < FPW; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) ring[((slot * 2 + j) * GMAXMT + a_frag[i]) * kWave + lane] = a[i][j];
#pragma unroll
    for (int h = 0; h < 2; ++h) wring[slot * WSLOT + w_lds[h]] = b[h];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4_t bf = wring[slot * WSLOT + f_row * 8 + ((4 * j + q) ^ ((f_row >> 1) & 7))];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = mfma16x16x32_bf16(ring[((slot * 2 + j) * GMAXMT + mt) * kWave + lane], bf, acc[mt]);
    }
  };

  __syncthreads();   // the previous tile's readers are done with both rings
#pragma unroll
  for (int u = 0; u < D; ++u) load_step(max(0, min(u, ns - 1)), ra[u], rb[u]);
  int s0 = 0;
  for (; s0 + D <= ns; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      step((s0 + u) & 1, ra[u], rb[u]);
      load_step(min(s0 + u + D, ns - 1), ra[u], rb[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < D - 1; ++u)
    if (u < ns - s0) step((s0 + u) & 1, ra[u], rb[u]);
  // partial last step: chunks at or past K enter the MFMA as zeros on both sides
  if (ktail) {
    load_step(ns, ra[0], rb[0]);
    const bool w_past = 8 * w_c >= ktail;
#pragma unroll
    for (int h = 0; h < 2; ++h) rb[0][h] = w_past ? u32x4_t{0u, 0u, 0u, 0u} : rb[0][h];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool past = 32 * j + 8 * q >= ktail;
#pragma unroll
      for (int i = 0; i < FPW; ++i) ra[0][i][j] = past ? u32x4_t{0u, 0u, 0u, 0u} : ra[0][i][j];
    }
    step(ns & 1, ra[0], rb[0]);
  }

  grouped_store<MT, EPI>(C, acc, N, n_lim, e, r_begin, rows, n0 + wave * 16 + r16, q, ep);
}

// Persistent workgroups over the same tile list, weights through LDS (above).
template <int W, int D, int OCC, bool EPI>
__global__ __launch_bounds__(W * kWave, OCC) void grouped_bf16_wl_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ a_off,
    const uint16_t* __restrict__ B, const int32_t* __restrict__ ids, int N, int K, int num_active,
    int tiles_n, int per_xcd, Planes pl, Epilogue ep) {
  __shared__ __attribute__((aligned(16))) u32x4_t ring[2 * 2 * GMAXMT * kWave];
  __shared__ __attribute__((aligned(16))) u32x4_t wring[2 * 16 * W * 8];
  constexpr int GBN = 16 * W;
  const int total = count_tiles(a_off, ids, num_active, GBM, tiles_n);
  const int xcd = blockIdx.x & 7;
  const int lo = (int)(((long)total * xcd) >> 3), hi = (int)(((long)total * (xcd + 1)) >> 3);
  for (int t = lo + (int)(blockIdx.x >> 3); t < hi; t += per_xcd) {
    const TileLoc loc = locate_tile(t, a_off, ids, num_active, GBM, tiles_n);
    const int g = loc.g;
    const int chunk = loc.local / tiles_n, nt = loc.local % tiles_n;
    // uniform values in SGPRs: buffer descriptors and row-tile dispatch stay scalar
    const int e = __builtin_amdgcn_readfirstlane(ids[g]);
    const int r_begin = __builtin_amdgcn_readfirstlane((int)a_off[g] + chunk * GBM);
    const int rows = __builtin_amdgcn_readfirstlane(min(GBM, (int)a_off[g + 1] - r_begin));
    const PlaneTile pt = plane_tile(pl, nt, N, GBN);
    const int n0 = pt.n0, n_lim = pt.n_lim;
    const uint16_t* Ap = A + (size_t)pt.plane * pl.plane_rows * K;
    // two activation fragments per wave per sub-step beyond four row tiles
    // (four waves): half as many steps in flight
    constexpr int D5 = W >= 8 ? D : (D + 1) / 2;
    switch ((rows + 15) >> 4) {
      case 1: grouped_tile_wl<W, 1, D, EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      case 2: grouped_tile_wl<W, 2, D, EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      case 3: grouped_tile_wl<W, 3, D, EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      case 4: grouped_tile_wl<W, 4, D, EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      case 5: grouped_tile_wl<W, 5, D5, EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      case 6: grouped_tile_wl<W, 6, D5, EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      case 7: grouped_tile_wl<W, 7, D5, EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      default: grouped_tile_wl<W, 8, D5, EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
    }
  }
}

template <int D, int P>
constexpr int fit_group() { return D % P == 0 ? P : (D % 2 == 0 ? 2 : 1); }

// Persistent workgroups over the tile list, weights stored [E, K, N] (above).
template <int W, int D, int OCC, int P, bool EPI>
__global__ __launch_bounds__(W * kWave, OCC) void grouped_bf16_kernel(
    uint16_t* __restrict__ C, const uint16_t* __restrict__ A, const uint32_t* __restrict__ a_off,
    const uint16_t* __restrict__ B, const int32_t* __restrict__ ids, int N, int K, int num_active,
    int tiles_n, int per_xcd, Planes pl, Epilogue ep) {
  __shared__ __attribute__((aligned(16))) u32x4_t ring[2 * GMAXMT * kWave];
  __shared__ __attribute__((aligned(16))) u32x4_t wring[2 * WRing<W>::SLOT];

  constexpr int GBN = 16 * W;   // columns per work tile: 16 per wave
  // every wave scans the group table itself (one group per lane), so no
  // workgroup waits on a serial walk of it
  const int total = count_tiles(a_off, ids, num_active, GBM, tiles_n);
  const int xcd = blockIdx.x & 7;
  const int lo = (int)(((long)total * xcd) >> 3), hi = (int)(((long)total * (xcd + 1)) >> 3);

  for (int t = lo + (int)(blockIdx.x >> 3); t < hi; t += per_xcd) {
    const TileLoc loc = locate_tile(t, a_off, ids, num_active, GBM, tiles_n);
    const int g = loc.g;
    const int chunk = loc.local / tiles_n, nt = loc.local % tiles_n;
    // uniform values in SGPRs: buffer descriptors and row-tile dispatch stay scalar
    const int e = __builtin_amdgcn_readfirstlane(ids[g]);
    const int r_begin = __builtin_amdgcn_readfirstlane((int)a_off[g] + chunk * GBM);
    const int rows = __builtin_amdgcn_readfirstlane(min(GBM, (int)a_off[g + 1] - r_begin));
    const PlaneTile pt = plane_tile(pl, nt, N, GBN);
    const int n0 = pt.n0, n_lim = pt.n_lim;
    const uint16_t* Ap = A + (size_t)pt.plane * pl.plane_rows * K;
    // With four waves, tiles of more than four row tiles load two activation
    // fragments per wave per step, so they run half as many steps ahead: the
    // same registers and about the same bytes in flight.
    constexpr int D5 = W >= 8 ? D : D / 2;
    switch ((rows + 15) >> 4) {
      case 1: grouped_tile<W, 1, D, fit_group<D, P>(), EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      case 2: grouped_tile<W, 2, D, fit_group<D, P>(), EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      case 3: grouped_tile<W, 3, D, fit_group<D, P>(), EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      case 4: grouped_tile<W, 4, D, fit_group<D, P>(), EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      case 5: grouped_tile<W, 5, D5, fit_group<D5, P>(), EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      case 6: grouped_tile<W, 6, D5, fit_group<D5, P>(), EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      case 7: grouped_tile<W, 7, D5, fit_group<D5, P>(), EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
      default: grouped_tile<W, 8, D5, fit_group<D5, P>(), EPI>(C, Ap, B, ring, wring, N, K, e, r_begin, rows, n0, n_lim, ep); break;
    }
  }
}

// Launch: persistent workgroups, a whole number per XCD. Weights [E, N, K]:
// eight waves (128 columns), three 64-deep steps in flight, two workgroups per
// CU. Weights [E, K, N]: eight waves, eight 32-deep steps in flight issued in
// pairs, one workgroup per CU.
hipError_t launch_grouped_bf16(const GroupedArgs& p, hipStream_t stream) {
  constexpr int W = 8, GBN = 16 * W;
  // column tiles per row chunk: each plane's columns in tiles of their own
  const int tiles_n = (int)((p.planes.pb1 + GBN - 1) / GBN + (p.planes.pb2 - p.planes.pb1 + GBN - 1) / GBN +
                            (p.N - p.planes.pb2 + GBN - 1) / GBN);
  if (p.transpose_b) {
    constexpr int D = 3, OCC = 2;
    const int grid = 8 * ((OCC * p.num_cus + 7) / 8);
    if (p.epi.flags)
      hipLaunchKernelGGL((grouped_bf16_wl_kernel<W, D, OCC, true>), dim3(grid), dim3(W * kWave), 0, stream, p.C,
                         p.A, p.a_offsets, p.B, p.expert_ids, (int)p.N, (int)p.K, p.num_active, tiles_n, grid / 8,
                         p.planes, p.epi);
    else
      hipLaunchKernelGGL((grouped_bf16_wl_kernel<W, D, OCC, false>), dim3(grid), dim3(W * kWave), 0, stream, p.C,
                         p.A, p.a_offsets, p.B, p.expert_ids, (int)p.N, (int)p.K, p.num_active, tiles_n, grid / 8,
                         p.planes, p.epi);
  } else {
    constexpr int D = 8, OCC = 1, P = 2;
    const int grid = 8 * ((OCC * p.num_cus + 7) / 8);
    if (p.epi.flags)
      hipLaunchKernelGGL((grouped_bf16_kernel<W, D, OCC, P, true>), dim3(grid), dim3(W * kWave), 0, stream, p.C,
                         p.A, p.a_offsets, p.B, p.expert_ids, (int)p.N, (int)p.K, p.num_active, tiles_n, grid / 8,
                         p.planes, p.epi);
    else
      hipLaunchKernelGGL((grouped_bf16_kernel<W, D, OCC, P, false>), dim3(grid), dim3(W * kWave), 0, stream, p.C,
                         p.A, p.a_offsets, p.B, p.expert_ids, (int)p.N, (int)p.K, p.num_active, tiles_n, grid / 8,
                         p.planes, p.epi);
  }
  return hipGetLastError();
}

}  // namespace qg
