// Ragged, block-scaled K-projection written into a paged KV cache, after the
// Modular page "k_matmul_ragged_paged_scale" (Args: hidden_state,
// input_row_offsets, weight, input_scale, weight_scale, kv_collection,
// layer_idx; Parameters: scales_granularity_mnk).
//
//   K[t][n] = sum_kb is[t][kb] * ws[kb][n/128] * sum_{k in kb} h[t][k] * W[k][n]
//
// with 128 x 128 weight-scale blocks and 1 x 128 input-scale blocks. Tokens of
// all sequences are one flat row dimension (raggedness costs nothing in the
// GEMM); the sequence only matters for where a finished row is stored.
//   * Two tiled designs on BM x 128 tiles with 4 * BM / 48 waves: the
//     raw-weight design (bf16 hidden rows) and the e4m3-hidden design (both
//     MFMA operands e4m3). Each 128-deep K stage is exactly one scale block,
//     so the stage's MFMA partial is scaled once, in fp32, by
//     is[t][kb] * ws[kb][nb] (ws is uniform over the tile) and added to the
//     accumulator. Activations are never re-rounded. The tile rows' input
//     scales sit in LDS, 32 blocks at a time (refilled every 32 stages).
//   * The fp8 weight tile [128 k][128 n] is fetched with coalesced 16-byte row
//     loads, copied into LDS as it is, and MFMA B fragments are read with
//     8-bit transpose reads.
//   * Hidden rows are staged through LDS with an XOR swizzle, one barrier per
//     stage: on 144-row tiles straight from global memory into three LDS
//     stage buffers (global_load_lds), on smaller tiles through registers into
//     two.
//   * Column tile t of a wave holds 16 consecutive columns (the transpose
//     read's order); fp32 accumulation.
//   * Epilogue: token t -> sequence b (binary search of the row offsets) ->
//     position cache_lengths[b] + (t - offs[b]) -> (page_table entry, slot);
//     the row lands in its plane (keys, or values for the second half of
//     [W_k | W_v]) of layer layer_idx, as bf16 or as e4m3 codes with per-run
//     scales. Nothing else in the cache is written.
#include "device_common.h"
#include "launch.h"

namespace qg {

namespace {

constexpr int KBN = 128;      // columns per tile (one weight-scale column block)
constexpr int KBK = 128;      // K per stage (one scale block)
constexpr int KCH = KBK / 8;  // 16-byte chunks per LDS row (16)
constexpr int KSW = 32;       // input-scale blocks held in LDS at a time

// hidden rows: chunk c of row r lives at chunk c ^ (r & 15)
__device__ __forceinline__ int swz_a(int r, int c) { return c ^ (r & 15); }
// 128-byte rows (the fp8 tiles of the direct-to-LDS kernels): chunk c of row r lives at
// chunk c ^ (r & 7) ^ (bit 3 of r), so rows r and r + 8, which share LDS banks, differ too
__device__ __forceinline__ int swz8(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }
// the e4m3-hidden kernel's weight tile: its transpose reads take K rows 32 apart in
// one read phase, so bit 5 of the row (not bit 3) goes into chunk bit 0
__device__ __forceinline__ int swz8b5(int r, int c) { return c ^ (r & 7) ^ ((r >> 5) & 1); }

}  // namespace

// Epilogue shared by the tiled designs: each token row of the tile
// goes to (layer, plane, page, slot) of the cache, as bf16 or as e4m3 codes with
// per-run scales (described below). acc holds a wave's 48 x 32 tile: rows
// wm * 48 + mt * 16 + 4q + i, columns wn * 32 + 16 j + r16 (column tile j holds
// 16 consecutive columns). `scratch` is LDS of at least 4 * BM floats that no
// wave reads any more.
template <int BM, bool Q8>
__device__ __forceinline__ void kproj_store_tile(
    const float4_t (&acc)[3][2], long long* row_dst, float* scratch, int tid, int m0, int n0, int T,
    const uint32_t* __restrict__ offs, const uint32_t* __restrict__ cache_len,
    const uint32_t* __restrict__ page_table, int batch, int max_pages, int num_pages, int page_size, int layer,
    int n_plane, void* __restrict__ blocks_v, float* __restrict__ kv_scales, int qgran) {
  constexpr int MT = 3;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int q = lane >> 4, r16 = lane & 15;
  const int plane = n0 / n_plane, colp = n0 - plane * n_plane;   // the tile's plane and column there
  if (tid < BM) {
    const int t = m0 + tid;
    long long dst = -1;   // cache row (layer, plane, page, slot) of token t
    if (t < T) {
      int lo = 0, hi = batch;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int)offs[mid] <= t) lo = mid; else hi = mid;
      }
      const int pos = (int)cache_len[lo] + (t - (int)offs[lo]);
      const int page = (int)page_table[(size_t)lo * max_pages + pos / page_size];
      const int slot = pos % page_size;
      dst = (((long long)layer * 2 + plane) * num_pages + page) * page_size + slot;
    }
    row_dst[tid] = dst;
  }
  __syncthreads();
  const int col = colp + wn * 32 + r16;   // column of acc[.][0]; acc[.][1]: +16
  if constexpr (!Q8) {
    uint16_t* __restrict__ blocks = static_cast<uint16_t*>(blocks_v);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long long d = row_dst[wm * 48 + mt * 16 + q * 4 + i];
        if (d >= 0) {
          blocks[d * n_plane + col] = f2bf_rn(acc[mt][0][i]);
          blocks[d * n_plane + col + 16] = f2bf_rn(acc[mt][1][i]);
        }
      }
    }
  } else {
    uint8_t* __restrict__ blocks = static_cast<uint8_t*>(blocks_v);
    // amax of each of the lane's rows over the wave's 32 columns
    float am[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = fmaxf(fabsf(acc[mt][0][i]), fabsf(acc[mt][1][i]));
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
        am[mt][i] = a;
      }
    }
    const int gw = qgran / 32;   // waves per run of qgran columns: 1, 2 or 4 (workgroup-uniform)
    if (gw > 1) {
      float* amx = scratch;      // [wave column][row]
      if (r16 == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) amx[wn * BM + wm * 48 + mt * 16 + q * 4 + i] = am[mt][i];
      }
      __syncthreads();
      const int w0 = wn & ~(gw - 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wm * 48 + mt * 16 + q * 4 + i;
          float a = amx[w0 * BM + row];
          for (int w = 1; w < gw; ++w) a = fmaxf(a, amx[(w0 + w) * BM + row]);
          am[mt][i] = a;
        }
      }
    }
    const int nsc = n_plane / qgran;   // scales per cache row
    const bool scale_writer = r16 == 0 && (wn & (gw - 1)) == 0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long long d = row_dst[wm * 48 + mt * 16 + q * 4 + i];
        if (d < 0) continue;
        const float sc = am[mt][i] / 448.0f;   // correctly rounded fp32 division
        const float v0 = sc > 0.f ? acc[mt][0][i] / sc : 0.f;
        const float v1 = sc > 0.f ? acc[mt][1][i] / sc : 0.f;
        const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);   // nearest even, low half
        blocks[d * n_plane + col] = (uint8_t)pk;
        blocks[d * n_plane + col + 16] = (uint8_t)(pk >> 8);
        if (scale_writer) kv_scales[d * nsc + (colp + wn * 32) / qgran] = sc;
      }
    }
  }
}

// e4m3-hidden design: fp8 (e4m3) hidden rows, so both operands are fp8 and one
// v_mfma_scale_f32_16x16x128_f8f6f4 (unit block scales) covers a 16 x 16 output
// tile over a whole 128-deep scale block; its fp32 result is scaled by
// is[t][kb] * ws[kb][nb] and added to the accumulator, as in the raw-weight design below,
// whose tiles, waves and epilogue it shares (BM = 48 * WM rows x 128 columns,
// 48 x 32 wave tiles).
//   * Both tiles stay fp8 in LDS, copied as they are: hidden rows [BM][128 B]
//     and the weight tile [128 k][128 n], 16-byte chunks XOR-swizzled by the
//     low three row bits. No conversion, no transposed writes.
//   * A fragment (row r16, K 32q .. 32q + 31): two 16-byte reads. B fragment
//     (column r16, the same K): four 8-bit transpose reads
//     (ds_read_b64_tr_b8); within each 16-lane group, lane m names K row
//     32q + 8s + m / 2 and byte 8 (m % 2) of the column chunk, and lane i
//     receives the eight K values of column i.
//   * Staging: the stage's hidden and weight chunks form one list dealt to the
//     threads round-robin; every thread issues the same number of loads (the
//     last round re-reads its own chunks where the list runs out) so the
//     compiler's in-order load counting sees one fixed sequence, and only
//     in-list chunks are stored. PD stages are in flight in registers: stage
//     kb + PD is requested while stage kb is multiplied, and stage kb + 1,
//     requested PD - 1 stages earlier, is stored after it (a stage's MFMAs take
//     far less time than a global load's latency).
template <int WM, bool Q8, int PD>
__global__ __launch_bounds__(WM * 256) void kproj_f8f8_kernel(
    const uint8_t* __restrict__ H, const uint32_t* __restrict__ offs, const uint8_t* __restrict__ W,
    const float* __restrict__ in_scale, const float* __restrict__ w_scale, void* __restrict__ blocks_v,
    const uint32_t* __restrict__ cache_len, const uint32_t* __restrict__ page_table, int T, int Kh, int N,
    int batch, int max_pages, int num_pages, int page_size, int layer, int tiles_m, int tiles_n, int n_plane,
    float* __restrict__ kv_scales, int qgran) {
  constexpr int BM = 48 * WM;
  constexpr int NTHR = WM * 256;
  constexpr int MT = 3;
  constexpr int ACH = BM * 8;                          // 16-byte hidden chunks per stage
  constexpr int BCH = 128 * 8;                         // 16-byte weight chunks per stage
  constexpr int LOADS = (ACH + BCH + NTHR - 1) / NTHR;  // loads per thread per stage
  __shared__ __attribute__((aligned(16))) u32x4_t lds_a[2][ACH];
  __shared__ __attribute__((aligned(16))) u32x4_t lds_b[2][BCH];
  __shared__ __attribute__((aligned(16))) float lds_is[KSW * BM];   // [kb % KSW][row]: a window of KSW blocks
  __shared__ long long row_dst[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int q = lane >> 4, r16 = lane & 15;

  const int tiles = tiles_m * tiles_n;
  const int per = (tiles + 7) >> 3;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= tiles) return;
  const int m0 = (lin / tiles_n) * BM;   // N-fastest: the column tiles of a row block share an XCD
  const int nb = lin % tiles_n;
  const int n0 = nb * KBN;
  const int KB = Kh / KBK;

  // this thread's chunks: source (byte offset at stage 0, bytes per stage) and LDS slot
  const uint8_t* src[LOADS];
  uint32_t sstep[LOADS];
  int slot[LOADS];   // index into lds_a (< ACH) or ACH + index into lds_b; -1: not stored
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int id0 = tid + i * NTHR;
    const bool in_list = id0 < ACH + BCH;
    const int id = in_list ? id0 : id0 - NTHR;   // re-read this thread's previous chunk
    if (id < ACH) {
      const int row = id >> 3, ch = id & 7;
      src[i] = H + (size_t)min(m0 + row, T - 1) * Kh + ch * 16;
      sstep[i] = KBK;
      slot[i] = row * 8 + (ch ^ (row & 7));
    } else {
      const int j = id - ACH, kr = j >> 3, ch = j & 7;
      src[i] = W + (size_t)kr * N + n0 + ch * 16;
      sstep[i] = (uint32_t)KBK * (uint32_t)N;
      slot[i] = ACH + kr * 8 + (ch ^ (kr & 7));
    }
    if (!in_list) slot[i] = -1;
  }
  auto load_stage = [&](int kb, u32x4_t (&r)[LOADS]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      r[i] = *reinterpret_cast<const u32x4_t*>(src[i] + (size_t)kb * sstep[i]);
  };
  auto store_stage = [&](int buf, const u32x4_t (&r)[LOADS]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if (slot[i] < 0) continue;
      if (slot[i] < ACH) lds_a[buf][slot[i]] = r[i];
      else lds_b[buf][slot[i] - ACH] = r[i];
    }
  };

  // input scales of the tile's rows, KSW blocks at a time (refilled every KSW stages)
  auto fill_is = [&](int kb0) {
    const int nb_is = min(KSW, KB - kb0);
    for (int e = tid; e < nb_is * BM; e += NTHR) {
      const int row = e % BM, kb = e / BM;
      lds_is[kb * BM + row] = in_scale[(size_t)min(m0 + row, T - 1) * KB + kb0 + kb];
    }
  };
  fill_is(0);

  float4_t acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i][0] = acc[i][1] = float4_t{0.f, 0.f, 0.f, 0.f};

  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  auto compute = [&](int kb, int buf) {
    i32x8_t bf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int c = wn * 2 + t;   // the column chunk of column tile t
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int kr = 32 * q + 8 * s4 + (r16 >> 1);
        const unsigned char* base = reinterpret_cast<const unsigned char*>(&lds_b[buf][kr * 8 + (c ^ (kr & 7))]) +
                                    8 * (r16 & 1);
        const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(__attribute__((address_space(3))) const unsigned char*)base);
        bf[t][2 * s4] = v.x;
        bf[t][2 * s4 + 1] = v.y;
      }
    }
    const float wsv = w_scale[(size_t)kb * (N / KBN) + nb];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = wm * 48 + mt * 16 + r16;
      const u32x4_t lo = lds_a[buf][row * 8 + ((2 * q) ^ (row & 7))];
      const u32x4_t hi = lds_a[buf][row * 8 + ((2 * q + 1) ^ (row & 7))];
      const i32x8_t av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const float4_t is4 = *reinterpret_cast<const float4_t*>(&lds_is[(kb % KSW) * BM + wm * 48 + mt * 16 + q * 4]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float4_t part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            av, bf[t], float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);   // e4m3 x e4m3, unit scales
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][t][i] += is4[i] * wsv * part[i];
      }
    }
  };

  u32x4_t rg[PD][LOADS];
#pragma unroll
  for (int p = 0; p < PD; ++p) load_stage(min(p, KB - 1), rg[p]);
  store_stage(0, rg[0]);
  __syncthreads();
  for (int kb = 0; kb < KB; kb += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int i = kb + p;   // stage multiplied now; rg[p] (stage i, stored) takes stage i + PD
      if (i < KB && i > 0 && i % KSW == 0) {   // the next window of input scales (uniform test;
        fill_is(i);                            // every wave left the previous one at the last barrier)
        __syncthreads();
      }
      if constexpr (PD > 1) load_stage(min(i + PD, KB - 1), rg[p]);   // past the end: re-reads, unstored
      else load_stage(min(i + 1, KB - 1), rg[0]);
      __builtin_amdgcn_sched_barrier(0);
      if (i < KB) compute(i, i & 1);
      if (i + 1 < KB) store_stage((i + 1) & 1, rg[(p + 1) % PD]);
      __syncthreads();
    }
  }

  // column tile t of a wave holds 16 consecutive columns (the transpose read's order)
  kproj_store_tile<BM, Q8>(acc, row_dst, lds_is, tid, m0, n0, T, offs, cache_len, page_table, batch,
                                 max_pages, num_pages, page_size, layer, n_plane, blocks_v, kv_scales, qgran);
}

// Raw-weight design for bf16 hidden rows: the e4m3-hidden design's staging
// (both tiles copied into LDS as they are, one round-robin list of 16-byte
// chunks, PD stages of loads in flight) with bf16 MFMAs.
//   * Hidden rows: [BM][256 B] per 128-deep stage, 16-byte chunks XOR-swizzled
//     by the low four row bits. A fragment (row r16, K 32s + 8q .. + 7): one
//     16-byte read.
//   * Weight tile: [128 k][128 n] e4m3, chunks swizzled by the low three row
//     bits. B fragment (column 16c + r16 of chunk c, the same K): one 8-bit
//     transpose read (lane m names K row 32s + 8q + m / 2 and byte 8 (m % 2) of
//     the chunk; lane i receives the eight K values of column i), then four
//     v_cvt_scalef32_pk_bf16_fp8 at scale 1 (exact: every e4m3 value is a bf16
//     value). Each wave converts its own fragments; nothing is transposed or
//     converted on the way into LDS.
//   * 16x16x32 bf16 MFMAs on 48 x 32 wave tiles (column tile t of a wave holds
//     16 consecutive columns), the stage's partials scaled once by
//     is[t][kb] * ws[kb][nb], and the shared epilogue.
template <int WM, bool Q8, int PD>
__global__ __launch_bounds__(WM * 256) void kproj_bf16_kernel(
    const uint16_t* __restrict__ H, const uint32_t* __restrict__ offs, const uint8_t* __restrict__ W,
    const float* __restrict__ in_scale, const float* __restrict__ w_scale, void* __restrict__ blocks_v,
    const uint32_t* __restrict__ cache_len, const uint32_t* __restrict__ page_table, int T, int Kh, int N,
    int batch, int max_pages, int num_pages, int page_size, int layer, int tiles_m, int tiles_n, int n_plane,
    float* __restrict__ kv_scales, int qgran) {
  constexpr int BM = 48 * WM;
  constexpr int NTHR = WM * 256;
  constexpr int MT = 3;
  constexpr int ACH = BM * KCH;                        // 16-byte hidden chunks per stage (16 per row)
  constexpr int BCH = 128 * 8;                         // 16-byte weight chunks per stage (8 per K row)
  constexpr int LOADS = (ACH + BCH + NTHR - 1) / NTHR;  // loads per thread per stage
  __shared__ __attribute__((aligned(16))) u32x4_t lds_a[2][ACH];
  __shared__ __attribute__((aligned(16))) u32x4_t lds_b[2][BCH];
  __shared__ __attribute__((aligned(16))) float lds_is[KSW * BM];   // [kb % KSW][row]: a window of KSW blocks
  __shared__ long long row_dst[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int q = lane >> 4, r16 = lane & 15;

  const int tiles = tiles_m * tiles_n;
  const int per = (tiles + 7) >> 3;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= tiles) return;
  const int m0 = (lin / tiles_n) * BM;   // N-fastest: the column tiles of a row block share an XCD
  const int nb = lin % tiles_n;
  const int n0 = nb * KBN;
  const int KB = Kh / KBK;

  // this thread's chunks: source at stage 0, bytes per stage, LDS slot
  const uint8_t* src[LOADS];
  uint32_t sstep[LOADS];
  int slot[LOADS];   // index into lds_a (< ACH) or ACH + index into lds_b; -1: not stored
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int id0 = tid + i * NTHR;
    const bool in_list = id0 < ACH + BCH;
    const int id = in_list ? id0 : id0 - NTHR;   // re-read this thread's previous chunk
    if (id < ACH) {
      const int row = id / KCH, ch = id % KCH;
      src[i] = reinterpret_cast<const uint8_t*>(H + (size_t)min(m0 + row, T - 1) * Kh) + ch * 16;
      sstep[i] = KBK * 2;
      slot[i] = row * KCH + swz_a(row, ch);
    } else {
      const int j = id - ACH, kr = j >> 3, ch = j & 7;
      src[i] = W + (size_t)kr * N + n0 + ch * 16;
      sstep[i] = (uint32_t)KBK * (uint32_t)N;
      slot[i] = ACH + kr * 8 + (ch ^ (kr & 7));
    }
    if (!in_list) slot[i] = -1;
  }
  auto load_stage = [&](int kb, u32x4_t (&r)[LOADS]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      r[i] = *reinterpret_cast<const u32x4_t*>(src[i] + (size_t)kb * sstep[i]);
  };
  auto store_stage = [&](int buf, const u32x4_t (&r)[LOADS]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if (slot[i] < 0) continue;
      if (slot[i] < ACH) lds_a[buf][slot[i]] = r[i];
      else lds_b[buf][slot[i] - ACH] = r[i];
    }
  };

  // input scales of the tile's rows, KSW blocks at a time (refilled every KSW stages)
  auto fill_is = [&](int kb0) {
    const int nb_is = min(KSW, KB - kb0);
    for (int e = tid; e < nb_is * BM; e += NTHR) {
      const int row = e % BM, kb = e / BM;
      lds_is[kb * BM + row] = in_scale[(size_t)min(m0 + row, T - 1) * KB + kb0 + kb];
    }
  };
  fill_is(0);

  float4_t acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i][0] = acc[i][1] = float4_t{0.f, 0.f, 0.f, 0.f};

  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  auto compute = [&](int kb, int buf) {
    float4_t part[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i) part[i][0] = part[i][1] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t bf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int c = wn * 2 + t;   // the column chunk of column tile t
        const int kr = 32 * s + 8 * q + (r16 >> 1);
        const unsigned char* base =
            reinterpret_cast<const unsigned char*>(&lds_b[buf][kr * 8 + (c ^ (kr & 7))]) + 8 * (r16 & 1);
        const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(__attribute__((address_space(3))) const unsigned char*)base);
        bf[t] = u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true))};
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = wm * 48 + mt * 16 + r16;
        const u32x4_t av = lds_a[buf][row * KCH + swz_a(row, s * 4 + q)];
        part[mt][0] = mfma16x16x32_bf16(av, bf[0], part[mt][0]);
        part[mt][1] = mfma16x16x32_bf16(av, bf[1], part[mt][1]);
      }
    }
    const float wsv = w_scale[(size_t)kb * (N / KBN) + nb];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float4_t is4 = *reinterpret_cast<const float4_t*>(&lds_is[(kb % KSW) * BM + wm * 48 + mt * 16 + q * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f = is4[i] * wsv;
        acc[mt][0][i] += f * part[mt][0][i];
        acc[mt][1][i] += f * part[mt][1][i];
      }
    }
  };

  u32x4_t rg[PD][LOADS];
#pragma unroll
  for (int p = 0; p < PD; ++p) load_stage(min(p, KB - 1), rg[p]);
  store_stage(0, rg[0]);
  __syncthreads();
  for (int kb = 0; kb < KB; kb += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int i = kb + p;   // stage multiplied now; rg[p] (stage i, stored) takes stage i + PD
      if (i < KB && i > 0 && i % KSW == 0) {   // the next window of input scales (uniform test;
        fill_is(i);                            // every wave left the previous one at the last barrier)
        __syncthreads();
      }
      if constexpr (PD > 1) load_stage(min(i + PD, KB - 1), rg[p]);   // past the end: re-reads, unstored
      else load_stage(min(i + 1, KB - 1), rg[0]);
      __builtin_amdgcn_sched_barrier(0);
      if (i < KB) compute(i, i & 1);
      if (i + 1 < KB) store_stage((i + 1) & 1, rg[(p + 1) % PD]);
      __syncthreads();
    }
  }

  kproj_store_tile<BM, Q8>(acc, row_dst, lds_is, tid, m0, n0, T, offs, cache_len, page_table, batch,
                                 max_pages, num_pages, page_size, layer, n_plane, blocks_v, kv_scales, qgran);
}



// Direct-to-LDS design for 144-row tiles (bf16 hidden rows).
//   * Staging: every 16-byte chunk of the hidden and weight tiles, and the
//     tile rows' input scales, go from global memory straight into LDS with
//     global_load_lds (a wave's instruction fills 1 KiB of LDS, lane l at
//     byte 16 l, so each lane fetches the chunk that the swizzled layout puts
//     there). No registers hold staged data, so three stage buffers keep two
//     stages of loads in flight behind the one being multiplied.
//   * Twelve waves on 48 x 32 tiles, fragments and conversions as in
//     kproj_bf16_kernel.
//   * A stage's partials are scaled by is[t][kb] * ws[kb][nb] and added to the
//     accumulators during the next stage, among its MFMAs, so no wave waits
//     for its last MFMAs before the stage barrier.
template <bool Q8>
__global__ __launch_bounds__(768) void kproj_bf16_dma_kernel(
    const uint16_t* __restrict__ H, const uint32_t* __restrict__ offs, const uint8_t* __restrict__ W,
    const float* __restrict__ in_scale, const float* __restrict__ w_scale, void* __restrict__ blocks_v,
    const uint32_t* __restrict__ cache_len, const uint32_t* __restrict__ page_table, int T, int Kh, int N,
    int batch, int max_pages, int num_pages, int page_size, int layer, int tiles_m, int tiles_n, int n_plane,
    float* __restrict__ kv_scales, int qgran) {
  constexpr int BM = 144, MT = 3, NBUF = 3;
  constexpr int ACH = BM * KCH;   // 16-byte hidden chunks per stage: 36 wave loads of 1 KiB
  constexpr int BCH = 128 * 8;    // 16-byte weight chunks per stage: 16 wave loads
  __shared__ __attribute__((aligned(1024))) u32x4_t lds_a[NBUF][ACH];
  __shared__ __attribute__((aligned(1024))) u32x4_t lds_b[NBUF][BCH];
  __shared__ __attribute__((aligned(16))) float lds_is[NBUF][BM];
  __shared__ long long row_dst[BM];
  static_assert(sizeof(lds_b) >= 4 * BM * sizeof(float), "room for the epilogue's scratch");
  static_assert(ACH == 36 * 64 && BCH == 16 * 64, "wave loads per stage");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int q = lane >> 4, r16 = lane & 15;

  const int tiles = tiles_m * tiles_n;
  const int per = (tiles + 7) >> 3;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= tiles) return;
  const int m0 = (lin / tiles_n) * BM;   // N-fastest: the column tiles of a row block share an XCD
  const int nb = lin % tiles_n;
  const int n0 = nb * KBN;
  const int KB = Kh / KBK;

  // wave loads: hidden 1 KiB blocks wave, wave + 12, wave + 24 (rows 4a .. 4a + 3 each);
  // weight blocks wave and, for waves 0-3, wave + 12 (K rows 8b .. 8b + 7 each);
  // waves 4-6: the input scales of rows 64 (wave - 4) + lane
  const uint8_t* hb = reinterpret_cast<const uint8_t*>(H + (size_t)m0 * Kh);
  uint32_t aoff[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int row = 4 * (wave + 12 * j) + (lane >> 4);
    const int ch = (lane & 15) ^ (row & 15);
    aoff[j] = (uint32_t)(min(m0 + row, T - 1) - m0) * (uint32_t)(Kh * 2) + ch * 16;
  }
  uint32_t boff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int kr = 8 * (wave + 12 * j) + (lane >> 3);
    boff[j] = (uint32_t)kr * (uint32_t)N + swz8(kr, lane & 7) * 16;
  }
  const int is_row = 64 * (wave - 4) + lane;
  const bool is_loader = wave >= 4 && wave < 7;
  const uint32_t is_off = (uint32_t)(min(m0 + (is_loader ? is_row : 0), T - 1) - m0) * (uint32_t)KB * 4u;
  // LDS byte address of a __shared__ location (the global_load_lds destination base, in M0)
  auto lds_addr = [](const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
  };
  auto issue = [&](int kb, int buf) {
    const uint8_t* ha = hb + (size_t)kb * (KBK * 2);
    const uint8_t* wk = W + (size_t)kb * KBK * N + n0;
#pragma unroll
    for (int j = 0; j < 3; ++j) dma16(ha, aoff[j], lds_addr(&lds_a[buf][(wave + 12 * j) * 64]));
    dma16(wk, boff[0], lds_addr(&lds_b[buf][wave * 64]));
    if (wave < 4) dma16(wk, boff[1], lds_addr(&lds_b[buf][(wave + 12) * 64]));
    if (is_loader) dma4_lanes(in_scale + (size_t)m0 * KB + kb, is_off, lds_addr(&lds_is[buf][64 * (wave - 4)]), is_row < BM);
  };
  // wait until at most the last stage's loads of this wave are in flight
  auto wait_all_but_one_stage = [&]() {
    if (wave < 7) __builtin_amdgcn_s_waitcnt(0xF75);   // vmcnt(5): waves 0-6 issue five loads per stage
    else __builtin_amdgcn_s_waitcnt(0xF74);            // vmcnt(4)
  };

  float4_t acc[MT][2], pp[MT][2];   // accumulators; the previous stage's partials
  float pf[MT][4];                   // and their factors is * ws
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    acc[i][0] = acc[i][1] = pp[i][0] = pp[i][1] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) pf[i][j] = 0.f;
  }
  auto fold_prev = [&]() {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[mt][0][i] += pf[mt][i] * pp[mt][0][i];
        acc[mt][1][i] += pf[mt][i] * pp[mt][1][i];
      }
    // keep the additions here: left to itself the compiler sinks them to the
    // end of the unrolled loop and keeps every stage's partials alive
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) asm volatile("" : "+v"(acc[mt][0]), "+v"(acc[mt][1]));
  };

  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  auto compute = [&](int kb, int buf) {
    float4_t part[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i) part[i][0] = part[i][1] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t bf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int c = wn * 2 + t;   // the column chunk of column tile t
        const int kr = 32 * s + 8 * q + (r16 >> 1);
        const unsigned char* base =
            reinterpret_cast<const unsigned char*>(&lds_b[buf][kr * 8 + swz8(kr, c)]) + 8 * (r16 & 1);
        const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(__attribute__((address_space(3))) const unsigned char*)base);
        bf[t] = u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true))};
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = wm * 48 + mt * 16 + r16;
        const u32x4_t av = lds_a[buf][row * KCH + swz_a(row, s * 4 + q)];
        part[mt][0] = mfma16x16x32_bf16(av, bf[0], part[mt][0]);
        part[mt][1] = mfma16x16x32_bf16(av, bf[1], part[mt][1]);
      }
      if (s == 1) fold_prev();   // the previous stage's partials, while these MFMAs run
    }
    const float wsv = w_scale[(size_t)kb * (N / KBN) + nb];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float4_t is4 = *reinterpret_cast<const float4_t*>(&lds_is[buf][wm * 48 + mt * 16 + q * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) pf[mt][i] = is4[i] * wsv;
      pp[mt][0] = part[mt][0];
      pp[mt][1] = part[mt][1];
    }
  };

  issue(0, 0);
  if (KB > 1) {
    issue(1, 1);
    wait_all_but_one_stage();
  } else {
    __builtin_amdgcn_s_waitcnt(0xF70);
  }
  __syncthreads();
  // one stage: loads for stage i + 2 (into the buffer that stage i - 1 left at the
  // last barrier), the MFMAs of stage i, then wait until stage i + 1 has landed
  auto stage = [&](int i, int buf) {
    if (i + 2 < KB) issue(i + 2, (buf + 2) % NBUF);
    compute(i, buf);
    if (i + 2 < KB) wait_all_but_one_stage();
    else __builtin_amdgcn_s_waitcnt(0xF70);
    __syncthreads();
  };
  int kb0 = 0;
  for (; kb0 + 2 * NBUF <= KB; kb0 += 2 * NBUF) {   // two rounds of the buffers: the partials alternate too
#pragma unroll
    for (int u = 0; u < 2 * NBUF; ++u) stage(kb0 + u, u % NBUF);
  }
  for (; kb0 < KB; ++kb0) stage(kb0, kb0 % NBUF);
  fold_prev();

  kproj_store_tile<BM, Q8>(acc, row_dst, reinterpret_cast<float*>(&lds_b[0][0]), tid, m0, n0, T, offs, cache_len,
                           page_table, batch, max_pages, num_pages, page_size, layer, n_plane, blocks_v, kv_scales,
                           qgran);
}

// Direct-to-LDS design of the e4m3-hidden kernel for 144-row tiles: staging as
// in kproj_bf16_dma_kernel (hidden, weight and input-scale chunks straight into
// NBUF LDS stage buffers, NBUF - 1 stages of loads in flight), fragments and
// MFMAs as in kproj_f8f8_kernel, and each stage's six MFMA results scaled and
// added during the next stage.
template <bool Q8, int NBUF>
__global__ __launch_bounds__(768) void kproj_f8f8_dma_kernel(
    const uint8_t* __restrict__ H, const uint32_t* __restrict__ offs, const uint8_t* __restrict__ W,
    const float* __restrict__ in_scale, const float* __restrict__ w_scale, void* __restrict__ blocks_v,
    const uint32_t* __restrict__ cache_len, const uint32_t* __restrict__ page_table, int T, int Kh, int N,
    int batch, int max_pages, int num_pages, int page_size, int layer, int tiles_m, int tiles_n, int n_plane,
    float* __restrict__ kv_scales, int qgran) {
  constexpr int BM = 144, MT = 3;
  constexpr int ACH = BM * 8;     // 16-byte hidden chunks per stage: 18 wave loads of 1 KiB
  constexpr int BCH = 128 * 8;    // 16-byte weight chunks per stage: 16 wave loads
  __shared__ __attribute__((aligned(1024))) u32x4_t lds_a[NBUF][ACH];
  __shared__ __attribute__((aligned(1024))) u32x4_t lds_b[NBUF][BCH];
  __shared__ __attribute__((aligned(16))) float lds_is[NBUF][BM];
  __shared__ long long row_dst[BM];
  static_assert(sizeof(lds_b) >= 4 * BM * sizeof(float), "room for the epilogue's scratch");
  static_assert(ACH == 18 * 64 && BCH == 16 * 64, "wave loads per stage");
  static_assert(NBUF == 3 || NBUF == 4, "stage buffers");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int q = lane >> 4, r16 = lane & 15;

  const int tiles = tiles_m * tiles_n;
  const int per = (tiles + 7) >> 3;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= tiles) return;
  const int m0 = (lin / tiles_n) * BM;   // N-fastest: the column tiles of a row block share an XCD
  const int nb = lin % tiles_n;
  const int n0 = nb * KBN;
  const int KB = Kh / KBK;

  // wave loads: hidden 1 KiB blocks wave and, for waves 0-5, wave + 12 (rows 8a .. 8a + 7 each);
  // weight blocks wave and, for waves 0-3, wave + 12 (K rows 8b .. 8b + 7 each);
  // waves 6-8: the input scales of rows 64 (wave - 6) + lane
  const uint8_t* hb = H + (size_t)m0 * Kh;
  uint32_t aoff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 8 * (wave + 12 * j) + (lane >> 3);
    const int ch = swz8(row, lane & 7);
    aoff[j] = (uint32_t)(min(m0 + row, T - 1) - m0) * (uint32_t)Kh + ch * 16;
  }
  uint32_t boff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int kr = 8 * (wave + 12 * j) + (lane >> 3);
    boff[j] = (uint32_t)kr * (uint32_t)N + swz8b5(kr, lane & 7) * 16;
  }
  const int is_row = 64 * (wave - 6) + lane;
  const bool is_loader = wave >= 6 && wave < 9;
  const uint32_t is_off = (uint32_t)(min(m0 + (is_loader ? is_row : 0), T - 1) - m0) * (uint32_t)KB * 4u;
  const int nw = 2 + (wave < 6) + (wave < 4) + is_loader;   // loads per stage of this wave: 2 .. 4
  auto lds_addr = [](const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
  };
  auto issue = [&](int kb, int buf) {
    const uint8_t* ha = hb + (size_t)kb * KBK;
    const uint8_t* wk = W + (size_t)kb * KBK * N + n0;
    dma16(ha, aoff[0], lds_addr(&lds_a[buf][wave * 64]));
    if (wave < 6) dma16(ha, aoff[1], lds_addr(&lds_a[buf][(wave + 12) * 64]));
    dma16(wk, boff[0], lds_addr(&lds_b[buf][wave * 64]));
    if (wave < 4) dma16(wk, boff[1], lds_addr(&lds_b[buf][(wave + 12) * 64]));
    if (is_loader) dma4_lanes(in_scale + (size_t)m0 * KB + kb, is_off, lds_addr(&lds_is[buf][64 * (wave - 6)]), is_row < BM);
  };
  // wait until at most `n` of this wave's loads are in flight (n: 0 .. 8, uniform)
  auto wait_loads = [](int n) {
    switch (n) {
      case 0: __builtin_amdgcn_s_waitcnt(0xF70); break;
      case 1: __builtin_amdgcn_s_waitcnt(0xF71); break;
      case 2: __builtin_amdgcn_s_waitcnt(0xF72); break;
      case 3: __builtin_amdgcn_s_waitcnt(0xF73); break;
      case 4: __builtin_amdgcn_s_waitcnt(0xF74); break;
      case 5: __builtin_amdgcn_s_waitcnt(0xF75); break;
      case 6: __builtin_amdgcn_s_waitcnt(0xF76); break;
      case 7: __builtin_amdgcn_s_waitcnt(0xF77); break;
      default: __builtin_amdgcn_s_waitcnt(0xF78); break;
    }
  };

  float4_t acc[MT][2], pp[MT][2];   // accumulators; the previous stage's MFMA results
  float pf[MT][4];                   // and their factors is * ws
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    acc[i][0] = acc[i][1] = pp[i][0] = pp[i][1] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) pf[i][j] = 0.f;
  }
  auto fold_prev = [&]() {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[mt][0][i] += pf[mt][i] * pp[mt][0][i];
        acc[mt][1][i] += pf[mt][i] * pp[mt][1][i];
      }
    // keep the additions here (see kproj_bf16_dma_kernel)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) asm volatile("" : "+v"(acc[mt][0]), "+v"(acc[mt][1]));
  };

  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  auto compute = [&](int kb, int buf) {
    i32x8_t bf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int c = wn * 2 + t;   // the column chunk of column tile t
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int kr = 32 * q + 8 * s4 + (r16 >> 1);
        const unsigned char* base = reinterpret_cast<const unsigned char*>(&lds_b[buf][kr * 8 + swz8b5(kr, c)]) +
                                    8 * (r16 & 1);
        const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(__attribute__((address_space(3))) const unsigned char*)base);
        bf[t][2 * s4] = v.x;
        bf[t][2 * s4 + 1] = v.y;
      }
    }
    float4_t part[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = wm * 48 + mt * 16 + r16;
      const u32x4_t lo = lds_a[buf][row * 8 + swz8(row, 2 * q)];
      const u32x4_t hi = lds_a[buf][row * 8 + swz8(row, 2 * q + 1)];
      const i32x8_t av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
      for (int t = 0; t < 2; ++t)
        part[mt][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            av, bf[t], float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);   // e4m3 x e4m3, unit scales
      if (mt == 0) fold_prev();   // the previous stage's results, while these MFMAs run
    }
    const float wsv = w_scale[(size_t)kb * (N / KBN) + nb];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float4_t is4 = *reinterpret_cast<const float4_t*>(&lds_is[buf][wm * 48 + mt * 16 + q * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) pf[mt][i] = is4[i] * wsv;
      pp[mt][0] = part[mt][0];
      pp[mt][1] = part[mt][1];
    }
  };

  // prologue: stages 0 .. NBUF - 2 in flight, stage 0 landed
  for (int p = 0; p < NBUF - 1; ++p)
    if (p < KB) issue(p, p);
  wait_loads(nw * (min(NBUF - 1, KB) - 1));
  __syncthreads();
  // one stage: loads for stage i + NBUF - 1 (into the buffer that stage i - 1 left
  // at the last barrier), the MFMAs of stage i, then wait until stage i + 1 has landed
  auto stage = [&](int i, int buf) {
    const bool more = i + NBUF - 1 < KB;
    if (more) issue(i + NBUF - 1, (buf + NBUF - 1) % NBUF);
    compute(i, buf);
    wait_loads(nw * max(0, min(NBUF - 2, KB - 2 - i)));   // stages i + 2 .. may stay in flight
    __syncthreads();
  };
  constexpr int UNR = NBUF % 2 ? 2 * NBUF : NBUF;   // whole rounds of the buffers and of the alternating partials
  int kb0 = 0;
  for (; kb0 + UNR <= KB; kb0 += UNR) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) stage(kb0 + u, u % NBUF);
  }
  for (; kb0 < KB; ++kb0) stage(kb0, kb0 % NBUF);
  fold_prev();

  kproj_store_tile<BM, Q8>(acc, row_dst, reinterpret_cast<float*>(&lds_b[0][0]), tid, m0, n0, T, offs, cache_len,
                           page_table, batch, max_pages, num_pages, page_size, layer, n_plane, blocks_v, kv_scales,
                           qgran);
}

template <int WM, int PD>
static hipError_t launch_kproj_bf16(const KProjArgs& p, hipStream_t stream) {
  constexpr int BM = 48 * WM;
  const int tiles_m = (int)((p.T + BM - 1) / BM), tiles_n = (int)(p.N / KBN);
  const int grid = ((tiles_m * tiles_n + 7) / 8) * 8;
  // 144-row tiles: the direct-to-LDS design; 48 and 96 rows: staging through registers
  if constexpr (WM == 3) {
    if (p.fp8)
      hipLaunchKernelGGL((kproj_bf16_dma_kernel<true>), dim3(grid), dim3(768), 0, stream, p.hidden, p.row_offsets,
                         p.weight, p.input_scale, p.weight_scale, p.blocks, p.cache_lengths, p.page_table, (int)p.T,
                         (int)p.Kh, (int)p.N, (int)p.batch, (int)p.max_pages, (int)p.num_pages, (int)p.page_size,
                         (int)p.layer_idx, tiles_m, tiles_n, (int)p.n_plane, p.kv_scales, p.qgran);
    else
      hipLaunchKernelGGL((kproj_bf16_dma_kernel<false>), dim3(grid), dim3(768), 0, stream, p.hidden, p.row_offsets,
                         p.weight, p.input_scale, p.weight_scale, p.blocks, p.cache_lengths, p.page_table, (int)p.T,
                         (int)p.Kh, (int)p.N, (int)p.batch, (int)p.max_pages, (int)p.num_pages, (int)p.page_size,
                         (int)p.layer_idx, tiles_m, tiles_n, (int)p.n_plane, nullptr, 0);
  } else {
    if (p.fp8)
      hipLaunchKernelGGL((kproj_bf16_kernel<WM, true, PD>), dim3(grid), dim3(WM * 256), 0, stream, p.hidden,
                         p.row_offsets, p.weight, p.input_scale, p.weight_scale, p.blocks, p.cache_lengths,
                         p.page_table, (int)p.T, (int)p.Kh, (int)p.N, (int)p.batch, (int)p.max_pages,
                         (int)p.num_pages, (int)p.page_size, (int)p.layer_idx, tiles_m, tiles_n, (int)p.n_plane,
                         p.kv_scales, p.qgran);
    else
      hipLaunchKernelGGL((kproj_bf16_kernel<WM, false, PD>), dim3(grid), dim3(WM * 256), 0, stream, p.hidden,
                         p.row_offsets, p.weight, p.input_scale, p.weight_scale, p.blocks, p.cache_lengths,
                         p.page_table, (int)p.T, (int)p.Kh, (int)p.N, (int)p.batch, (int)p.max_pages,
                         (int)p.num_pages, (int)p.page_size, (int)p.layer_idx, tiles_m, tiles_n, (int)p.n_plane,
                         nullptr, 0);
  }
  return hipGetLastError();
}

template <int WM, int PD>
static hipError_t launch_kproj_f8f8(const KProjArgs& p, hipStream_t stream) {
  constexpr int BM = 48 * WM;
  const int tiles_m = (int)((p.T + BM - 1) / BM), tiles_n = (int)(p.N / KBN);
  const int grid = ((tiles_m * tiles_n + 7) / 8) * 8;
  const uint8_t* h = static_cast<const uint8_t*>(static_cast<const void*>(p.hidden));
  // 144-row tiles: the direct-to-LDS design; 48 and 96 rows: staging through registers
  if constexpr (WM == 3) {
    constexpr int NB = 3;   // a fourth buffer measured slower
    if (p.fp8)
      hipLaunchKernelGGL((kproj_f8f8_dma_kernel<true, NB>), dim3(grid), dim3(768), 0, stream, h, p.row_offsets,
                         p.weight, p.input_scale, p.weight_scale, p.blocks, p.cache_lengths, p.page_table, (int)p.T,
                         (int)p.Kh, (int)p.N, (int)p.batch, (int)p.max_pages, (int)p.num_pages, (int)p.page_size,
                         (int)p.layer_idx, tiles_m, tiles_n, (int)p.n_plane, p.kv_scales, p.qgran);
    else
      hipLaunchKernelGGL((kproj_f8f8_dma_kernel<false, NB>), dim3(grid), dim3(768), 0, stream, h, p.row_offsets,
                         p.weight, p.input_scale, p.weight_scale, p.blocks, p.cache_lengths, p.page_table, (int)p.T,
                         (int)p.Kh, (int)p.N, (int)p.batch, (int)p.max_pages, (int)p.num_pages, (int)p.page_size,
                         (int)p.layer_idx, tiles_m, tiles_n, (int)p.n_plane, nullptr, 0);
  } else {
    if (p.fp8)
      hipLaunchKernelGGL((kproj_f8f8_kernel<WM, true, PD>), dim3(grid), dim3(WM * 256), 0, stream, h,
                         p.row_offsets, p.weight, p.input_scale, p.weight_scale, p.blocks, p.cache_lengths,
                         p.page_table, (int)p.T, (int)p.Kh, (int)p.N, (int)p.batch, (int)p.max_pages,
                         (int)p.num_pages, (int)p.page_size, (int)p.layer_idx, tiles_m, tiles_n, (int)p.n_plane,
                         p.kv_scales, p.qgran);
    else
      hipLaunchKernelGGL((kproj_f8f8_kernel<WM, false, PD>), dim3(grid), dim3(WM * 256), 0, stream, h,
                         p.row_offsets, p.weight, p.input_scale, p.weight_scale, p.blocks, p.cache_lengths,
                         p.page_table, (int)p.T, (int)p.Kh, (int)p.N, (int)p.batch, (int)p.max_pages,
                         (int)p.num_pages, (int)p.page_size, (int)p.layer_idx, tiles_m, tiles_n, (int)p.n_plane,
                         nullptr, 0);
  }
  return hipGetLastError();
}

// Row-tile height from the fill of the last pass over the CUs: the tallest
// candidate within 3% of the best fill (taller tiles reuse each weight
// fragment across more rows).
static int pick_kproj_rows(const KProjArgs& p, const int* cand, int n) {
  const long long tn = p.N / KBN;
  double eff[8];
  double best_eff = 0.0;
  for (int i = 0; i < n; ++i) {
    const int bm = cand[i];
    const long long tiles = ((p.T + bm - 1) / bm) * tn;
    const long long rounds = (tiles + p.num_cus - 1) / p.num_cus;
    eff[i] = (double)p.T * tn / ((double)rounds * p.num_cus * bm);
    if (eff[i] > best_eff) best_eff = eff[i];
  }
  for (int i = n - 1; i >= 0; --i)
    if (eff[i] >= best_eff - 0.03) return cand[i];
  return cand[n - 1];
}

hipError_t launch_kproj_fp8(const KProjArgs& p, hipStream_t stream) {
  static const int cand[] = {48, 96, 144};
  // the 144-row (direct-to-LDS) kernels address a tile's hidden rows and a
  // stage's weight rows with 32-bit offsets: up to 2^23 hidden columns and 2^24
  // output columns; beyond that the 48 / 96-row kernels (64-bit addresses)
  const int nc = (p.Kh <= (1 << 23) && p.N <= (1 << 24)) ? 3 : 2;
  if (p.hidden_fp8) {
    // e4m3 hidden rows: 48, 96 or 144-row tiles
    switch (pick_kproj_rows(p, cand, nc) / 48) {
      case 1: return launch_kproj_f8f8<1, 2>(p, stream);
      case 2: return launch_kproj_f8f8<2, 2>(p, stream);
      default: return launch_kproj_f8f8<3, 2>(p, stream);
    }
  }
  switch (pick_kproj_rows(p, cand, nc) / 48) {
    case 1: return launch_kproj_bf16<1, 2>(p, stream);
    case 2: return launch_kproj_bf16<2, 2>(p, stream);
    default: return launch_kproj_bf16<3, 2>(p, stream);
  }
}

}  // namespace qg
