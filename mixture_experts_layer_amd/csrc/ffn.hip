// Grouped SwiGLU expert GEMMs over ragged per-expert row counts, gfx950.
//
// "MoE 推理优化全景指南", section Expert GEMM 为什么经常不够大: experts with
// different row counts m_i run in one schedule, expert i computing
// [m_i, hidden] @ W_i.  Expert layout per the Moebius paper, section 3.1:
// W13 (E_loc, 2I, H) with gate and up stacked, W2 (E_loc, H, I).
//
// Row counts live on the device.  The grid is sized for the worst case and
// every block reads its (expert, row range) from a tile map built by the
// routing kernels; blocks past the map's length exit at once.  Nothing is
// read back to the host.
#include <type_traits>

#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

// 16 bytes of a weight stream that no other block reads again: a
// non-temporal load (the nt cache-policy bit).  In the direct-load kernels
// below, at decode-sized batches where every weight byte is read by exactly
// one block, it ran the HBM-bound expert GEMMs 8-10% faster than plain
// loads.  The LDS-tiled prefill GEMMs reuse weight tiles across an expert's
// row tiles through the L2 and must not use it (nt on their LDS-DMA loads
// doubled their time); the single-launch decode kernel measured 5-7% slower
// with it.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8_t ld_stream16(const void* p) {
  return __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(static_cast<const u32x4_t*>(p)));
}
__device__ __forceinline__ uint4 ld_stream16_u4(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 16-byte store with the non-temporal hint
__device__ __forceinline__ void st_stream16(bf16_t* p, const uint4& v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

struct DirectArgs {
  const bf16_t* X;          // activation rows, K contiguous
  const int32_t* src_token; // null: row r reads X row r; else X row src_token[r]
  const int4* tile_map;     // null: dense rows [0, M_dense) of expert 0
  const int32_t* n_tiles;
  int M_dense;
  const bf16_t* W;          // [E_loc][rows][K]
  long long w_stride;       // elements between experts
  int K;                    // contraction length (multiple of 32)
  int N_out;                // output columns (multiple of 16 * NT)
  int up_off;               // SwiGLU: row offset of the up half in W
  void* Y;                  // [rows][N_out]
  int map_bm;               // rows per tile-map entry (>= the kernel's row tile)
};

// ---------------------------------------------------------------------------
// Direct-load bf16 MFMA kernel.  A block owns BM = 16*MT rows of one expert
// and 16*NT output columns; its NW waves split the K dimension and each
// streams its weight rows straight from HBM into MFMA fragments (every weight
// element is used by all BM rows at once, so staging it through LDS would buy
// no reuse).  Partial sums meet in LDS in a fixed order.
//
// v_mfma_f32_16x16x32_bf16 with A = weight fragment (row n = lane % 16) and
// B = activation fragment (column m = lane % 16), both taking 8 consecutive
// K elements at offset 8 * (lane / 16); the accumulator lane l holds
// C[n = 4*(l/16) + i][m = l % 16].
//
// SWIGLU: W rows [n] (gate) and [up_off + n] (up) are multiplied together and
// the epilogue writes SiLU(gate) * up.
//
// Weight loads.  In the fragment layout a wave instruction reads 64 bytes of
// each of 16 rows, so each group of 16 consecutive lanes touches 16
// different cache lines.  Read as 8 rows x 128 bytes instead (8 consecutive
// lanes on one line: two K steps of one row), the same weight stream ran 9%
// faster at 2-8 rows per expert.  So when a load batch holds an even number
// of K steps, each pair of steps is loaded that way and regrouped into
// fragments through a small LDS area private to the wave.
// ---------------------------------------------------------------------------
// The regrouping area of one wave and (column tile, gate/up) holds two K
// steps of 16 rows x 64 B: step t at byte 1024 t, row r in the 64-byte slot
// (r + 2 t) % 16, its chunk g at 16 (g ^ (r / 4 % 4)).  Each 16-lane quarter
// of a write (2 rows x 2 steps x 4 chunks) and of a fragment read (16 rows,
// one chunk) then covers the 64 banks once.
constexpr int XP_AREA = 2048 / 16;                  // in 16-byte units

__device__ __forceinline__ int xp_slot(int t, int row, int g) {
  return t * 64 + ((row + 2 * t) & 15) * 4 + (g ^ ((row >> 2) & 3));
}

// Weight operands per 16-column output tile: gate and up apart (SwiGLU), or
// one (the down projection, or PACK: 8 gate and the matching 8 up rows in one
// 16-row operand, 8 output columns per tile)
template <bool SWIGLU, bool PACK>
constexpr int direct_ns() {
  return SWIGLU && !PACK ? 2 : 1;
}
// K steps per load batch: about 24 16-byte loads in flight per wave
template <int MT, int NT, bool SWIGLU, bool PACK = false>
constexpr int direct_u() {
  constexpr int lps = NT * direct_ns<SWIGLU, PACK>() + MT;   // loads per K step
  return 24 / lps < 2 ? 2 : (24 / lps > 8 ? 8 : 24 / lps);
}
// 16-byte LDS units of a block's regrouping areas (0: fragment-layout loads)
template <int MT, int NT, int NW, bool SWIGLU, bool PACK = false>
constexpr int direct_xp_units() {
  return direct_u<MT, NT, SWIGLU, PACK>() % 2 == 0
             ? NW * NT * direct_ns<SWIGLU, PACK>() * XP_AREA
             : 0;
}

// Rows [r0, r1) (at most 16 * MT) of expert e against output columns
// [n0, n0 + BN): BN = 16 * NT, or 8 with PACK (SwiGLU, one column tile, the
// gate rows n0 + [0, 8) and up rows up_off + n0 + [0, 8) as one operand, so
// the accumulator's lanes 32-63 hold the up sums of lanes 0-31's gate sums).
template <int MT, int NT, int NW, bool SWIGLU, bool OUT_BF16, bool PACK = false>
__device__ __forceinline__ void direct_rows(const DirectArgs& a, int e, int r0, int r1, int n0,
                                            float* red, uint4* xp_all) {
  static_assert(!PACK || (SWIGLU && NT == 1 && NW > 1), "PACK: SwiGLU, one tile, split K");
  constexpr int NS = direct_ns<SWIGLU, PACK>();
  constexpr int BM = 16 * MT;
  constexpr int BN = PACK ? 8 : 16 * NT;
  constexpr int NACC = MT * NT * NS;
  constexpr int PITCH = 65;
  constexpr int U = direct_u<MT, NT, SWIGLU, PACK>();
  constexpr bool PAIRED = U % 2 == 0;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int kg = 8 * (lane >> 4);

  // The rows' sources are loaded here but turned into addresses only after
  // the first batch of weight loads has been issued (set_xp below), so the
  // weight stream does not wait for the source-token round trip.
  const bf16_t* xp[MT];
  bool xv[MT];
  int xsrc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = r0 + 16 * mt + (lane & 15);
    xv[mt] = row < r1;
    xsrc[mt] = xv[mt] ? (a.src_token ? a.src_token[row] : row) : 0;
    xp[mt] = a.X;
  }
  auto set_xp = [&]() {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      // the weight loads above stay ahead of this point; the wait for the
      // source lands here
      asm volatile("" : "+v"(xsrc[mt]) :: "memory");
      // a source of -1 (a padding row) reads row 0 instead of memory before X
      xp[mt] = a.X + (size_t)max(xsrc[mt], 0) * a.K + kg;
    }
  };
  const bf16_t* We = a.W + (size_t)e * a.w_stride;
  const bf16_t* wg[NT];
  const bf16_t* wu[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = lane & 15;
    const int n = PACK ? n0 + (r & 7) + (r < 8 ? 0 : a.up_off) : n0 + 16 * nt + r;
    wg[nt] = We + (size_t)n * a.K + kg;
    wu[nt] = We + (size_t)(a.up_off + n) * a.K + kg;
  }

  f32x4_t acc[MT][NT][NS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int s = 0; s < NS; ++s) acc[mt][nt][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // this wave's contiguous share of the K steps (32 elements each), taken
  // U steps per batch: every load of a batch is issued before its first
  // MFMA.  Steps past the share re-read the share's last step (a valid
  // address) and multiply zeros, so a batch never waits step by step.
  const int S = a.K / 32;
  const int s_begin = (S * wid) / NW;
  const int s_end = (S * (wid + 1)) / NW;

  if constexpr (PAIRED) {
    // lane i loads row 8 h + i / 8 of a 16-row tile: 16 bytes at 16 (i % 4)
    // of step 2 p + (i / 4) % 2 of the batch (a step past the share re-reads
    // the share's last step, as the activation loads do)
    const int lt = (lane >> 2) & 1;
    const bf16_t* wq[NT][NS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + 16 * nt + (lane >> 3);
      wq[nt][0] = We + (size_t)n * a.K + 8 * (lane & 3);
      if (NS == 2) wq[nt][NS - 1] = We + (size_t)(a.up_off + n) * a.K + 8 * (lane & 3);
    }
    // the operand's upper 8 rows: the next 8 rows, or with PACK the up rows
    const size_t half = (size_t)(PACK ? a.up_off : 8) * a.K;
    bf16x8_t* area = reinterpret_cast<bf16x8_t*>(xp_all) + wid * (NT * NS * XP_AREA);
    int wi[2], ri[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) wi[h] = xp_slot(lt, 8 * h + (lane >> 3), lane & 3);
#pragma unroll
    for (int t = 0; t < 2; ++t) ri[t] = xp_slot(t, lane & 15, lane >> 4);

    for (int s = s_begin; s < s_end; s += U) {
      uint4 xa[U][MT];
      bf16x8_t wv[U / 2][NT][NS][2];
#pragma unroll
      for (int p = 0; p < U / 2; ++p) {
        const int ko = min(s + 2 * p + lt, s_end - 1) * 32;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int w = 0; w < NS; ++w)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              wv[p][nt][w][h] = ld_stream16(wq[nt][w] + h * half + ko);
      }
      if (s == s_begin) set_xp();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ko = min(s + u, s_end - 1) * 32;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          xa[u][mt] = xv[mt] ? *reinterpret_cast<const uint4*>(xp[mt] + ko) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s + u >= s_end) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) xa[u][mt] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int p = 0; p < U / 2; ++p) {
        bf16x8_t f[NT][NS][2];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int w = 0; w < NS; ++w) {
            bf16x8_t* ar = area + (nt * NS + w) * XP_AREA;
            ar[wi[0]] = wv[p][nt][w][0];
            ar[wi[1]] = wv[p][nt][w][1];
          }
        wave_lds_sync();
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int w = 0; w < NS; ++w) {
            const bf16x8_t* ar = area + (nt * NS + w) * XP_AREA;
            f[nt][w][0] = ar[ri[0]];
            f[nt][w][1] = ar[ri[1]];
          }
        wave_lds_sync();   // the next pair's writes stay behind these reads
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              acc[mt][nt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  f[nt][0][t], as_bf16x8(xa[2 * p + t][mt]), acc[mt][nt][0], 0, 0, 0);
              if (NS == 2)
                acc[mt][nt][NS - 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    f[nt][NS - 1][t], as_bf16x8(xa[2 * p + t][mt]), acc[mt][nt][NS - 1],
                    0, 0, 0);
            }
      }
    }
  } else
  for (int s = s_begin; s < s_end; s += U) {
    uint4 xa[U][MT], wa[U][NT], wb[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ko = min(s + u, s_end - 1) * 32;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        wa[u][nt] = ld_stream16_u4(wg[nt] + ko);
        if (NS == 2) wb[u][nt] = ld_stream16_u4(wu[nt] + ko);
      }
    }
    if (s == s_begin) set_xp();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ko = min(s + u, s_end - 1) * 32;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xa[u][mt] = xv[mt] ? *reinterpret_cast<const uint4*>(xp[mt] + ko) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s + u >= s_end) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) xa[u][mt] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[mt][nt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(wa[u][nt]), as_bf16x8(xa[u][mt]), acc[mt][nt][0], 0, 0, 0);
          if (NS == 2)
            acc[mt][nt][NS - 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                as_bf16x8(wb[u][nt]), as_bf16x8(xa[u][mt]), acc[mt][nt][NS - 1], 0, 0, 0);
        }
    }
  }

  if constexpr (NW == 1) {
    // a single wave holds the whole sum: lane l writes columns
    // n0 + 16*nt + 4*(l/16) + [0, 4) of row r0 + 16*mt + l%16
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = r0 + 16 * mt + (lane & 15);
      if (row >= r1) continue;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = SWIGLU ? silu_fast(acc[mt][nt][0][i]) * acc[mt][nt][NS - 1][i] : acc[mt][nt][0][i];
        const size_t yi = (size_t)row * a.N_out + n0 + 16 * nt + 4 * (lane >> 4);
        if (OUT_BF16)
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(a.Y) + yi) =
              make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        else
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.Y) + yi) =
              make_float4(o[0], o[1], o[2], o[3]);
      }
    }
    return;
  }

  // partial sums -> LDS: red[w][((mt*NT + nt)*NS + which)*4 + i][lane]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int w = 0; w < NS; ++w)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          red[(wid * NACC + (mt * NT + nt) * NS + w) * 4 * PITCH + i * PITCH + lane] =
              acc[mt][nt][w][i];
  __syncthreads();

  // reduce over waves in wave order and write BM x BN outputs, n fastest;
  // the up sum sits in the next accumulator, or with PACK 32 lanes on
  constexpr int UP = PACK ? 32 : 4 * PITCH;
  for (int o = threadIdx.x; o < BM * BN; o += NW * 64) {
    const int m = o / BN, n = o - m * BN;
    const int row = r0 + m;
    if (row >= r1) continue;
    const int mt = m >> 4, ml = m & 15, nt = n >> 4, nl = n & 15;
    const int i = nl & 3, src_lane = ml + 16 * (nl >> 2);
    const int base = ((mt * NT + nt) * NS) * 4 * PITCH + i * PITCH + src_lane;
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      g += red[w * NACC * 4 * PITCH + base];
      if (SWIGLU) u += red[w * NACC * 4 * PITCH + base + UP];
    }
    const float out = SWIGLU ? silu_fast(g) * u : g;
    const size_t yi = (size_t)row * a.N_out + n0 + n;
    if (OUT_BF16) reinterpret_cast<bf16_t*>(a.Y)[yi] = f32_to_bf16(out);
    else reinterpret_cast<float*>(a.Y)[yi] = out;
  }
}

// One launch may carry two problems of the same tile shape: blocks
// [0, grid0) take a0 and the rest a1 (the shared expert beside the routed
// experts, so that one grid covers the CUs).  WALK: a tile-map entry may
// cover more rows than the kernel's row tile (map_bm > 16 * MT: the down
// projection reading the gate/up GEMM's map), and the block walks them
// 16 * MT rows at a time (a separate instance: the loop cost the other
// launches a few percent).
//
// The 8-wave gate/up instance is held to four waves per SIMD (128 VGPRs), so
// that two of its blocks share a CU: left to itself the compiler took 130 and
// room for one block, and the Qwen3 TP share's gate/up GEMM at T = 8 ran
// 36.2 us instead of 33.8.
template <int MT, int NT, int NW, bool SWIGLU, bool OUT_BF16, bool WALK, bool PACK = false>
__global__ __launch_bounds__(NW * 64, (NW == 8 && SWIGLU) ? 4 : 1) void ffn_direct_kernel(
    DirectArgs a0, DirectArgs a1, int grid0) {
  const bool second = (int)blockIdx.x >= grid0;
  const DirectArgs a = second ? a1 : a0;
  const int bid = second ? (int)blockIdx.x - grid0 : (int)blockIdx.x;
  constexpr int BM = 16 * MT;
  constexpr int BN = PACK ? 8 : 16 * NT;
  constexpr int NACC = MT * NT * direct_ns<SWIGLU, PACK>();
  constexpr int XPU = direct_xp_units<MT, NT, NW, SWIGLU, PACK>();
  __shared__ float red[NW > 1 ? NW * NACC * 4 * 65 : 1];
  __shared__ uint4 xp_lds[XPU > 0 ? XPU : 1];

  const int n_ntiles = a.N_out / BN;
  const int tile = bid / n_ntiles;
  const int ntile = bid - tile * n_ntiles;
  int e, r0, r1;
  if (a.tile_map) {
    if (tile >= a.n_tiles[0]) return;
    const int4 tm = a.tile_map[tile];
    e = tm.x; r0 = tm.y + (tile - tm.w) * a.map_bm; r1 = min(r0 + a.map_bm, tm.z);
  } else {
    e = 0; r0 = tile * BM; r1 = min(r0 + BM, a.M_dense);
    if (r0 >= a.M_dense) return;
  }
  if constexpr (WALK) {
    for (int rs = r0; rs < r1; rs += BM) {
      direct_rows<MT, NT, NW, SWIGLU, OUT_BF16>(a, e, rs, min(rs + BM, r1), ntile * BN, red,
                                                xp_lds);
      if (NW > 1) __syncthreads();    // red is written again by the next rows
    }
  } else {
    direct_rows<MT, NT, NW, SWIGLU, OUT_BF16, PACK>(a, e, r0, r1, ntile * BN, red, xp_lds);
  }
}

// ---------------------------------------------------------------------------
// Down projection over at most 16 rows per tile-map entry with a contraction
// of at most 2048 (a few rows per expert).  In ffn_direct_kernel every 16 x 16
// output tile is its own block, and every one of them loads the same 16
// activation rows: as many activation bytes as weight bytes cross each CU's
// L1.  Here a block's 8 waves take 8 column tiles of the same rows: the rows'
// activation fragments are loaded once, by the 8 waves together, into LDS
// (global -> LDS, one 1 KB fragment per K step of 32), and each wave streams
// only its own weight rows into MFMA fragments.  Each wave sums its whole
// contraction, so no partial sums meet; a wave whose column tile is past the
// output width only helps with the activation loads.  The weights are read
// in step pairs and regrouped as in direct_rows (2 KB of LDS per wave).
// Beyond that the LDS holds exactly the K / 32 fragments (1 KB each), so a
// short contraction leaves room for more blocks per CU, and more weight
// streams in flight.
// ---------------------------------------------------------------------------
constexpr int DCOLS_WAVES = 8;       // column tiles per block
constexpr int DCOLS_MAX_K = 2048;    // activation fragments held in LDS (64 KB)
typedef __attribute__((address_space(3))) void dlds_void_t;
typedef __attribute__((address_space(1))) void dgbl_void_t;

template <bool OUT_BF16>
__global__ __launch_bounds__(DCOLS_WAVES * 64) void ffn_direct_cols_kernel(DirectArgs a0,
                                                                          DirectArgs a1,
                                                                          int grid0) {
  constexpr int U = 8;               // K steps per weight load batch
  const bool second = (int)blockIdx.x >= grid0;
  const DirectArgs a = second ? a1 : a0;
  const int bid = second ? (int)blockIdx.x - grid0 : (int)blockIdx.x;
  extern __shared__ __attribute__((aligned(16))) uint4 s_x[];   // [K / 32][64]
  __shared__ bf16x8_t s_xp[DCOLS_WAVES * XP_AREA];               // regrouping areas
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n_ct = a.N_out / 16;
  const int n_cb = (n_ct + DCOLS_WAVES - 1) / DCOLS_WAVES;
  const int tile = bid / n_cb;
  const int cb = bid - tile * n_cb;
  int e, r0, r1;
  if (a.tile_map) {
    if (tile >= a.n_tiles[0]) return;
    const int4 tm = a.tile_map[tile];
    e = tm.x; r0 = tm.y + (tile - tm.w) * a.map_bm; r1 = min(r0 + a.map_bm, tm.z);
  } else {
    e = 0; r0 = tile * 16; r1 = min(r0 + 16, a.M_dense);
    if (r0 >= a.M_dense) return;
  }
  const int S = a.K / 32;
  // the rows' activation fragments: fragment s holds, in lane l, row
  // r0 + l % 16 and K elements 32 s + 8 (l / 16) + [0, 8); rows past r1
  // read row r0 (their outputs are not stored)
  {
    const int row = r0 + (lane & 15) < r1 ? r0 + (lane & 15) : r0;
    const int src = a.src_token ? max(a.src_token[row], 0) : row;
    const bf16_t* xp = a.X + (size_t)src * a.K + 8 * (lane >> 4);
    const int wu = __builtin_amdgcn_readfirstlane(wid);
    for (int st = wu; st < S; st += DCOLS_WAVES)
      __builtin_amdgcn_global_load_lds((dgbl_void_t*)(xp + 32 * st), (dlds_void_t*)&s_x[st * 64], 16,
                                       0, 0);
  }
  const int ct = cb * DCOLS_WAVES + wid;
  const bool live = ct < n_ct;
  const int n0 = 16 * (live ? ct : 0);
  // weight step pairs as in direct_rows: lane i reads row 8 h + i / 8 of the
  // column tile, 16 bytes at 16 (i % 4) of step (i / 4) % 2 of the pair (a
  // step past the end re-reads the last one and is not multiplied), then the
  // pair is regrouped into fragments through this wave's LDS area
  const int lt = (lane >> 2) & 1;
  const bf16_t* wp =
      a.W + (size_t)e * a.w_stride + (size_t)(n0 + (lane >> 3)) * a.K + 8 * (lane & 3);
  const size_t half = (size_t)8 * a.K;
  bf16x8_t* area = s_xp + wid * XP_AREA;
  const int wi0 = xp_slot(lt, lane >> 3, lane & 3), wi1 = xp_slot(lt, 8 + (lane >> 3), lane & 3);
  const int ri0 = xp_slot(0, lane & 15, lane >> 4), ri1 = xp_slot(1, lane & 15, lane >> 4);
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += U) {
    bf16x8_t wv[U / 2][2];
    if (live) {
#pragma unroll
      for (int p = 0; p < U / 2; ++p) {
        const int ko = min(s0 + 2 * p + lt, S - 1) * 32;
        wv[p][0] = ld_stream16(wp + ko);
        wv[p][1] = ld_stream16(wp + half + ko);
      }
    }
    if (s0 == 0) {
      // every wave's activation loads (and its first weight batch) have
      // landed before any wave reads the fragments
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    if (live) {
#pragma unroll
      for (int p = 0; p < U / 2; ++p) {
        const int sp = s0 + 2 * p;
        if (sp >= S) break;
        area[wi0] = wv[p][0];
        area[wi1] = wv[p][1];
        wave_lds_sync();
        const bf16x8_t f0 = area[ri0], f1 = area[ri1];
        wave_lds_sync();   // the next pair's writes stay behind these reads
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f0, as_bf16x8(s_x[sp * 64 + lane]), acc, 0,
                                                      0, 0);
        if (sp + 1 < S)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              f1, as_bf16x8(s_x[(sp + 1) * 64 + lane]), acc, 0, 0, 0);
      }
    }
  }
  if (!live) return;
  // lane l holds columns n0 + 4 (l / 16) + [0, 4) of row r0 + l % 16
  const int row = r0 + (lane & 15);
  if (row >= r1) return;
  const size_t yi = (size_t)row * a.N_out + n0 + 4 * (lane >> 4);
  if (OUT_BF16)
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(a.Y) + yi) =
        make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
  else
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.Y) + yi) =
        make_float4(acc[0], acc[1], acc[2], acc[3]);
}

// ---------------------------------------------------------------------------
// LDS-tiled bf16 MFMA kernel for prefill-sized row counts.
//
// Block tile: TM rows x TN weight rows, K in chunks of TK, WM x WN waves,
// each wave (TM/WM) rows x (TN/WN) weight rows of v_mfma_f32_32x32x16_bf16
// (A = weight fragment, B = activation fragment; accumulator lane l holds
// row m = l % 32 and weight rows 8*q + 4*(l/32) + r, register 4*q + r).
//
// Operands reach LDS through global_load_lds_dwordx4: each lane copies 16
// bytes from any global address (so the token gather of the gate/up GEMM
// happens inside the load) to LDS slot base + 16 * lane; one wave
// instruction fills 1 KB.  Rows are XOR-swizzled in 16-byte chunks (chunk c
// of row r sits at c ^ ((r / R) % C), R rows per 256 bytes, C chunks per
// row) so that 16 lanes reading one column chunk of 16 rows hit 16 distinct
// 4-bank groups.  STAGES buffers: while stage s is multiplied, the next
// STAGES-1 are in flight.
//
// SWIGLU: the TN weight rows are TN/2 gate rows [n0, n0 + TN/2) followed by
// the matching up rows; each wave holds gate and up accumulators for the
// same (row, column) and writes SiLU(gate) * up.
//
// Block order: blocks of one expert are numbered M-tile-fastest inside
// groups of G N-tiles, so the M-tiles sharing a weight tile run together;
// consecutive numbers are mapped to one XCD (workgroups are dealt to the 8
// XCDs round-robin) so that they share that XCD's L2.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

struct TileArgs {
  const bf16_t* X;
  const int32_t* src_token;
  const int4* tile_map;     // {expert, first row, end row, first tile of expert}
  const int32_t* n_tiles;
  int M_dense;
  const bf16_t* W;
  long long w_stride;
  int K;
  int N_out;                // output columns: I_loc (SWIGLU) or H
  int up_off;
  void* Y;
  int group;                // N-tiles per group
  long long x_bytes;        // extent of X in bytes (buffer-load path)
};

template <int TM_, int TN_, int TK_, int STAGES_, int WM_, int WN_, int MINB_>
struct TileCfg {
  static constexpr int TM = TM_, TN = TN_, TK = TK_, STAGES = STAGES_, WM = WM_, WN = WN_;
  static constexpr int MINB = MINB_;
  static constexpr int NWAVE = WM * WN, NTHR = NWAVE * 64;
  static constexpr int RB = TK * 2;                 // bytes per LDS row
  static constexpr int CPR = RB / 16;               // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;              // rows per load instruction
  static constexpr int RP256 = 256 / RB;            // rows per 256 bytes
  static constexpr int XBYTES = TM * RB, WBYTES = TN * RB, SBYTES = XBYTES + WBYTES;
  static constexpr int XLOADS = TM / RPI / NWAVE;   // load instructions per wave per stage
  static constexpr int WLOADS = TN / RPI / NWAVE;
  static constexpr int NLOADS = XLOADS + WLOADS;
  // a tile holding at most TM/2 rows ("half" tile) loads only the x-load
  // instructions of its first TM/2 rows
  static constexpr bool HALF_OK = (TM / 2) % (RPI * NWAVE) == 0 && WM == 2;
  static constexpr int XLOADS_H = HALF_OK ? (TM / 2) / RPI / NWAVE : XLOADS;
  static constexpr int NLOADS_H = XLOADS_H + WLOADS;
  static constexpr int WTM = TM / WM, WTN = TN / WN;  // wave tile
  static constexpr int MFM = WTM / 32, MFN = WTN / 32;
  // A half tile of the 256 x 256 two-stage configuration runs "wide": its
  // TM/2 rows against 2 TN weight rows (two adjacent N-tiles), its 8 waves
  // in one row of wave tiles of the usual shape.  Its stage holds TM/2 x rows
  // and 2 TN weight rows, so every stage buffer is sized for the larger one.
  static constexpr bool WIDE = TM == 256 && TN == 256 && STAGES == 2 && WM == 2 && WN == 4;
  static constexpr int WLOADS_W = 2 * WLOADS;
  static constexpr int NLOADS_W = XLOADS_H + WLOADS_W;
  static constexpr int SSTRIDE =
      WIDE ? (SBYTES > XBYTES / 2 + 2 * WBYTES ? SBYTES : XBYTES / 2 + 2 * WBYTES) : SBYTES;
  static constexpr int LDS = STAGES * SSTRIDE;
  static_assert(TM % (RPI * NWAVE) == 0 && TN % (RPI * NWAVE) == 0, "load split");
  static_assert(WTM % 32 == 0 && WTN % 64 == 0, "wave tile");
  static_assert(TK % 16 == 0, "k step");
};


// 16 bytes per lane from base + voff + soff into LDS at lds + 16 * lane, as a
// raw-buffer load of a buffer of nbytes: the address is a scalar base, one
// 32-bit lane offset and a scalar step, so a load costs no vector
// instructions; bytes past nbytes read as zero.
template <int AUX = 0>
__device__ __forceinline__ void buffer_load_lds16(const void* base, uint32_t nbytes, void* lds,
                                                  uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, AUX);
#endif
}

template <class C>
__device__ __forceinline__ int tile_swz(int r) { return (r / C::RP256) % C::CPR; }

// Wait until at most N vector-memory loads of this wave are outstanding and
// all its LDS reads have returned, then meet the other waves.
template <int N>
__device__ __forceinline__ void wait_stage_barrier() {
  static_assert(N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
  // The same lgkmcnt(0) where the compiler can see it (a no-op at run time):
  // its wait insertion does not read the asm, and believing an older scalar
  // load still pending, it had made the stage's first MFMAs wait for every
  // LDS read issued ahead of them instead of only their own.
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt(63) expcnt(7) lgkmcnt(0)
}

// A bf16 output tile leaves through LDS: the block's finished tile is staged
// row by row (rows padded by 16 bytes so the column-wise writes spread over
// the banks) and stored 16 bytes per lane along rows, instead of 8-byte
// pieces scattered over 32 rows per instruction, with the non-temporal hint
// (whole 128-byte lines).  That ran the down GEMM 5-8% faster.  The gate/up
// tile (half as wide) had lost as much to the two extra barriers as it
// gained; with the hint on its whole-line stores it measured even at T = 8192
// and 2% faster per layer at the Qwen3 EP view's T = 1024 (the same hint on
// its 8-byte direct stores had cost 6-15%).
template <class C, bool SWIGLU, bool OUT_BF16>
struct TileOut {
  static constexpr int OC = SWIGLU ? C::TN / 2 : C::TN;   // output columns per block
  static constexpr int PITCH = OC * 2 + 16;                // staged row bytes
  static constexpr int PITCH_W = 2 * OC * 2 + 16;          // wide half tile: TM/2 rows, 2 OC
  static constexpr bool STAGED = OUT_BF16;
  static constexpr int OUT_BYTES =
      C::WIDE && C::TM / 2 * PITCH_W > C::TM * PITCH ? C::TM / 2 * PITCH_W : C::TM * PITCH;
  static constexpr int LDS = (STAGED && OUT_BYTES > C::LDS) ? OUT_BYTES : C::LDS;
  static_assert(LDS <= 160 * 1024, "LDS per block");
};

// BUF: operands reach LDS by raw-buffer loads (X and each expert's weights
// within 4 GiB); otherwise by global loads from 64-bit per-lane pointers.
// As in the direct kernel, blocks [0, grid0) take a0 and the rest a1.
// WNT: weight loads with the non-temporal hint (aux 2 = nt on gfx950), for
// launches whose experts fill about one row tile each, so that no other
// block of the launch reads a weight tile again.
template <class C, bool SWIGLU, bool OUT_BF16, bool BUF, bool LS = false, bool WNT = false>
__global__ __launch_bounds__(C::NTHR, C::MINB) void ffn_tile_kernel(TileArgs a0, TileArgs a1,
                                                                    int grid0) {
  const bool second = (int)blockIdx.x >= grid0;
  const TileArgs a = second ? a1 : a0;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n_cols_tile = SWIGLU ? C::TN / 2 : C::TN;
  const int NTn = a.N_out / n_cols_tile;

  // ---- which (expert, M-tile, N-tile) this block computes
  int e = 0, off = 0, end = a.M_dense, ms = 0, n_active;
  if (a.tile_map) n_active = a.n_tiles[0] * NTn;
  else n_active = ((a.M_dense + C::TM - 1) / C::TM) * NTn;
  int b = second ? (int)blockIdx.x - grid0 : (int)blockIdx.x;
  if (b >= n_active) return;
  {
    const int per = n_active >> 3;                 // XCD-contiguous numbering
    if (b < per * 8) b = (b & 7) * per + (b >> 3);
  }
  const int mi = b / NTn;
  if (a.tile_map) {
    const int4 tm = a.tile_map[mi];
    e = tm.x; off = tm.y; end = tm.z; ms = tm.w;
  }
  const int te = (end - off + C::TM - 1) / C::TM;
  const int li = b - ms * NTn;
  const int G = a.group;
  const int g = li / (te * G);
  const int rem = li - g * te * G;
  const int Gc = min(G, NTn - g * G);
  const int m_t = rem / Gc;
  const int n_t = g * G + (rem - m_t * Gc);
  const int r0 = off + m_t * C::TM;
  const int r1 = min(r0 + C::TM, end);
  const int n0 = n_t * n_cols_tile;
  // A tile of at most TM/2 rows (an expert's last) in a configuration that
  // allows it takes two adjacent N-tiles at once: the block of the even one
  // runs wide, the block of the odd one has nothing left to do.  (Its cost
  // then matches a full tile's, which keeps the blocks of an expert running
  // in step; a half tile finishing early had let them drift apart and fetch
  // shared weight and token tiles again from beyond L2.)
  const bool half_rows = C::HALF_OK && r1 - r0 <= C::TM / 2;
  bool wide = false;
  if constexpr (C::WIDE) {
    if (half_rows) {
      if (n_t & 1) return;
      wide = n_t + 1 < NTn;
    }
  }

  // ---- per-lane global source pointers for the load instructions
  const int prow = lane / C::CPR;    // row inside a load instruction's row group
  const int pchunk = lane % C::CPR;  // LDS chunk slot written by this lane
  const bf16_t* xsrc[C::XLOADS];
#pragma unroll
  for (int j = 0; j < C::XLOADS; ++j) {
    const int rt = (wid + C::NWAVE * j) * C::RPI + prow;
    int row = r0 + rt;
    if (row >= r1) row = r0;                          // padding rows read a valid row
    const int src = a.src_token ? max(a.src_token[row], 0) : row;
    xsrc[j] = a.X + (size_t)src * a.K + (pchunk ^ tile_swz<C>(rt)) * 8;
  }
  const bf16_t* We = a.W + (size_t)e * a.w_stride;
  constexpr int WLA = C::WIDE ? C::WLOADS_W : C::WLOADS;   // weight loads of the widest mode
  const bf16_t* wsrc[WLA];
  // gate rows first (TN/2, or TN when wide), then the matching up rows
  const int gate_rows = wide ? C::TN : C::TN / 2;
#pragma unroll
  for (int j = 0; j < WLA; ++j) {
    const int rt = (wid + C::NWAVE * j) * C::RPI + prow;
    int wrow;
    if (SWIGLU) wrow = rt < gate_rows ? n0 + rt : a.up_off + n0 + (rt - gate_rows);
    else wrow = n0 + rt;
    if (j >= C::WLOADS && !wide) wrow = n0;           // unused
    wsrc[j] = We + (size_t)wrow * a.K + (pchunk ^ tile_swz<C>(rt)) * 8;
  }

  // An expert's last tile is often at most half full: then the x rows of the
  // upper half (padding) are not loaded and the waves that own them skip
  // their LDS reads and MFMAs, leaving their SIMD's MFMA pipe to the other
  // wave.  They still take part in the loads of weights and in every barrier.
  const bool half = half_rows && !wide;
  // buffer path: byte offsets of the same addresses from the buffers' bases
  uint32_t xo[C::XLOADS], wo[WLA];
  if constexpr (BUF) {
#pragma unroll
    for (int j = 0; j < C::XLOADS; ++j)
      xo[j] = (uint32_t)(reinterpret_cast<const unsigned char*>(xsrc[j]) -
                         reinterpret_cast<const unsigned char*>(a.X));
#pragma unroll
    for (int j = 0; j < WLA; ++j)
      wo[j] = (uint32_t)(reinterpret_cast<const unsigned char*>(wsrc[j]) -
                         reinterpret_cast<const unsigned char*>(We));
  }
  const uint32_t x_nbytes = (uint32_t)a.x_bytes;
  const uint32_t w_nbytes = (uint32_t)(a.w_stride * 2);
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);
  // LS: of the two waves on a SIMD (w and w ^ NWAVE/2), one issues both
  // waves' operand loads and the other issues none, so that one of them
  // always has MFMAs to issue while the other is held up issuing loads (a
  // timing copy whose loads were never waited for had run no faster than the
  // kernel: the cost sat in issuing and moving them, not in waiting).  In
  // full and wide tiles waves [0, NWAVE/2) load; in half tiles the waves
  // that own the empty upper rows (and compute nothing) load.
  constexpr bool LSX = LS && BUF && C::NWAVE == 8;
  constexpr int HW = C::NWAVE / 2;
  uint32_t xo1[LSX ? C::XLOADS : 1], wo1[LSX ? WLA : 1];
  if constexpr (LSX) {
    const int pw = wid ^ HW;
#pragma unroll
    for (int j = 0; j < C::XLOADS; ++j) {
      const int rt = (pw + C::NWAVE * j) * C::RPI + prow;
      int row = r0 + rt;
      if (row >= r1) row = r0;
      const int src = a.src_token ? max(a.src_token[row], 0) : row;
      xo1[j] = (uint32_t)(((size_t)src * a.K + (pchunk ^ tile_swz<C>(rt)) * 8) * 2);
    }
#pragma unroll
    for (int j = 0; j < WLA; ++j) {
      const int rt = (pw + C::NWAVE * j) * C::RPI + prow;
      int wrow;
      if (SWIGLU) wrow = rt < gate_rows ? n0 + rt : a.up_off + n0 + (rt - gate_rows);
      else wrow = n0 + rt;
      if (j >= C::WLOADS && !wide) wrow = n0;           // unused
      wo1[j] = (uint32_t)(((size_t)wrow * a.K + (pchunk ^ tile_swz<C>(rt)) * 8) * 2);
    }
  }
  // mode 0: full tile, 1: half tile, 2: wide half tile; role 0: this wave's
  // share, 1: this wave's and its partner's, 2: none
  auto issue = [&](int ks, int buf, auto mode_c, auto role_c) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr int ROLE = decltype(role_c)::value;
    constexpr int XL = MODE == 0 ? C::XLOADS : C::XLOADS_H;
    constexpr int WL = MODE == 2 ? C::WLOADS_W : C::WLOADS;
    if constexpr (ROLE == 2) return;
    unsigned char* sx = smem + buf * C::SSTRIDE;
    unsigned char* sw = sx + (MODE == 2 ? C::XBYTES / 2 : C::XBYTES);
    if constexpr (BUF) {
      const uint32_t soff = (uint32_t)ks * (C::TK * 2);
      const int pw_u = wid_u ^ HW;
#pragma unroll
      for (int j = 0; j < XL; ++j) {
        buffer_load_lds16(a.X, x_nbytes, sx + (wid_u + C::NWAVE * j) * 1024, xo[j], soff);
        if constexpr (ROLE == 1)
          buffer_load_lds16(a.X, x_nbytes, sx + (pw_u + C::NWAVE * j) * 1024, xo1[j], soff);
      }
#pragma unroll
      for (int j = 0; j < WL; ++j) {
        buffer_load_lds16<WNT ? 2 : 0>(We, w_nbytes, sw + (wid_u + C::NWAVE * j) * 1024, wo[j],
                                       soff);
        if constexpr (ROLE == 1)
          buffer_load_lds16<WNT ? 2 : 0>(We, w_nbytes, sw + (pw_u + C::NWAVE * j) * 1024, wo1[j],
                                         soff);
      }
    } else {
      const int ko = ks * C::TK;
#pragma unroll
      for (int j = 0; j < XL; ++j)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(xsrc[j] + ko),
                                         (lds_void_t*)(sx + (wid_u + C::NWAVE * j) * 1024), 16, 0, 0);
#pragma unroll
      for (int j = 0; j < WL; ++j)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(wsrc[j] + ko),
                                         (lds_void_t*)(sw + (wid_u + C::NWAVE * j) * 1024), 16, 0, 0);
    }
  };

  // wide: one row of 8 wave tiles (same shape) across 2 TN weight rows
  const int wm = wide ? 0 : wid / C::WN, wn = wide ? wid : wid % C::WN;
  const int lrow = lane & 31;
  const bool idle = half && wm * C::WTM >= C::TM / 2;
  const int khalf = lane >> 5;
  // weight-row bases of the wave's N subtiles inside the TN-row tile
  int nbase[C::MFN];
#pragma unroll
  for (int ni = 0; ni < C::MFN; ++ni) {
    if (SWIGLU) {
      constexpr int HALF = C::MFN / 2;
      nbase[ni] = (ni < HALF ? 0 : gate_rows) + wn * (C::WTN / 2) + (ni % HALF) * 32;
    } else {
      nbase[ni] = wn * C::WTN + ni * 32;
    }
  }
  int xoff[C::MFM], woff[C::MFN];    // row offsets; the swizzle term is per row
  int xsw[C::MFM], wsw[C::MFN];
#pragma unroll
  for (int mi = 0; mi < C::MFM; ++mi) {
    const int r = wm * C::WTM + mi * 32 + lrow;
    xoff[mi] = r * C::RB;
    xsw[mi] = tile_swz<C>(r);
  }
#pragma unroll
  for (int ni = 0; ni < C::MFN; ++ni) {
    const int r = nbase[ni] + lrow;
    woff[ni] = r * C::RB;
    wsw[ni] = tile_swz<C>(r);
  }

  f32x16_t acc[C::MFM][C::MFN];
#pragma unroll
  for (int i = 0; i < C::MFM; ++i)
#pragma unroll
    for (int j = 0; j < C::MFN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  constexpr int KK = C::TK / 16;     // MFMA K steps per stage
  const int nk = a.K / C::TK;
  auto load_frags = [&](const unsigned char* sx, const unsigned char* sw, int kk, bf16x8_t* xf,
                        bf16x8_t* wf) {
    const int c = kk * 2 + khalf;
#pragma unroll
    for (int mi = 0; mi < C::MFM; ++mi)
      xf[mi] = *reinterpret_cast<const bf16x8_t*>(sx + xoff[mi] + ((c ^ xsw[mi]) * 16));
#pragma unroll
    for (int ni = 0; ni < C::MFN; ++ni)
      wf[ni] = *reinterpret_cast<const bf16x8_t*>(sw + woff[ni] + ((c ^ wsw[ni]) * 16));
  };
  // One stage loop, instantiated for full tiles, for the computing waves of
  // half tiles, for their idle waves and for wide half tiles; the choice is
  // made once per wave.
  auto stage_loop = [&](auto mode_c, auto compute_c, auto role_c) {
  constexpr int MODE = decltype(mode_c)::value;
  constexpr int ROLE = decltype(role_c)::value;
  constexpr int NL1 = MODE == 0 ? C::NLOADS : MODE == 1 ? C::NLOADS_H : C::NLOADS_W;
  constexpr int NL = ROLE == 0 ? NL1 : ROLE == 1 ? 2 * NL1 : 0;   // this wave's loads per stage
#pragma unroll
  for (int s0 = 0; s0 < C::STAGES - 1; ++s0)
    if (s0 < nk) issue(s0, s0, mode_c, role_c);
  for (int ks = 0; ks < nk; ++ks) {
    // Stage ks has landed for this wave once at most the loads of the
    // STAGES-2 younger stages are outstanding; the barrier makes that true
    // for every wave.  The fragments of the previous stage were consumed by
    // its MFMAs, so no LDS read of the buffer refilled below is in flight.
    // (A __syncthreads() here would also drain the younger stages.)
    // (NL loads per stage: a half tile issues fewer)
    const int younger = min(nk - 1 - ks, C::STAGES - 2);
    switch (younger) {
      case 0: wait_stage_barrier<0>(); break;
      case 1: wait_stage_barrier<NL>(); break;
      case 2: wait_stage_barrier<(C::STAGES > 3 ? 2 : 1) * NL>(); break;
      case 3: wait_stage_barrier<(C::STAGES > 4 ? 3 : 1) * NL>(); break;
      default: wait_stage_barrier<(C::STAGES > 5 ? 4 : 1) * NL>(); break;
    }
    if (ks + C::STAGES - 1 < nk)
      issue(ks + C::STAGES - 1, (ks + C::STAGES - 1) % C::STAGES, mode_c, role_c);
    if constexpr (!decltype(compute_c)::value) continue;
    const unsigned char* sx = smem + (ks % C::STAGES) * C::SSTRIDE;
    const unsigned char* sw = sx + (MODE == 2 ? C::XBYTES / 2 : C::XBYTES);
    bf16x8_t xf[2][C::MFM], wf[2][C::MFN];
    load_frags(sx, sw, 0, xf[0], wf[0]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < KK) load_frags(sx, sw, kk + 1, xf[cur ^ 1], wf[cur ^ 1]);
      // keep the next step's LDS reads ahead of this step's MFMAs
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mi = 0; mi < C::MFM; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::MFN; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][ni], xf[cur][mi],
                                                                acc[mi][ni], 0, 0, 0);
    }
  }
  };
  using Full = std::integral_constant<int, 0>;
  using Half = std::integral_constant<int, 1>;
  using Wide = std::integral_constant<int, 2>;
  using Own = std::integral_constant<int, 0>;
  using Both = std::integral_constant<int, 1>;
  using None = std::integral_constant<int, 2>;
  if constexpr (LSX) {
    const bool lo = wid < HW;
    bool done = false;
    if constexpr (C::WIDE) {
      if (wide) {
        if (lo) stage_loop(Wide{}, std::true_type{}, Both{});
        else stage_loop(Wide{}, std::true_type{}, None{});
        done = true;
      }
    }
    if (!done) {
      if (!half) {
        if (lo) stage_loop(Full{}, std::true_type{}, Both{});
        else stage_loop(Full{}, std::true_type{}, None{});
      } else if (!idle) {
        stage_loop(Half{}, std::true_type{}, None{});
      } else {
        stage_loop(Half{}, std::false_type{}, Both{});
      }
    }
  } else if constexpr (C::WIDE) {
    if (wide) stage_loop(Wide{}, std::true_type{}, Own{});
    else if (!half) stage_loop(Full{}, std::true_type{}, Own{});
    else if (!idle) stage_loop(Half{}, std::true_type{}, Own{});
    else stage_loop(Half{}, std::false_type{}, Own{});
  } else {
    if (!half) stage_loop(Full{}, std::true_type{}, Own{});
    else if (!idle) stage_loop(Half{}, std::true_type{}, Own{});
    else stage_loop(Half{}, std::false_type{}, Own{});
  }

  // ---- epilogue
  using O = TileOut<C, SWIGLU, OUT_BF16>;
  if constexpr (O::STAGED) {
    // every wave is done reading the stage buffers (their loads all landed
    // before the last stage) before the tile is staged over them
    lds_barrier();
    const int pitch = wide ? O::PITCH_W : O::PITCH;
#pragma unroll
    for (int mi = 0; mi < C::MFM; ++mi) {
      if (idle) break;
      unsigned char* so = smem + (wm * C::WTM + mi * 32 + lrow) * pitch;
      if (SWIGLU) {
        constexpr int HALF = C::MFN / 2;
#pragma unroll
        for (int ni = 0; ni < HALF; ++ni) {
          const int lc = wn * (C::WTN / 2) + ni * 32 + 4 * khalf;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float h[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              h[r] = silu_fast(acc[mi][ni][4 * q + r]) * acc[mi][ni + HALF][4 * q + r];
            *reinterpret_cast<uint2*>(so + (lc + 8 * q) * 2) =
                make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
          }
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < C::MFN; ++ni) {
          const int lc = wn * C::WTN + ni * 32 + 4 * khalf;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<uint2*>(so + (lc + 8 * q) * 2) =
                make_uint2(pack_bf16x2(acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1]),
                           pack_bf16x2(acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]));
        }
      }
    }
    lds_barrier();
    const int nrows = r1 - r0;
    bf16_t* Y = reinterpret_cast<bf16_t*>(a.Y);
    // Non-temporal stores: the output rows are read next by another launch
    // (the down projection or the combine), and allocating them in L2 had
    // evicted operand tiles that other blocks of this launch still read
    // (Qwen3 EP view: down projection 0.337 -> 0.302 ms at T = 1024, 0.953
    // -> 0.93 ms at T = 8192).
    auto store_rows = [&](auto cpr_c, int rows, int pitch_b) {
      constexpr int CPR_OUT = decltype(cpr_c)::value;   // 16-byte chunks per row
      for (int c = threadIdx.x; c < rows * CPR_OUT; c += C::NTHR) {
        const int r = c / CPR_OUT, cc = c - r * CPR_OUT;
        if (r < nrows)
          st_stream16(Y + (size_t)(r0 + r) * a.N_out + n0 + cc * 8,
                      *reinterpret_cast<const uint4*>(smem + r * pitch_b + cc * 16));
      }
    };
    if (wide) store_rows(std::integral_constant<int, 2 * O::OC / 8>{}, C::TM / 2, O::PITCH_W);
    else store_rows(std::integral_constant<int, O::OC / 8>{}, C::TM, O::PITCH);
    return;
  }
#pragma unroll
  for (int mi = 0; mi < C::MFM; ++mi) {
    const int row = r0 + wm * C::WTM + mi * 32 + lrow;
    if (row >= r1) continue;
    if (SWIGLU) {
      constexpr int HALF = C::MFN / 2;
#pragma unroll
      for (int ni = 0; ni < HALF; ++ni) {
        const int col0 = n0 + wn * (C::WTN / 2) + ni * 32 + 4 * khalf;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            h[r] = silu_fast(acc[mi][ni][4 * q + r]) * acc[mi][ni + HALF][4 * q + r];
          uint2 o = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(a.Y) + (size_t)row * a.N_out +
                                    col0 + 8 * q) = o;
        }
      }
    } else {
#pragma unroll
      for (int ni = 0; ni < C::MFN; ++ni) {
        const int col0 = n0 + wn * C::WTN + ni * 32 + 4 * khalf;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const size_t yi = (size_t)row * a.N_out + col0 + 8 * q;
          if (OUT_BF16) {
            uint2 o = make_uint2(pack_bf16x2(acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1]),
                                 pack_bf16x2(acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]));
            *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(a.Y) + yi) = o;
          } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.Y) + yi) =
                make_float4(acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                            acc[mi][ni][4 * q + 3]);
          }
        }
      }
    }
  }
}

// Tile shapes for prefill-sized expert GEMMs (8 waves: two per SIMD, so one
// wave's waits on LDS or on the stage barrier overlap the other's MFMAs).
// Experts with >= 384 expected rows take 256-row tiles; smaller ones take
// 128-row tiles, which waste less on each expert's partial last tile.
using TileBig = TileCfg<256, 256, 64, 2, 2, 4, 1>;
using TileMed = TileCfg<128, 256, 64, 3, 2, 4, 1>;
// gate/up with an output width that is a multiple of 64 but not of 128 (a
// tensor-parallel share such as 1536 / 8 = 192): 64 gate + 64 up rows per
// tile, four waves of 64 x 64
using TileNarrow = TileCfg<128, 128, 64, 3, 2, 2, 1>;
constexpr int BIG_TILE_MIN_ROWS = 384;
static_assert(TileBig::TN == TileMed::TN && TileBig::TK == TileMed::TK, "shared shape limits");
constexpr int TL_N = TileMed::TN, TL_K = TileMed::TK;

// ---------------------------------------------------------------------------
// float32 layer: one thread per output element of a 16 x 16 tile, plain FMA
// dot products over K (the fp32 configuration is small).
// ---------------------------------------------------------------------------
struct F32Args {
  const float* X;
  const int32_t* src_token;
  const int4* tile_map;
  const int32_t* n_tiles;
  int M_dense;
  const float* W;
  long long w_stride;
  int K, N_out, up_off;
  float* Y;
};

template <bool SWIGLU>
__global__ __launch_bounds__(256) void ffn_f32_kernel(F32Args a) {
  const int n_ntiles = a.N_out / 16;
  const int tile = blockIdx.x / n_ntiles;
  const int ntile = blockIdx.x - tile * n_ntiles;
  int e, r0, r1;
  if (a.tile_map) {
    if (tile >= a.n_tiles[0]) return;
    const int4 tm = a.tile_map[tile];
    e = tm.x; r0 = tm.y + (tile - tm.w) * 16; r1 = min(r0 + 16, tm.z);
  } else {
    e = 0; r0 = tile * 16; r1 = min(r0 + 16, a.M_dense);
    if (r0 >= a.M_dense) return;
  }
  const int row = r0 + (threadIdx.x >> 4);
  const int n = ntile * 16 + (threadIdx.x & 15);
  if (row >= r1) return;
  const int src = a.src_token ? max(a.src_token[row], 0) : row;
  const float4* xr = reinterpret_cast<const float4*>(a.X + (size_t)src * a.K);
  const float* We = a.W + (size_t)e * a.w_stride;
  const float4* wg = reinterpret_cast<const float4*>(We + (size_t)n * a.K);
  const float4* wu = reinterpret_cast<const float4*>(We + (size_t)(a.up_off + n) * a.K);
  float g = 0.f, u = 0.f;
  for (int q = 0; q < a.K / 4; ++q) {
    const float4 xv = xr[q];
    const float4 gv = wg[q];
    g = fmaf(xv.x, gv.x, g); g = fmaf(xv.y, gv.y, g); g = fmaf(xv.z, gv.z, g); g = fmaf(xv.w, gv.w, g);
    if (SWIGLU) {
      const float4 uv = wu[q];
      u = fmaf(xv.x, uv.x, u); u = fmaf(xv.y, uv.y, u); u = fmaf(xv.z, uv.z, u); u = fmaf(xv.w, uv.w, u);
    }
  }
  a.Y[(size_t)row * a.N_out + n] = SWIGLU ? silu(g) * u : g;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool ffn_tile_ok(int H, int I_loc) {
  return H % TL_K == 0 && H % TL_N == 0 && I_loc % TL_K == 0 && I_loc % (TileNarrow::TN / 2) == 0;
}

int ffn_row_tile(int dt, int mean_rows, int H, int I_loc, int experts) {
  if (dt == 0) return 16;
  if (ffn_tile_ok(H, I_loc)) {
    // (256-row tiles need gate/up widths that are multiples of 128)
    if (mean_rows >= 64)
      return mean_rows >= BIG_TILE_MIN_ROWS && I_loc % (TL_N / 2) == 0 ? TileBig::TM : TileMed::TM;
    // From a few rows per expert up, the LDS-tiled kernel streams each
    // expert's weights faster than the direct kernel (its 256-row weight
    // tiles move in 1 KB contiguous loads shared by all 8 waves; a mostly
    // empty tile skips its padding's work): 3-35% per layer at 4-48 rows per
    // expert, and from 2 rows with a long contraction (H >= 6144), where the
    // direct kernel's per-wave streams fall further behind.  The condition:
    // 16 rows per expert, or enough down-projection blocks (one per 128-row
    // tile and 256 columns) to cover the 256 CUs -- with few experts (8) and
    // a handful of rows each the direct kernel stays ahead.
    // (narrow gate/up tiles -- widths not a multiple of 128 -- run one wave
    // per SIMD and only pay from 16 rows per expert)
    // With the long contraction the LDS-tiled kernel pays from one row per
    // expert once the touched experts' gate/up tiles give every CU two
    // blocks: DeepSeek-V3 shape at T = 8 and 32 (about one row per touched
    // expert), gate/up GEMM 12-16% faster; with 8 touched experts (T = 1)
    // its 128 blocks left the CUs short and the direct kernel stayed ahead.
    int min_rows = 4;
    if (I_loc % (TL_N / 2) != 0) min_rows = 16;
    else if (H >= 6144) min_rows = (long long)experts * (I_loc / (TL_N / 2)) >= 512 ? 1 : 2;
    const long long blocks = (long long)experts * ((mean_rows + TileMed::TM - 1) / TileMed::TM) *
                             (H / TileMed::TN);
    if (mean_rows >= min_rows && (blocks >= 256 || mean_rows >= 16)) return TileMed::TM;
  }
  // routed counts spread well past the mean, so the tile is sized for about
  // twice the mean: an expert split over two tiles streams its weights twice
  if (mean_rows <= 8) return 16;
  if (mean_rows <= 16) return 32;
  return 64;
}

static bool is_tile_bm(int BM) { return BM == TileBig::TM || BM == TileMed::TM; }

template <class C, bool SWIGLU, bool OUT_BF16, bool BUF, bool LS, bool WNT>
static hipError_t launch_tile_ls(const TileArgs& a, int max_tiles, const TileArgs* b, int b_tiles,
                                 hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t err = ensure_lds_limit(
      reinterpret_cast<const void*>(&ffn_tile_kernel<C, SWIGLU, OUT_BF16, BUF, LS, WNT>),
      TileOut<C, SWIGLU, OUT_BF16>::LDS, lds_set);
  if (err != hipSuccess) return err;
  constexpr int cols = SWIGLU ? C::TN / 2 : C::TN;
  const int grid0 = max_tiles * (a.N_out / cols);
  const int grid1 = b ? b_tiles * (b->N_out / cols) : 0;
  ffn_tile_kernel<C, SWIGLU, OUT_BF16, BUF, LS, WNT>
      <<<grid0 + grid1, C::NTHR, TileOut<C, SWIGLU, OUT_BF16>::LDS, st>>>(a, b ? *b : a, grid0);
  return hipGetLastError();
}

// The two-stage 256-row tiles load through one wave per SIMD (LS): Qwen3
// shape T = 8192, gate/up GEMM 1.648 -> 1.591 ms and down 0.961 -> 0.945 ms,
// Mixtral T = 4096 layer 2.89 -> 2.78 ms (same box, alternating runs).  The
// three-stage 128-row tiles measured the same or 1-2% slower with it.
// Three-stage tiles (128 rows) of a launch whose experts hold fewer rows than
// one tile on average (mean_rows < TM) load their weights non-temporally: the
// Qwen3 EP view at T = 128, 256 and 1024 ran 4-8% faster and Mixtral T = 256
// about 3% (same box, alternating runs).  With 128 or more rows per expert
// (DeepSeek-V3 T = 4096) an expert's row tiles share weight tiles through the
// L2, and the hint measured the same or slower there.
template <class C, bool SWIGLU, bool OUT_BF16, bool BUF>
static hipError_t launch_tile_buf(const TileArgs& a, int max_tiles, const TileArgs* b, int b_tiles,
                                  int mean_rows, hipStream_t st) {
  constexpr bool LS = BUF && C::NWAVE == 8 && C::STAGES == 2;
  if constexpr (BUF && C::STAGES == 3) {
    // (not with a second problem riding along: the shared expert's dense
    // rows reuse its weight tiles)
    if (mean_rows < C::TM && !b)
      return launch_tile_ls<C, SWIGLU, OUT_BF16, BUF, LS, true>(a, max_tiles, b, b_tiles, st);
  }
  return launch_tile_ls<C, SWIGLU, OUT_BF16, BUF, LS, false>(a, max_tiles, b, b_tiles, st);
}

// Raw-buffer loads (no vector address arithmetic per load: the gate/up GEMM
// ran 7-9% faster) whenever X's extent is known and X and one expert's
// weights each fit the 32-bit buffer range (for both problems of a shared
// launch).
static bool tile_buf_ok(const TileArgs& a) {
  return a.x_bytes > 0 && a.x_bytes <= 0xffffffffLL && a.w_stride * 2 <= 0xffffffffLL;
}

template <class C, bool SWIGLU, bool OUT_BF16>
static hipError_t launch_tile_cfg(const TileArgs& a, int max_tiles, const TileArgs* b, int b_tiles,
                                  int mean_rows, hipStream_t st) {
  const bool buf = tile_buf_ok(a) && (!b || tile_buf_ok(*b));
  if (buf)
    return launch_tile_buf<C, SWIGLU, OUT_BF16, true>(a, max_tiles, b, b_tiles, mean_rows, st);
  return launch_tile_buf<C, SWIGLU, OUT_BF16, false>(a, max_tiles, b, b_tiles, mean_rows, st);
}

// N-tiles per group.  One N-tile per group (all M-tiles of an expert that
// share a weight tile numbered consecutively, on one XCD) fetched the least
// from beyond L2 and ran fastest among groups of 1, 2, 4 and all N-tiles.
static int tile_group(int /*mean_rows*/, int /*tm*/, int /*ntn*/) { return 1; }

// Tile shape for a row tile and output width: 256-row tiles, 128-row tiles,
// or (gate/up widths not a multiple of 128) the narrow 128x128 tiles.
enum TileShape { TILE_BIG, TILE_MED, TILE_NARROW };
static TileShape tile_shape(int BM, bool swiglu, int N_out) {
  if (BM == TileBig::TM) return TILE_BIG;
  if (swiglu && N_out % (TL_N / 2) != 0) return TILE_NARROW;
  return TILE_MED;
}

template <bool SWIGLU, bool OUT_BF16>
static hipError_t launch_tile(TileArgs a, int BM, int mean_rows, int max_tiles, const TileArgs* b,
                              int b_tiles, hipStream_t st) {
  const int ntn = a.N_out / (SWIGLU ? TL_N / 2 : TL_N);
  a.group = tile_group(mean_rows, BM, ntn);
  switch (tile_shape(BM, SWIGLU, a.N_out)) {
    case TILE_BIG:
      return launch_tile_cfg<TileBig, SWIGLU, OUT_BF16>(a, max_tiles, b, b_tiles, mean_rows, st);
    case TILE_NARROW:
      if constexpr (SWIGLU)
        return launch_tile_cfg<TileNarrow, SWIGLU, OUT_BF16>(a, max_tiles, b, b_tiles, mean_rows, st);
      [[fallthrough]];
    default:
      return launch_tile_cfg<TileMed, SWIGLU, OUT_BF16>(a, max_tiles, b, b_tiles, mean_rows, st);
  }
}

// Waves per block: enough that each wave's K share is one load batch where
// the block size allows it, and never shares of fewer than 4 steps.
static int pick_nw(int steps, int max_nw, int batch) {
  int nw = 1;
  while (nw * 2 <= max_nw && (steps + nw - 1) / nw > batch && steps / (nw * 2) >= 4) nw *= 2;
  return nw;
}

template <int MT, int NT, int NW, bool SWIGLU, bool OUT_BF16, bool PACK = false>
static hipError_t launch_direct_t(const DirectArgs& a, int max_tiles, const DirectArgs* b,
                                  int b_tiles, hipStream_t st) {
  constexpr int BN = PACK ? 8 : 16 * NT;
  if (a.N_out % BN != 0 || (b && b->N_out % BN != 0)) return hipErrorInvalidValue;
  const int grid0 = max_tiles * (a.N_out / BN);
  const int grid1 = b ? b_tiles * (b->N_out / BN) : 0;
  if constexpr (!SWIGLU && MT == 1 && NT == 1) {
    if (a.map_bm > 16 || (b && b->map_bm > 16)) {
      ffn_direct_kernel<MT, NT, NW, SWIGLU, OUT_BF16, true><<<grid0 + grid1, NW * 64, 0, st>>>(
          a, b ? *b : a, grid0);
      return hipGetLastError();
    }
  }
  if (a.map_bm > 16 * MT || (b && b->map_bm > 16 * MT)) return hipErrorInvalidValue;
  ffn_direct_kernel<MT, NT, NW, SWIGLU, OUT_BF16, false, PACK>
      <<<grid0 + grid1, NW * 64, 0, st>>>(a, b ? *b : a, grid0);
  return hipGetLastError();
}

template <int MT, int NT, bool SWIGLU, bool OUT_BF16, bool PACK = false>
static hipError_t launch_direct_nw(const DirectArgs& a, int nw, int max_tiles, const DirectArgs* b,
                                   int b_tiles, hipStream_t st) {
  switch (nw) {
    case 1:
      if constexpr (PACK) return hipErrorInvalidValue;   // PACK sums over waves
      else return launch_direct_t<MT, NT, 1, SWIGLU, OUT_BF16>(a, max_tiles, b, b_tiles, st);
    case 2: return launch_direct_t<MT, NT, 2, SWIGLU, OUT_BF16, PACK>(a, max_tiles, b, b_tiles, st);
    case 4: return launch_direct_t<MT, NT, 4, SWIGLU, OUT_BF16, PACK>(a, max_tiles, b, b_tiles, st);
    default:
      return launch_direct_t<MT, NT, 8, SWIGLU, OUT_BF16, PACK>(a, max_tiles, b, b_tiles, st);
  }
}

// 16-column output tiles per block for each row tile (BM = 16, 32, 64).  With
// 32 or 64 rows, two output tiles per wave share each activation fragment:
// the activation loads had been as many as the weight loads, and halving
// them ran the layer 14-15% faster at 16-32 rows per expert; with 16 rows
// the extra registers cost more than the loads saved.
constexpr int DIRECT_NT16 = 1, DIRECT_NT32 = 2, DIRECT_NT64 = 2;

template <int MT, int NT, bool SWIGLU>
constexpr int direct_batch() {
  return direct_u<MT, NT, SWIGLU>();
}

// Waves per block of the direct kernel for a row tile and contraction.
template <bool SWIGLU>
static int direct_nw(int BM, int K) {
  const int steps = K / 32;
  // 16-row tiles: at most 8 waves, so two blocks share a CU: one block's LDS
  // reduction and stores overlap the other's weight loads (16-wave blocks
  // left the CU's loads idle during them; 8 ran the gate/up GEMM 9-11%
  // faster).  Measured further: the gate/up GEMM over a long K (>= 192
  // steps, e.g. H = 7168) ran 6% faster with 4 waves; the down projection
  // 10-18% faster with 2 waves (longer per-wave streams, a cheaper
  // reduction) -- up to a contraction of 256 steps: over I = 14336 (Mixtral
  // shape, 448 steps) each of 2 waves chained 28 load batches, and 4 waves
  // ran the down projection 5-18% faster at T = 1-16 (T = 1: 53.6 -> 44.1 us).
  const int max_nw16 = SWIGLU ? (steps >= 192 ? 4 : 8) : (steps >= 256 ? 4 : 2);
  // 32- and 64-row tiles (more MFMA work per load): 4 waves for gate/up, 2
  // for the down projection ran the layer 3-15% faster than 8 at 16-32 rows
  // per expert
  const int max_nw_big = SWIGLU ? 4 : 2;
  if (BM == 16) return pick_nw(steps, max_nw16, direct_batch<1, DIRECT_NT16, SWIGLU>());
  if (BM == 32) return pick_nw(steps, max_nw_big, direct_batch<2, DIRECT_NT32, SWIGLU>());
  return pick_nw(steps, max_nw_big, direct_batch<4, DIRECT_NT64, SWIGLU>());
}

// b (optional, b_tiles row tiles): a second problem in the same launch; its
// waves per block must equal a's (the caller checks).
// Whether a direct down projection runs as ffn_direct_cols_kernel: 16-row
// tiles (no walk over a larger map entry), the activation fragments within
// the LDS it reserves, output columns in whole tiles.
static bool direct_cols_ok(const DirectArgs& a, bool swiglu, int BM) {
  return !swiglu && BM == 16 && a.map_bm <= 16 && a.K <= DCOLS_MAX_K && a.N_out % 16 == 0;
}

// Whether a gate/up launch the plan gave 8-column tiles (PACK) can take
// them: the partial sums meet over waves, and whole 8-column tiles.
static bool direct_pack_ok(const DirectArgs& a, int nw, const DirectArgs* b) {
  return nw >= 2 && a.N_out % 8 == 0 && (!b || b->N_out % 8 == 0);
}

template <bool SWIGLU, bool OUT_BF16>
static hipError_t launch_direct(const DirectArgs& a, int BM, int max_tiles, const DirectArgs* b,
                                int b_tiles, hipStream_t st, bool pack = false) {
  if constexpr (!SWIGLU) {
    if (direct_cols_ok(a, false, BM) && (!b || direct_cols_ok(*b, false, BM))) {
      const int cb = (a.N_out / 16 + DCOLS_WAVES - 1) / DCOLS_WAVES;
      const int grid0 = max_tiles * cb;
      const int grid1 = b ? b_tiles * ((b->N_out / 16 + DCOLS_WAVES - 1) / DCOLS_WAVES) : 0;
      const int lds = (b ? std::max(a.K, b->K) : a.K) / 32 * 1024;
      static std::atomic<uint64_t> lds_set{0};
      hipError_t err = ensure_lds_limit(
          reinterpret_cast<const void*>(&ffn_direct_cols_kernel<OUT_BF16>), DCOLS_MAX_K / 32 * 1024,
          lds_set);
      if (err != hipSuccess) return err;
      ffn_direct_cols_kernel<OUT_BF16><<<grid0 + grid1, DCOLS_WAVES * 64, lds, st>>>(a, b ? *b : a,
                                                                                   grid0);
      return hipGetLastError();
    }
  }
  const int nw = direct_nw<SWIGLU>(BM, a.K);
  if constexpr (SWIGLU && DIRECT_NT16 == 1) {
    if (pack && BM == 16 && direct_pack_ok(a, nw, b))
      return launch_direct_nw<1, 1, true, OUT_BF16, true>(a, nw, max_tiles, b, b_tiles, st);
  }
  if (BM == 16)
    return launch_direct_nw<1, DIRECT_NT16, SWIGLU, OUT_BF16>(a, nw, max_tiles, b, b_tiles, st);
  if (BM == 32)
    return launch_direct_nw<2, DIRECT_NT32, SWIGLU, OUT_BF16>(a, nw, max_tiles, b, b_tiles, st);
  return launch_direct_nw<4, DIRECT_NT64, SWIGLU, OUT_BF16>(a, nw, max_tiles, b, b_tiles, st);
}

static DirectArgs gate_up_direct(const FfnArgs& a, int BM) {
  return DirectArgs{(const bf16_t*)a.x, a.src_token, a.tile_map, a.n_tiles, a.M_dense,
                    (const bf16_t*)a.w13, 2LL * a.I_loc * a.H, a.H, a.I_loc, a.I_loc, a.h,
                    a.map_bm > 0 ? a.map_bm : BM};
}
static DirectArgs down_direct(const FfnArgs& a, int BM) {
  return DirectArgs{(const bf16_t*)a.h, nullptr, a.tile_map, a.n_tiles, a.M_dense,
                    (const bf16_t*)a.w2, (long long)a.H * a.I_loc, a.I_loc, a.H, 0, a.y,
                    a.map_bm > 0 ? a.map_bm : BM};
}
static TileArgs gate_up_tile(const FfnArgs& a) {
  return TileArgs{(const bf16_t*)a.x, a.src_token, a.tile_map, a.n_tiles, a.M_dense,
                  (const bf16_t*)a.w13, 2LL * a.I_loc * a.H, a.H, a.I_loc, a.I_loc, a.h, 1,
                  a.x_rows * a.H * 2};
}
static TileArgs down_tile(const FfnArgs& a) {
  return TileArgs{(const bf16_t*)a.h, nullptr, a.tile_map, a.n_tiles, a.M_dense,
                  (const bf16_t*)a.w2, (long long)a.H * a.I_loc, a.I_loc, a.H, 0, a.y, 1,
                  a.h_rows * a.I_loc * 2};
}

bool ffn_can_share_gemm(const FfnArgs& a, int BM, const FfnArgs& b, int b_BM, bool gate_up) {
  if (a.dt != 1 || b.dt != 1 || a.y_dt != b.y_dt || BM != b_BM) return false;
  if (a.max_tiles <= 0 || b.max_tiles <= 0) return false;
  if (is_tile_bm(BM))
    return tile_shape(BM, gate_up, gate_up ? a.I_loc : a.H) ==
               tile_shape(BM, gate_up, gate_up ? b.I_loc : b.H) &&
           ffn_tile_ok(a.H, a.I_loc) && ffn_tile_ok(b.H, b.I_loc) && a.map_bm <= 0 &&
           b.map_bm <= 0;
  if (gate_up) return direct_nw<true>(BM, a.H) == direct_nw<true>(BM, b.H);
  // both in ffn_direct_cols_kernel, or both in ffn_direct_kernel with the
  // same waves per block (launch_direct takes the first only if both can)
  if (direct_cols_ok(down_direct(a, BM), false, BM) && direct_cols_ok(down_direct(b, BM), false, BM))
    return true;
  return direct_nw<false>(BM, a.I_loc) == direct_nw<false>(BM, b.I_loc);
}

int ffn_down_row_tile(int dt, int mean_rows, int H, int I_loc, int BM) {
  // the one-row rule of ffn_row_tile (long contraction, fewer than 2 rows
  // per expert) put the gate/up GEMM on LDS tiles: DeepSeek-V3 shape at
  // T = 4, 8 and 16, down projection 4-9% faster in the direct kernel
  if (dt == 1 && is_tile_bm(BM) && H >= 6144 && mean_rows < 2 && I_loc % 32 == 0) return 16;
  return BM;
}

// Columns per block of the 128-row LDS-tiled down projection.  With few
// experts of at most ~100 rows each (Mixtral shape, T = 64-256: 8 experts, one
// row tile each) the 256-column tiles give 8 x 16 = 128 blocks and leave half
// the CUs idle over a 14336-long contraction; 128-column tiles give every CU
// one block: down projection 0.21-0.25 -> 0.18-0.19 ms, layer 6-8% faster.
// At T = 512 (about 128 rows per expert, so many experts need a second,
// mostly empty tile) they needed two rounds of blocks and ran 20% slower, so
// they are taken only while the expected blocks fill at most one round.  The
// column split leaves every output's sum over K in the same order, so the
// results are the same bits either way.
int ffn_down_cols(int dt, int BM_dn, int mean_rows, int experts, int H) {
  if (dt != 1 || BM_dn != TileMed::TM || H % TileNarrow::TN != 0 || mean_rows <= 0) return 0;
  const long long rows = (long long)mean_rows + mean_rows / 4;
  const long long tiles = (long long)experts * ((rows + TileMed::TM - 1) / TileMed::TM);
  return tiles * (H / TileNarrow::TN) <= 256 ? TileNarrow::TN : 0;
}

// 8-column gate/up tiles.  One 16-row operand carries 8 gate and the matching
// 8 up rows, so a block streams half the weight bytes of a 16-column one and
// its blocks spread more evenly over the CUs.  Measured on the Qwen3 TP share
// (graph-replayed, same box): T = 4 47.3 -> 44.4 us, T = 8 62.7-62.9 -> 61.4-
// 61.8 us (about 49 touched experts x 12 column tiles = 588 blocks of 16
// columns for 256 CUs: some CUs streamed three, most two); Qwen3 EP view T = 1
// (8 experts x 96 tiles, three per CU, narrowed as 7.8 are expected) 1%
// faster.  At T = 16 and 64, EP T = 16 and Mixtral T = 1 (4-30 blocks per CU)
// it was within about 1% either way (EP T = 16 1.2% slower): every weight load
// then comes with its own activation load.  The expected touched experts
// assume uniform routing.
int ffn_gate_up_pack(int dt, int BM, int T, int k, int E, int E_loc, int I_loc) {
  if (dt != 1 || BM != 16 || T <= 0 || k <= 0 || E <= 0 || I_loc % 16 != 0) return 0;
  const double touched = E_loc * (1.0 - __builtin_pow(1.0 - 1.0 / E, (double)T * k));
  return touched * (I_loc / 16) < 3.0 * 256 ? 1 : 0;
}

long long ffn_gate_up_blocks(const FfnArgs& a, int BM) {
  if (a.dt == 0) return (long long)a.max_tiles * (a.I_loc / 16);
  if (is_tile_bm(BM)) {
    const int cols = tile_shape(BM, true, a.I_loc) == TILE_NARROW ? TileNarrow::TN / 2 : TL_N / 2;
    return (long long)a.max_tiles * (a.I_loc / cols);
  }
  return (long long)a.max_tiles * (a.I_loc / (BM == 16 ? 16 * DIRECT_NT16 : 32));
}

hipError_t launch_ffn_gate_up(const FfnArgs& a, int BM, hipStream_t st, const FfnArgs* also) {
  if (also) {
    if (is_tile_bm(BM)) {
      const TileArgs t2 = gate_up_tile(*also);
      return launch_tile<true, true>(gate_up_tile(a), BM, a.mean_rows, a.max_tiles, &t2,
                                     also->max_tiles, st);
    }
    const DirectArgs g2 = gate_up_direct(*also, BM);
    return launch_direct<true, true>(gate_up_direct(a, BM), BM, a.max_tiles, &g2, also->max_tiles, st,
                                     a.gate_up_pack != 0);
  }
  if (a.max_tiles <= 0) return hipSuccess;
  if (a.dt == 0) {
    if (a.map_bm > 0 && a.map_bm != 16) return hipErrorInvalidValue;
    F32Args g1{(const float*)a.x, a.src_token, a.tile_map, a.n_tiles, a.M_dense,
               (const float*)a.w13, 2LL * a.I_loc * a.H, a.H, a.I_loc, a.I_loc, (float*)a.h};
    ffn_f32_kernel<true><<<a.max_tiles * (a.I_loc / 16), 256, 0, st>>>(g1);
    return hipGetLastError();
  }
  if (is_tile_bm(BM)) {
    if (a.map_bm > 0 && a.map_bm != BM) return hipErrorInvalidValue;
    return launch_tile<true, true>(gate_up_tile(a), BM, a.mean_rows, a.max_tiles, nullptr, 0, st);
  }
  return launch_direct<true, true>(gate_up_direct(a, BM), BM, a.max_tiles, nullptr, 0, st,
                                   a.gate_up_pack != 0);
}

template <bool OUT_BF16>
static hipError_t launch_down_bf16(const FfnArgs& a, int BM, const FfnArgs* also, hipStream_t st) {
  if (is_tile_bm(BM)) {
    if (a.map_bm > 0 && a.map_bm != BM) return hipErrorInvalidValue;
    if (a.down_cols != 0 && a.down_cols != TileMed::TN) {
      if (a.down_cols != TileNarrow::TN || BM != TileMed::TM || also || a.H % TileNarrow::TN != 0)
        return hipErrorInvalidValue;
      TileArgs t = down_tile(a);
      t.group = 1;
      return launch_tile_cfg<TileNarrow, false, OUT_BF16>(t, a.max_tiles, nullptr, 0, a.mean_rows,
                                                          st);
    }
    if (also) {
      const TileArgs t2 = down_tile(*also);
      return launch_tile<false, OUT_BF16>(down_tile(a), BM, a.mean_rows, a.max_tiles, &t2,
                                          also->max_tiles, st);
    }
    return launch_tile<false, OUT_BF16>(down_tile(a), BM, a.mean_rows, a.max_tiles, nullptr, 0, st);
  }
  if (also) {
    const DirectArgs g2 = down_direct(*also, BM);
    return launch_direct<false, OUT_BF16>(down_direct(a, BM), BM, a.max_tiles, &g2, also->max_tiles, st);
  }
  return launch_direct<false, OUT_BF16>(down_direct(a, BM), BM, a.max_tiles, nullptr, 0, st);
}

hipError_t launch_ffn_down(const FfnArgs& a, int BM, hipStream_t st, const FfnArgs* also) {
  if (!also && a.max_tiles <= 0) return hipSuccess;
  if (a.dt == 0) {
    if (a.map_bm > 0 && a.map_bm != 16) return hipErrorInvalidValue;
    F32Args g2{(const float*)a.h, nullptr, a.tile_map, a.n_tiles, a.M_dense,
               (const float*)a.w2, (long long)a.H * a.I_loc, a.I_loc, a.H, 0, (float*)a.y};
    ffn_f32_kernel<false><<<a.max_tiles * (a.H / 16), 256, 0, st>>>(g2);
    return hipGetLastError();
  }
  if (a.y_dt == 0) return launch_down_bf16<false>(a, BM, also, st);
  return launch_down_bf16<true>(a, BM, also, st);
}

GemmPlan plan_layer_gemms(int dt, int T, int k, int E, int E_loc, int H, int I_loc,
                          int I_shared) {
  auto cdiv = [](int a, int b) { return a / b + (a % b != 0); };   // a >= 0, no overflow
  GemmPlan p{};
  const int mean = cdiv(T * k, E);
  p.BM = ffn_row_tile(dt, mean, H, I_loc, T * k < E_loc ? T * k : E_loc);
  p.BM_dn = ffn_down_row_tile(dt, mean, H, I_loc, p.BM);
  p.dn_cols = ffn_down_cols(dt, p.BM_dn, mean, T * k < E_loc ? T * k : E_loc, H);
  p.up_pack = ffn_gate_up_pack(dt, p.BM, T, k, E, E_loc, I_loc);
  if (I_shared <= 0 || T <= 0) return p;
  // the routed problems as the launches see them (any tile count > 0)
  FfnArgs f{};
  f.dt = dt; f.y_dt = dt; f.H = H; f.I_loc = I_loc; f.max_tiles = 1;
  FfnArgs fd = f;
  if (p.BM_dn != p.BM) fd.map_bm = p.BM;
  FfnArgs g{};
  g.dt = dt; g.y_dt = dt; g.H = H; g.I_loc = I_shared; g.M_dense = T;
  p.BMs = ffn_row_tile(dt, T, H, I_shared, 1);
  g.max_tiles = cdiv(T, p.BMs);
  const bool thin = ffn_gate_up_blocks(g, p.BMs) < 256;   // fewer blocks than CUs
  auto pick = [&](const FfnArgs& r, int BMr, bool gate_up, int& BMo) {
    BMo = p.BMs;
    if (ffn_can_share_gemm(r, BMr, g, p.BMs, gate_up)) return (int)SHARE_OWN_TILE;
    if (!thin) return (int)SHARE_NONE;
    FfnArgs g2 = g;
    g2.max_tiles = cdiv(T, BMr);
    if (!ffn_can_share_gemm(r, BMr, g2, BMr, gate_up)) return (int)SHARE_NONE;
    BMo = BMr;
    return (int)SHARE_ROUTED_TILE;
  };
  p.up = pick(f, p.BM, true, p.BMs_up);
  p.dn = pick(fd, p.BM_dn, false, p.BMs_dn);
  return p;
}

hipError_t launch_grouped_ffn(const FfnArgs& a, int BM, hipStream_t st) {
  hipError_t err = launch_ffn_gate_up(a, BM, st);
  if (err != hipSuccess) return err;
  return launch_ffn_down(a, BM, st);
}

}  // namespace moe
