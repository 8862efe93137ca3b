// Router scores and top-k gating for gfx950.
//
// Router: s = W_r x ("MoE 推理优化全景指南", section 从 Dense FFN 到专家集合).
// Gating variants: "Lecture 8 · 混合专家模型的推理" (CS349D notes) section 1.2.
// Per-tile expert histogram and in-tile ranks feed the stable permutation of
// "MoE 推理优化全景指南", section Dispatch 并不是一次普通 all-to-all.
#include "moe_device.h"
#include "moe_gate.h"
#include "moe_kernels.h"
#include "moe_router.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits, matrix-vector form: one wave per (expert, pair of tokens),
// four per block (router_dot_wave: lanes split H, a fixed butterfly sums
// them, so results are bitwise repeatable and equal to the decode kernel's).
// Used for float32 inputs and for small token counts, where the whole of W_r
// must be streamed by many CUs.  Two tokens per wave keep each wave's loads to
// one round trip (8 chunks of the weight row and of each token per lane) and
// give the CUs many waves to switch between; W_r is read once per token pair,
// mostly from L2.
// ---------------------------------------------------------------------------
constexpr int RT_GEMV_TOK = 2;

template <typename Tin>
__global__ __launch_bounds__(256) void router_gemv_kernel(const Tin* __restrict__ x,
                                                          const Tin* __restrict__ wr, int T, int H,
                                                          int E, const float* __restrict__ bias,
                                                          float* __restrict__ logits) {
  const int ntg = (T + RT_GEMV_TOK - 1) / RT_GEMV_TOK;
  const int u = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u >= E * ntg) return;
  const int e = u / ntg, t0 = (u - e * ntg) * RT_GEMV_TOK;
  router_dot_wave<Tin, false, 8, RT_GEMV_TOK>(x, wr, H, E, e, t0, min(RT_GEMV_TOK, T - t0), bias,
                                              logits);
}

// ---------------------------------------------------------------------------
// Router logits on bf16 MFMA: one block (4 waves) per 64 tokens and all E
// experts (E = 32 * EW, E <= 256).  Token rows and W_r rows reach LDS in K
// chunks of 64 through global_load_lds_dwordx4, three chunks in flight, rows
// XOR-swizzled in 16-byte chunks against bank conflicts.  Each wave owns 16
// tokens: v_mfma_f32_16x16x32_bf16 with A = W_r fragment (row = expert),
// B = token fragment; accumulator lane l holds token l % 16 and experts
// 4*(l/16) + i, stored as one 16-byte vector.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

constexpr int RT_TOK = 64, RT_K = 64, RT_STAGES = 3;

__device__ __forceinline__ int rt_swz(int r) { return (r >> 1) & 7; }

template <int EW>
__global__ __launch_bounds__(256) void router_mfma_kernel(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wr, int T,
                                                          int H, int E_all,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits) {
  constexpr int E = 32 * EW;                // experts of this block: e0 .. e0 + E - 1
  const int e0 = blockIdx.y * E;
  constexpr int XB = RT_TOK * 128;          // token chunk bytes
  constexpr int WB = E * 128;               // W_r chunk bytes
  constexpr int SB = XB + WB;
  constexpr int NL = 2 + EW;                // loads per wave per stage
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int t0 = blockIdx.x * RT_TOK;
  const int prow = lane >> 3, pch = lane & 7;

  const bf16_t* xsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rt = (wid + 4 * j) * 8 + prow;
    const int t = min(t0 + rt, T - 1);
    xsrc[j] = x + (size_t)t * H + (pch ^ rt_swz(rt)) * 8;
  }
  const bf16_t* wsrc[EW];
#pragma unroll
  for (int j = 0; j < EW; ++j) {
    const int rt = (wid + 4 * j) * 8 + prow;
    // rows past E (a block covering the last E % 32 experts) read row E-1;
    // their results are never stored
    wsrc[j] = wr + (size_t)min(e0 + rt, E_all - 1) * H + (pch ^ rt_swz(rt)) * 8;
  }
  auto issue = [&](int ks, int buf) {
    unsigned char* sx = smem + buf * SB;
    unsigned char* sw = sx + XB;
    const int ko = ks * RT_K;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(xsrc[j] + ko),
                                       (lds_void_t*)(sx + (wid + 4 * j) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < EW; ++j)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(wsrc[j] + ko),
                                       (lds_void_t*)(sw + (wid + 4 * j) * 1024), 16, 0, 0);
  };

  f32x4_t acc[E / 16];
#pragma unroll
  for (int i = 0; i < E / 16; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int lrow = lane & 15, kq = lane >> 4;
  // this lane's four experts' bias per 16-expert group, loaded ahead of the
  // K loop (loaded in the epilogue, under its branches, each had cost a wait)
  float4 bv[E / 16];
#pragma unroll
  for (int nb = 0; nb < E / 16; ++nb) {
    const int e = e0 + nb * 16 + 4 * kq;
    bv[nb] = (bias && e < E_all) ? *reinterpret_cast<const float4*>(bias + e)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int nk = H / RT_K;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int ks = 0; ks < nk; ++ks) {
    // stage ks landed once at most the NL loads of stage ks+1 are pending;
    // the previous stage's fragments were consumed by its MFMAs
    if (ks + 1 < nk) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(NL) : "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (ks + 2 < nk) issue(ks + 2, (ks + 2) % RT_STAGES);
    const unsigned char* sx = smem + (ks % RT_STAGES) * SB;
    const unsigned char* sw = sx + XB;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + kq;
      const int xr = wid * 16 + lrow;
      const bf16x8_t xf = *reinterpret_cast<const bf16x8_t*>(sx + xr * 128 + ((c ^ rt_swz(xr)) * 16));
#pragma unroll
      for (int nb = 0; nb < E / 16; ++nb) {
        const int wrow = nb * 16 + lrow;
        const bf16x8_t wf =
            *reinterpret_cast<const bf16x8_t*>(sw + wrow * 128 + ((c ^ rt_swz(wrow)) * 16));
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf, acc[nb], 0, 0, 0);
      }
    }
  }
  const int t = t0 + wid * 16 + lrow;
  if (t < T) {
#pragma unroll
    for (int nb = 0; nb < E / 16; ++nb) {
      const int e = e0 + nb * 16 + 4 * kq;
      if (e >= E_all) continue;                 // E is a multiple of 4
      float4 v = make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
      if (bias) {
        v.x += bv[nb].x; v.y += bv[nb].y; v.z += bv[nb].z; v.w += bv[nb].w;
      }
      *reinterpret_cast<float4*>(logits + (size_t)t * E_all + e) = v;
    }
  }
}

// Each block covers 64 tokens and 32*EW experts; E is split over the grid's
// second dimension so that a large E gives more blocks (and each block a
// smaller share of W_r to stream through LDS).  EW = 2 when 64 divides E and
// the grid still has 128 blocks, else EW = 1 (with a partial last block when
// 32 does not divide E: few experts, the tokens still read once where a
// per-expert GEMV would read them E times).
template <int EW>
static hipError_t launch_router_mfma(const bf16_t* x, const bf16_t* wr, int T, int H, int E,
                                     const float* bias, float* logits, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  const int lds = RT_STAGES * (RT_TOK * 128 + 32 * EW * 128);
  hipError_t err =
      ensure_lds_limit(reinterpret_cast<const void*>(&router_mfma_kernel<EW>), lds, lds_set);
  if (err != hipSuccess) return err;
  const dim3 grid((T + RT_TOK - 1) / RT_TOK, (E + 32 * EW - 1) / (32 * EW));
  router_mfma_kernel<EW><<<grid, 256, lds, st>>>(x, wr, T, H, E, bias, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gating + routing metadata for one tile of TOK_TILE tokens.
//
// Selection: each 16-lane row of a wave owns one token (gate_row: k rounds
// of a row-wide arg-max); with 16 waves the tile's 64 tokens are all in
// flight at once (four waves per SIMD hide the DPP and LDS latencies).  Lane
// `sub` holds experts sub, sub + 16, ... (EPR of them).  The tile's logits
// are staged in LDS (E <= 256) with a row pitch that puts the 64 lanes of a
// wave in 64 distinct banks.  The gate weights are finished in the row and
// written straight out.
//
// Histogram and ranks: the tile's tokens routed to a local expert form a
// 64-bit mask (one bit per token of the tile; a token's k ids are distinct),
// built with one LDS atomic OR per pair -- the result does not depend on
// their order.  The expert's count is the mask's popcount, and the rank of
// pair (t, j) inside the expert's segment of the tile is the popcount of the
// bits below t, so rows keep ascending token order.
//
// single != 0 (the whole batch is this one tile): the block also finishes the
// permutation -- counts, offsets, dst_row, src_token and the GEMM tile map.
// Otherwise it writes the tile's counts and the pairs' in-tile ranks for the
// scan and scatter kernels.
// do_gate == 0: ids come from ids_in (permutation only, no gating).
// ---------------------------------------------------------------------------
constexpr int GATE_STAGE_E = 256;                       // largest E staged in LDS
constexpr int GATE_PITCH_MAX = GATE_STAGE_E + 4;

template <int EPR>
struct GateWaves {
  // 16 waves while a lane's experts fit comfortably in 128 VGPRs
  static constexpr int value = EPR <= 16 ? 16 : 4;
};

template <int EPR, bool STAGE>
__global__ __launch_bounds__(GateWaves<EPR>::value * 64) void gate_tile_kernel(GateTileArgs a) {
  constexpr int NW = GateWaves<EPR>::value;
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) int s_ids[TOK_TILE * KMAX];
  __shared__ int s_rank[TOK_TILE * KMAX];
  __shared__ __attribute__((aligned(16))) float s_logits[STAGE ? TOK_TILE * GATE_PITCH_MAX : 4];
  __shared__ int s_cnt[1024];
  __shared__ unsigned long long s_mask[1024];
  __shared__ int s_drop;
  __shared__ int s_off[1025];
  __shared__ int s_scr[1024];
  __shared__ int s_tmp[NT + 1];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int tpb = a.tok_per_block > 0 ? a.tok_per_block : TOK_TILE;
  const int t0 = tile * tpb;
  const int ntok = max(0, min(tpb, a.T - t0));
  const int k = a.k, E = a.E;
  const int mode = a.mode;

  if (a.do_gate) {
    const int P = ((E + 63) & ~63) + 4;               // LDS row pitch (floats)
    if (STAGE) {
      const float* src = a.logits + (size_t)t0 * E;
      const int nval = ntok * E;
      if ((E & 3) == 0) {
        // 16-byte loads, up to four in flight per thread; a 16-byte group
        // never straddles two rows when E is a multiple of 4
        const int nv4 = nval >> 2;
        const float4* src4 = reinterpret_cast<const float4*>(src);
        for (int i0 = threadIdx.x; i0 < nv4; i0 += 4 * NT) {
          float4 v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = src4[min(i0 + u * NT, nv4 - 1)];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = (i0 + u * NT) * 4;
            if (i < nval) {
              const int r = i / E, c = i - r * E;
              *reinterpret_cast<float4*>(s_logits + r * P + c) = v[u];
            }
          }
        }
      } else {
        for (int i = threadIdx.x; i < nval; i += NT) s_logits[(i / E) * P + i % E] = src[i];
      }
      lds_barrier();
    }
    const int row = lane >> 4, sub = lane & 15;
    if (ntok <= NW) {
      // a whole wave per token (gate_select64: a quarter of gate_row's keys
      // per lane, so shorter rounds); every row then finishes the weights
      // exactly as gate_row would, and row 0 keeps them
      constexpr int EPR64 = (EPR + 3) / 4;
      const int tt = wid;
      if (tt < ntok) {
        float s64[EPR64], s[EPR];
#pragma unroll
        for (int i = 0; i < EPR64; ++i) {
          const int e = lane + 64 * i;
          s64[i] = e < E ? (STAGE ? s_logits[tt * P + e] : a.logits[(size_t)(t0 + tt) * E + e])
                         : 0.f;
        }
#pragma unroll
        for (int i = 0; i < EPR; ++i) {
          const int e = sub + 16 * i;
          s[i] = e < E ? (STAGE ? s_logits[tt * P + e] : a.logits[(size_t)(t0 + tt) * E + e])
                       : 0.f;
        }
        unsigned long long c0, c1, first;
        gate_select64<EPR64>(s64, true, E, k, mode, a.sel_bias, c0, c1, first);
        int id0, id1;
        float g0, g1;
        gate_weights<EPR>(s, true, sub, E, k, mode, c0, c1, first, id0, g0, id1, g1);
        if (row == 0 && sub < k) {
          s_ids[tt * k + sub] = id0;
          a.ids_out[(size_t)(t0 + tt) * k + sub] = id0;
          a.w_out[(size_t)(t0 + tt) * k + sub] = g0;
        }
        if (row == 0 && sub + 16 < k) {
          s_ids[tt * k + sub + 16] = id1;
          a.ids_out[(size_t)(t0 + tt) * k + sub + 16] = id1;
          a.w_out[(size_t)(t0 + tt) * k + sub + 16] = g1;
        }
      }
    }
    for (int pass = 0; ntok > NW && pass * NW * 4 < ntok; ++pass) {
      if (pass * NW * 4 + wid * 4 >= ntok) break;   // no token of this wave left
      const int tt = pass * NW * 4 + wid * 4 + row;
      const bool live = tt < ntok;
      float s[EPR];
#pragma unroll
      for (int i = 0; i < EPR; ++i) {
        const int e = sub + 16 * i;
        s[i] = (live && e < E)
                   ? (STAGE ? s_logits[tt * P + e] : a.logits[(size_t)(t0 + tt) * E + e])
                   : 0.f;
      }
      int id0, id1;
      float g0, g1;
      gate_row<EPR>(s, live, sub, E, k, mode, a.sel_bias, id0, g0, id1, g1);
      const bool h0 = live && sub < k, h1 = live && sub + 16 < k;
      if (h0) {
        s_ids[tt * k + sub] = id0;
        a.ids_out[(size_t)(t0 + tt) * k + sub] = id0;
        a.w_out[(size_t)(t0 + tt) * k + sub] = g0;
      }
      if (h1) {
        s_ids[tt * k + sub + 16] = id1;
        a.ids_out[(size_t)(t0 + tt) * k + sub + 16] = id1;
        a.w_out[(size_t)(t0 + tt) * k + sub + 16] = g1;
      }
    }
  } else {
    for (int i = threadIdx.x; i < ntok * k; i += NT) s_ids[i] = a.ids_in[(size_t)t0 * k + i];
  }
  if (!a.do_permute) return;
  const int npair = ntok * k;
  const int E_loc = a.e_end - a.e_begin;
  for (int el = threadIdx.x; el < E_loc; el += NT) s_mask[el] = 0ull;
  if (threadIdx.x == 0) s_drop = 0;
  lds_barrier();
  for (int p = threadIdx.x; p < npair; p += NT) {
    const int el = s_ids[p] - a.e_begin;
    if (el >= 0 && el < E_loc) atomicOr(&s_mask[el], 1ull << (p / k));
  }
  lds_barrier();
  for (int el = threadIdx.x; el < E_loc; el += NT) s_cnt[el] = __popcll(s_mask[el]);
  for (int p = threadIdx.x; p < npair; p += NT) {
    const int el = s_ids[p] - a.e_begin;
    if (el >= 0 && el < E_loc) s_rank[p] = __popcll(s_mask[el] & ((1ull << (p / k)) - 1ull));
  }
  lds_barrier();

  if (!a.single) {
    for (int el = threadIdx.x; el < E_loc; el += NT)
      a.tile_counts[(size_t)tile * E_loc + el] = s_cnt[el];
    for (int p = threadIdx.x; p < npair; p += NT) {
      const int e = s_ids[p];
      const bool local = e >= a.e_begin && e < a.e_end;
      a.rank_out[(size_t)t0 * k + p] = local ? s_rank[p] : -1;
    }
    return;
  }

// single tile: finish the permutation here (an expert over capacity keeps
// its first pairs in token order: their ranks are below the capacity)
  if (E_loc <= 256) {
    // wave 0 alone (DPP scans; the block-wide scans below are for more
    // experts)
    if (wid == 0)
      wave_routing_metadata(s_cnt, E_loc, a.capacity, false, a.BM, a.max_rows, a.max_tiles, s_off,
                            a.counts, a.offsets, a.dropped, a.tile_map, a.n_tiles);
    lds_barrier();
    for (int p = threadIdx.x; p < npair; p += NT) {
      const int e = s_ids[p];
      int row = -1;
      if (e >= a.e_begin && e < a.e_end && s_rank[p] < a.capacity) {
        row = s_off[e - a.e_begin] + s_rank[p];
        a.src_token[row] = p / k;
      }
      a.dst_row[p] = row;
    }
    return;
  }
  int drop = 0;
  for (int el = threadIdx.x; el < E_loc; el += NT) {
    const int kept = min(s_cnt[el], a.capacity);
    drop += s_cnt[el] - kept;
    s_cnt[el] = kept;
    s_off[el] = kept;
  }
  if (a.dropped && drop) atomicAdd(&s_drop, drop);   // an integer total
  lds_barrier();
  if (a.dropped && threadIdx.x == 0) a.dropped[0] = s_drop;
  const int total = block_exclusive_scan(s_off, E_loc, s_tmp);
  if (threadIdx.x == 0) s_off[E_loc] = total;
  lds_barrier();
  for (int el = threadIdx.x; el < E_loc; el += NT) a.counts[el] = s_cnt[el];
  for (int el = threadIdx.x; el <= E_loc; el += NT) a.offsets[el] = s_off[el];
  for (int p = threadIdx.x; p < npair; p += NT) {
    const int e = s_ids[p];
    int row = -1;
    if (e >= a.e_begin && e < a.e_end && s_rank[p] < a.capacity) {
      row = s_off[e - a.e_begin] + s_rank[p];
      a.src_token[row] = p / k;
    }
    a.dst_row[p] = row;
  }
  if (a.tile_map)
    block_build_tile_map(s_cnt, s_off, E_loc, a.BM, a.max_rows, a.max_tiles, s_scr, s_tmp,
                         a.tile_map, a.n_tiles);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const void* x, const void* wr, int dt, int T, int H, int E,
                                const float* bias, float* logits, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  // bf16 prefill batches with E a multiple of 4 (16-byte logit stores).
  // The MFMA kernel has one block per 64 tokens and 64 experts, so with at
  // most 128 experts and a few hundred tokens it runs on a handful of CUs;
  // the per-expert dot products spread over E * T / 2 waves instead.  Up to
  // 256 tokens with E <= 128 they won (Qwen3 EP view T = 128 routing stage
  // 44.7 -> 31 us, T = 256 45 -> 40 us, Mixtral T = 256 32 -> 18 us); with
  // 256 experts (DeepSeek-V3 T = 256, 70 -> 84 us) and at T = 1024 (47 ->
  // 87 us) the MFMA kernel stays ahead.
  const int gemv_max_t = E <= 128 ? 256 : 64;
  const bool mfma_shape = dt == 1 && T > gemv_max_t && H % RT_K == 0 && E % 4 == 0;
  if (!mfma_shape) {
    const long long units = (long long)E * ((T + RT_GEMV_TOK - 1) / RT_GEMV_TOK);
    const int grid = (int)((units + 3) / 4);
    if (dt == 0)
      router_gemv_kernel<float><<<grid, 256, 0, st>>>((const float*)x, (const float*)wr, T, H, E,
                                                      bias, logits);
    else
      router_gemv_kernel<bf16_t><<<grid, 256, 0, st>>>((const bf16_t*)x, (const bf16_t*)wr, T, H,
                                                       E, bias, logits);
    return hipGetLastError();
  }
  const bf16_t* xb = (const bf16_t*)x;
  const bf16_t* wb = (const bf16_t*)wr;
  // 64 experts per block when that still gives half the CUs a block, else
  // 32 (twice the blocks, each with a smaller share of W_r to stream):
  // routing stage 49 -> 42 us at the Qwen3 EP view's T = 512 and 50 -> 43 us
  // at T = 1024, DeepSeek-V3 T = 1024 72 -> 68 us
  if (E % 64 == 0 && (long long)((T + RT_TOK - 1) / RT_TOK) * (E / 64) >= 128)
    return launch_router_mfma<2>(xb, wb, T, H, E, bias, logits, st);
  return launch_router_mfma<1>(xb, wb, T, H, E, bias, logits, st);
}

// E <= 256 (at most 16 experts per lane) stages the logits in LDS.
template <int EPR>
static void launch_gate_epr(const GateTileArgs& a, int grid, hipStream_t st) {
  constexpr bool stage = EPR * 16 <= GATE_STAGE_E;
  gate_tile_kernel<EPR, stage><<<grid, GateWaves<EPR>::value * 64, 0, st>>>(a);
}

hipError_t launch_gate_tiles(const GateTileArgs& a, int n_tiles_tok, hipStream_t st) {
  // a token count per block other than the tile's serves the gating alone
  if (a.tok_per_block < 0 || a.tok_per_block > TOK_TILE || (a.tok_per_block > 0 && a.do_permute))
    return hipErrorInvalidValue;
  const int grid = n_tiles_tok > 0 ? n_tiles_tok : 1;
  const int epr = (a.E + 15) / 16;          // experts per lane of a 16-lane row
  if (epr <= 1) launch_gate_epr<1>(a, grid, st);
  else if (epr <= 2) launch_gate_epr<2>(a, grid, st);
  else if (epr <= 4) launch_gate_epr<4>(a, grid, st);
  else if (epr <= 8) launch_gate_epr<8>(a, grid, st);
  else if (epr <= 16) launch_gate_epr<16>(a, grid, st);
  else if (epr <= 32) launch_gate_epr<32>(a, grid, st);
  else launch_gate_epr<64>(a, grid, st);
  return hipGetLastError();
}

}  // namespace moe
