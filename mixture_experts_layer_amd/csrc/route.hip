// Router scores and top-k gating for gfx950.
//
// Router: s = W_r x ("MoE 推理优化全景指南", section 从 Dense FFN 到专家集合).
// Gating variants: "Lecture 8 · 混合专家模型的推理" (CS349D notes) section 1.2.
// Per-tile expert histogram and in-tile ranks feed the stable permutation of
// "MoE 推理优化全景指南", section Dispatch 并不是一次普通 all-to-all.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits, matrix-vector form: one block per expert and group of up to
// TT tokens.  The 256 threads split H; partial dot products are reduced with
// a fixed butterfly + LDS tree, so results are bitwise repeatable.  Used for
// float32 inputs and for small token counts, where the whole of W_r must be
// streamed once by many CUs.
// ---------------------------------------------------------------------------
template <typename Tin, int TT>
__global__ __launch_bounds__(256) void router_gemv_kernel(const Tin* __restrict__ x,
                                                          const Tin* __restrict__ wr, int T, int H,
                                                          int E, const float* __restrict__ bias,
                                                          float* __restrict__ logits) {
  constexpr int VEC = 16 / sizeof(Tin);  // elements per 16-byte load
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * TT;
  const int ntok = min(TT, T - t0);
  float acc[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = 0.f;

  for (int h = threadIdx.x * VEC; h < H; h += 256 * VEC) {
    float wv[8];
    const uint4 wraw = *reinterpret_cast<const uint4*>(wr + (size_t)e * H + h);
    if constexpr (VEC == 8) {
      unpack_bf16x8(wraw, wv);
    } else {
      wv[0] = __uint_as_float(wraw.x); wv[1] = __uint_as_float(wraw.y);
      wv[2] = __uint_as_float(wraw.z); wv[3] = __uint_as_float(wraw.w);
    }
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      if (i < ntok) {
        const uint4 xraw = *reinterpret_cast<const uint4*>(x + (size_t)(t0 + i) * H + h);
        float xv[8];
        if constexpr (VEC == 8) {
          unpack_bf16x8(xraw, xv);
        } else {
          xv[0] = __uint_as_float(xraw.x); xv[1] = __uint_as_float(xraw.y);
          xv[2] = __uint_as_float(xraw.z); xv[3] = __uint_as_float(xraw.w);
        }
        float a = acc[i];
#pragma unroll
        for (int q = 0; q < VEC; ++q) a = fmaf(xv[q], wv[q], a);
        acc[i] = a;
      }
    }
  }
  __shared__ float red[4][TT];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    float v = acc[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) red[wid][i] = v;
  }
  __syncthreads();
  if (threadIdx.x < ntok) {
    const int i = threadIdx.x;
    float v = (red[0][i] + red[1][i]) + (red[2][i] + red[3][i]);
    if (bias) v += bias[e];
    logits[(size_t)(t0 + i) * E + e] = v;
  }
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
                                                          int H, const float* __restrict__ bias,
                                                          float* __restrict__ logits) {
  constexpr int E = 32 * EW;
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
    wsrc[j] = wr + (size_t)rt * H + (pch ^ rt_swz(rt)) * 8;
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
      const int e = nb * 16 + 4 * kq;
      float4 v = make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
      if (bias) {
        v.x += bias[e]; v.y += bias[e + 1]; v.z += bias[e + 2]; v.w += bias[e + 3];
      }
      *reinterpret_cast<float4*>(logits + (size_t)t * E + e) = v;
    }
  }
}

template <int EW>
static hipError_t launch_router_mfma(const bf16_t* x, const bf16_t* wr, int T, int H,
                                     const float* bias, float* logits, hipStream_t st) {
  static bool attr_set = false;
  const int lds = RT_STAGES * (RT_TOK * 128 + 32 * EW * 128);
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&router_mfma_kernel<EW>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  router_mfma_kernel<EW><<<(T + RT_TOK - 1) / RT_TOK, 256, lds, st>>>(x, wr, T, H, bias, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Wave-wide reductions: DPP inside each 16-lane row (pairs at distance 1, 2,
// then the half-row and row mirrors), then the four row results via
// readlane.  Every lane ends with the result; the combination order is fixed,
// so float sums are the same on every run.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

// (key, id) arg-max: larger key wins, equal keys go to the smaller id.
__device__ __forceinline__ bool better(float ok, int oi, float k, int i) {
  return ok > k || (ok == k && oi < i);
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& k, int& i) {
  const float ok = dpp_f<CTRL>(k);
  const int oi = dpp_i<CTRL>(i);
  if (better(ok, oi, k, i)) { k = ok; i = oi; }
}
__device__ __forceinline__ void wave_argmax(float& k, int& i) {
  argmax_step<DPP_XOR1>(k, i);
  argmax_step<DPP_XOR2>(k, i);
  argmax_step<DPP_HALF_MIRROR>(k, i);
  argmax_step<DPP_MIRROR>(k, i);
  float bk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, k), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const float ok = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, k), r));
    const int oi = __builtin_amdgcn_readlane(i, r);
    if (better(ok, oi, bk, bi)) { bk = ok; bi = oi; }
  }
  k = bk;
  i = bi;
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<DPP_XOR1>(v);
  v += dpp_f<DPP_XOR2>(v);
  v += dpp_f<DPP_HALF_MIRROR>(v);
  v += dpp_f<DPP_MIRROR>(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<DPP_XOR1>(v));
  v = fmaxf(v, dpp_f<DPP_XOR2>(v));
  v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f<DPP_MIRROR>(v));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// ---------------------------------------------------------------------------
// Gating + routing metadata for one tile of TOK_TILE tokens (NW waves; a
// wave takes tokens wid, wid + NW, ...; the next token's logits are loaded
// while the current one is processed).
//
// Selection: k rounds of a wave-wide arg-max over (key descending, id
// ascending); the key is the logit, or logit + sel_bias in float32 for the
// sigmoid mode.  Exact comparisons only, so the chosen ids are a function of
// the float32 logits alone.
//
// Histogram and ranks (no atomics): after the tile's ids are in LDS, thread
// e walks the tile's (token, slot) pairs in order and numbers the ones routed
// to local expert e.  The rank of a pair inside its expert's segment of the
// tile is that number, so rows keep ascending token order.
//
// single != 0 (the whole batch is this one tile): the block also finishes the
// permutation -- counts, offsets, dst_row, src_token and the GEMM tile map.
// Otherwise it writes the tile's counts and the pairs' in-tile ranks for the
// scan and scatter kernels.
// do_gate == 0: ids come from ids_in (permutation only, no gating).
// ---------------------------------------------------------------------------
template <int EPL, int NW>
__global__ __launch_bounds__(NW * 64) void gate_tile_kernel(GateTileArgs a) {
  __shared__ __attribute__((aligned(16))) int s_ids[TOK_TILE * KMAX];
  __shared__ int s_rank[TOK_TILE * KMAX];
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1025];
  __shared__ int s_scr[1024];
  __shared__ int s_tmp[NW * 64 + 1];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int t0 = tile * TOK_TILE;
  const int ntok = max(0, min(TOK_TILE, a.T - t0));
  const int k = a.k, E = a.E;
  const bool sig = a.mode == 3;

  if (a.do_gate) {
    float s_next[EPL];
    auto load = [&](int tt, float* s) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        s[i] = (tt < ntok && e < E) ? a.logits[(size_t)(t0 + tt) * E + e] : 0.f;
      }
    };
    load(wid, s_next);
    for (int tt = wid; tt < ntok; tt += NW) {
      const int t = t0 + tt;
      float s[EPL], key[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) s[i] = s_next[i];
      load(tt + NW, s_next);
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < E ? s[i] : -INFINITY;
        if (sig && a.sel_bias && e < E) key[i] = s[i] + a.sel_bias[e];
      }
      bool avail[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) avail[i] = lane + 64 * i < E;
      int sel_id = -1;       // lane j < k keeps the j-th choice
      float sel_s = 0.f;
      for (int r = 0; r < k; ++r) {
        float bk = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          const int e = lane + 64 * i;
          if (avail[i] && better(key[i], e, bk, bi)) { bk = key[i]; bi = e; }
        }
        wave_argmax(bk, bi);
        // the owner lane retires the winner; every lane learns its logit
        float win_s = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (lane + 64 * i == bi) {
            avail[i] = false;
            win_s = s[i];
          }
        win_s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, win_s),
                                                                    bi & 63));
        if (lane == r) {
          sel_id = bi;
          sel_s = win_s;
        }
      }
      // gate weights of the k choices (lanes 0..k-1)
      const bool mine = lane < k;
      float wv;
      if (a.mode == 0) {
        const float m = wave_max(mine ? sel_s : -INFINITY);
        const float ev = mine ? expf(sel_s - m) : 0.f;
        wv = ev / wave_sum(ev);
      } else if (a.mode == 1 || a.mode == 2) {
        // softmax over all E; the largest logit is the first choice
        const float m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sel_s), 0));
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (lane + 64 * i < E) z += expf(s[i] - m);
        z = wave_sum(z);
        float p = mine ? expf(sel_s - m) / z : 0.f;
        if (a.mode == 2) p = p / wave_sum(p);
        wv = p;
      } else {
        const float sg = mine ? 1.0f / (1.0f + expf(-sel_s)) : 0.f;
        wv = sg / wave_sum(sg);
      }
      if (mine) {
        a.ids_out[(size_t)t * k + lane] = sel_id;
        a.w_out[(size_t)t * k + lane] = wv;
        s_ids[tt * k + lane] = sel_id;
      }
    }
  } else {
    for (int i = threadIdx.x; i < ntok * k; i += NW * 64) s_ids[i] = a.ids_in[(size_t)t0 * k + i];
  }
  if (!a.do_permute) return;
  const int npair = ntok * k;
  // pad the id list to a multiple of 16 with an id no expert has
  for (int p = npair + threadIdx.x; p < ((npair + 15) & ~15); p += NW * 64) s_ids[p] = -1;
  __syncthreads();

  // atomic-free histogram and in-tile ranks, 16 ids per LDS pass
  const int E_loc = a.e_end - a.e_begin;
  for (int el = threadIdx.x; el < E_loc; el += NW * 64) {
    const int e = a.e_begin + el;
    int c = 0;
    for (int p = 0; p < npair; p += 16) {
      const int4* q = reinterpret_cast<const int4*>(s_ids + p);
      const int4 v0 = q[0], v1 = q[1], v2 = q[2], v3 = q[3];
      const int ids16[16] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w,
                             v2.x, v2.y, v2.z, v2.w, v3.x, v3.y, v3.z, v3.w};
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (ids16[j] == e) s_rank[p + j] = c++;
    }
    s_cnt[el] = c;
  }
  __syncthreads();

  if (!a.single) {
    for (int el = threadIdx.x; el < E_loc; el += NW * 64)
      a.tile_counts[(size_t)tile * E_loc + el] = s_cnt[el];
    for (int p = threadIdx.x; p < npair; p += NW * 64) {
      const int e = s_ids[p];
      const bool local = e >= a.e_begin && e < a.e_end;
      a.rank_out[(size_t)t0 * k + p] = local ? s_rank[p] : -1;
    }
    return;
  }

  // single tile: finish the permutation here
  for (int el = threadIdx.x; el < E_loc; el += NW * 64) s_off[el] = s_cnt[el];
  __syncthreads();
  const int total = block_exclusive_scan(s_off, E_loc, s_tmp);
  if (threadIdx.x == 0) s_off[E_loc] = total;
  __syncthreads();
  for (int el = threadIdx.x; el < E_loc; el += NW * 64) a.counts[el] = s_cnt[el];
  for (int el = threadIdx.x; el <= E_loc; el += NW * 64) a.offsets[el] = s_off[el];
  for (int p = threadIdx.x; p < npair; p += NW * 64) {
    const int e = s_ids[p];
    int row = -1;
    if (e >= a.e_begin && e < a.e_end) {
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
  const bool mfma_shape = dt == 1 && T > 32 && H % RT_K == 0 &&
                          (E == 32 || E == 64 || E == 128 || E == 256);
  if (!mfma_shape) {
    dim3 grid(E, (T + 7) / 8);
    if (dt == 0)
      router_gemv_kernel<float, 8><<<grid, 256, 0, st>>>((const float*)x, (const float*)wr, T, H,
                                                         E, bias, logits);
    else
      router_gemv_kernel<bf16_t, 8><<<grid, 256, 0, st>>>((const bf16_t*)x, (const bf16_t*)wr, T,
                                                          H, E, bias, logits);
    return hipGetLastError();
  }
  const bf16_t* xb = (const bf16_t*)x;
  const bf16_t* wb = (const bf16_t*)wr;
  switch (E) {
    case 32: return launch_router_mfma<1>(xb, wb, T, H, bias, logits, st);
    case 64: return launch_router_mfma<2>(xb, wb, T, H, bias, logits, st);
    case 128: return launch_router_mfma<4>(xb, wb, T, H, bias, logits, st);
    default: return launch_router_mfma<8>(xb, wb, T, H, bias, logits, st);
  }
}

template <int NW>
static void launch_gate_nw(const GateTileArgs& a, int grid, hipStream_t st) {
  const int epl = (a.E + 63) / 64;
  if (epl <= 1) gate_tile_kernel<1, NW><<<grid, NW * 64, 0, st>>>(a);
  else if (epl <= 2) gate_tile_kernel<2, NW><<<grid, NW * 64, 0, st>>>(a);
  else if (epl <= 4) gate_tile_kernel<4, NW><<<grid, NW * 64, 0, st>>>(a);
  else if (epl <= 8) gate_tile_kernel<8, NW><<<grid, NW * 64, 0, st>>>(a);
  else gate_tile_kernel<16, NW><<<grid, NW * 64, 0, st>>>(a);
}

hipError_t launch_gate_tiles(const GateTileArgs& a, int n_tiles_tok, hipStream_t st) {
  const int grid = n_tiles_tok > 0 ? n_tiles_tok : 1;
  // one tile (decode-sized batch): 16 waves share its 64 tokens
  if (grid == 1) launch_gate_nw<16>(a, grid, st);
  else launch_gate_nw<4>(a, grid, st);
  return hipGetLastError();
}

}  // namespace moe
