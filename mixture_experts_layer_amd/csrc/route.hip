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
// experts (E <= 256).  W_r is staged through LDS in K chunks of 64 and shared
// by the 4 waves; each wave owns 16 tokens.  v_mfma_f32_16x16x32_bf16 with
// A = x fragment (row = token), B = W_r fragment (column = expert); the
// accumulator lane l holds token 4*(l/16)+i, expert l%16.
// ---------------------------------------------------------------------------
constexpr int RT_KC = 64;          // K chunk
constexpr int RT_LD = RT_KC + 8;   // LDS row pitch (bf16), padded against bank conflicts

__global__ __launch_bounds__(256) void router_mfma_kernel(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wr, int T,
                                                          int H, int E,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) bf16_t sw[256 * RT_LD];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int Ep = (E + 15) & ~15;
  const int nb = Ep >> 4;
  const int t0 = blockIdx.x * 64 + wid * 16;
  const int my_tok = t0 + (lane & 15);
  const bool tok_ok = my_tok < T;
  const int kg = (lane >> 4) * 8;

  f32x4_t acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < H; k0 += RT_KC) {
    __syncthreads();
    // stage W_r[0:Ep, k0:k0+64): Ep rows x 8 chunks of 16 bytes
    for (int c = threadIdx.x; c < Ep * 8; c += 256) {
      const int r = c >> 3, q = (c & 7) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < E) v = *reinterpret_cast<const uint4*>(wr + (size_t)r * H + k0 + q);
      *reinterpret_cast<uint4*>(sw + r * RT_LD + q) = v;
    }
    uint4 a0 = make_uint4(0, 0, 0, 0), a1 = make_uint4(0, 0, 0, 0);
    if (tok_ok) {
      const bf16_t* xp = x + (size_t)my_tok * H + k0 + kg;
      a0 = *reinterpret_cast<const uint4*>(xp);
      a1 = *reinterpret_cast<const uint4*>(xp + 32);
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      if (n < nb) {
        const bf16_t* bp = sw + (n * 16 + (lane & 15)) * RT_LD + kg;
        const uint4 b0 = *reinterpret_cast<const uint4*>(bp);
        const uint4 b1 = *reinterpret_cast<const uint4*>(bp + 32);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(b0), acc[n], 0, 0, 0);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(b1), acc[n], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    if (n < nb) {
      const int e = n * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = blockIdx.x * 64 + wid * 16 + (lane >> 4) * 4 + i;
        if (t < T && e < E) logits[(size_t)t * E + e] = acc[n][i] + (bias ? bias[e] : 0.f);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Gating + routing metadata for one tile of TOK_TILE tokens (4 waves, one
// token per wave at a time).
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
template <int EPL>
__global__ __launch_bounds__(256) void gate_tile_kernel(GateTileArgs a) {
  __shared__ int s_ids[TOK_TILE * KMAX];
  __shared__ int s_rank[TOK_TILE * KMAX];
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1025];
  __shared__ int s_scr[1024];
  __shared__ int s_tmp[257];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int t0 = tile * TOK_TILE;
  const int ntok = max(0, min(TOK_TILE, a.T - t0));
  const int k = a.k, E = a.E;

  if (a.do_gate) {
    for (int tt = wid; tt < ntok; tt += 4) {
      const int t = t0 + tt;
      float key[EPL], s[EPL];
      bool avail[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        avail[i] = e < E;
        s[i] = avail[i] ? a.logits[(size_t)t * E + e] : 0.f;
        key[i] = s[i];
        if (a.mode == 3 && a.sel_bias && avail[i]) key[i] = s[i] + a.sel_bias[e];
      }
      int sel_id = -1;       // lane j < k keeps the j-th choice
      float sel_s = 0.f;
      for (int r = 0; r < k; ++r) {
        // local best among available entries
        float bk = 0.f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          const int e = lane + 64 * i;
          if (avail[i] && (bi == 0x7fffffff || key[i] > bk)) {
            bk = key[i];
            bi = e;
          }
        }
        // wave arg-max: larger key wins, equal keys -> smaller id
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float ok = __shfl_xor(bk, o);
          const int oi = __shfl_xor(bi, o);
          const bool take = (oi != 0x7fffffff) &&
                            (bi == 0x7fffffff || ok > bk || (ok == bk && oi < bi));
          if (take) {
            bk = ok;
            bi = oi;
          }
        }
        // owner lane retires the winner and reports its logit
        float win_s = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (lane + 64 * i == bi) {
            avail[i] = false;
            win_s = s[i];
          }
        const int owner = bi & 63;
        win_s = __shfl(win_s, owner);
        if (lane == r) {
          sel_id = bi;
          sel_s = win_s;
        }
      }
      // gate weights of the k choices (lanes 0..k-1)
      const bool mine = lane < k;
      float wv = 0.f;
      if (a.mode == 0) {
        float m = mine ? sel_s : -INFINITY;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        float ev = mine ? expf(sel_s - m) : 0.f;
        float z = ev;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
        wv = ev / z;
      } else if (a.mode == 1 || a.mode == 2) {
        // softmax over all E: the maximum logit is the first choice
        const float m = __shfl(sel_s, 0);
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (lane + 64 * i < E) z += expf(s[i] - m);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
        float p = mine ? expf(sel_s - m) / z : 0.f;
        if (a.mode == 2) {
          float ps = p;
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) ps += __shfl_xor(ps, o);
          p = p / ps;
        }
        wv = p;
      } else {
        float sg = mine ? 1.0f / (1.0f + expf(-sel_s)) : 0.f;
        float ss = sg;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        wv = sg / ss;
      }
      if (mine) {
        a.ids_out[(size_t)t * k + lane] = sel_id;
        a.w_out[(size_t)t * k + lane] = wv;
        s_ids[tt * k + lane] = sel_id;
      }
    }
  } else {
    for (int i = threadIdx.x; i < ntok * k; i += 256) s_ids[i] = a.ids_in[(size_t)t0 * k + i];
  }
  if (!a.do_permute) return;
  __syncthreads();

  // atomic-free histogram and in-tile ranks
  const int E_loc = a.e_end - a.e_begin;
  const int npair = ntok * k;
  for (int el = threadIdx.x; el < E_loc; el += 256) {
    const int e = a.e_begin + el;
    int c = 0;
    for (int p = 0; p < npair; ++p)
      if (s_ids[p] == e) s_rank[p] = c++;
    s_cnt[el] = c;
  }
  __syncthreads();

  if (!a.single) {
    for (int el = threadIdx.x; el < E_loc; el += 256)
      a.tile_counts[(size_t)tile * E_loc + el] = s_cnt[el];
    for (int p = threadIdx.x; p < npair; p += 256) {
      const int e = s_ids[p];
      const bool local = e >= a.e_begin && e < a.e_end;
      a.rank_out[(size_t)t0 * k + p] = local ? s_rank[p] : -1;
    }
    return;
  }

  // single tile: finish the permutation here
  for (int el = threadIdx.x; el < E_loc; el += 256) s_off[el] = s_cnt[el];
  __syncthreads();
  const int total = block_exclusive_scan(s_off, E_loc, s_tmp);
  if (threadIdx.x == 0) s_off[E_loc] = total;
  __syncthreads();
  for (int el = threadIdx.x; el < E_loc; el += 256) a.counts[el] = s_cnt[el];
  for (int el = threadIdx.x; el <= E_loc; el += 256) a.offsets[el] = s_off[el];
  for (int p = threadIdx.x; p < npair; p += 256) {
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
  if (dt == 0) {
    dim3 grid(E, (T + 7) / 8);
    router_gemv_kernel<float, 8><<<grid, 256, 0, st>>>((const float*)x, (const float*)wr, T, H,
                                                       E, bias, logits);
  } else if (T <= 32 || E > 256 || H % RT_KC) {
    dim3 grid(E, (T + 7) / 8);
    router_gemv_kernel<bf16_t, 8><<<grid, 256, 0, st>>>((const bf16_t*)x, (const bf16_t*)wr, T,
                                                        H, E, bias, logits);
  } else {
    router_mfma_kernel<<<(T + 63) / 64, 256, 0, st>>>((const bf16_t*)x, (const bf16_t*)wr, T, H, E,
                                                      bias, logits);
  }
  return hipGetLastError();
}

hipError_t launch_gate_tiles(const GateTileArgs& a, int n_tiles_tok, hipStream_t st) {
  const int epl = (a.E + 63) / 64;
  const int grid = n_tiles_tok > 0 ? n_tiles_tok : 1;
  if (epl <= 1) gate_tile_kernel<1><<<grid, 256, 0, st>>>(a);
  else if (epl <= 2) gate_tile_kernel<2><<<grid, 256, 0, st>>>(a);
  else if (epl <= 4) gate_tile_kernel<4><<<grid, 256, 0, st>>>(a);
  else if (epl <= 8) gate_tile_kernel<8><<<grid, 256, 0, st>>>(a);
  else gate_tile_kernel<16><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
