// Token copies packed by destination rank for the expert-parallel dispatch,
// and the source rank's sum after the return.
//
// "MoE 推理优化全景指南", section 一个 token 为什么要跨 GPU: before the dispatch
// all-to-all the tokens are counted, prefix-summed and permuted by destination
// so that each destination's copies are contiguous.  "Lecture 8 · 混合专家模型
// 的推理" (CS349D notes) section 3.1: a token that chose two experts held by
// one device is sent there once, its gate weights travelling with it, and the
// results come back to be added.
//
// Rank r holds experts [r*E/P, (r+1)*E/P).  A copy is a (rank, token) pair;
// copies are ordered by rank, then by token.  Each token's destinations are a
// 64-bit mask (P <= 64), so per rank a wave ballot over a 64-token tile gives
// the tile's count (popcount) and every token's place in it (popcount of the
// lanes below): no sort and no atomics.
#include <algorithm>

#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int PK_TILE = 64;   // tokens per wave tile

__device__ __forceinline__ unsigned long long lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// A token's routing held in registers (KP >= k slots, loaded once): every
// copy of the token is written from these, with no load between its stores.
template <int KP>
struct TokenRoute {
  int id[KP];
  float w[KP];
  unsigned long long mask;   // destination ranks (ids outside [0, E) are not sent)

  // k a multiple of 4 (every shape here): 16-byte loads and stores of the
  // routing rows (the buffers are 16-byte aligned, rows k * 4 bytes long)
  __device__ __forceinline__ void load(const PackArgs& a, int t, bool live) {
    mask = 0ull;
    if ((a.k & 3) == 0) {
#pragma unroll
      for (int j = 0; j < KP; j += 4) {
        int4 iv = make_int4(-1, -1, -1, -1);
        float4 wv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (live && j < a.k) {
          iv = *reinterpret_cast<const int4*>(a.ids + (size_t)t * a.k + j);
          if (a.send_w) wv = *reinterpret_cast<const float4*>(a.w + (size_t)t * a.k + j);
        }
        id[j] = iv.x; id[j + 1] = iv.y; id[j + 2] = iv.z; id[j + 3] = iv.w;
        w[j] = wv.x; w[j + 1] = wv.y; w[j + 2] = wv.z; w[j + 3] = wv.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        id[j] = (live && j < a.k) ? a.ids[(size_t)t * a.k + j] : -1;
        w[j] = (live && j < a.k && a.send_w) ? a.w[(size_t)t * a.k + j] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < KP; ++j)
      if (id[j] >= 0 && id[j] < a.E) mask |= 1ull << (id[j] / a.per);
  }

  // token t's copy to rank r at `row`: the token, its routing (all k slots,
  // so the receiving rank can pick its own experts), and the row of every
  // slot the copy serves
  __device__ __forceinline__ void write_copy(const PackArgs& a, int t, int r, int row) const {
    a.send_token[row] = t;
    if ((a.k & 3) == 0) {
#pragma unroll
      for (int j = 0; j < KP; j += 4) {
        if (j < a.k) {
          if (a.send_ids)
            *reinterpret_cast<int4*>(a.send_ids + (size_t)row * a.k + j) =
                make_int4(id[j], id[j + 1], id[j + 2], id[j + 3]);
          if (a.send_w)
            *reinterpret_cast<float4*>(a.send_w + (size_t)row * a.k + j) =
                make_float4(w[j], w[j + 1], w[j + 2], w[j + 3]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        if (j < a.k) {
          if (a.send_ids) a.send_ids[(size_t)row * a.k + j] = id[j];
          if (a.send_w) a.send_w[(size_t)row * a.k + j] = w[j];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KP; ++j)
      if (j < a.k && id[j] >= 0 && id[j] < a.E && id[j] / a.per == r)
        a.send_row[(size_t)t * a.k + j] = row;
  }

  __device__ __forceinline__ void clear_rows(const PackArgs& a, int t) const {
#pragma unroll
    for (int j = 0; j < KP; ++j)
      if (j < a.k) a.send_row[(size_t)t * a.k + j] = -1;
  }
};

// ---------------------------------------------------------------------------
// One wave, T <= 64: counts, offsets and the copy table in one pass.
// ---------------------------------------------------------------------------
template <int KP>
__global__ __launch_bounds__(64) void pack_single_kernel(PackArgs a) {
  const int t = threadIdx.x;
  const bool live = t < a.T;
  TokenRoute<KP> tr;
  tr.load(a, t, live);
  const unsigned long long m = tr.mask;
  if (live) tr.clear_rows(a, t);
  // lane r ends with rank r's count; exclusive scan over the lanes
  int cnt = 0;
  for (int r = 0; r < a.P; ++r) {
    const unsigned long long b = __ballot((m >> r) & 1ull);
    if (t == r) cnt = __popcll(b);
  }
  const int inc = wave_inclusive_scan(cnt);
  const int off = inc - cnt;
  if (t < a.P) {
    a.send_counts[t] = cnt;
    a.send_offsets[t] = off;
  }
  if (t == a.P - 1) a.send_offsets[a.P] = inc;
  for (int r = 0; r < a.P; ++r) {
    const unsigned long long b = __ballot((m >> r) & 1ull);
    const int base = __builtin_amdgcn_readlane(off, r);
    if ((m >> r) & 1ull) tr.write_copy(a, t, r, base + __popcll(b & lanes_below()));
  }
}

// ---------------------------------------------------------------------------
// Multi-tile path.  1: per tile and rank, the number of copies.
// ---------------------------------------------------------------------------
template <int KP>
__global__ __launch_bounds__(256) void pack_count_kernel(PackArgs a) {
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n_tiles = (a.T + PK_TILE - 1) / PK_TILE;
  if (tile >= n_tiles) return;
  const int t = tile * PK_TILE + lane;
  const bool live = t < a.T;
  TokenRoute<KP> tr;
  tr.load(a, t, live);
  const unsigned long long m = tr.mask;
  if (live) {
    a.masks[t] = m;
    tr.clear_rows(a, t);
  }
  int cnt = 0;
  for (int r = 0; r < a.P; ++r) {
    const unsigned long long b = __ballot((m >> r) & 1ull);
    if (lane == r) cnt = __popcll(b);
  }
  if (lane < a.P) a.tile_counts[(size_t)tile * a.P + lane] = cnt;
}

// 2: per rank, exclusive scan of its tile counts (one wave per rank, 64
// tiles per step with a carry), then the rank offsets.
__global__ __launch_bounds__(1024) void pack_scan_kernel(PackArgs a) {
  __shared__ int s_total[64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int n_tiles = (a.T + PK_TILE - 1) / PK_TILE;
  for (int r = wid; r < a.P; r += nw) {
    int carry = 0;
    for (int t0 = 0; t0 < n_tiles; t0 += 64) {
      const int tile = t0 + lane;
      const int c = tile < n_tiles ? a.tile_counts[(size_t)tile * a.P + r] : 0;
      const int inc = wave_inclusive_scan(c);
      if (tile < n_tiles) a.tile_base[(size_t)tile * a.P + r] = carry + inc - c;
      carry += __builtin_amdgcn_readlane(inc, 63);
    }
    if (lane == 0) s_total[r] = carry;
  }
  __syncthreads();
  if (wid == 0) {
    const int c = lane < a.P ? s_total[lane] : 0;
    const int inc = wave_inclusive_scan(c);
    if (lane < a.P) {
      a.send_counts[lane] = c;
      a.send_offsets[lane] = inc - c;
    }
    if (lane == a.P - 1) a.send_offsets[a.P] = inc;
  }
}

// 3: the copy table.
template <int KP>
__global__ __launch_bounds__(256) void pack_scatter_kernel(PackArgs a) {
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n_tiles = (a.T + PK_TILE - 1) / PK_TILE;
  if (tile >= n_tiles) return;
  const int t = tile * PK_TILE + lane;
  const bool live = t < a.T;
  TokenRoute<KP> tr;
  tr.load(a, t, live);
  const unsigned long long m = tr.mask;
  const int rb = lane < a.P ? a.send_offsets[lane] + a.tile_base[(size_t)tile * a.P + lane] : 0;
  for (int r = 0; r < a.P; ++r) {
    const unsigned long long b = __ballot((m >> r) & 1ull);
    const int base = __builtin_amdgcn_readlane(rb, r);
    if ((m >> r) & 1ull) tr.write_copy(a, t, r, base + __popcll(b & lanes_below()));
  }
}

// x_send[row] = x[t] for each copy row of each token t (its distinct
// send_row[t][j]).  A wave takes one token, or one of `splits` column slices
// of a token when the batch is small, loads that part of the token's row once
// and stores it to every copy, every 16-byte load of a lane issued before its
// stores.  (One wave per copy row had read each token's row once per copy:
// 4.7 times at DeepSeek-V3 routing over 8 ranks.)  Rows are read and
// written once, with the non-temporal hint (pack 1%, the return sum 3%
// faster at DeepSeek-V3 T = 4096).
template <int KP>
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint4* __restrict__ x,
                                                        const int32_t* __restrict__ send_row,
                                                        int T, int k, int row_vecs, int splits,
                                                        uint4* __restrict__ out) {
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t = gw / splits;
  if (t >= T) return;
  const int chunk = (row_vecs + splits - 1) / splits;
  const int cb = (gw - t * splits) * chunk;
  const int ce = min(cb + chunk, row_vecs);
  // the token's distinct copy rows (slots sent to one rank share a row)
  int rows[KP];
  int n = 0;
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    const int r = j < k ? send_row[(size_t)t * k + j] : -1;
    bool fresh = r >= 0;
#pragma unroll
    for (int i = 0; i < KP; ++i)
      if (i < n && rows[i] == r) fresh = false;
    if (fresh) rows[n++] = r;
  }
  if (n == 0 || cb >= ce) return;
  // 16-byte vectors as a clang vector type: an array of them stays in
  // registers (an array of the HIP uint4 struct would go to scratch)
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const v4u* src = reinterpret_cast<const v4u*>(x) + (size_t)t * row_vecs;
  constexpr int B = 8;
  for (int c0 = cb + lane; c0 < ce; c0 += 64 * B) {
    v4u v[B];
#pragma unroll
    for (int i = 0; i < B; ++i) v[i] = __builtin_nontemporal_load(&src[min(c0 + 64 * i, ce - 1)]);
#pragma unroll
    for (int q = 0; q < KP; ++q) {
      if (q >= n) break;
      v4u* dst = reinterpret_cast<v4u*>(out) + (size_t)rows[q] * row_vecs;
#pragma unroll
      for (int i = 0; i < B; ++i)
        if (c0 + 64 * i < ce) __builtin_nontemporal_store(v[i], &dst[c0 + 64 * i]);
    }
  }
}

// 16 bytes read once (the non-temporal hint): the returned rows are summed
// once and not read again.
__device__ __forceinline__ uint4 ld_once16(const uint32_t* p) {
  typedef uint32_t v4x __attribute__((ext_vector_type(4)));
  const v4x v = __builtin_nontemporal_load(reinterpret_cast<const v4x*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// y[t] = sum of y_ret over t's distinct copy rows, ascending (rank order),
// in float32, rounded once.  One 256-thread block per token; thread i takes
// the 16-byte columns i, i + 256, ...
template <int KP, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void unpack_sum_kernel(const void* __restrict__ y_ret,
                                                         const int32_t* __restrict__ send_row,
                                                         int T, int k, int H,
                                                         void* __restrict__ y) {
  const int t = blockIdx.x;
  // t's distinct copy rows, ascending, computed by every thread in registers
  int rj[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) rj[j] = j < k ? send_row[(size_t)t * k + j] : -1;
  int rows[KP];
  int n_rows = 0, last = -1;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    int row = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < KP; ++j)
      if (rj[j] > last && rj[j] < row) row = rj[j];
    rows[i] = row;
    if (row != 0x7fffffff) {
      last = row;
      n_rows = i + 1;
    }
  }
  constexpr int EPV = 8;                            // columns per step (8 bf16 or 2 x 4 f32)
  const int nv = H / EPV;
  // rows past n_rows repeat the last row's address (a valid one) and are not
  // added, so that a group's loads need no branch (a load under a branch per
  // row had waited for each row in turn)
  int rr[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) rr[i] = i < n_rows ? rows[i] : last;   // last: the largest row
#pragma unroll 2
  for (int c = threadIdx.x; c < nv; c += 256) {
    float acc[EPV];
#pragma unroll
    for (int q = 0; q < EPV; ++q) acc[q] = 0.f;
    // rows in groups of 8: every load of a group is issued before its adds
    constexpr int G = KP < 8 ? KP : 8;
#pragma unroll
    for (int g = 0; g < KP; g += G) {
      if (g >= n_rows) break;
      if constexpr (IN_BF16) {
        uint4 raw[G];
#pragma unroll
        for (int i = 0; i < G; ++i)
          raw[i] = ld_once16(reinterpret_cast<const uint32_t*>(y_ret) +
                             ((size_t)rr[g + i] * nv + c) * 4);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          if (g + i < n_rows) {
            float v[EPV];
            unpack_bf16x8(raw[i], v);
#pragma unroll
            for (int q = 0; q < EPV; ++q) acc[q] += v[q];
          }
        }
      } else {
        float4 u0[G], u1[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const float4* p = reinterpret_cast<const float4*>(y_ret) + ((size_t)rr[g + i] * nv + c) * 2;
          u0[i] = p[0];
          u1[i] = p[1];
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
          if (g + i < n_rows) {
            acc[0] += u0[i].x; acc[1] += u0[i].y; acc[2] += u0[i].z; acc[3] += u0[i].w;
            acc[4] += u1[i].x; acc[5] += u1[i].y; acc[6] += u1[i].z; acc[7] += u1[i].w;
          }
        }
      }
    }
    if constexpr (OUT_BF16) {
      reinterpret_cast<uint4*>(y)[(size_t)t * nv + c] =
          make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    } else {
      float4* p = reinterpret_cast<float4*>(y) + ((size_t)t * nv + c) * 2;
      p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

template <int KP>
hipError_t launch_unpack_kp(const void* y_ret, int y_ret_dt, const int32_t* send_row, int T, int k,
                            int H, void* y, int dt, hipStream_t st) {
  const int blocks = T;
  if (y_ret_dt == 1 && dt == 1)
    unpack_sum_kernel<KP, true, true><<<blocks, 256, 0, st>>>(y_ret, send_row, T, k, H, y);
  else if (y_ret_dt == 1)
    unpack_sum_kernel<KP, true, false><<<blocks, 256, 0, st>>>(y_ret, send_row, T, k, H, y);
  else if (dt == 1)
    unpack_sum_kernel<KP, false, true><<<blocks, 256, 0, st>>>(y_ret, send_row, T, k, H, y);
  else
    unpack_sum_kernel<KP, false, false><<<blocks, 256, 0, st>>>(y_ret, send_row, T, k, H, y);
  return hipGetLastError();
}

template <int KP>
void launch_pack_kp(const PackArgs& a, hipStream_t st) {
  if (a.T <= PK_TILE) {   // also T = 0: zero counts and offsets
    pack_single_kernel<KP><<<1, 64, 0, st>>>(a);
  } else {
    const int n_tiles = (a.T + PK_TILE - 1) / PK_TILE;
    const int blocks = (n_tiles + 3) / 4;
    pack_count_kernel<KP><<<blocks, 256, 0, st>>>(a);
    pack_scan_kernel<<<1, 1024, 0, st>>>(a);
    pack_scatter_kernel<KP><<<blocks, 256, 0, st>>>(a);
  }
}

}  // namespace

hipError_t launch_pack_by_rank(const PackArgs& a, const void* x, int H, int elt_bytes, void* x_send,
                               int max_rows, hipStream_t st) {
  if (a.k <= 8) launch_pack_kp<8>(a, st);
  else launch_pack_kp<32>(a, st);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !x || max_rows <= 0 || a.T <= 0) return err;
  // small batches: split each token's row over several waves (64 vectors of
  // 16 bytes at least), so that about 2048 waves share the copies
  const int row_vecs = H * elt_bytes / 16;
  int splits = 2048 / a.T;
  splits = std::max(1, std::min(splits, row_vecs / 64));
  const long long waves = (long long)a.T * splits;
  const int blocks = (int)((waves + 3) / 4);
  if (a.k <= 8)
    copy_rows_kernel<8><<<blocks, 256, 0, st>>>(static_cast<const uint4*>(x), a.send_row, a.T,
                                                 a.k, row_vecs, splits,
                                                 static_cast<uint4*>(x_send));
  else
    copy_rows_kernel<32><<<blocks, 256, 0, st>>>(static_cast<const uint4*>(x), a.send_row, a.T,
                                                  a.k, row_vecs, splits,
                                                  static_cast<uint4*>(x_send));
  return hipGetLastError();
}

hipError_t launch_unpack_sum(const void* y_ret, int y_ret_dt, const int32_t* send_row, int T, int k,
                             int H, void* y, int dt, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (k <= 8) return launch_unpack_kp<8>(y_ret, y_ret_dt, send_row, T, k, H, y, dt, st);
  return launch_unpack_kp<32>(y_ret, y_ret_dt, send_row, T, k, H, y, dt, st);
}

}  // namespace moe
