// Prefix sums and the stable scatter of token copies for gfx950.
//
// "MoE 推理优化全景指南", section Dispatch 并不是一次普通 all-to-all:
// histogram -> prefix sum -> permute, each expert's copies contiguous and in
// token order.  The per-tile histograms and in-tile ranks come from the gating
// kernel; here one block turns them into offsets and per-tile bases, and a
// wide kernel writes dst_row / src_token.  No atomics anywhere, so the
// permutation is the same on every run.  An optional capacity keeps each
// expert's first pairs in token order and drops the rest ("MoE 推理优化全景
// 指南", section Capacity、padding 与 token dropping); in the padded layout of
// that section every expert owns a fixed block of `capacity` rows, its kept
// pairs first, then padding rows whose source is -1.
#include <climits>

#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

// One block: for every local expert, an exclusive scan of its counts over the
// token tiles (tile_base), its total (counts), then the exclusive scan over
// experts (offsets; el * capacity in the padded layout) and the GEMM tile map.
//
// The tiles are cut into NC chunks (NC * E_loc <= blockDim.x), thread
// (chunk c, expert el) = c * E_loc + el, so that neighbouring threads read
// neighbouring counts.  A thread loads its chunk's counts in batches of
// SCAN_BATCH, all loads of a batch before their sums, so a chunk of up to
// SCAN_BATCH tiles costs one memory round trip (walking 128 tiles four at a
// time had cost 32 round trips, 15 us at T = 8192).  The chunk totals meet
// in LDS; each thread adds those of the chunks before its own and walks its
// chunk again (a second round trip, to the L2) to write tile_base.
constexpr int SCAN_BATCH = 16;
constexpr int SCAN_MAX_CHUNKS = 64;

__global__ __launch_bounds__(1024) void permute_scan_kernel(const int32_t* __restrict__ tile_counts,
                                                            int n_tt, int E_loc,
                                                            int32_t* __restrict__ tile_base,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets, int BM,
                                                            int max_rows, int max_tiles,
                                                            int4* __restrict__ tile_map,
                                                            int32_t* __restrict__ n_tiles,
                                                            int capacity, int padded,
                                                            int32_t* __restrict__ dropped) {
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1025];
  __shared__ int s_scr[1024];
  __shared__ int s_tmp[1025];
  __shared__ int s_chunk[1024];           // [chunk][expert] chunk totals
  const int nthr = blockDim.x;
  int NC = nthr / E_loc;                  // chunks per expert
  if (NC > SCAN_MAX_CHUNKS) NC = SCAN_MAX_CHUNKS;
  if (NC > n_tt) NC = n_tt;
  if (NC < 1) NC = 1;
  const int L = (n_tt + NC - 1) / NC;     // tiles per chunk
  // pass 1: chunk totals
  for (int i = threadIdx.x; i < NC * E_loc; i += nthr) {
    const int c = i / E_loc, el = i - c * E_loc;
    const int tb = c * L, te = min(tb + L, n_tt);
    int sum = 0;
    for (int t0 = tb; t0 < te; t0 += SCAN_BATCH) {
      int v[SCAN_BATCH];
#pragma unroll
      for (int j = 0; j < SCAN_BATCH; ++j)
        v[j] = t0 + j < te ? tile_counts[(size_t)(t0 + j) * E_loc + el] : 0;
#pragma unroll
      for (int j = 0; j < SCAN_BATCH; ++j) sum += v[j];
    }
    s_chunk[i] = sum;
  }
  lds_barrier();
  // pass 2: bases
  for (int i = threadIdx.x; i < NC * E_loc; i += nthr) {
    const int c = i / E_loc, el = i - c * E_loc;
    int run = 0;
    for (int c2 = 0; c2 < c; ++c2) run += s_chunk[c2 * E_loc + el];
    const int tb = c * L, te = min(tb + L, n_tt);
    for (int t0 = tb; t0 < te; t0 += SCAN_BATCH) {
      int v[SCAN_BATCH];
#pragma unroll
      for (int j = 0; j < SCAN_BATCH; ++j)
        v[j] = t0 + j < te ? tile_counts[(size_t)(t0 + j) * E_loc + el] : 0;
#pragma unroll
      for (int j = 0; j < SCAN_BATCH; ++j) {
        if (t0 + j < te) tile_base[(size_t)(t0 + j) * E_loc + el] = run;
        run += v[j];
      }
    }
    if (c == NC - 1) s_cnt[el] = run;   // the expert's total
  }
  lds_barrier();
  if (E_loc <= 256) {
    // wave 0 alone (DPP scans) finishes counts, offsets, the dropped total
    // and the tile map
    if (threadIdx.x < 64)
      wave_routing_metadata(s_cnt, E_loc, capacity, padded != 0, BM, max_rows, max_tiles, s_off,
                            counts, offsets, dropped, tile_map, n_tiles);
    return;
  }
  // an expert over capacity keeps its first `capacity` pairs
  for (int el = threadIdx.x; el < E_loc; el += nthr) {
    const int run = s_cnt[el], kept = min(run, capacity);
    s_cnt[el] = kept;
    s_off[el] = kept;
    s_scr[el] = run - kept;
  }
  lds_barrier();
  const int n_dropped = block_exclusive_scan(s_scr, E_loc, s_tmp);
  if (dropped && threadIdx.x == 0) dropped[0] = n_dropped;
  const int total = block_exclusive_scan(s_off, E_loc, s_tmp);
  if (padded) {
    // the host has checked that E_loc * capacity fits an int
    for (int el = threadIdx.x; el <= E_loc; el += blockDim.x) s_off[el] = el * capacity;
  } else if (threadIdx.x == 0) {
    s_off[E_loc] = total;
  }
  lds_barrier();
  for (int el = threadIdx.x; el < E_loc; el += blockDim.x) counts[el] = s_cnt[el];
  for (int el = threadIdx.x; el <= E_loc; el += blockDim.x) offsets[el] = s_off[el];
  if (tile_map)
    block_build_tile_map(s_cnt, s_off, E_loc, BM, max_rows, max_tiles, s_scr, s_tmp, tile_map,
                         n_tiles);
}

// One thread per (token, slot): row = offsets[e] + tile_base[tile][e] + rank.
__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ tile_base, const int32_t* __restrict__ offsets, int T, int k,
    int e_begin, int e_end, int capacity, int32_t* __restrict__ dst_row,
    int32_t* __restrict__ src_token) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= T * k) return;
  const int t = p / k;
  const int e = ids[p];
  int row = -1;
  if (e >= e_begin && e < e_end) {
    const int el = e - e_begin;
    const int E_loc = e_end - e_begin;
    // place of the pair in its expert's token order; beyond capacity it is
    // dropped
    const int pos = tile_base[(size_t)(t / TOK_TILE) * E_loc + el] + rank[p];
    if (pos < capacity) {
      row = offsets[el] + pos;
      src_token[row] = t;
    }
  }
  dst_row[p] = row;
}

// Padded layout: src_token = -1 on the rows of every expert block past its
// kept pairs (row r is row r % capacity of expert r / capacity).  The kept
// rows are the scatter kernel's, so the two write disjoint rows.
__global__ __launch_bounds__(256) void pad_rows_kernel(const int32_t* __restrict__ counts,
                                                       int n_rows, int capacity,
                                                       int32_t* __restrict__ src_token) {
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < n_rows; r += gridDim.x * blockDim.x) {
    const int el = r / capacity;
    if (r - el * capacity >= counts[el]) src_token[r] = -1;
  }
}

// x_perm[row] = x[src_token[row]] for rows < offsets[E_loc], a zero row where
// the source is -1 (padding); 16-byte copies.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ x,
                                                          const int32_t* __restrict__ src_token,
                                                          const int32_t* __restrict__ offsets,
                                                          int E_loc, int row_vecs,
                                                          uint4* __restrict__ x_perm) {
  const int row = blockIdx.x;
  if (row >= offsets[E_loc]) return;
  const int t = src_token[row];
  if (t < 0) {
    for (int c = threadIdx.x; c < row_vecs; c += blockDim.x)
      x_perm[(size_t)row * row_vecs + c] = make_uint4(0, 0, 0, 0);
    return;
  }
  for (int c = threadIdx.x; c < row_vecs; c += blockDim.x)
    x_perm[(size_t)row * row_vecs + c] = x[(size_t)t * row_vecs + c];
}

// Checks of the routing metadata, for callers that ask for them ("MoE 推理优化
// 全景指南", section Dispatch 并不是一次普通 all-to-all: wrong counts or
// offsets misroute rows without any error).  One block; err[0] receives
//   bit 0  an id outside [0, E)
//   bit 1  offsets that do not start at 0 or disagree with counts (padded
//          layout: offsets[i] != i * capacity)
//   bit 2  counts that do not add up to the local pairs less the dropped
//          ones (without a dropped word and with a capacity: more than them)
//   bit 3  a count below 0 or above the capacity
// or 0.  Integer sums only; the result does not depend on thread timing.
__global__ __launch_bounds__(256) void validate_meta_kernel(
    const int32_t* __restrict__ ids, int npair, int E, int e_begin, int e_end,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int capacity,
    int padded, const int32_t* __restrict__ dropped, int32_t* __restrict__ err) {
  __shared__ int s_bits, s_local, s_sum;
  if (threadIdx.x == 0) {
    s_bits = 0;
    s_local = 0;
    s_sum = 0;
  }
  __syncthreads();
  int bits = 0, local = 0, sum = 0;
  for (int p = threadIdx.x; p < npair; p += blockDim.x) {
    const int e = ids[p];
    if (e < 0 || e >= E) bits |= 1;
    if (e >= e_begin && e < e_end) ++local;
  }
  const int E_loc = e_end - e_begin;
  for (int el = threadIdx.x; el < E_loc; el += blockDim.x) {
    const int c = counts[el], o0 = offsets[el], o1 = offsets[el + 1];
    sum += c;
    if (c < 0 || c > capacity) bits |= 8;
    if (padded) {
      // the host has checked that E_loc * capacity fits an int
      if (o0 != el * capacity || o1 != (el + 1) * capacity) bits |= 2;
    } else if (o1 - o0 != c) {
      bits |= 2;
    }
  }
  if (threadIdx.x == 0 && offsets[0] != 0) bits |= 2;
  atomicOr(&s_bits, bits);
  atomicAdd(&s_local, local);
  atomicAdd(&s_sum, sum);
  __syncthreads();
  if (threadIdx.x == 0) {
    int b = s_bits;
    const int d = dropped ? dropped[0] : -1;
    const bool bad = d >= 0 ? s_sum + d != s_local
                            : (capacity == INT_MAX ? s_sum != s_local : s_sum > s_local);
    if (bad) b |= 4;
    err[0] = b;
  }
}

// Tile map for a standalone grouped-FFN call, from device offsets.
__global__ __launch_bounds__(256) void tile_map_kernel(const int32_t* __restrict__ offsets,
                                                       int E_loc, int BM, int max_rows,
                                                       int max_tiles,
                                                       int4* __restrict__ tile_map,
                                                       int32_t* __restrict__ n_tiles) {
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1025];
  __shared__ int s_scr[1024];
  __shared__ int s_tmp[257];
  for (int e = threadIdx.x; e <= E_loc; e += blockDim.x) s_off[e] = offsets[e];
  lds_barrier();
  for (int e = threadIdx.x; e < E_loc; e += blockDim.x) s_cnt[e] = s_off[e + 1] - s_off[e];
  lds_barrier();
  block_build_tile_map(s_cnt, s_off, E_loc, BM, max_rows, max_tiles, s_scr, s_tmp, tile_map,
                       n_tiles);
}

hipError_t launch_permute_scan(const int32_t* tile_counts, int n_tt, int E_loc,
                               int32_t* tile_base, int32_t* counts, int32_t* offsets, int BM,
                               int max_rows, int max_tiles, int4* tile_map, int32_t* n_tiles,
                               int capacity, int padded, int32_t* dropped, hipStream_t st) {
  const int threads = 1024;
  permute_scan_kernel<<<1, threads, 0, st>>>(tile_counts, n_tt, E_loc, tile_base, counts, offsets,
                                             BM, max_rows, max_tiles, tile_map, n_tiles, capacity,
                                             padded, dropped);
  return hipGetLastError();
}

hipError_t launch_pad_rows(const int32_t* counts, int E_loc, int capacity, int32_t* src_token,
                           hipStream_t st) {
  const long long n = (long long)E_loc * capacity;
  if (n <= 0) return hipSuccess;
  const long long blocks = (n + 255) / 256;
  pad_rows_kernel<<<(int)(blocks < 2048 ? blocks : 2048), 256, 0, st>>>(counts, (int)n, capacity,
                                                                         src_token);
  return hipGetLastError();
}

hipError_t launch_permute_scatter(const int32_t* ids, const int32_t* rank, const int32_t* tile_base,
                                  const int32_t* offsets, int T, int k, int e_begin, int e_end,
                                  int capacity, int32_t* dst_row, int32_t* src_token,
                                  hipStream_t st) {
  const int n = T * k;
  if (n <= 0) return hipSuccess;
  permute_scatter_kernel<<<(n + 255) / 256, 256, 0, st>>>(ids, rank, tile_base, offsets, T, k,
                                                          e_begin, e_end, capacity, dst_row,
                                                          src_token);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* src_token, const int32_t* offsets,
                              int E_loc, int max_rows, int H, int elt_bytes, void* x_perm,
                              hipStream_t st) {
  if (max_rows <= 0) return hipSuccess;
  const int row_vecs = H * elt_bytes / 16;
  gather_rows_kernel<<<max_rows, 256, 0, st>>>((const uint4*)x, src_token, offsets, E_loc,
                                               row_vecs, (uint4*)x_perm);
  return hipGetLastError();
}

hipError_t launch_validate_meta(const int32_t* ids, int npair, int E, int e_begin, int e_end,
                                const int32_t* counts, const int32_t* offsets, int capacity,
                                int padded, const int32_t* dropped, int32_t* err, hipStream_t st) {
  validate_meta_kernel<<<1, 256, 0, st>>>(ids, npair, E, e_begin, e_end, counts, offsets, capacity,
                                          padded, dropped, err);
  return hipGetLastError();
}

hipError_t launch_tile_map_from_offsets(const int32_t* offsets, int E_loc, int BM, int max_rows,
                                        int max_tiles, int4* tile_map, int32_t* n_tiles,
                                        hipStream_t st) {
  tile_map_kernel<<<1, 256, 0, st>>>(offsets, E_loc, BM, max_rows, max_tiles, tile_map, n_tiles);
  return hipGetLastError();
}

}  // namespace moe
