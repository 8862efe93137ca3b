// Device helpers for the gfx950 kernels: bf16 conversion, 16-byte vector
// loads, MFMA fragment types, and block-wide scans used by the routing
// metadata kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include "moe_kernels.h"

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest, ties to even (finite inputs).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Expand 8 packed bf16 (one 16-byte load) into floats.
__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// Hardware exp and reciprocal (about 1 ulp each): for epilogues whose result
// is rounded to bfloat16 anyway.  Large negative z gives exp -> inf and
// rcp -> 0, so the result tends to -0 as it should.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Workgroup barrier for LDS traffic: each wave's LDS operations have
// completed when the others pass it.  __syncthreads() also drains every
// outstanding global store of the wave (vmcnt(0)), a memory round trip that
// the routing kernels -- which never read back what they store -- need not
// pay at each of their barriers.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Order one wave's LDS accesses across its lanes: what any lane wrote before
// this point is what every lane reads after it.  The hardware keeps a wave's
// LDS operations in order; the fences and the wave barrier stop the compiler
// from moving a lane's reads above other lanes' writes (it may, for a lane
// that skips those writes, in its single-thread view).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive prefix sum over the 64 lanes of a wave: a Hillis-Steele scan
// inside each 16-lane row by DPP row shifts (a lane with no source lane in
// its row adds 0), then the totals of the rows below, read with readlane.
// Sum over the 64 lanes of a wave, the same bits in every lane: DPP steps
// inside each 16-lane row (pairs, quads, half-row and row mirrors), then the
// rows' sums across row pairs and halves with v_permlane16_swap and
// v_permlane32_swap.  Each step adds two values that the two lanes concerned
// hold in opposite roles, and float addition is commutative, so no lane
// disagrees; the order of the additions is fixed.
__device__ __forceinline__ float wave_sum_f(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, x), decltype(ctrl)::value, 0xF,
                                         0xF, false));
  };
  v += dpp(v, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
  v += dpp(v, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
  v += dpp(v, std::integral_constant<int, 0x141>{});   // row_half_mirror
  v += dpp(v, std::integral_constant<int, 0x140>{});   // row_mirror
  const uint32_t u = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const uint32_t w = __float_as_uint(v);
  const auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31),
            t2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of n ints held in LDS (n <= 4 * blockDim.x,
// blockDim.x a multiple of 64 and at most 1024).  `data` is replaced by its
// exclusive prefix sums; returns the total.  Per-thread chunk sums are
// scanned inside each wave with shuffles, then across waves through `tmp`
// (at least blockDim.x / 64 ints): one barrier in the middle, one at the end.
// All threads of the block must call it, after `data` is visible to all.
// ---------------------------------------------------------------------------
__device__ inline int block_exclusive_scan(int* data, int n, int* tmp) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int lane = tid & 63, wid = tid >> 6, nw = nt >> 6;
  const int per = (n + nt - 1) / nt;
  const int b = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (b + i < n) local += data[b + i];
  const int v = wave_inclusive_scan(local);  // inclusive scan inside the wave
  if (lane == 63) tmp[wid] = v;
  lds_barrier();
  int wbase = 0, total = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = tmp[w];
    if (w < wid) wbase += t;
    total += t;
  }
  int run = wbase + v - local;
  for (int i = 0; i < per; ++i)
    if (b + i < n) {
      const int x = data[b + i];
      data[b + i] = run;
      run += x;
    }
  lds_barrier();
  return total;
}

// ---------------------------------------------------------------------------
// GEMM tile map: for every local expert, ceil(count / BM) row tiles of at most
// BM rows.  Every entry of expert e is {e, first row of e, end row of e,
// index of e's first entry}; tile q of e covers rows [first + q*BM,
// min(first + (q+1)*BM, end)).  n_tiles[0] = number of entries.  cnt[] holds counts and off[] exclusive offsets (both in LDS).
// An expert whose rows fall outside [0, max_rows) gets no tiles, and at most
// max_tiles entries are written, so a GEMM driven by the map never indexes
// outside its buffers even if the offsets were inconsistent.
// scratch: E_loc ints of LDS, tmp: blockDim.x + 1 ints of LDS.
// ---------------------------------------------------------------------------
__device__ inline int tiles_of(int c, int o, int BM, int max_rows) {
  if (c <= 0 || o < 0 || o + c > max_rows) return 0;
  return (c + BM - 1) / BM;
}

__device__ inline void block_build_tile_map(const int* cnt, const int* off, int E_loc, int BM,
                                            int max_rows, int max_tiles, int* scratch, int* tmp,
                                            int4* tile_map, int* n_tiles) {
  for (int e = threadIdx.x; e < E_loc; e += blockDim.x)
    scratch[e] = tiles_of(cnt[e], off[e], BM, max_rows);
  lds_barrier();
  const int total = block_exclusive_scan(scratch, E_loc, tmp);
  for (int e = threadIdx.x; e < E_loc; e += blockDim.x) {
    const int nt = tiles_of(cnt[e], off[e], BM, max_rows);
    const int4 entry = make_int4(e, off[e], off[e] + cnt[e], scratch[e]);
    for (int q = 0; q < nt; ++q) {
      const int slot = scratch[e] + q;
      if (slot >= max_tiles) break;
      tile_map[slot] = entry;
    }
  }
  if (threadIdx.x == 0) n_tiles[0] = min(total, max_tiles);
}

// ---------------------------------------------------------------------------
// Routing metadata from per-expert pair totals, by one wave (E_loc <= 256;
// lane l owns local experts 4l .. 4l + 3): kept = min(total, capacity) per
// expert into counts; offsets = exclusive prefix sums of kept (el * capacity
// when padded), offsets[E_loc] their end; the dropped total; and the GEMM
// tile map (tile_map may be null).  DPP scans give the same values as
// block_exclusive_scan and block_build_tile_map.  s_off (E_loc + 1 ints of
// LDS) receives the offsets for the caller.  The host has checked that
// E_loc * capacity fits an int in the padded layout.
// ---------------------------------------------------------------------------
__device__ inline void wave_routing_metadata(const int* total, int E_loc, int capacity, bool padded,
                                             int BM, int max_rows, int max_tiles, int* s_off,
                                             int32_t* counts, int32_t* offsets, int32_t* dropped,
                                             int4* tile_map, int32_t* n_tiles) {
  const int lane = threadIdx.x & 63;
  int c[4], rows = 0, drop = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int el = 4 * lane + j;
    const int n = el < E_loc ? total[el] : 0;
    c[j] = min(n, capacity);
    drop += n - c[j];
    rows += c[j];
  }
  const int rs = wave_inclusive_scan(rows);
  const int end = padded ? E_loc * capacity : __builtin_amdgcn_readlane(rs, 63);
  int off = rs - rows, o[4], nt[4], tiles = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int el = 4 * lane + j;
    o[j] = padded ? el * capacity : off;
    nt[j] = 0;
    if (el < E_loc) {
      s_off[el] = o[j];
      counts[el] = c[j];
      offsets[el] = o[j];
      if (tile_map) nt[j] = tiles_of(c[j], o[j], BM, max_rows);
    }
    tiles += nt[j];
    off += c[j];
  }
  if (dropped) {
    const int ds = wave_inclusive_scan(drop);
    if (lane == 63) dropped[0] = ds;
  }
  if (lane == 0) {
    s_off[E_loc] = end;
    offsets[E_loc] = end;
  }
  if (tile_map) {
    const int ts = wave_inclusive_scan(tiles);
    int tb = ts - tiles;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int4 entry = make_int4(4 * lane + j, o[j], o[j] + c[j], tb);
      for (int q = 0; q < nt[j] && tb + q < max_tiles; ++q) tile_map[tb + q] = entry;
      tb += nt[j];
    }
    if (lane == 63) n_tiles[0] = min(ts, max_tiles);
  }
}

}  // namespace moe
