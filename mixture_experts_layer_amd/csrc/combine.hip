// Inverse permutation with the gate-weighted sum, gfx950.
//
// "MoE 推理优化全景指南", section Dispatch 并不是一次普通 all-to-all: combine
// restores token order and applies the routing weights.  Moebius reading
// notes, eq. (1): y = sum over the chosen experts of g_i * FFN_i(x).
// "Lecture 8 · 混合专家模型的推理" (CS349D notes) section 1.2: a shared expert
// every token passes through, added here with weight 1.
//
// Each thread owns 8 consecutive columns of one token: it reads the k permuted
// rows with 16-byte loads, accumulates w * y_perm in float32 in slot order
// and rounds once.  Memory-bound gather; no atomics.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

// A permuted row segment is read once, by the thread that sums its token:
// non-temporal loads (combine at Qwen3 T = 8192: 0.119 -> 0.104 ms).
__device__ __forceinline__ uint4 ld_once16(const bf16_t* p) {
  typedef uint32_t v4x __attribute__((ext_vector_type(4)));
  const v4x v = __builtin_nontemporal_load(reinterpret_cast<const v4x*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_perm,
                                                      const int32_t* __restrict__ dst_row,
                                                      const float* __restrict__ w, int T, int k,
                                                      int H, const void* __restrict__ y_shared,
                                                      void* __restrict__ y) {
  const int t = blockIdx.y;
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (c0 >= H) return;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  // the shared expert's row segment is loaded first: its latency overlaps
  // the routing loads below instead of following the sum
  uint4 sh_raw[OUT_BF16 ? 1 : 2];
  if (y_shared) {
    if (OUT_BF16) {
      sh_raw[0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(y_shared) +
                                                  (size_t)t * H + c0);
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(y_shared) +
                                                      (size_t)t * H + c0);
      sh_raw[0] = p[0];
      sh_raw[OUT_BF16 ? 0 : 1] = p[1];
    }
  }
  // up to 8 permuted rows per batch: their loads are all in flight before the
  // first multiply-add; the sum still runs in slot order
  for (int j0 = 0; j0 < k; j0 += 8) {
    int rows[8];
    float wj[8];
    uint4 raw[8][IN_BF16 ? 1 : 2];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      rows[u] = j < k ? dst_row[(size_t)t * k + j] : -1;
      wj[u] = j < k ? w[(size_t)t * k + j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (rows[u] < 0) continue;
      if (IN_BF16) {
        raw[u][0] = ld_once16(reinterpret_cast<const bf16_t*>(y_perm) + (size_t)rows[u] * H + c0);
      } else {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(y_perm) +
                                                        (size_t)rows[u] * H + c0);
        raw[u][0] = p[0];
        raw[u][IN_BF16 ? 0 : 1] = p[1];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (rows[u] < 0) continue;
      float v[8];
      if (IN_BF16) {
        unpack_bf16x8(raw[u][0], v);
      } else {
        const uint4 lo = raw[u][0], hi = raw[u][IN_BF16 ? 0 : 1];
        v[0] = __uint_as_float(lo.x); v[1] = __uint_as_float(lo.y);
        v[2] = __uint_as_float(lo.z); v[3] = __uint_as_float(lo.w);
        v[4] = __uint_as_float(hi.x); v[5] = __uint_as_float(hi.y);
        v[6] = __uint_as_float(hi.z); v[7] = __uint_as_float(hi.w);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(wj[u], v[q], acc[q]);
    }
  }
  if (y_shared) {
    float v[8];
    if (OUT_BF16) {
      unpack_bf16x8(sh_raw[0], v);
    } else {
      const uint4 lo = sh_raw[0], hi = sh_raw[OUT_BF16 ? 0 : 1];
      v[0] = __uint_as_float(lo.x); v[1] = __uint_as_float(lo.y);
      v[2] = __uint_as_float(lo.z); v[3] = __uint_as_float(lo.w);
      v[4] = __uint_as_float(hi.x); v[5] = __uint_as_float(hi.y);
      v[6] = __uint_as_float(hi.z); v[7] = __uint_as_float(hi.w);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += v[q];
  }
  if (OUT_BF16) {
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(y) + (size_t)t * H + c0) = o;
  } else {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + (size_t)t * H + c0);
    p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

hipError_t launch_combine(const void* y_perm, int y_perm_dt, const int32_t* dst_row,
                          const float* w, int T, int k, int H, const void* y_shared, void* y,
                          int dt, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  dim3 grid((H / 8 + 255) / 256, T);
  const bool in_bf = y_perm_dt == 1, out_bf = dt == 1;
  if (in_bf && out_bf) combine_kernel<true, true><<<grid, 256, 0, st>>>(y_perm, dst_row, w, T, k, H, y_shared, y);
  else if (in_bf) combine_kernel<true, false><<<grid, 256, 0, st>>>(y_perm, dst_row, w, T, k, H, y_shared, y);
  else if (out_bf) combine_kernel<false, true><<<grid, 256, 0, st>>>(y_perm, dst_row, w, T, k, H, y_shared, y);
  else combine_kernel<false, false><<<grid, 256, 0, st>>>(y_perm, dst_row, w, T, k, H, y_shared, y);
  return hipGetLastError();
}

}  // namespace moe
