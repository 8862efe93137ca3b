// Router scores by one wave, shared by the staged router kernel and the
// single-launch decode kernel, so both paths produce bit-identical logits
// (and therefore the same top-k choices).
//
// s = W_r x ("MoE 推理优化全景指南", section 从 Dense FFN 到专家集合).
#pragma once
#include "moe_device.h"

namespace moe {

// Logits of tokens t0 .. t0 + nt - 1 (nt <= NTM <= 8) against expert e, computed by
// the calling wave (all 64 lanes): lane l takes the 16-byte chunks l, l + 64,
// ... of the H axis and accumulates them in H order with fmaf; wave_sum_f
// then sums the 64 lanes in a fixed order.  Lane 0 stores logits[t][e]
// (+ bias[e]).
// The chunks are taken in groups, and a group's weight loads and every
// token's loads are issued before the first multiply, so a group costs one
// memory round trip: 8 chunks per group for a single token, GM for several
// (GM * (nt + 1) loads in flight per lane).  Every lane visits its chunks in
// the same order whatever the grouping, so the logits are bit-identical.
// COHERENT: store with a device-scope atomic (visible to other workgroups of
// the running kernel once the store has completed); same value either way.
template <typename Tin>
__device__ __forceinline__ void router_fma_chunk(const uint4& wraw, const uint4& xraw, float& a) {
  constexpr int VEC = 16 / sizeof(Tin);
  float wv[8], xv[8];
  if constexpr (VEC == 8) {
    unpack_bf16x8(wraw, wv);
    unpack_bf16x8(xraw, xv);
  } else {
    wv[0] = __uint_as_float(wraw.x); wv[1] = __uint_as_float(wraw.y);
    wv[2] = __uint_as_float(wraw.z); wv[3] = __uint_as_float(wraw.w);
    xv[0] = __uint_as_float(xraw.x); xv[1] = __uint_as_float(xraw.y);
    xv[2] = __uint_as_float(xraw.z); xv[3] = __uint_as_float(xraw.w);
  }
#pragma unroll
  for (int q = 0; q < VEC; ++q) a = fmaf(xv[q], wv[q], a);
}

template <typename Tin, bool COHERENT = false, int GM = 2, int NTM = 8>
__device__ __forceinline__ void router_dot_wave(const Tin* __restrict__ x, const Tin* __restrict__ wr,
                                       int H, int E, int e, int t0, int nt,
                                       const float* __restrict__ bias, float* __restrict__ logits) {
  constexpr int VEC = 16 / sizeof(Tin);  // elements per 16-byte load
  const int lane = threadIdx.x & 63;
  const Tin* wrow = wr + (size_t)e * H;
  const float bias_e = bias ? bias[e] : 0.f;   // loaded ahead of the dot products
  float acc[NTM];
#pragma unroll
  for (int i = 0; i < NTM; ++i) acc[i] = 0.f;
  auto ld = [&](const Tin* p, int h) {
    return h < H ? *reinterpret_cast<const uint4*>(p + h) : make_uint4(0, 0, 0, 0);
  };
  if (nt == 1) {
    constexpr int G = 8;
    const Tin* xr = x + (size_t)t0 * H;
    for (int h0 = VEC * lane; h0 < H; h0 += G * 64 * VEC) {
      uint4 wraw[G], xraw[G];
#pragma unroll
      for (int c = 0; c < G; ++c) wraw[c] = ld(wrow, h0 + c * 64 * VEC);
#pragma unroll
      for (int c = 0; c < G; ++c) xraw[c] = ld(xr, h0 + c * 64 * VEC);
#pragma unroll
      for (int c = 0; c < G; ++c)
        if (h0 + c * 64 * VEC < H) router_fma_chunk<Tin>(wraw[c], xraw[c], acc[0]);
    }
  } else {
    for (int h0 = VEC * lane; h0 < H; h0 += GM * 64 * VEC) {
      uint4 wraw[GM], xraw[NTM][GM];
#pragma unroll
      for (int c = 0; c < GM; ++c) wraw[c] = ld(wrow, h0 + c * 64 * VEC);
#pragma unroll
      for (int i = 0; i < NTM; ++i)
#pragma unroll
        for (int c = 0; c < GM; ++c)
          xraw[i][c] = i < nt ? ld(x + (size_t)(t0 + i) * H, h0 + c * 64 * VEC)
                              : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < NTM; ++i)
        if (i < nt) {
#pragma unroll
          for (int c = 0; c < GM; ++c)
            if (h0 + c * 64 * VEC < H) router_fma_chunk<Tin>(wraw[c], xraw[i][c], acc[i]);
        }
    }
  }
#pragma unroll
  for (int i = 0; i < NTM; ++i) {
    if (i < nt) {
      const float v = wave_sum_f(acc[i]);
      if (lane == 0) {
        const float out = bias ? v + bias_e : v;
        float* dst = logits + (size_t)(t0 + i) * E + e;
        if constexpr (COHERENT)
          __hip_atomic_store(reinterpret_cast<uint32_t*>(dst), __float_as_uint(out),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *dst = out;
      }
    }
  }
}

}  // namespace moe
