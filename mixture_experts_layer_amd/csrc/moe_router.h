// Router scores by one wave, shared by the staged router kernel and the
// single-launch decode kernel, so both paths produce bit-identical logits
// (and therefore the same top-k choices).
//
// s = W_r x ("MoE 推理优化全景指南", section 从 Dense FFN 到专家集合).
#pragma once
#include "moe_device.h"

namespace moe {

// Logits of tokens t0 .. t0 + nt - 1 (nt <= 8) against expert e, computed by
// the calling wave (all 64 lanes): lane l takes the 16-byte chunks l, l + 64,
// ... of the H axis and accumulates them in H order with fmaf; a fixed xor
// butterfly then sums the 64 lanes.  Lane 0 stores logits[t][e] (+ bias[e]).
// The chunks are taken 8 at a time, the weight row's loads and then every
// token's loads issued before the first multiply, so a group costs one
// memory round trip rather than one per chunk.
// COHERENT: store with a device-scope atomic (visible to other workgroups of
// the running kernel once the store has completed); same value either way.
template <typename Tin, bool COHERENT = false>
__device__ __forceinline__ void router_dot_wave(const Tin* __restrict__ x, const Tin* __restrict__ wr,
                                       int H, int E, int e, int t0, int nt,
                                       const float* __restrict__ bias, float* __restrict__ logits) {
  constexpr int VEC = 16 / sizeof(Tin);  // elements per 16-byte load
  constexpr int G = 8;                   // chunks per group
  const int lane = threadIdx.x & 63;
  const Tin* wrow = wr + (size_t)e * H;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int h0 = VEC * lane; h0 < H; h0 += G * 64 * VEC) {
    uint4 wraw[G];
#pragma unroll
    for (int c = 0; c < G; ++c) {
      const int h = h0 + c * 64 * VEC;
      wraw[c] = h < H ? *reinterpret_cast<const uint4*>(wrow + h) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nt) {
        uint4 xraw[G];
#pragma unroll
        for (int c = 0; c < G; ++c) {
          const int h = h0 + c * 64 * VEC;
          xraw[c] = h < H ? *reinterpret_cast<const uint4*>(x + (size_t)(t0 + i) * H + h)
                          : make_uint4(0, 0, 0, 0);
        }
        float a = acc[i];
#pragma unroll
        for (int c = 0; c < G; ++c) {
          if (h0 + c * 64 * VEC < H) {
            float wv[8], xv[8];
            if constexpr (VEC == 8) {
              unpack_bf16x8(wraw[c], wv);
              unpack_bf16x8(xraw[c], xv);
            } else {
              wv[0] = __uint_as_float(wraw[c].x); wv[1] = __uint_as_float(wraw[c].y);
              wv[2] = __uint_as_float(wraw[c].z); wv[3] = __uint_as_float(wraw[c].w);
              xv[0] = __uint_as_float(xraw[c].x); xv[1] = __uint_as_float(xraw[c].y);
              xv[2] = __uint_as_float(xraw[c].z); xv[3] = __uint_as_float(xraw[c].w);
            }
#pragma unroll
            for (int q = 0; q < VEC; ++q) a = fmaf(xv[q], wv[q], a);
          }
        }
        acc[i] = a;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < nt) {
      float v = acc[i];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0) {
        const float out = bias ? v + bias[e] : v;
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
