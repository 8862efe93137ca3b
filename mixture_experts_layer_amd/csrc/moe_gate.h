// Top-k gating of one token by one 16-lane row of a wave, shared by the
// gate-tile kernel and the single-launch decode kernel.
//
// Gating variants: "Lecture 8 · 混合专家模型的推理" (CS349D notes) section 1.2;
// the key/tie rule (key descending, equal keys to the lower expert id) makes
// the chosen ids a function of the float32 logits alone.
#pragma once
#include "moe_device.h"

namespace moe {

// ---------------------------------------------------------------------------
// Row reductions: DPP inside each 16-lane row -- pairs at distance 1 and 2,
// then the half-row and row mirrors -- leave every lane of the row with the
// row's result; the combination order is fixed, so float sums are the same
// on every run.
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

// Sum over each 16-lane row.
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<DPP_XOR1>(v);
  v += dpp_f<DPP_XOR2>(v);
  v += dpp_f<DPP_HALF_MIRROR>(v);
  v += dpp_f<DPP_MIRROR>(v);
  return v;
}

// ---------------------------------------------------------------------------
// Selection keys as one unsigned 64-bit integer: the float key mapped to an
// order-preserving 32-bit pattern (sign flipped for positives, all bits for
// negatives; -0 counted as +0) in the high word and ~id in the low word, so
// that "larger key, then smaller id" is plain unsigned order and 0 stands
// below every real key.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned long long pack_key(float key, int id) {
  const uint32_t u = __float_as_uint(key == 0.0f ? 0.0f : key);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (uint32_t)(0xffffffffu - (uint32_t)id);
}
__device__ __forceinline__ int packed_id(unsigned long long p) {
  return (int)(0xffffffffu - (uint32_t)p);
}
__device__ __forceinline__ float packed_key(unsigned long long p) {
  const uint32_t o = (uint32_t)(p >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
template <int CTRL>
__device__ __forceinline__ void max64_step(unsigned long long& v) {
  const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(v >> 32));
  const unsigned long long o = ((unsigned long long)hi << 32) | lo;
  v = o > v ? o : v;
}

// ---------------------------------------------------------------------------
// Gate one token.  The 16 lanes of a row call this together; lane `sub` holds
// the logits of experts sub, sub + 16, ... in s[0..EPR) (any value where the
// expert id is >= E).  `live` is false for a padding row (its lanes still take
// part in the row reductions and get no choice).
//
// k rounds of a row-wide arg-max over (key descending, id ascending) on the
// packed keys -- a local maximum, then four DPP steps -- pick the experts in
// order; every lane of the row sees the winner, the lane holding it retires
// it, and lane r % 16 keeps choice r.  The key is the logit, or logit +
// sel_bias in float32 for the sigmoid mode.  The round loop is not unrolled:
// gating runs once per layer call, so its code is kept small.
//
// Out: choice `sub` in (id0, g0) and choice sub + 16 in (id1, g1), valid
// when live and sub < k (sub + 16 < k); k <= 32.
// Weights by mode: 0 softmax over the k chosen logits; 1 softmax over all E
// taken at the chosen ids; 2 as 1, renormalised over the k chosen; 3
// sigmoid(logit) of the chosen, renormalised (no bias in the weights).
// ---------------------------------------------------------------------------
// The gate weights of one token from its chosen keys, on the 16-lane row
// layout of gate_row: lane `sub` holds the logits of experts sub, sub + 16,
// ... in s[], choice sub in c0 and choice sub + 16 in c1 (packed keys), and
// `first` is the largest key.
template <int EPR>
__device__ __forceinline__ void gate_weights(const float (&s)[EPR], bool live, int sub, int E,
                                             int k, int mode, unsigned long long c0,
                                             unsigned long long c1, unsigned long long first,
                                             int& id0, float& g0, int& id1, float& g1) {
  const bool h0 = live && sub < k, h1 = live && sub + 16 < k;
  id0 = h0 ? packed_id(c0) : -1;
  id1 = h1 ? packed_id(c1) : -1;
  if (mode == 3) {
    // the chosen experts' logits, from the lanes of this row that hold them
    const int row0 = (threadIdx.x & 63) & ~15;
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int j = 0; j < EPR; ++j) {
      const float a0 = __shfl(s[j], row0 + (id0 & 15));
      const float a1 = __shfl(s[j], row0 + (id1 & 15));
      if (h0 && (id0 >> 4) == j) v0 = a0;
      if (h1 && (id1 >> 4) == j) v1 = a1;
    }
    g0 = h0 ? 1.0f / (1.0f + expf(-v0)) : 0.f;
    g1 = h1 ? 1.0f / (1.0f + expf(-v1)) : 0.f;
    const float z = row_sum(g0 + g1);
    g0 = g0 / z;
    g1 = g1 / z;
    return;
  }
  // modes 0-2: the key is the logit itself
  const float v0 = packed_key(c0), v1 = packed_key(c1), first_s = packed_key(first);
  if (mode == 0) {
    // softmax over the k chosen logits; the first choice is the largest
    g0 = h0 ? expf(v0 - first_s) : 0.f;
    g1 = h1 ? expf(v1 - first_s) : 0.f;
    const float z = row_sum(g0 + g1);
    g0 = g0 / z;
    g1 = g1 / z;
  } else {
    // softmax over all E, then (mode 2) renormalised over the k chosen
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < EPR; ++i)
      if (live && sub + 16 * i < E) z += expf(s[i] - first_s);
    z = row_sum(z);
    g0 = h0 ? expf(v0 - first_s) / z : 0.f;
    g1 = h1 ? expf(v1 - first_s) / z : 0.f;
    if (mode == 2) {
      const float ps = row_sum(g0 + g1);
      g0 = g0 / ps;
      g1 = g1 / ps;
    }
  }
}

template <int EPR>
__device__ __forceinline__ void gate_row(const float (&s)[EPR], bool live, int sub, int E, int k, int mode,
                                const float* __restrict__ sel_bias, int& id0, float& g0, int& id1,
                                float& g1) {
  const bool sig = mode == 3;
  // the selection bias is loaded for all slots before any key is formed: a
  // load per slot under the mode's branch had waited for each slot in turn
  float sb[EPR];
#pragma unroll
  for (int i = 0; i < EPR; ++i) sb[i] = 0.f;
  if (sig && sel_bias) {
#pragma unroll
    for (int i = 0; i < EPR; ++i) {
      const int e = sub + 16 * i;
      sb[i] = e < E ? sel_bias[e] : 0.f;
    }
  }
  unsigned long long cand[EPR];
#pragma unroll
  for (int i = 0; i < EPR; ++i) {
    const int e = sub + 16 * i;
    const bool ok = live && e < E;
    cand[i] = ok ? pack_key((sig && sel_bias) ? s[i] + sb[i] : s[i], e) : 0ull;
  }
  unsigned long long c0 = 0ull, c1 = 0ull, first = 0ull;
  for (int r = 0; r < k; ++r) {
    unsigned long long best = cand[0];
#pragma unroll
    for (int i = 1; i < EPR; ++i) best = cand[i] > best ? cand[i] : best;
    max64_step<DPP_XOR1>(best);
    max64_step<DPP_XOR2>(best);
    max64_step<DPP_HALF_MIRROR>(best);
    max64_step<DPP_MIRROR>(best);
    if (r == 0) first = best;
    if (sub == (r & 15)) {
      if (r < 16) c0 = best;
      else c1 = best;
    }
#pragma unroll
    for (int i = 0; i < EPR; ++i) cand[i] = cand[i] == best ? 0ull : cand[i];
  }
  gate_weights<EPR>(s, live, sub, E, k, mode, c0, c1, first, id0, g0, id1, g1);
}

// ---------------------------------------------------------------------------
// The same choice for one token made by a whole wave (all 64 lanes, one token
// per wave): lane l holds the logits of experts l, l + 64, ... in s64[].
// Each round's arg-max takes four DPP steps inside the rows and two
// row-exchange steps (v_permlane16_swap, then v_permlane32_swap) across them,
// with a quarter of gate_row's keys per lane.  Every lane leaves with the
// row layout's (c0, c1, first): choice (lane % 16) and (lane % 16) + 16, and
// the largest key -- the same keys gate_row finds, since they are distinct.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned long long max64_across_rows(unsigned long long v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  {
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const unsigned long long a = ((unsigned long long)h[0] << 32) | l[0];
    const unsigned long long b = ((unsigned long long)h[1] << 32) | l[1];
    v = a > b ? a : b;                 // the row pair's largest
  }
  const uint32_t lo2 = (uint32_t)v, hi2 = (uint32_t)(v >> 32);
  const auto l = __builtin_amdgcn_permlane32_swap(lo2, lo2, false, false);
  const auto h = __builtin_amdgcn_permlane32_swap(hi2, hi2, false, false);
  const unsigned long long a = ((unsigned long long)h[0] << 32) | l[0];
  const unsigned long long b = ((unsigned long long)h[1] << 32) | l[1];
  return a > b ? a : b;                // the two halves' largest
}

template <int EPR64>
__device__ __forceinline__ void gate_select64(const float (&s64)[EPR64], bool live, int E, int k,
                                              int mode, const float* __restrict__ sel_bias,
                                              unsigned long long& c0, unsigned long long& c1,
                                              unsigned long long& first) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const bool sig = mode == 3;
  float sb[EPR64];                      // the selection bias, all loads first
#pragma unroll
  for (int i = 0; i < EPR64; ++i) sb[i] = 0.f;
  if (sig && sel_bias) {
#pragma unroll
    for (int i = 0; i < EPR64; ++i) {
      const int e = lane + 64 * i;
      sb[i] = e < E ? sel_bias[e] : 0.f;
    }
  }
  unsigned long long cand[EPR64];
#pragma unroll
  for (int i = 0; i < EPR64; ++i) {
    const int e = lane + 64 * i;
    const bool ok = live && e < E;
    cand[i] = ok ? pack_key((sig && sel_bias) ? s64[i] + sb[i] : s64[i], e) : 0ull;
  }
  c0 = c1 = first = 0ull;
  for (int r = 0; r < k; ++r) {
    unsigned long long best = cand[0];
#pragma unroll
    for (int i = 1; i < EPR64; ++i) best = cand[i] > best ? cand[i] : best;
    max64_step<DPP_XOR1>(best);
    max64_step<DPP_XOR2>(best);
    max64_step<DPP_HALF_MIRROR>(best);
    max64_step<DPP_MIRROR>(best);
    best = max64_across_rows(best);
    if (r == 0) first = best;
    if (sub == (r & 15)) {
      if (r < 16) c0 = best;
      else c1 = best;
    }
#pragma unroll
    for (int i = 0; i < EPR64; ++i) cand[i] = cand[i] == best ? 0ull : cand[i];
  }
}

}  // namespace moe
