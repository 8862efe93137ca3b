// Local halves of the expert-parallel <-> tensor-parallel weight reshard.
//
// Moebius notes (Zhongzhu Zhou), section 3: EP and TP are two layouts of the
// same expert weights, eq. (6)-(8).  Algorithm 1 (EP -> TP) packs, for every
// peer p, the slice of this rank's experts that p holds after the switch,
// before an All-to-All; its output needs no further step.  Algorithm 2
// (TP -> EP) sends contiguous expert ranges and interleaves the received
// slices back into whole experts.  These kernels are the two data movements
// on one rank (pack, interleave); the exchange between ranks is not here.
//
// Layouts (elements of dtype dt, n = E/P experts per rank, s = I/P):
//   EP:      W13[n][2I][H] (gate rows [0, I), up rows [I, 2I)), W2[n][H][I]
//   chunks:  C13[P][n][2s][H] (peer p: gate rows p*s .. p*s+s-1, then the same
//            up rows), C2[P][n][H][s] (peer p: input columns p*s .. p*s+s-1)
// Peer p's slice cuts the same intermediate range from both halves of the
// stacked axis, so that SwiGLU stays local to a TP rank.
//
// Pure data movement, HBM-bound: each thread copies 16-byte vectors, the
// consecutive threads of a wave consecutive vectors of one row (or of one W2
// row segment of s elements), all of its loads before its stores.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int RS_THREADS = 256;
constexpr int RS_PER_THREAD = 4;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Vector offsets of element vector `idx` of the chunk layout, in the chunk
// buffer and in the EP buffer.
__device__ __forceinline__ void w13_offsets(int idx, int hv, int s, int n, int I,
                                            long long& chunk, long long& ep) {
  const int v = idx % hv;
  int rest = idx / hv;
  const int j = rest % (2 * s);
  rest /= 2 * s;
  const int e = rest % n;
  const int p = rest / n;
  const int row = j < s ? p * s + j : I + p * s + (j - s);
  chunk = (long long)idx;
  ep = ((long long)e * 2 * I + row) * hv + v;
}

__device__ __forceinline__ void w2_offsets(int idx, int sv, int iv, int H, int n,
                                           long long& chunk, long long& ep) {
  const int v = idx % sv;
  int rest = idx / sv;
  const int h = rest % H;
  rest /= H;
  const int e = rest % n;
  const int p = rest / n;
  chunk = (long long)idx;
  ep = ((long long)e * H + h) * iv + (long long)p * sv + v;
}

// PACK: EP -> chunks; otherwise chunks -> EP.  W2: the W2 layouts, else W13.
template <bool PACK, bool W2>
__global__ __launch_bounds__(RS_THREADS) void reshard_kernel(const v4u* __restrict__ src,
                                                             v4u* __restrict__ dst, int total,
                                                             int a0, int a1, int a2, int a3) {
  const int base = blockIdx.x * RS_THREADS * RS_PER_THREAD + threadIdx.x;
  v4u v[RS_PER_THREAD];
  long long d[RS_PER_THREAD];
#pragma unroll
  for (int u = 0; u < RS_PER_THREAD; ++u) {
    const int idx = min(base + u * RS_THREADS, total - 1);
    long long chunk, ep;
    if constexpr (W2) w2_offsets(idx, a0, a1, a2, a3, chunk, ep);
    else w13_offsets(idx, a0, a1, a2, a3, chunk, ep);
    v[u] = PACK ? src[ep] : src[chunk];
    d[u] = PACK ? chunk : ep;
  }
#pragma unroll
  for (int u = 0; u < RS_PER_THREAD; ++u)
    if (base + u * RS_THREADS < total) dst[d[u]] = v[u];
}

template <bool PACK>
hipError_t launch_reshard_dir(const void* w13_src, const void* w2_src, int n, int I, int H, int P,
                              int elt, void* w13_dst, void* w2_dst, hipStream_t st) {
  const int s = I / P;
  const int per_block = RS_THREADS * RS_PER_THREAD;
  if (w13_src) {
    const int hv = H * elt / 16;
    const long long total = (long long)P * n * 2 * s * hv;
    if (total > 0)
      reshard_kernel<PACK, false><<<(int)((total + per_block - 1) / per_block), RS_THREADS, 0, st>>>(
          static_cast<const v4u*>(w13_src), static_cast<v4u*>(w13_dst), (int)total, hv, s, n, I);
  }
  if (w2_src) {
    const int sv = s * elt / 16, iv = I * elt / 16;
    const long long total = (long long)P * n * H * sv;
    if (total > 0)
      reshard_kernel<PACK, true><<<(int)((total + per_block - 1) / per_block), RS_THREADS, 0, st>>>(
          static_cast<const v4u*>(w2_src), static_cast<v4u*>(w2_dst), (int)total, sv, iv, H, n);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reshard(bool pack, const void* w13_src, const void* w2_src, int n, int I, int H,
                          int P, int elt_bytes, void* w13_dst, void* w2_dst, hipStream_t st) {
  if (pack)
    return launch_reshard_dir<true>(w13_src, w2_src, n, I, H, P, elt_bytes, w13_dst, w2_dst, st);
  return launch_reshard_dir<false>(w13_src, w2_src, n, I, H, P, elt_bytes, w13_dst, w2_dst, st);
}

}  // namespace moe
