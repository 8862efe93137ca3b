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
// consecutive threads of a wave consecutive vectors of one row (or of
// consecutive W2 row segments of s elements), all of a batch's loads before
// its stores.  The layout arithmetic is done once per block (and per thread
// for W2), not per vector with four integer divisions as in the first
// version (1-3% faster).  Every byte is read once and written once, so the
// loads and stores carry the non-temporal hint: 0.65 -> 0.72 of HBM for one
// Qwen3 rank share (pack 232 -> 205 us, interleave 229 -> 209 us).
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int RS_THREADS = 256;
constexpr int RS_BATCH = 4;            // vectors per thread per load batch
constexpr int RS_W2_ROWS = 256;        // W2 rows (h) per block

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// W13: one block per chunk row r = (p, e, j), j < 2s; the row's hv vectors
// are contiguous in both layouts (EP row p*s + j of the gate half for j < s,
// else I + p*s + (j - s)), so the index arithmetic is once per block.
template <bool PACK>
__global__ __launch_bounds__(RS_THREADS) void reshard_w13_kernel(const v4u* __restrict__ src,
                                                                 v4u* __restrict__ dst, int hv,
                                                                 int s, int n, int I) {
  const int r = blockIdx.x;
  const int j = r % (2 * s);
  const int pe = r / (2 * s);
  const int e = pe % n, p = pe / n;
  const int row = j < s ? p * s + j : I + p * s + (j - s);
  const long long c_off = (long long)r * hv;
  const long long e_off = ((long long)e * 2 * I + row) * hv;
  const v4u* sp = src + (PACK ? e_off : c_off);
  v4u* dp = dst + (PACK ? c_off : e_off);
  for (int v0 = threadIdx.x; v0 < hv; v0 += RS_THREADS * RS_BATCH) {
    v4u v[RS_BATCH];
#pragma unroll
    for (int u = 0; u < RS_BATCH; ++u) v[u] = __builtin_nontemporal_load(&sp[min(v0 + u * RS_THREADS, hv - 1)]);
#pragma unroll
    for (int u = 0; u < RS_BATCH; ++u)
      if (v0 + u * RS_THREADS < hv) __builtin_nontemporal_store(v[u], &dp[v0 + u * RS_THREADS]);
  }
}

// W2: one block per (p, e) and RS_W2_ROWS rows h.  The chunk's rows are
// contiguous (sv vectors each); in the EP layout row h's segment p starts at
// (e*H + h)*iv + p*sv.  Each thread walks its vectors f = tid, tid + 256, ...
// of the block's range, advancing (row, column) without a division.
template <bool PACK>
__global__ __launch_bounds__(RS_THREADS) void reshard_w2_kernel(const v4u* __restrict__ src,
                                                                v4u* __restrict__ dst, int sv,
                                                                int iv, int H, int n) {
  const int nhb = (H + RS_W2_ROWS - 1) / RS_W2_ROWS;
  const int hb = blockIdx.x % nhb;
  const int pe = blockIdx.x / nhb;
  const int e = pe % n, p = pe / n;
  const int h0 = hb * RS_W2_ROWS;
  const int total = (min(h0 + RS_W2_ROWS, H) - h0) * sv;
  const long long c_base = ((long long)pe * H + h0) * sv;
  const long long e_base = ((long long)e * H + h0) * iv + (long long)p * sv;
  const int step_h = RS_THREADS / sv, step_v = RS_THREADS - step_h * sv;
  int f = threadIdx.x;
  int hh = f / sv, vv = f - hh * sv;
  while (f < total) {
    long long cs[RS_BATCH], es[RS_BATCH];
    int nb = 0;
#pragma unroll
    for (int u = 0; u < RS_BATCH; ++u) {
      cs[u] = c_base + f;
      es[u] = e_base + (long long)hh * iv + vv;
      if (f < total) nb = u + 1;
      f += RS_THREADS;
      hh += step_h;
      vv += step_v;
      if (vv >= sv) {
        vv -= sv;
        ++hh;
      }
    }
    v4u v[RS_BATCH];
#pragma unroll
    for (int u = 0; u < RS_BATCH; ++u)
      if (u < nb) v[u] = __builtin_nontemporal_load(&src[PACK ? es[u] : cs[u]]);
#pragma unroll
    for (int u = 0; u < RS_BATCH; ++u)
      if (u < nb) __builtin_nontemporal_store(v[u], &dst[PACK ? cs[u] : es[u]]);
  }
}

template <bool PACK>
hipError_t launch_reshard_dir(const void* w13_src, const void* w2_src, int n, int I, int H, int P,
                              int elt, void* w13_dst, void* w2_dst, hipStream_t st) {
  const int s = I / P;
  if (w13_src) {
    const int hv = H * elt / 16;
    const long long rows = (long long)P * n * 2 * s;
    if (rows > 0 && hv > 0)
      reshard_w13_kernel<PACK><<<(int)rows, RS_THREADS, 0, st>>>(
          static_cast<const v4u*>(w13_src), static_cast<v4u*>(w13_dst), hv, s, n, I);
  }
  if (w2_src) {
    const int sv = s * elt / 16, iv = I * elt / 16;
    const long long blocks = (long long)P * n * ((H + RS_W2_ROWS - 1) / RS_W2_ROWS);
    if (blocks > 0 && sv > 0)
      reshard_w2_kernel<PACK><<<(int)blocks, RS_THREADS, 0, st>>>(
          static_cast<const v4u*>(w2_src), static_cast<v4u*>(w2_dst), sv, iv, H, n);
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
