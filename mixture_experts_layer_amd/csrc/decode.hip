// The whole layer share in one kernel launch, for decode-sized batches.
//
// "MoE 推理优化全景指南", section 一个 token 为什么要跨 GPU: route, dispatch
// metadata, expert MLPs and the weighted combine run one after the other; at
// decode each is small, so separate launches leave the GPU idle between
// dependent steps.  "Lecture 8 · 混合专家模型的推理" (CS349D notes) section 6
// names the remedy: one persistent kernel with device-side dependencies.
//
// One grid of one 16-wave block per CU, every block resident at once (the
// host sizes the grid from the occupancy of this kernel).  Phases:
//   1. Router: wave units (expert, 2 tokens) write float32 logits; every block
//      then arrives at a counter and waits for all blocks.
//   2. Gating, repeated by every block for all T <= 64 tokens (a whole wave per
//      token while T <= 16, gate_select64; else a 16-lane row, gate_row), and
//      the routing metadata in LDS: a 64-bit token mask per local expert gives
//      counts = popcount, offsets by a scan, and the row of (t, j) as
//      offset + popcount of the mask below bit t -- the stable order of the
//      permutation with no sort.  Active experts (count > 0) get slots, the
//      shared expert (if any) slot 0.
//   3. Gate/up units (slot, 8 columns of h): 8 gate + the matching 8 up rows
//      of W13 form the 16-row MFMA operand, the block's 16 waves split H, and
//      SiLU(gate) * up is rounded to bf16 into h.  A block adds the number of
//      units it finished to a counter once, after its last unit.
//   4. Down units (16 rows of H, all slots): the block's waves form groups of
//      KS that split each slot's K range (KS from the host: 1 when I is
//      short, up to 8 for a long I with few experts); a wave issues its first
//      batch of W2 loads, waits until every gate/up unit is counted, then
//      loads h and streams.  Results stay in LDS, where the block combines
//      them per token in slot order (plus the shared expert, weight 1) and
//      writes 16 columns of y.
// Units are dealt statically (every block derives the same lists from the
// same routing): gate/up unit u to block u mod NB, down unit v to block
// NB - 1 - v, so that the blocks the gate/up phase leaves idle start the down
// projection's loads early.
//
// Data that crosses workgroups (logits, h) moves only through device-scope
// atomic loads and stores (relaxed): coherent across the XCDs' L2s without
// any L2 write-back or invalidate, which a release/acquire fence would cost
// at every hand-over.  A producer's coherent stores have completed when its
// workgroup barrier passes (vmcnt(0)); only then does one lane add to a
// counter.  The workgroup whose add completes the count (fetch_add returns
// it) writes every workgroup's go flag -- one 128-byte line each, so that
// waiting workgroups poll distinct addresses instead of hammering one -- and
// a consumer issues its coherent loads only after its flag is up.  Flags
// carry the launch's epoch (2e + 1 after the router, 2e + 2 after the
// gate/up units), so they never need clearing.
//
// Waits are bounded (about 0.1-1 s): one that runs out sets a bit in the
// error word of the sync block and lets the block finish, so the grid always
// drains.
//
// Sync block (at the start of the workspace): ints [0] parity p, [1] error
// bits, [2] epoch e, then two counter sets; a launch uses set p, block 0
// clears set 1 - p, flips p and advances e once every block has read them
// (after the router wait).  Go flags follow the 4 KiB header.  A zeroed block
// is a valid first state, and every launch leaves a valid one.
#include "moe_device.h"
#include "moe_gate.h"
#include "moe_kernels.h"
#include "moe_router.h"

namespace moe {

namespace {

constexpr int DEC_WAVES = 16;
constexpr int DEC_THREADS = DEC_WAVES * 64;
constexpr int DEC_PAIRS = DECODE_MAX_PAIRS;
constexpr int DEC_EMAX = DECODE_MAX_E;
constexpr int DEC_TMAX = DECODE_MAX_T;
constexpr int DEC_SLOTS = DEC_EMAX + 1;
constexpr int DEC_YROWS = DEC_PAIRS + DEC_TMAX;
constexpr int DEC_YP = 17;          // LDS row pitch of expert outputs (floats)
constexpr int DEC_U = 8;            // K steps (32 elements) per load batch
constexpr int DEC_SPIN = 1 << 18;   // polls before a wait gives up

constexpr int SYNC_HDR = 64;        // ints before the counter sets
constexpr int SYNC_SET = 64;        // [0] router arrivals, [1] gate/up units done
constexpr int SYNC_FLAGS = 1024;    // int offset of the go flags (4 KiB)
constexpr int FLAG_STRIDE = 32;     // ints per go flag (128 bytes)
static_assert((SYNC_HDR + 2 * SYNC_SET) <= SYNC_FLAGS, "sync header too small");
static_assert((SYNC_FLAGS + DECODE_MAX_BLOCKS * FLAG_STRIDE) * 4 <= DECODE_SYNC_BYTES,
              "sync block too small");

__device__ __forceinline__ int load_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_relaxed(int* p, int v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// device-coherent 4- and 16-byte accesses for data shared between workgroups
__device__ __forceinline__ void store_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent_f32(const float* p) {
  return __uint_as_float(
      __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ uint4 load_coherent16(const bf16_t* p) {
  const unsigned long long* q = reinterpret_cast<const unsigned long long*>(p);
  const unsigned long long lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long hi =
      __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
}

__device__ __forceinline__ void set_error(int* sync, int bit) {
  __hip_atomic_fetch_or(sync + DECODE_ERR_INT, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll a go flag until it holds `want` or, if `alt_ok`, want + 1; false
// after DEC_SPIN polls.
__device__ bool wait_flag(const int* p, uint32_t want, bool alt_ok) {
  for (int i = 0; i < DEC_SPIN; ++i) {
    const uint32_t v = (uint32_t)load_relaxed(p);
    if (v == want || (alt_ok && v == want + 1u)) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// Count `inc` arrivals at *ctr; the workgroup that completes `target` raises
// every workgroup's go flag to `val`.  Called by the whole block after its
// stores have completed; returns true in the block that raised the flags.
__device__ bool arrive(int* ctr, int inc, int target, int* flags, int nb, uint32_t val,
                       int* s_last) {
  if (threadIdx.x == 0) {
    const int old = inc > 0 ? __hip_atomic_fetch_add(ctr, inc, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                            : -1;
    *s_last = (inc > 0 && old + inc == target) ? 1 : 0;
  }
  __syncthreads();
  const bool last = *s_last != 0;
  if (last)
    for (int i = threadIdx.x; i < nb; i += blockDim.x)
      store_coherent(reinterpret_cast<uint32_t*>(flags + i * FLAG_STRIDE), val);
  return last;
}

__device__ __forceinline__ uint4 ld16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

}  // namespace

struct DecodeArgs {
  const bf16_t* x;          // [T][H]
  const bf16_t* wr;         // [E][H]
  const float* logit_bias;  // [E] or null
  const float* sel_bias;    // [E] or null
  const bf16_t* w13;        // [E_loc][2I][H]
  const bf16_t* w2;         // [E_loc][H][I]
  const bf16_t* w13s;       // [2Is][H] or null
  const bf16_t* w2s;        // [H][Is] or null
  bf16_t* y;                // [T][H]
  float* logits;            // [T][E]
  bf16_t* h;                // routed rows [R][I]
  bf16_t* hs;               // shared-expert rows [T][Is]
  int* sync;                // sync block
  int32_t* ids_out;         // optional copies, written by block 0
  float* w_out;
  int32_t* counts_out;
  int32_t* offsets_out;
  int32_t* src_out;
  int32_t* dst_out;
  int T, H, E, k, mode, I, Is, e_begin, e_end;
  int ks2;                  // waves splitting each slot's K in the down units (1, 2, 4, 8)
};

template <int EPR>
__global__ __launch_bounds__(DEC_THREADS, DEC_WAVES / 4) void moe_decode_kernel(DecodeArgs a) {
  __shared__ int s_ids[DEC_PAIRS];
  __shared__ float s_w[DEC_PAIRS];
  __shared__ int s_dst[DEC_PAIRS];
  __shared__ unsigned long long s_mask[DEC_EMAX];
  __shared__ int s_cnt[DEC_EMAX];
  __shared__ int s_off[DEC_EMAX + 1];
  __shared__ int s_slot_e[DEC_SLOTS], s_slot_off[DEC_SLOTS], s_slot_n[DEC_SLOTS];
  __shared__ int s_src[DEC_YROWS];
  __shared__ int s_nslot;
  __shared__ int s_last;
  __shared__ __attribute__((aligned(16))) float s_red[DEC_WAVES * 64 * 4];
  __shared__ float s_y[DEC_YROWS * DEC_YP];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int NB = gridDim.x, b = blockIdx.x;
  const int T = a.T, H = a.H, E = a.E, k = a.k;
  int* sync = a.sync;
  const int p = load_relaxed(sync) & 1;
  const uint32_t ep = (uint32_t)load_relaxed(sync + 2);
  int* set = sync + SYNC_HDR + p * SYNC_SET;
  int* flags = sync + SYNC_FLAGS;
  const int* my_flag = flags + b * FLAG_STRIDE;

  // ---- 1. router logits: wave unit (expert e, tokens t0, t0 + 1), dealt
  // over the blocks first so that as many CUs as possible stream W_r --------
  {
    const int ntg = (T + 1) >> 1;
    for (int u = b + wid * NB; u < E * ntg; u += NB * DEC_WAVES) {
      const int e = u / ntg, t0 = (u - e * ntg) * 2;
      router_dot_wave<bf16_t, true, 4, 2>(a.x, a.wr, H, E, e, t0, min(2, T - t0), a.logit_bias,
                                          a.logits);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's logit stores completed
  __syncthreads();
  if (!arrive(set, 1, NB, flags, NB, 2u * ep + 1u, &s_last)) {
    // the gate/up flag (2e + 2) can only follow this one
    if (tid == 0 && !wait_flag(my_flag, 2u * ep + 1u, true)) set_error(sync, 1);
    __syncthreads();
  }

  // ---- 2. gating of all T tokens: one per wave while T <= 16, else four per
  // wave per pass ------------------------------------------------------------
  {
    const int row = lane >> 4, sub = lane & 15;
    if (T <= DEC_WAVES) {
      // the whole wave makes the choice (gate_select64: a quarter of
      // gate_row's keys per lane, so shorter rounds), and every row then
      // finishes the weights exactly as gate_row would; row 0 keeps them
      constexpr int EPR64 = (EPR + 3) / 4;
      const int tt = wid;
      if (tt < T) {
        float s64[EPR64], s[EPR];
#pragma unroll
        for (int i = 0; i < EPR64; ++i) {
          const int e = lane + 64 * i;
          s64[i] = e < E ? load_coherent_f32(a.logits + (size_t)tt * E + e) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < EPR; ++i) {
          const int e = sub + 16 * i;
          s[i] = e < E ? load_coherent_f32(a.logits + (size_t)tt * E + e) : 0.f;
        }
        unsigned long long c0, c1, first;
        gate_select64<EPR64>(s64, true, E, k, a.mode, a.sel_bias, c0, c1, first);
        int id0, id1;
        float g0, g1;
        gate_weights<EPR>(s, true, sub, E, k, a.mode, c0, c1, first, id0, g0, id1, g1);
        if (row == 0 && sub < k) {
          s_ids[tt * k + sub] = id0;
          s_w[tt * k + sub] = g0;
        }
      }
    } else
    for (int tt0 = wid * 4; tt0 < T; tt0 += DEC_WAVES * 4) {
      const int tt = tt0 + row;
      const bool live = tt < T;
      float s[EPR];
#pragma unroll
      for (int i = 0; i < EPR; ++i) {
        const int e = sub + 16 * i;
        s[i] = (live && e < E) ? load_coherent_f32(a.logits + (size_t)tt * E + e) : 0.f;
      }
      int id0, id1;
      float g0, g1;
      gate_row<EPR>(s, live, sub, E, k, a.mode, a.sel_bias, id0, g0, id1, g1);
      if (live && sub < k) {
        s_ids[tt * k + sub] = id0;
        s_w[tt * k + sub] = g0;
      }
    }
  }
  lds_barrier();
  // ---- routing metadata in LDS, by wave 0 alone (no block barriers) --------
  const int E_loc = a.e_end - a.e_begin;
  const int npair = T * k;
  const bool has_sh = a.Is > 0;
  const int base = has_sh ? 1 : 0;
  if (wid == 0) {
    for (int i = lane; i < E_loc; i += 64) s_mask[i] = 0ull;
    wave_lds_sync();
    for (int q = lane; q < npair; q += 64) {
      const int el = s_ids[q] - a.e_begin;
      if (el >= 0 && el < E_loc) atomicOr(&s_mask[el], 1ull << (q / k));
    }
    wave_lds_sync();
    // lane l owns experts [4l, 4l + 4) (E_loc <= 256): counts, then
    // exclusive scans of rows and of active experts across the wave
    int c[4], rows = 0, act = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * lane + j;
      c[j] = i < E_loc ? __popcll(s_mask[i]) : 0;
      rows += c[j];
      act += c[j] > 0 ? 1 : 0;
    }
    const int rs = wave_inclusive_scan(rows), as = wave_inclusive_scan(act);
    const int R_all = __builtin_amdgcn_readlane(rs, 63), n_all = __builtin_amdgcn_readlane(as, 63);
    int off = rs - rows, sl = base + as - act;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * lane + j;
      if (i < E_loc) {
        s_cnt[i] = c[j];
        s_off[i] = off;
        if (c[j] > 0) {
          s_slot_e[sl] = i;
          s_slot_off[sl] = off;
          s_slot_n[sl] = c[j];
          ++sl;
        }
        off += c[j];
      }
    }
    if (lane == 0) {
      s_off[E_loc] = R_all;
      s_nslot = n_all + base;
      if (has_sh) {
        s_slot_e[0] = -1;
        s_slot_off[0] = R_all;
        s_slot_n[0] = T;
      }
    }
    wave_lds_sync();
    for (int q = lane; q < npair; q += 64) {
      const int t = q / k, el = s_ids[q] - a.e_begin;
      int row = -1;
      if (el >= 0 && el < E_loc) {
        row = s_off[el] + __popcll(s_mask[el] & ((1ull << t) - 1ull));
        s_src[row] = t;
      }
      s_dst[q] = row;
    }
    if (has_sh)
      for (int t = lane; t < T; t += 64) s_src[R_all + t] = t;
  }
  __syncthreads();
  const int R = s_off[E_loc];
  const int nslot = s_nslot;
  const int nact = nslot - base;
  if (b == 0) {
    if (a.ids_out)
      for (int q = tid; q < npair; q += DEC_THREADS) a.ids_out[q] = s_ids[q];
    if (a.w_out)
      for (int q = tid; q < npair; q += DEC_THREADS) a.w_out[q] = s_w[q];
    if (a.counts_out)
      for (int i = tid; i < E_loc; i += DEC_THREADS) a.counts_out[i] = s_cnt[i];
    if (a.offsets_out)
      for (int i = tid; i <= E_loc; i += DEC_THREADS) a.offsets_out[i] = s_off[i];
    if (a.src_out)
      for (int r = tid; r < R; r += DEC_THREADS) a.src_out[r] = s_src[r];
    if (a.dst_out)
      for (int q = tid; q < npair; q += DEC_THREADS) a.dst_out[q] = s_dst[q];
    // every block has read p and e (it arrived at the router counter): clear
    // the other set for the next launch and hand both over
    int* other = sync + SYNC_HDR + (1 - p) * SYNC_SET;
    for (int i = tid; i < SYNC_SET; i += DEC_THREADS) other[i] = 0;
    if (tid == 0) {
      sync[0] = 1 - p;
      sync[2] = (int)(ep + 1u);
    }
  }
  const int r16 = lane & 15, kg = 8 * (lane >> 4);
  const int C8r = a.I / 8, C8s = a.Is / 8;
  const int U1 = nact * C8r + (has_sh ? C8s : 0);

  // ---- 3. gate/up units (slot, 8 columns of h) ------------------------------
  bool g1_last = false;
  {
    const int S = H / 32;
    const int sb = (S * wid) / DEC_WAVES, se = (S * (wid + 1)) / DEC_WAVES;
    int done = 0;
    for (int u = b; u < U1; u += NB) {
      int slot, c8;
      if (has_sh && u < C8s) {
        slot = 0;
        c8 = u;
      } else {
        const int v = u - (has_sh ? C8s : 0);
        slot = base + v / C8r;
        c8 = v - (v / C8r) * C8r;
      }
      const int el = s_slot_e[slot];
      const int Ia = el < 0 ? a.Is : a.I;
      const bf16_t* W = el < 0 ? a.w13s : a.w13 + (size_t)el * 2 * a.I * H;
      bf16_t* hp = el < 0 ? a.hs : a.h + (size_t)s_slot_off[slot] * a.I;
      const int* srcs = s_src + s_slot_off[slot];
      const int n = s_slot_n[slot];
      // operand row r16: gate row 8*c8 + r16 (r16 < 8) or the matching up row
      const int wr_i = r16 < 8 ? 8 * c8 + r16 : Ia + 8 * c8 + (r16 - 8);
      const bf16_t* wp = W + (size_t)wr_i * H + kg;
      for (int m0 = 0; m0 < n; m0 += 16) {
        const bool mv = m0 + r16 < n;
        const bf16_t* xp = a.x + (size_t)(mv ? srcs[m0 + r16] : 0) * H + kg;
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int s = sb; s < se; s += DEC_U) {
          uint4 wv[DEC_U], xv[DEC_U];
          // only the batch's own steps are loaded; the rest multiply zeros
#pragma unroll
          for (int q = 0; q < DEC_U; ++q) {
            const bool in = s + q < se;
            wv[q] = in ? ld16(wp + (s + q) * 32) : make_uint4(0, 0, 0, 0);
            xv[q] = mv && in ? ld16(xp + (s + q) * 32) : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int q = 0; q < DEC_U; ++q)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[q]), as_bf16x8(xv[q]), acc,
                                                          0, 0, 0);
        }
        // accumulator lane l: operand rows 4*(l/16) + i (gate 0..7, up 8..15)
        // of token m0 + l % 16; waves' partial sums meet in LDS in wave order
        *reinterpret_cast<float4*>(&s_red[(wid * 64 + lane) * 4]) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
        lds_barrier();
        if (tid < 64) {
          // thread (column pair jp, row mm) writes columns 2jp, 2jp + 1
          const int jp = tid >> 4, mm = tid & 15;
          float o[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int j = 2 * jp + c;
            const int gl = (j >> 2) * 16 + mm, ri = j & 3;
            float g = 0.f, uu = 0.f;
#pragma unroll
            for (int w = 0; w < DEC_WAVES; ++w) {
              g += s_red[(w * 64 + gl) * 4 + ri];
              uu += s_red[(w * 64 + gl + 32) * 4 + ri];
            }
            o[c] = silu_fast(g) * uu;
          }
          if (m0 + mm < n)
            store_coherent(
                reinterpret_cast<uint32_t*>(hp + (size_t)(m0 + mm) * Ia + 8 * c8 + 2 * jp),
                pack_bf16x2(o[0], o[1]));
        }
        lds_barrier();
      }
      ++done;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's h stores completed
    __syncthreads();
    if (U1 > 0) g1_last = arrive(set + 1, done, U1, flags, NB, 2u * ep + 2u, &s_last);
  }

  // ---- 4. down units (16 rows of H, all slots) + combine -------------------
  {
    const int nhb = H / 16;
    const int KS = a.ks2, G = DEC_WAVES / KS;
    const int grp = wid / KS, kq = wid - grp * KS;
    const int rounds = (nslot + G - 1) / G;
    int max_n = 0;
    for (int sl = 0; sl < nslot; ++sl) max_n = max(max_n, s_slot_n[sl]);
    const int v0 = NB - 1 - b;
    // Each wave waits for the gate/up units inside its first batch, between
    // that batch's W2 loads (which do not depend on h) and its h loads, so
    // the weights are in flight during the wait; a wave that reads no h does
    // not wait.  (Touching the first W2 loads into L2 before a block-wide
    // wait instead left the first batches of a workgroup's 16 waves to
    // complete one SIMD slot after another, about a memory round trip apart.)
    bool waiting = v0 < nhb && U1 > 0 && !g1_last;
    for (int v = v0; v < nhb; v += NB) {
      const int hr0 = 16 * v;
      for (int r = 0; r < rounds; ++r) {
        const int sl = grp + r * G;
        const bool live = sl < nslot;
        const int el = live ? s_slot_e[sl] : 0;
        const int Ia = el < 0 ? a.Is : a.I;
        const bf16_t* wp =
            (el < 0 ? a.w2s : a.w2 + (size_t)el * H * a.I) + (size_t)(hr0 + r16) * Ia + kg;
        const bf16_t* hp = el < 0 ? a.hs : a.h + (size_t)(live ? s_slot_off[sl] : 0) * a.I;
        const int n = live ? s_slot_n[sl] : 0, yr0 = live ? s_slot_off[sl] : 0;
        const int S2 = Ia / 32;
        const int kb = (S2 * kq) / KS, ke = (S2 * (kq + 1)) / KS;
        for (int m0 = 0; m0 < (KS == 1 ? n : max_n); m0 += 16) {
          const bool mv = m0 + r16 < n;
          f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (m0 < n) {
            const bf16_t* hq = hp + (size_t)(mv ? m0 + r16 : 0) * Ia + kg;
            for (int s = kb; s < ke; s += DEC_U) {
              uint4 wv[DEC_U], hv[DEC_U];
              // only the batch's own steps are loaded (a share of a few
              // steps, as at one token per slot, no longer issues DEC_U
              // loads of W2 and of h); the rest multiply zeros
#pragma unroll
              for (int q = 0; q < DEC_U; ++q)
                wv[q] = s + q < ke ? ld16(wp + (s + q) * 32) : make_uint4(0, 0, 0, 0);
              if (waiting) {
                if (lane == 0 && !wait_flag(my_flag, 2u * ep + 2u, false)) set_error(sync, 2);
                waiting = false;
                // no h load may be moved above the wait
                asm volatile("" ::: "memory");
              }
#pragma unroll
              for (int q = 0; q < DEC_U; ++q)
                hv[q] = mv && s + q < ke ? load_coherent16(hq + (s + q) * 32)
                                         : make_uint4(0, 0, 0, 0);
#pragma unroll
              for (int q = 0; q < DEC_U; ++q)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[q]), as_bf16x8(hv[q]),
                                                              acc, 0, 0, 0);
            }
          }
          // lane l: H rows hr0 + 4*(l/16) + i of token row m0 + l % 16
          if (KS == 1) {
            if (mv) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                s_y[(yr0 + m0 + r16) * DEC_YP + 4 * (lane >> 4) + i] = acc[i];
            }
          } else {
            // the KS waves of a group add their K parts in wave order
            *reinterpret_cast<float4*>(&s_red[(wid * 64 + lane) * 4]) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
            lds_barrier();
            if (kq == 0 && mv) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                float t = 0.f;
                for (int w = 0; w < KS; ++w) t += s_red[((wid + w) * 64 + lane) * 4 + i];
                s_y[(yr0 + m0 + r16) * DEC_YP + 4 * (lane >> 4) + i] = t;
              }
            }
            lds_barrier();
          }
        }
      }
      __syncthreads();
      for (int o = tid; o < T * 16; o += DEC_THREADS) {
        const int t = o >> 4, c = o & 15;
        float acc = 0.f;
        for (int j = 0; j < k; ++j) {
          const int row = s_dst[t * k + j];
          if (row >= 0) acc = fmaf(s_w[t * k + j], s_y[row * DEC_YP + c], acc);
        }
        if (has_sh) acc += s_y[(R + t) * DEC_YP + c];
        a.y[(size_t)t * H + hr0 + c] = f32_to_bf16(acc);
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

struct DecodeGrid {
  std::atomic<int> nb[64];
};

template <int EPR>
hipError_t decode_grid(int& nb_out) {
  static DecodeGrid cache{};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < 64) {
    const int c = cache.nb[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      nb_out = c;
      return hipSuccess;
    }
  }
  int occ = 0, cus = 0;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &occ, reinterpret_cast<const void*>(&moe_decode_kernel<EPR>), DEC_THREADS, 0);
  if (err != hipSuccess) return err;
  err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  if (occ < 1 || cus < 1) return hipErrorInvalidConfiguration;
  int nb = occ * cus;
  if (nb > DECODE_MAX_BLOCKS) nb = DECODE_MAX_BLOCKS;
  if (dev >= 0 && dev < 64) cache.nb[dev].store(nb, std::memory_order_relaxed);
  nb_out = nb;
  return hipSuccess;
}

template <int EPR>
hipError_t launch_decode_epr(const DecodeArgs& a, hipStream_t st) {
  int nb = 0;
  hipError_t err = decode_grid<EPR>(nb);
  if (err != hipSuccess) return err;
  moe_decode_kernel<EPR><<<nb, DEC_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

bool decode_supported(int dt, int T, int E, int E_loc, int k, int H, int I, int Is) {
  return dt == 1 && T >= 1 && T <= DECODE_MAX_T && E <= DECODE_MAX_E && E_loc <= DECODE_MAX_E &&
         k <= DECODE_MAX_K && T * k <= DECODE_MAX_PAIRS && H % 32 == 0 && I % 32 == 0 &&
         Is % 32 == 0;
}

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t st) {
  DecodeArgs a{};
  a.x = static_cast<const bf16_t*>(d.x);
  a.wr = static_cast<const bf16_t*>(d.w_router);
  a.logit_bias = d.logit_bias;
  a.sel_bias = d.sel_bias;
  a.w13 = static_cast<const bf16_t*>(d.w13);
  a.w2 = static_cast<const bf16_t*>(d.w2);
  a.w13s = static_cast<const bf16_t*>(d.w13_shared);
  a.w2s = static_cast<const bf16_t*>(d.w2_shared);
  a.y = static_cast<bf16_t*>(d.y);
  a.logits = d.logits;
  a.h = static_cast<bf16_t*>(d.h);
  a.hs = static_cast<bf16_t*>(d.h_shared);
  a.sync = d.sync;
  a.ids_out = d.ids_out;
  a.w_out = d.w_out;
  a.counts_out = d.counts_out;
  a.offsets_out = d.offsets_out;
  a.src_out = d.src_out;
  a.dst_out = d.dst_out;
  a.T = d.T; a.H = d.H; a.E = d.E; a.k = d.k; a.mode = d.mode;
  a.I = d.I_loc; a.Is = d.I_shared; a.e_begin = d.e_begin; a.e_end = d.e_end;
  // down units: KS waves split a slot's K so that the block's waves stay busy
  // when at most DEC_WAVES / KS slots can be active, while each wave keeps at
  // least one full load batch of the routed contraction (a split below that
  // costs its cross-wave reduction and barriers for nothing: TP share T = 1,
  // I = 192, KS 2 -> 1 took the layer from 24.0 to 23.5 us)
  const int E_loc = d.e_end - d.e_begin;
  const int slots = (d.T * d.k < E_loc ? d.T * d.k : E_loc) + (d.I_shared > 0 ? 1 : 0);
  a.ks2 = 1;
  while (a.ks2 < DEC_WAVES && 2 * a.ks2 * slots <= DEC_WAVES &&
         d.I_loc / 32 / (2 * a.ks2) >= DEC_U)
    a.ks2 *= 2;
  const int epr = (a.E + 15) / 16;
  if (epr <= 1) return launch_decode_epr<1>(a, st);
  if (epr <= 2) return launch_decode_epr<2>(a, st);
  if (epr <= 4) return launch_decode_epr<4>(a, st);
  if (epr <= 8) return launch_decode_epr<8>(a, st);
  return launch_decode_epr<16>(a, st);
}

}  // namespace moe
