// C ABI entry points: argument checks, workspace layout and kernel sequencing.
// Declarations and the full contract are in include/moe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <climits>
#include <mutex>

#include "moe.h"
#include "moe_kernels.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int elt_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }
inline bool valid_dt(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
inline int cdiv(int a, int b) { return a / b + (a % b != 0); }   // a >= 0, b > 0, no overflow

// Bump allocator over the caller's workspace (or a size count when base == 0).
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t bytes) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += align_up(bytes);
    return p;
  }
};

// Token-pair and logit counts are int on the device: T * E (logits; k <= E,
// so this bounds the T * k pairs as well) must fit an int.
bool fits_int(long long a, long long b) { return a * b <= INT_MAX; }

int check_route_shape(int T, int E, int k, int mode) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (mode < 0 || mode > 3) return MOE_ERR_INVALID_ARG;
  if (E > 1024 || k > KMAX) return MOE_ERR_UNSUPPORTED;
  if (!fits_int(T, E)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_hidden(int H) {
  if (H <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 32) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Expected rows per expert, used to pick the GEMM row tile.
int mean_rows(int T, int k, int E) { return cdiv(T * k, E); }

int max_tiles_for(int max_rows, int E_loc, int BM) {
  if (max_rows <= 0) return 1;
  const long long bound = ((long long)max_rows + (long long)E_loc * (BM - 1)) / BM;
  return (int)(bound < max_rows ? bound : max_rows);
}

struct LayerWs {
  int* sync;                 // DECODE_SYNC_BYTES at offset 0
  float* logits;
  int32_t *ids, *counts, *offsets, *src_token, *dst_row;
  float* w;
  int32_t *tile_counts, *tile_base, *rank, *n_tiles;
  int4* tile_map;
  void *h, *y_perm, *h_s, *y_s;
  int BM, max_tiles, max_rows, n_tt;
};

int check_desc(const moe_layer_desc* d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (!valid_dt(d->dt)) return MOE_ERR_INVALID_ARG;
  int st = check_hidden(d->H);
  if (st) return st;
  if (d->E < 1 || d->k < 1 || d->k > d->E) return MOE_ERR_INVALID_ARG;
  if (d->mode < 0 || d->mode > 3) return MOE_ERR_INVALID_ARG;
  if (d->E > 1024 || d->k > KMAX) return MOE_ERR_UNSUPPORTED;
  if (d->I_loc <= 0 || d->e_begin < 0 || d->e_end > d->E || d->e_begin >= d->e_end)
    return MOE_ERR_INVALID_ARG;
  if (d->I_loc % 32) return MOE_ERR_UNSUPPORTED;
  if (d->I_shared < 0) return MOE_ERR_INVALID_ARG;
  if (d->I_shared % 32) return MOE_ERR_UNSUPPORTED;
  if (!d->w_router || !d->w13 || !d->w2) return MOE_ERR_INVALID_ARG;
  if (!aligned16(d->w_router) || !aligned16(d->w13) || !aligned16(d->w2))
    return MOE_ERR_INVALID_ARG;
  if (d->I_shared > 0) {
    if (!d->w13_shared || !d->w2_shared) return MOE_ERR_INVALID_ARG;
    if (!aligned16(d->w13_shared) || !aligned16(d->w2_shared)) return MOE_ERR_INVALID_ARG;
  }
  if ((d->logit_bias && !aligned16(d->logit_bias)) || (d->sel_bias && !aligned16(d->sel_bias)))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// pad_rows >= 0: the padded capacity layout, whose h and y_perm hold pad_rows
// (E_loc * capacity) rows; the GEMM tiles still cover only kept rows.
size_t layer_layout(const moe_layer_desc* d, int T, void* base, LayerWs* w, int pad_rows = -1) {
  const int E_loc = d->e_end - d->e_begin;
  const int eb = elt_bytes(d->dt);
  const int real_rows = T * (d->k < E_loc ? d->k : E_loc);
  const int max_rows = pad_rows >= 0 ? pad_rows : real_rows;
  const int n_tt = cdiv(T, TOK_TILE);
  const int BM = ffn_row_tile(d->dt, mean_rows(T, d->k, d->E), d->H, d->I_loc,
                              T * d->k < E_loc ? T * d->k : E_loc);
  const int max_tiles = max_tiles_for(real_rows < max_rows ? real_rows : max_rows, E_loc, BM);
  Carver c(base);
  LayerWs l;
  // the single-launch decode path keeps its counters here, ahead of
  // everything the other path writes, so the two can share a workspace
  l.sync = c.take<int>(DECODE_SYNC_BYTES);
  l.logits = c.take<float>((size_t)T * d->E * 4);
  l.ids = c.take<int32_t>((size_t)T * d->k * 4);
  l.w = c.take<float>((size_t)T * d->k * 4);
  l.tile_counts = c.take<int32_t>((size_t)n_tt * E_loc * 4);
  l.tile_base = c.take<int32_t>((size_t)n_tt * E_loc * 4);
  l.rank = c.take<int32_t>((size_t)T * d->k * 4);
  l.counts = c.take<int32_t>((size_t)E_loc * 4);
  l.offsets = c.take<int32_t>((size_t)(E_loc + 1) * 4);
  l.src_token = c.take<int32_t>((size_t)(pad_rows >= 0 ? pad_rows : T * d->k) * 4);
  l.dst_row = c.take<int32_t>((size_t)T * d->k * 4);
  l.tile_map = c.take<int4>((size_t)max_tiles * sizeof(int4));
  l.n_tiles = c.take<int32_t>(4);
  l.h = c.take<char>((size_t)max_rows * d->I_loc * eb);
  l.y_perm = c.take<char>((size_t)max_rows * d->H * eb);
  l.h_s = l.y_s = nullptr;
  if (d->I_shared > 0) {
    l.h_s = c.take<char>((size_t)T * d->I_shared * eb);
    l.y_s = c.take<char>((size_t)T * d->H * eb);
  }
  l.BM = BM;
  l.max_tiles = max_tiles;
  l.max_rows = max_rows;
  l.n_tt = n_tt;
  if (w) *w = l;
  return c.used;
}

#define MOE_TRY(expr)                      \
  do {                                     \
    hipError_t _e = (expr);                \
    if (_e != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool decode_shape_ok(const moe_layer_desc* d, int T) {
  return decode_supported(d->dt, T, d->E, d->e_end - d->e_begin, d->k, d->H, d->I_loc,
                          d->I_shared);
}

// moe_layer takes the single-launch path while the expert weights a call can
// touch -- min(E_loc, T*k) routed experts plus the shared one -- stay under
// this many bytes: there the launch and dependency chain of the staged path
// costs more than the single launch's lower streaming rate.  Measured
// crossover on MI355X, since the staged path's direct GEMMs stream their
// weights non-temporally: between 75 MB (Qwen3 TP share T = 2: 35.7 µs
// staged, 35.1 µs single-launch) and 151 MB (T = 4: 47.8 against 50.3 µs).
constexpr double DECODE_AUTO_BYTES = 100e6;

bool decode_preferred(const moe_layer_desc* d, int T) {
  const int E_loc = d->e_end - d->e_begin;
  const long long pairs = (long long)T * d->k;
  const double experts = (double)(pairs < E_loc ? pairs : E_loc);
  const double bytes = 2.0 * 3.0 * (double)d->H * (experts * d->I_loc + (double)d->I_shared);
  return bytes <= DECODE_AUTO_BYTES;
}

int check_layer_call(const moe_layer_desc* d, int T, const void* x, void* y, void* ws,
                     size_t ws_bytes, const moe_debug_out* dbg, int pad_rows = -1) {
  int st = check_desc(d);
  if (st) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (!fits_int(T, d->E)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !y || !aligned16(x) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  const size_t need = layer_layout(d, T, nullptr, nullptr, pad_rows);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_INVALID_ARG;
  if (dbg) {
    const void* ptrs[] = {dbg->logits, dbg->topk_ids, dbg->topk_w, dbg->counts,
                          dbg->offsets, dbg->src_token, dbg->dst_row};
    for (const void* p : ptrs)
      if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

// MOE_VALIDATE=1 in the environment (read at every call): after the routing
// metadata is built, check it on the device and return MOE_ERR_METADATA if it
// is inconsistent.  The check copies its result word to the host and waits
// for the stream, so such calls cannot be captured in a graph.
// Single-tile batches from this many tokens gate over several blocks of
// GATE_SPLIT_TPB tokens before the one-block metadata pass.
constexpr int GATE_SPLIT_MIN_T = 16;
constexpr int GATE_SPLIT_TPB = 4;

bool validate_on() {
  const char* v = getenv("MOE_VALIDATE");
  return v && v[0] == '1' && v[1] == '\0';
}
constexpr size_t VALIDATE_BYTES = 256;   // the result word, at a 256-byte boundary
constexpr int LAYER_VALIDATE_INT = 8;    // its int index in the layer's sync block

int check_meta(const int32_t* ids, int npair, int E, int e_begin, int e_end, const int32_t* counts,
               const int32_t* offsets, int capacity, int padded, const int32_t* dropped,
               int32_t* err, hipStream_t s) {
  MOE_TRY(launch_validate_meta(ids, npair, E, e_begin, e_end, counts, offsets, capacity, padded,
                               dropped, err, s));
  int32_t word = 0;
  MOE_TRY(hipMemcpyAsync(&word, err, sizeof(word), hipMemcpyDeviceToHost, s));
  MOE_TRY(hipStreamSynchronize(s));
  return word ? MOE_ERR_METADATA : MOE_OK;
}

// The decode path's error word (int 1 of the synchronisation block): read it
// after the stream's work, clear it if set, and return MOE_ERR_WAIT if it was.
// Synchronises the stream.
int take_wait_word(int* sync, hipStream_t s) {
  int32_t word = 0;
  MOE_TRY(hipMemcpyAsync(&word, sync + DECODE_ERR_INT, sizeof(word), hipMemcpyDeviceToHost, s));
  MOE_TRY(hipStreamSynchronize(s));
  if (word == 0) return MOE_OK;
  static const int32_t zero = 0;
  MOE_TRY(hipMemcpyAsync(sync + DECODE_ERR_INT, &zero, sizeof(zero), hipMemcpyHostToDevice, s));
  MOE_TRY(hipStreamSynchronize(s));
  return MOE_ERR_WAIT;
}

int run_decode(const moe_layer_desc* d, int T, const void* x, void* y, const LayerWs& l,
               moe_debug_out* dbg, hipStream_t s) {
  auto mark = [&](int i) -> hipError_t {
    if (dbg && dbg->stage_events[i])
      return hipEventRecord(static_cast<hipEvent_t>(dbg->stage_events[i]), s);
    return hipSuccess;
  };
  DecodeLaunch a{};
  a.x = x; a.w_router = d->w_router; a.logit_bias = d->logit_bias; a.sel_bias = d->sel_bias;
  a.w13 = d->w13; a.w2 = d->w2; a.w13_shared = d->w13_shared; a.w2_shared = d->w2_shared;
  a.y = y;
  a.logits = (dbg && dbg->logits) ? dbg->logits : l.logits;
  a.h = l.h;
  a.h_shared = l.h_s;
  a.sync = l.sync;
  if (dbg) {
    a.ids_out = dbg->topk_ids; a.w_out = dbg->topk_w; a.counts_out = dbg->counts;
    a.offsets_out = dbg->offsets; a.src_out = dbg->src_token; a.dst_out = dbg->dst_row;
  }
  a.T = T; a.H = d->H; a.E = d->E; a.k = d->k; a.mode = d->mode;
  a.I_loc = d->I_loc; a.I_shared = d->I_shared; a.e_begin = d->e_begin; a.e_end = d->e_end;
  const bool check = validate_on();
  if (check) {
    // the kernel's metadata lives in LDS; have it written out to be checked
    if (!a.ids_out) a.ids_out = l.ids;
    if (!a.counts_out) a.counts_out = l.counts;
    if (!a.offsets_out) a.offsets_out = l.offsets;
  }
  MOE_TRY(mark(0));
  MOE_TRY(launch_decode(a, s));
  for (int i = 1; i < MOE_STAGE_EVENTS; ++i) MOE_TRY(mark(i));
  if (check) {
    const int st = check_meta(a.ids_out, T * d->k, d->E, d->e_begin, d->e_end, a.counts_out,
                              a.offsets_out, INT_MAX, 0, nullptr, l.sync + LAYER_VALIDATE_INT, s);
    // a wait that ran out is the cause of any other inconsistency: report it first
    const int wst = take_wait_word(l.sync, s);
    return wst != MOE_OK ? wst : st;
  }
  return MOE_OK;
}


// ---------------------------------------------------------------------------
// Workspace of the allocation-free entry point: one array per GPU, reserved
// when the code object is loaded on it and held until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// its device address comes from hipGetSymbolAddress, once per device, and
// only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ void zero_words_kernel(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// The current device's scratch address; at the first call on a device, look
// it up and clear its decode synchronisation block on `s` (a fill kernel,
// stream-ordered before the call's own launches).
int static_scratch(void** out, hipStream_t s) {
  int dev = 0;
  MOE_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    MOE_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || !aligned16(p)) return MOE_ERR_HIP;
    zero_words_kernel<<<32, 256, 0, s>>>(static_cast<int*>(p), DECODE_SYNC_BYTES / 4);
    MOE_TRY(hipGetLastError());
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

#ifndef MOE_SOURCE_SHA256
#define MOE_SOURCE_SHA256 "unstamped"
#endif
const char* moe_source_sha256(void) { return MOE_SOURCE_SHA256; }

const char* moe_status_str(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape, dtype or mode";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch error";
    case MOE_ERR_METADATA: return "routing metadata check failed";
    case MOE_ERR_WAIT: return "a decode-path wait for another workgroup ran out (outputs undefined)";
    default: return "unknown status";
  }
}

int moe_route(const void* x, const void* w_router, int dt, int T, int H, int E, int k, int mode,
              const float* logit_bias, const float* sel_bias, float* logits, int32_t* topk_ids,
              float* topk_w, void* stream) {
  int st = check_route_shape(T, E, k, mode);
  if (st) return st;
  const bool given_logits = (x == nullptr && w_router == nullptr);
  if (!given_logits) {
    if (!x || !w_router || !valid_dt(dt)) return MOE_ERR_INVALID_ARG;
    if ((st = check_hidden(H))) return st;
    if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID_ARG;
    if (logit_bias && !aligned16(logit_bias)) return MOE_ERR_INVALID_ARG;
  }
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w)) return MOE_ERR_INVALID_ARG;
  if (sel_bias && !aligned16(sel_bias)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!given_logits) MOE_TRY(launch_router_logits(x, w_router, dt, T, H, E, logit_bias, logits, s));
  GateTileArgs a{};
  a.logits = logits;
  a.sel_bias = sel_bias;
  a.ids_out = topk_ids;
  a.w_out = topk_w;
  a.T = T; a.E = E; a.k = k; a.mode = mode;
  a.do_gate = 1; a.do_permute = 0;
  a.e_begin = 0; a.e_end = E;
  a.capacity = INT_MAX;
  return hip_status(launch_gate_tiles(a, cdiv(T, TOK_TILE), s));
}

static size_t permute_ws_base(int T, int k, int E_loc) {
  const int n_tt = cdiv(T, TOK_TILE);
  return align_up((size_t)n_tt * E_loc * 4) * 2 + align_up((size_t)T * k * 4);
}

size_t moe_permute_workspace_size(int T, int k, int E_loc) {
  if (T < 0 || k < 1 || E_loc < 1 || !fits_int(T, k)) return 0;
  return permute_ws_base(T, k, E_loc) + (validate_on() ? VALIDATE_BYTES : 0);
}

// Rows of the padded capacity layout (E_loc * capacity), or -1 if that does
// not fit an int.
static int padded_rows(int E_loc, int capacity) {
  const long long n = (long long)E_loc * capacity;
  return n > INT_MAX ? -1 : (int)n;
}

static int permute_impl(const int32_t* topk_ids, int T, int k, int E, int e_begin, int e_end,
                        int capacity, int padded, const void* x, int H, int dt, int32_t* counts,
                        int32_t* offsets, int32_t* src_token, int32_t* dst_row, void* x_perm,
                        int32_t* dropped, void* ws, size_t ws_bytes, void* stream) {
  if (capacity < 0 || (padded != 0 && padded != 1)) return MOE_ERR_INVALID_ARG;
  if (dropped && !aligned16(dropped)) return MOE_ERR_INVALID_ARG;
  int st = check_route_shape(T, E, k, 0);
  if (st) return st;
  if (e_begin < 0 || e_end > E || e_begin >= e_end) return MOE_ERR_INVALID_ARG;
  const int E_loc = e_end - e_begin;
  const int pad_rows = padded ? padded_rows(E_loc, capacity) : 0;
  if (pad_rows < 0) return MOE_ERR_INVALID_ARG;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !src_token || !dst_row)) return MOE_ERR_INVALID_ARG;
  if (pad_rows > 0 && !src_token) return MOE_ERR_INVALID_ARG;
  {
    const void* ptrs[] = {topk_ids, counts, offsets, src_token, dst_row};
    for (const void* p : ptrs)
      if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  }
  if (x) {
    if (!valid_dt(dt) || !x_perm) return MOE_ERR_INVALID_ARG;
    if ((st = check_hidden(H))) return st;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  }
  const size_t need = moe_permute_workspace_size(T, k, E_loc);
  const bool check = validate_on();      // the result word needs the workspace
  // the padded layout's offsets come from the scan kernel
  const bool single = T <= TOK_TILE && !padded;
  if ((!single || check) && need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n_tt = cdiv(T, TOK_TILE);
  Carver c(ws);
  int32_t* tile_counts = c.take<int32_t>((size_t)n_tt * E_loc * 4);
  int32_t* tile_base = c.take<int32_t>((size_t)n_tt * E_loc * 4);
  int32_t* rank = c.take<int32_t>((size_t)T * k * 4);

  GateTileArgs a{};
  a.ids_in = topk_ids;
  a.T = T; a.E = E; a.k = k; a.mode = 0;
  a.do_gate = 0; a.do_permute = 1;
  a.e_begin = e_begin; a.e_end = e_end;
  a.tile_counts = tile_counts; a.rank_out = rank;
  a.single = single ? 1 : 0;
  a.counts = counts; a.offsets = offsets; a.src_token = src_token; a.dst_row = dst_row;
  a.BM = 16; a.tile_map = nullptr; a.n_tiles = nullptr;
  a.capacity = capacity; a.dropped = dropped;
  // with no tokens the multi-tile path has no tile to count (its workspace
  // is empty); the scan still writes counts, offsets and the dropped word
  if (single || T > 0) MOE_TRY(launch_gate_tiles(a, n_tt, s));
  if (!single) {
    MOE_TRY(launch_permute_scan(tile_counts, n_tt, E_loc, tile_base, counts, offsets, 16, 0, 0,
                                nullptr, nullptr, capacity, padded, dropped, s));
    MOE_TRY(launch_permute_scatter(topk_ids, rank, tile_base, offsets, T, k, e_begin, e_end,
                                   capacity, dst_row, src_token, s));
    if (padded) MOE_TRY(launch_pad_rows(counts, E_loc, capacity, src_token, s));
  }
  const int gather_rows = padded ? pad_rows : T * (k < E_loc ? k : E_loc);
  if (x && gather_rows > 0)
    MOE_TRY(launch_gather_rows(x, src_token, offsets, E_loc, gather_rows, H, elt_bytes(dt), x_perm,
                               s));
  if (check)
    return check_meta(topk_ids, T * k, E, e_begin, e_end, counts, offsets, capacity, padded,
                      dropped,
                      reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                                 permute_ws_base(T, k, E_loc)),
                      s);
  return MOE_OK;
}

int moe_permute(const int32_t* topk_ids, int T, int k, int E, int e_begin, int e_end,
                const void* x, int H, int dt, int32_t* counts, int32_t* offsets,
                int32_t* src_token, int32_t* dst_row, void* x_perm, void* ws, size_t ws_bytes,
                void* stream) {
  return permute_impl(topk_ids, T, k, E, e_begin, e_end, INT_MAX, 0, x, H, dt, counts, offsets,
                      src_token, dst_row, x_perm, nullptr, ws, ws_bytes, stream);
}

int moe_permute_capacity(const int32_t* topk_ids, int T, int k, int E, int e_begin, int e_end,
                         int capacity, int padded, const void* x, int H, int dt, int32_t* counts,
                         int32_t* offsets, int32_t* src_token, int32_t* dst_row, void* x_perm,
                         int32_t* dropped, void* ws, size_t ws_bytes, void* stream) {
  return permute_impl(topk_ids, T, k, E, e_begin, e_end, capacity, padded, x, H, dt, counts,
                      offsets, src_token, dst_row, x_perm, dropped, ws, ws_bytes, stream);
}

size_t moe_grouped_ffn_workspace_size(int max_rows, int E_loc, int H, int I_loc, int dt) {
  if (max_rows < 0 || E_loc < 1 || H <= 0 || I_loc <= 0 || !valid_dt(dt)) return 0;
  const int BM = ffn_row_tile(dt, cdiv(max_rows, E_loc), H, I_loc,
                              max_rows < E_loc ? max_rows : E_loc);
  const int mt = max_tiles_for(max_rows, E_loc, BM);
  return align_up((size_t)max_rows * I_loc * elt_bytes(dt)) + align_up((size_t)mt * sizeof(int4)) +
         align_up(4);
}

int moe_grouped_ffn(const void* x_perm, const void* x, const int32_t* src_token,
                    const int32_t* offsets, int E_loc, int max_rows, int H, int I_loc,
                    const void* w13, const void* w2, int dt, void* y_perm, int y_dt, void* ws,
                    size_t ws_bytes, void* stream) {
  if (!valid_dt(dt) || !valid_dt(y_dt) || E_loc < 1 || max_rows < 0 || I_loc <= 0)
    return MOE_ERR_INVALID_ARG;
  int st = check_hidden(H);
  if (st) return st;
  if (I_loc % 32 || E_loc > 1024) return MOE_ERR_UNSUPPORTED;
  if (dt == MOE_F32 && y_dt != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (!offsets || !w13 || !w2 || !y_perm) return MOE_ERR_INVALID_ARG;
  if (!x_perm && (!x || !src_token)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {x_perm, x, src_token, offsets, w13, w2, y_perm, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  if (max_rows == 0) return MOE_OK;
  const size_t need = moe_grouped_ffn_workspace_size(max_rows, E_loc, H, I_loc, dt);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  const int BM = ffn_row_tile(dt, cdiv(max_rows, E_loc), H, I_loc,
                              max_rows < E_loc ? max_rows : E_loc);
  const int mt = max_tiles_for(max_rows, E_loc, BM);
  Carver c(ws);
  void* h = c.take<char>((size_t)max_rows * I_loc * elt_bytes(dt));
  int4* tile_map = c.take<int4>((size_t)mt * sizeof(int4));
  int32_t* n_tiles = c.take<int32_t>(4);
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(launch_tile_map_from_offsets(offsets, E_loc, BM, max_rows, mt, tile_map, n_tiles, s));
  FfnArgs a{};
  a.x = x_perm ? x_perm : x;
  a.src_token = x_perm ? nullptr : src_token;
  a.tile_map = tile_map; a.n_tiles = n_tiles; a.M_dense = 0; a.max_tiles = mt;
  a.mean_rows = cdiv(max_rows, E_loc);
  a.H = H; a.I_loc = I_loc; a.w13 = w13; a.w2 = w2; a.h = h; a.y = y_perm;
  a.dt = dt; a.y_dt = y_dt;
  a.x_rows = x_perm ? max_rows : 0;     // the token count behind src_token is not passed
  a.h_rows = max_rows;
  return hip_status(launch_grouped_ffn(a, BM, s));
}

int moe_combine(const void* y_perm, int y_perm_dt, const int32_t* dst_row, const float* topk_w,
                int T, int k, int H, const void* y_shared, void* y, int dt, void* stream) {
  if (!valid_dt(dt) || !valid_dt(y_perm_dt) || T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
  int st = check_hidden(H);
  if (st) return st;
  if (k > KMAX || !fits_int(T, k)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_perm || !dst_row || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {y_perm, dst_row, topk_w, y, y_shared};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(y_perm, y_perm_dt, dst_row, topk_w, T, k, H, y_shared, y, dt,
                                   static_cast<hipStream_t>(stream)));
}

size_t moe_pack_workspace_size(int T, int k, int P) {
  if (T < 0 || k < 1 || P < 1 || P > 64 || !fits_int(T, k)) return 0;
  const size_t n_tiles = (size_t)cdiv(T, 64);
  return align_up((size_t)T * 8) + 2 * align_up(n_tiles * P * 4);
}

int moe_pack_by_rank(const int32_t* topk_ids, const float* topk_w, int T, int k, int E, int P,
                     const void* x, int H, int dt, int32_t* send_counts, int32_t* send_offsets,
                     int32_t* send_token, int32_t* send_row, int32_t* send_ids, float* send_w,
                     void* x_send, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || E < 1 || k > E || P < 1) return MOE_ERR_INVALID_ARG;
  if (E % P) return MOE_ERR_INVALID_ARG;
  if (k > KMAX || E > 1024 || P > 64 || !fits_int(T, k)) return MOE_ERR_UNSUPPORTED;
  if (!send_counts || !send_offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !send_token || !send_row)) return MOE_ERR_INVALID_ARG;
  if (send_w && !topk_w) return MOE_ERR_INVALID_ARG;
  int st = MOE_OK;
  if (x) {
    if (!valid_dt(dt) || !x_send) return MOE_ERR_INVALID_ARG;
    if ((st = check_hidden(H))) return st;
  }
  {
    const void* ptrs[] = {topk_ids, topk_w, send_counts, send_offsets, send_token, send_row,
                          send_ids, send_w, x, x_send, ws};
    for (const void* p : ptrs)
      if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  }
  const bool single = T <= 64;
  if (!single && (!ws || ws_bytes < moe_pack_workspace_size(T, k, P))) return MOE_ERR_WORKSPACE;
  PackArgs a{};
  a.ids = topk_ids; a.w = topk_w;
  a.T = T; a.k = k; a.E = E; a.P = P; a.per = E / P;
  a.send_counts = send_counts; a.send_offsets = send_offsets; a.send_token = send_token;
  a.send_row = send_row; a.send_ids = send_ids; a.send_w = send_w;
  if (!single) {
    Carver c(ws);
    const size_t n_tiles = (size_t)cdiv(T, 64);
    a.masks = c.take<unsigned long long>((size_t)T * 8);
    a.tile_counts = c.take<int32_t>(n_tiles * P * 4);
    a.tile_base = c.take<int32_t>(n_tiles * P * 4);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    // zero counts and offsets, as for moe_permute
    a.T = 0;
    return hip_status(launch_pack_by_rank(a, nullptr, 0, 0, nullptr, 0, s));
  }
  const int max_rows = T * (k < P ? k : P);
  return hip_status(launch_pack_by_rank(a, x, H, elt_bytes(dt), x_send, max_rows, s));
}

int moe_unpack_sum(const void* y_ret, int y_ret_dt, const int32_t* send_row, int T, int k, int H,
                   void* y, int dt, void* stream) {
  if (!valid_dt(dt) || !valid_dt(y_ret_dt) || T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
  int st = check_hidden(H);
  if (st) return st;
  if (k > KMAX || !fits_int(T, k)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_ret || !send_row || !y) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {y_ret, send_row, y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARG;
  return hip_status(
      launch_unpack_sum(y_ret, y_ret_dt, send_row, T, k, H, y, dt, static_cast<hipStream_t>(stream)));
}

static int reshard_call(bool pack, const void* w13_src, const void* w2_src, int n, int I, int H,
                        int P, int dt, void* w13_dst, void* w2_dst, void* stream) {
  if (!valid_dt(dt) || n < 1 || I <= 0 || P < 1 || H <= 0) return MOE_ERR_INVALID_ARG;
  if (I % P) return MOE_ERR_INVALID_ARG;
  if (!w13_src != !w13_dst || !w2_src != !w2_dst) return MOE_ERR_INVALID_ARG;
  if (!w13_src && !w2_src) return MOE_ERR_INVALID_ARG;
  const int elt = elt_bytes(dt);
  if ((H * elt) % 16 || ((I / P) * elt) % 16) return MOE_ERR_UNSUPPORTED;
  const long long v13 = (long long)n * 2 * I * H * elt / 16;
  const long long v2 = (long long)n * H * I * elt / 16;
  if (v13 >= (1ll << 31) || v2 >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  const void* ptrs[] = {w13_src, w2_src, w13_dst, w2_dst};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_reshard(pack, w13_src, w2_src, n, I, H, P, elt, w13_dst, w2_dst,
                                   static_cast<hipStream_t>(stream)));
}

int moe_reshard_ep_to_tp_pack(const void* w13_ep, const void* w2_ep, int E_rank, int I, int H,
                              int P, int dt, void* w13_send, void* w2_send, void* stream) {
  return reshard_call(true, w13_ep, w2_ep, E_rank, I, H, P, dt, w13_send, w2_send, stream);
}

int moe_reshard_tp_to_ep_interleave(const void* w13_recv, const void* w2_recv, int E_rank, int I,
                                    int H, int P, int dt, void* w13_ep, void* w2_ep,
                                    void* stream) {
  return reshard_call(false, w13_recv, w2_recv, E_rank, I, H, P, dt, w13_ep, w2_ep, stream);
}

int moe_layer_status(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || !aligned16(ws) || ws_bytes < (size_t)DECODE_SYNC_BYTES) return MOE_ERR_INVALID_ARG;
  return take_wait_word(static_cast<int*>(ws), static_cast<hipStream_t>(stream));
}

size_t moe_layer_workspace_size(const moe_layer_desc* d, int T_max) {
  if (check_desc(d) != MOE_OK || T_max < 0 || !fits_int(T_max, d->E)) return 0;
  return layer_layout(d, T_max, nullptr, nullptr);
}

int moe_layer_decode(const moe_layer_desc* d, int T, const void* x, void* y, void* ws,
                     size_t ws_bytes, moe_debug_out* dbg, void* stream) {
  int st = check_layer_call(d, T, x, y, ws, ws_bytes, dbg);
  if (st || T == 0) return st;
  if (!decode_shape_ok(d, T)) return MOE_ERR_UNSUPPORTED;
  LayerWs l;
  layer_layout(d, T, ws, &l);
  return run_decode(d, T, x, y, l, dbg, static_cast<hipStream_t>(stream));
}

int moe_layer_path(const moe_layer_desc* d, int T) {
  const int st = check_desc(d);
  if (st) return -st;
  if (T < 0) return -MOE_ERR_INVALID_ARG;
  if (!fits_int(T, d->E)) return -MOE_ERR_UNSUPPORTED;
  return (T > 0 && decode_shape_ok(d, T) && decode_preferred(d, T)) ? 1 : 0;
}

int moe_layer(const moe_layer_desc* d, int T, const void* x, void* y, void* ws, size_t ws_bytes,
              moe_debug_out* dbg, void* stream) {
  if (moe_layer_path(d, T) == 1) return moe_layer_decode(d, T, x, y, ws, ws_bytes, dbg, stream);
  return moe_layer_staged(d, T, x, y, ws, ws_bytes, dbg, stream);
}

int moe_layer_static(const moe_layer_desc* d, int T, const void* x, void* y, moe_debug_out* dbg,
                     void* stream) {
  const int st = check_desc(d);
  if (st) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (!fits_int(T, d->E)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (layer_layout(d, T, nullptr, nullptr) > (size_t)MOE_STATIC_SCRATCH_BYTES)
    return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const int sst = static_scratch(&ws, static_cast<hipStream_t>(stream));
  if (sst) return sst;
  return moe_layer(d, T, x, y, ws, MOE_STATIC_SCRATCH_BYTES, dbg, stream);
}

static int layer_staged_impl(const moe_layer_desc* d, int T, const void* x, void* y, void* ws,
                             size_t ws_bytes, moe_debug_out* dbg, int capacity, int padded,
                             int32_t* dropped, void* stream) {
  // padded: expert blocks of `capacity` rows in h and y_perm (pad_rows >= 0);
  // a missing desc is reported by check_layer_call
  const int pad_rows = padded && d ? padded_rows(d->e_end - d->e_begin, capacity) : -1;
  int st = check_layer_call(d, T, x, y, ws, ws_bytes, dbg, pad_rows);
  if (st || T == 0) return st;
  LayerWs l;
  layer_layout(d, T, ws, &l, pad_rows);
  if (dbg) {
    if (dbg->logits) l.logits = dbg->logits;
    if (dbg->topk_ids) l.ids = dbg->topk_ids;
    if (dbg->topk_w) l.w = dbg->topk_w;
    if (dbg->counts) l.counts = dbg->counts;
    if (dbg->offsets) l.offsets = dbg->offsets;
    if (dbg->src_token) l.src_token = dbg->src_token;
    if (dbg->dst_row) l.dst_row = dbg->dst_row;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E_loc = d->e_end - d->e_begin;
  auto mark = [&](int i) -> hipError_t {
    if (dbg && dbg->stage_events[i])
      return hipEventRecord(static_cast<hipEvent_t>(dbg->stage_events[i]), s);
    return hipSuccess;
  };

  MOE_TRY(mark(0));
  // a1: router logits
  MOE_TRY(launch_router_logits(x, d->w_router, d->dt, T, d->H, d->E, d->logit_bias, l.logits, s));
  // a2-a5: gating, histogram, prefix sum, permutation, GEMM tile map
  const bool single = T <= TOK_TILE && !padded;
  GateTileArgs a{};
  a.logits = l.logits; a.sel_bias = d->sel_bias;
  a.ids_out = l.ids; a.w_out = l.w;
  a.T = T; a.E = d->E; a.k = d->k; a.mode = d->mode;
  a.do_gate = 1; a.do_permute = 1;
  a.e_begin = d->e_begin; a.e_end = d->e_end;
  a.tile_counts = l.tile_counts; a.rank_out = l.rank;
  a.single = single ? 1 : 0;
  a.counts = l.counts; a.offsets = l.offsets; a.src_token = l.src_token; a.dst_row = l.dst_row;
  a.BM = l.BM; a.tile_map = l.tile_map; a.n_tiles = l.n_tiles;
  a.max_rows = l.max_rows; a.max_tiles = l.max_tiles;
  a.capacity = capacity; a.dropped = dropped;
  if (single && T >= GATE_SPLIT_MIN_T && E_loc <= 256) {
    // The k arg-max rounds of a whole tile on one CU are bound by its vector
    // ALUs (16 waves, four per SIMD): gate GATE_SPLIT_TPB tokens per block
    // over several CUs, then build the metadata from the chosen ids in a
    // one-block pass, as moe_permute does.
    GateTileArgs g = a;
    g.do_permute = 0;
    g.tok_per_block = GATE_SPLIT_TPB;
    MOE_TRY(launch_gate_tiles(g, cdiv(T, GATE_SPLIT_TPB), s));
    a.do_gate = 0;
    a.ids_in = l.ids;
    MOE_TRY(launch_gate_tiles(a, 1, s));
  } else {
    MOE_TRY(launch_gate_tiles(a, l.n_tt, s));
  }
  if (!single) {
    MOE_TRY(launch_permute_scan(l.tile_counts, l.n_tt, E_loc, l.tile_base, l.counts, l.offsets,
                                l.BM, l.max_rows, l.max_tiles, l.tile_map, l.n_tiles, capacity,
                                padded, dropped, s));
    MOE_TRY(launch_permute_scatter(l.ids, l.rank, l.tile_base, l.offsets, T, d->k, d->e_begin,
                                   d->e_end, capacity, l.dst_row, l.src_token, s));
    // the GEMMs never read padding rows; mark them only for a caller who asks
    if (padded && dbg && dbg->src_token)
      MOE_TRY(launch_pad_rows(l.counts, E_loc, capacity, l.src_token, s));
  }
  MOE_TRY(mark(1));
  // a6-a7: grouped SwiGLU GEMMs, gather fused into the first
  FfnArgs f{};
  f.x = x; f.src_token = l.src_token; f.tile_map = l.tile_map; f.n_tiles = l.n_tiles;
  f.M_dense = 0; f.max_tiles = l.max_tiles; f.mean_rows = mean_rows(T, d->k, d->E);
  f.H = d->H; f.I_loc = d->I_loc; f.w13 = d->w13; f.w2 = d->w2;
  f.h = l.h; f.y = l.y_perm; f.dt = d->dt; f.y_dt = d->dt;
  f.x_rows = T; f.h_rows = l.max_rows;
  // the launches: routed row tiles, and whether the shared expert's GEMMs
  // ride in the routed launches (a8: the shared expert over every token)
  const GemmPlan plan = plan_layer_gemms(d->dt, T, d->k, d->E, E_loc, d->H, d->I_loc,
                                         d->I_shared);
  if (plan.BM != l.BM) return MOE_ERR_HIP;   // the workspace's tile map was sized for l.BM
  // the down projection may walk the gate/up GEMM's tile map with a smaller
  // row tile of its own
  const int BM_dn = plan.BM_dn;
  FfnArgs fd = f;
  if (BM_dn != l.BM) fd.map_bm = l.BM;
  if (plan.dn == SHARE_NONE) fd.down_cols = plan.dn_cols;
  FfnArgs g{};
  const int BMs = plan.BMs;
  const bool share_up = plan.up != SHARE_NONE, share_dn = plan.dn != SHARE_NONE;
  FfnArgs g_up{}, g_dn{};
  int BMs_dn = plan.BMs_dn;
  if (d->I_shared > 0) {
    g.x = x; g.src_token = nullptr; g.tile_map = nullptr; g.n_tiles = nullptr;
    g.M_dense = T; g.max_tiles = cdiv(T, BMs); g.mean_rows = T;
    g.H = d->H; g.I_loc = d->I_shared; g.w13 = d->w13_shared; g.w2 = d->w2_shared;
    g.h = l.h_s; g.y = l.y_s; g.dt = d->dt; g.y_dt = d->dt;
    g.x_rows = T; g.h_rows = T;
    g_up = g;
    g_up.max_tiles = cdiv(T, plan.BMs_up);
    g_dn = g;
    g_dn.max_tiles = cdiv(T, BMs_dn);
  }
  f.gate_up_pack = plan.up_pack;
  MOE_TRY(launch_ffn_gate_up(f, l.BM, s, share_up ? &g_up : nullptr));
  MOE_TRY(mark(2));
  // the shared expert's h must be complete before a launch that reads it
  if (d->I_shared > 0 && !share_up && share_dn) MOE_TRY(launch_ffn_gate_up(g, BMs, s));
  MOE_TRY(launch_ffn_down(fd, BM_dn, s, share_dn ? &g_dn : nullptr));
  MOE_TRY(mark(3));
  if (d->I_shared > 0 && !share_up && !share_dn) MOE_TRY(launch_grouped_ffn(g, BMs, s));
  else if (d->I_shared > 0 && !share_dn) MOE_TRY(launch_ffn_down(g_dn, BMs_dn, s));
  MOE_TRY(mark(4));
  // a9: inverse permutation + weighted sum (+ shared expert)
  MOE_TRY(launch_combine(l.y_perm, d->dt, l.dst_row, l.w, T, d->k, d->H,
                         d->I_shared > 0 ? l.y_s : nullptr, y, d->dt, s));
  MOE_TRY(mark(5));
  if (validate_on())
    return check_meta(l.ids, T * d->k, d->E, d->e_begin, d->e_end, l.counts, l.offsets, capacity,
                      padded, dropped, l.sync + LAYER_VALIDATE_INT, s);
  return MOE_OK;
}

int moe_layer_staged(const moe_layer_desc* d, int T, const void* x, void* y, void* ws,
                     size_t ws_bytes, moe_debug_out* dbg, void* stream) {
  return layer_staged_impl(d, T, x, y, ws, ws_bytes, dbg, INT_MAX, 0, nullptr, stream);
}

size_t moe_layer_capacity_workspace_size(const moe_layer_desc* d, int T_max, int capacity,
                                         int padded) {
  if (check_desc(d) != MOE_OK || T_max < 0 || capacity < 0 || (padded != 0 && padded != 1))
    return 0;
  if (!fits_int(T_max, d->E)) return 0;
  if (!padded) return layer_layout(d, T_max, nullptr, nullptr);
  const int pad_rows = padded_rows(d->e_end - d->e_begin, capacity);
  if (pad_rows < 0) return 0;
  return layer_layout(d, T_max, nullptr, nullptr, pad_rows);
}

int moe_layer_capacity(const moe_layer_desc* d, int T, int capacity, int padded, const void* x,
                       void* y, void* ws, size_t ws_bytes, moe_debug_out* dbg, int32_t* dropped,
                       void* stream) {
  if (capacity < 0 || (padded != 0 && padded != 1)) return MOE_ERR_INVALID_ARG;
  if (dropped && !aligned16(dropped)) return MOE_ERR_INVALID_ARG;
  if (padded && d && d->e_end > d->e_begin && padded_rows(d->e_end - d->e_begin, capacity) < 0)
    return MOE_ERR_INVALID_ARG;
  return layer_staged_impl(d, T, x, y, ws, ws_bytes, dbg, capacity, padded, dropped, stream);
}

}  // extern "C"
