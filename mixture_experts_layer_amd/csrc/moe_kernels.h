// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <stdint.h>

namespace moe {

// Raise a kernel's dynamic-LDS limit on the current device, once per
// (kernel, device): the attribute belongs to the device, so a process that
// drives several GPUs sets it on each.  `done` holds one bit per device id
// below 64 (higher ids set it on every launch); a lost race only repeats the
// call.
inline hipError_t ensure_lds_limit(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (err == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return err;
}

constexpr int TOK_TILE = 64;   // tokens per routing-metadata tile
constexpr int KMAX = 32;       // largest supported top-k

struct GateTileArgs {
  // gating
  const float* logits;      // [T][E]
  const float* sel_bias;    // [E] or null (mode 3)
  const int32_t* ids_in;    // [T][k] when do_gate == 0
  int32_t* ids_out;         // [T][k]
  float* w_out;             // [T][k]
  int T, E, k, mode;
  int do_gate, do_permute;
  int e_begin, e_end;
  // multi-tile outputs
  int32_t* tile_counts;     // [n_tiles_tok][E_loc]
  int32_t* rank_out;        // [T][k]
  // single-tile outputs
  int single;
  int32_t* counts;          // [E_loc]
  int32_t* offsets;         // [E_loc + 1]
  int32_t* src_token;       // [T*k]
  int32_t* dst_row;         // [T][k]
  int BM;                   // GEMM row tile for the tile map
  int max_rows, max_tiles;  // bounds of the GEMM buffers the map drives
  int4* tile_map;           // [max_tiles] or null
  int32_t* n_tiles;         // [1]
  int capacity;             // pairs kept per expert (INT_MAX: dropless)
  int32_t* dropped;         // [1] or null: local pairs dropped by the capacity
  // gating only (do_permute == 0): tokens per block, 0 = TOK_TILE
  int tok_per_block;
};

hipError_t launch_router_logits(const void* x, const void* wr, int dt, int T, int H, int E,
                                const float* bias, float* logits, hipStream_t st);
hipError_t launch_gate_tiles(const GateTileArgs& a, int n_tiles_tok, hipStream_t st);

// Multi-tile permutation: per-expert scan over tiles, then scatter.
// capacity: pairs kept per expert, the first in token order (INT_MAX:
// dropless); dropped (nullable) receives the number of local pairs dropped.
hipError_t launch_permute_scan(const int32_t* tile_counts, int n_tiles_tok, int E_loc,
                               int32_t* tile_base, int32_t* counts, int32_t* offsets, int BM,
                               int max_rows, int max_tiles, int4* tile_map, int32_t* n_tiles,
                               int capacity, int padded, int32_t* dropped, hipStream_t st);
// Padded capacity layout: src_token = -1 on every expert block's rows past its
// kept pairs (E_loc * capacity rows).
hipError_t launch_pad_rows(const int32_t* counts, int E_loc, int capacity, int32_t* src_token,
                           hipStream_t st);
hipError_t launch_permute_scatter(const int32_t* ids, const int32_t* rank, const int32_t* tile_base,
                                  const int32_t* offsets, int T, int k, int e_begin, int e_end,
                                  int capacity, int32_t* dst_row, int32_t* src_token,
                                  hipStream_t st);
hipError_t launch_gather_rows(const void* x, const int32_t* src_token, const int32_t* offsets,
                              int E_loc, int max_rows, int H, int elt_bytes, void* x_perm,
                              hipStream_t st);
// Routing-metadata checks into err[0] (0: consistent); see permute.hip.
hipError_t launch_validate_meta(const int32_t* ids, int npair, int E, int e_begin, int e_end,
                                const int32_t* counts, const int32_t* offsets, int capacity,
                                int padded, const int32_t* dropped, int32_t* err, hipStream_t st);
hipError_t launch_tile_map_from_offsets(const int32_t* offsets, int E_loc, int BM, int max_rows,
                                        int max_tiles, int4* tile_map, int32_t* n_tiles,
                                        hipStream_t st);

// Grouped expert GEMMs.
struct FfnArgs {
  const void* x;            // activations: x_perm rows, or token rows gathered via src_token
  const int32_t* src_token; // null: row r reads x row r
  const int4* tile_map;     // null: dense rows [0, M) of expert 0 in BM tiles
  const int32_t* n_tiles;
  int M_dense;              // rows when tile_map is null
  int max_tiles;
  int mean_rows;            // expected rows per expert (block-order heuristics)
  int H, I_loc;
  const void* w13;          // [E_loc][2*I_loc][H]
  const void* w2;           // [E_loc][H][I_loc]
  void* h;                  // [rows][I_loc], dtype dt
  void* y;                  // [rows][H], dtype y_dt
  int dt, y_dt;
  long long x_rows;         // rows of x (0: not known)
  long long h_rows;         // rows of h
  int map_bm;               // rows per tile-map entry when it differs from the
                            // launch's row tile (direct kernel only); 0: the same
  int down_cols;            // output columns per block of the LDS-tiled down
                            // projection with 128-row tiles: 128, or 0 for 256
  int gate_up_pack;         // 1: a 16-row direct gate/up launch takes 8-column
                            // tiles (8 gate + 8 up rows in one MFMA operand)
};
// Row tile of the expert GEMMs: 16/32/64 (direct kernel) or 128/256 (LDS-
// tiled kernel), from the expected rows per expert and the number of experts
// the rows spread over.
int ffn_row_tile(int dt, int mean_rows, int H, int I_loc, int experts);
// `also` (optional): a second problem run in the same launch, for which
// ffn_can_share_gemm(a, BM, *also, BM, ...) holds -- the shared expert beside
// the routed experts at a few tokens, where its own launches would leave most
// CUs idle.
hipError_t launch_ffn_gate_up(const FfnArgs& a, int BM, hipStream_t st,
                              const FfnArgs* also = nullptr);
hipError_t launch_ffn_down(const FfnArgs& a, int BM, hipStream_t st, const FfnArgs* also = nullptr);
// Row tile of the down projection after a gate/up GEMM with row tile BM
// over the same tile map: BM, except at about one row per expert with a
// long contraction, where the gate/up GEMM takes LDS tiles and the down
// projection's short one streams faster in the direct kernel (16-row tiles
// walking the gate/up GEMM's map: FfnArgs::map_bm = BM).
int ffn_down_row_tile(int dt, int mean_rows, int H, int I_loc, int BM);
// Output columns per block of the routed down projection when it runs 128-row
// LDS tiles (FfnArgs::down_cols): 128 where 256-column tiles would leave CUs
// idle (few experts, one row tile each), else 0 (256 columns).  experts: the
// experts the rows spread over.
int ffn_down_cols(int dt, int BM_dn, int mean_rows, int experts, int H);
// FfnArgs::gate_up_pack of the routed gate/up GEMM: 1 where its 16-row direct
// tiles of 16 columns would give the CUs fewer than three blocks each on
// average, so that whole blocks leave some CUs a third more bytes than
// others; 8-column tiles halve that step.
int ffn_gate_up_pack(int dt, int BM, int T, int k, int E, int E_loc, int I_loc);
// Whether b can ride in a's launch of one GEMM (gate_up: the gate/up GEMM,
// else the down projection): both bf16 with one row tile and the same kernel
// configuration (tile shape, or waves per block of the direct kernel).
bool ffn_can_share_gemm(const FfnArgs& a, int BM, const FfnArgs& b, int b_BM, bool gate_up);
// Blocks of a's gate/up launch with row tile BM (a.max_tiles row tiles).
long long ffn_gate_up_blocks(const FfnArgs& a, int BM);
hipError_t launch_grouped_ffn(const FfnArgs& a, int BM, hipStream_t st);

// The expert-GEMM launches of one staged layer call: the routed row tiles and
// how the shared expert's two GEMMs run.  A shared GEMM either rides in the
// routed launch (SHARE_OWN_TILE: its own row tile is the routed one's
// configuration; SHARE_ROUTED_TILE: its own tile would give it fewer blocks
// than there are CUs, so it takes the routed row tile) or has a launch of its
// own (SHARE_NONE).
enum SharedLaunch { SHARE_NONE = 0, SHARE_OWN_TILE = 1, SHARE_ROUTED_TILE = 2 };
struct GemmPlan {
  int BM;         // routed gate/up row tile
  int BM_dn;      // routed down row tile (walks the gate/up tile map when != BM)
  int BMs;        // the shared expert's own row tile (0: no shared expert)
  int up, dn;     // SharedLaunch of the shared gate/up and down GEMMs
  int BMs_up;     // row tile the shared gate/up GEMM runs with
  int BMs_dn;     // row tile the shared down GEMM runs with
  int dn_cols;    // FfnArgs::down_cols of the routed down projection
  int up_pack;    // FfnArgs::gate_up_pack of the routed gate/up GEMM
};
GemmPlan plan_layer_gemms(int dt, int T, int k, int E, int E_loc, int H, int I_loc, int I_shared);

hipError_t launch_combine(const void* y_perm, int y_perm_dt, const int32_t* dst_row,
                          const float* w, int T, int k, int H, const void* y_shared, void* y,
                          int dt, hipStream_t st);

// Token copies packed by destination rank (dispatch.hip).
struct PackArgs {
  const int32_t* ids;       // [T][k]
  const float* w;           // [T][k] or null (when send_w is null)
  int T, k, E, P, per;      // per = E / P experts per rank
  int32_t* send_counts;     // [P]
  int32_t* send_offsets;    // [P + 1]
  int32_t* send_token;      // [rows]
  int32_t* send_row;        // [T][k]
  int32_t* send_ids;        // [rows][k] or null
  float* send_w;            // [rows][k] or null
  unsigned long long* masks;  // [T] (multi-tile path)
  int32_t* tile_counts;     // [n_tiles][P]
  int32_t* tile_base;       // [n_tiles][P]
};
hipError_t launch_pack_by_rank(const PackArgs& a, const void* x, int H, int elt_bytes, void* x_send,
                               int max_rows, hipStream_t st);
hipError_t launch_unpack_sum(const void* y_ret, int y_ret_dt, const int32_t* send_row, int T, int k,
                             int H, void* y, int dt, hipStream_t st);

// EP <-> TP weight reshard, local halves (reshard.hip).  pack: EP weights ->
// per-peer chunks; otherwise per-peer chunks -> EP weights.  Either pair of
// pointers may be null.
hipError_t launch_reshard(bool pack, const void* w13_src, const void* w2_src, int n, int I, int H,
                          int P, int elt_bytes, void* w13_dst, void* w2_dst, hipStream_t st);

// Single-launch decode path (decode.hip).
constexpr int DECODE_MAX_T = 64;         // tokens: one 64-bit mask per expert
constexpr int DECODE_MAX_E = 256;        // E and E_loc
constexpr int DECODE_MAX_K = 16;
constexpr int DECODE_MAX_PAIRS = 512;    // T * k
constexpr int DECODE_MAX_BLOCKS = 1024;  // grid bound (workgroups resident at once)
// sync block at the start of the workspace: a 4 KiB header, then one
// 128-byte go-flag line per workgroup
constexpr int DECODE_SYNC_BYTES = 4096 + DECODE_MAX_BLOCKS * 128;
constexpr int DECODE_ERR_INT = 1;        // int index of the wait error word in the sync block

struct DecodeLaunch {
  const void* x;
  const void* w_router;
  const float* logit_bias;
  const float* sel_bias;
  const void* w13;
  const void* w2;
  const void* w13_shared;
  const void* w2_shared;
  void* y;
  float* logits;            // [T][E]
  void* h;                  // [T*min(k, E_loc)][I_loc]
  void* h_shared;           // [T][I_shared] or null
  int* sync;                // DECODE_SYNC_BYTES, zeroed before first use
  int32_t* ids_out;         // optional copies (may be null)
  float* w_out;
  int32_t* counts_out;
  int32_t* offsets_out;
  int32_t* src_out;
  int32_t* dst_out;
  int T, H, E, k, mode, I_loc, I_shared, e_begin, e_end;
};
bool decode_supported(int dt, int T, int E, int E_loc, int k, int H, int I, int Is);
hipError_t launch_decode(const DecodeLaunch& d, hipStream_t st);

}  // namespace moe
