/*
 * moe.h -- C ABI of a single-GPU Mixture-of-Experts layer forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes one GPU's share of an MoE layer: router scores, top-k
 * gating, per-expert histogram, prefix sum and permutation of token copies,
 * grouped SwiGLU expert GEMMs, and the inverse permutation with the
 * gate-weighted combine.  Passages cited below:
 *
 *   [Moebius notes]  Zhongzhu Zhou, reading notes "Moebius：为 MoE 大模型推理服务
 *                    实现无缝运行时并行策略切换" (zhongzhuzhou.org).
 *   [MoE guide]      "MoE 推理优化全景指南" (charlestar.github.io).
 *   [Moebius paper]  "Moebius: Serving Mixture-of-Expert Models with Seamless
 *                    Runtime Parallelism Switch".
 *   [CS349D L8]      "Lecture 8 · 混合专家模型的推理" (CS349D notes).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named x, w_*, y*, logits, topk_*, counts, offsets, src_token,
 *   dst_row, ws are DEVICE pointers; the caller owns every buffer.  The
 *   library never allocates or frees memory and keeps no state of its own
 *   between calls (the layer workspace's synchronisation block, below, lives
 *   in the caller's buffer).
 * - Every device pointer must be 16-byte aligned.  Matrices are row-major with
 *   the contraction (K) dimension contiguous:
 *     x[T][H], w_router[E][H], w13[e][2*I_loc][H], w2[e][H][I_loc].
 *   In w13, rows [0, I_loc) are the gate projection and rows [I_loc, 2*I_loc)
 *   the up projection ([Moebius paper] section 3.1 stacks the two; the order
 *   is this library's convention).  The expert MLP is
 *     y = W2 * (SiLU(W_gate x) * (W_up x)),  SiLU(z) = z / (1 + exp(-z)).
 * - `stream` is a hipStream_t (NULL = the null stream).  Calls are enqueued
 *   on it asynchronously; no call copies between host and device or
 *   synchronises (except in the MOE_VALIDATE=1 mode below), so every call
 *   may be captured in a HIP graph.
 * - Arguments are checked on the host before anything is enqueued; a failed
 *   check returns an error and enqueues nothing.  A kernel launch failure
 *   returns MOE_ERR_HIP.  T = 0 is a successful no-op (moe_permute still
 *   writes zero counts and offsets).
 * - Shape limits: 1 <= k <= 32, k <= E <= 1024, H and I_loc multiples of 32.
 *   The device counts logits and token pairs in int: T * E (the layer,
 *   moe_route, moe_permute) and T * k (moe_combine, moe_pack_by_rank,
 *   moe_unpack_sum) must not exceed 2^31 - 1.  Other shapes return
 *   MOE_ERR_UNSUPPORTED; the size queries return 0 for them.
 * - Results are bitwise repeatable: no kernel uses atomics to combine
 *   floating-point values or to order rows (the decode path's atomics only
 *   count finished work).
 * - Inference is dropless: every (token, slot) pair routed to a local expert
 *   is computed ([CS349D L8] section 1.4), except through the explicit
 *   capacity entry points.
 * - Metadata checks ([MoE guide] section "Dispatch 并不是一次普通 all-to-all":
 *   counts and offsets must be exact, or rows are misrouted silently).  With
 *   MOE_VALIDATE=1 in the environment (read at every call), moe_permute,
 *   moe_permute_capacity and the layer entry points check on the device, after
 *   the metadata is built, that every id is in [0, E), that the offsets start
 *   at 0 and step by the counts (padded layout: i * capacity), that the counts
 *   add up to the local pairs (less the dropped ones) and stay within the
 *   capacity.  The result word is copied to the host and the call waits for
 *   its stream, then returns MOE_ERR_METADATA if a check failed (the call's
 *   outputs are written either way).  Such calls synchronise and cannot be
 *   captured in a graph.  The word lives in the caller's workspace: the
 *   permute workspace grows by 256 bytes in this mode (and is then needed at
 *   every T), the layer uses bytes 32..35 of its synchronisation block.
 * - Non-finite inputs are outside the contract.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null / misaligned pointer, negative or inconsistent size */
  MOE_ERR_UNSUPPORTED = 2,   /* valid but outside the shape / dtype / mode limits above */
  MOE_ERR_WORKSPACE = 3,     /* workspace pointer null or smaller than the size query */
  MOE_ERR_HIP = 4,           /* a HIP launch returned an error */
  MOE_ERR_METADATA = 5,      /* the metadata check of MOE_VALIDATE=1 failed (below) */
  MOE_ERR_WAIT = 6           /* a decode-path wait for another workgroup ran out; the call's
                                outputs are undefined (moe_layer_status, MOE_VALIDATE=1) */
} moe_status;

typedef enum {
  MOE_F32 = 0,               /* float32 */
  MOE_BF16 = 1               /* bfloat16; products accumulate in float32 */
} moe_dtype;

/* Gating variants, [CS349D L8] section 1.2. */
typedef enum {
  MOE_GATE_TOPK_SOFTMAX = 0,         /* softmax over the k selected logits (weights sum to 1)     */
  MOE_GATE_SOFTMAX_TOPK = 1,         /* softmax over all E, keep k, no renormalisation (sum < 1)   */
  MOE_GATE_SOFTMAX_TOPK_RENORM = 2,  /* softmax over all E, keep k, divide by their sum            */
  MOE_GATE_SIGMOID_BIAS_RENORM = 3   /* select on logit + sel_bias, weight sigmoid(logit) / sum    */
} moe_gating;

/* ABI version of the loaded library (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static description of a status code; never NULL. */
const char* moe_status_str(int status);

/* SHA-256 (hex) of the sources and compile flags the library was built from,
 * or "unstamped".  The Python binding refuses a library whose stamp differs
 * from the sources beside it, so a stale binary is never run. */
const char* moe_source_sha256(void);

/*
 * moe_route -- router scores and top-k gating.
 *   [MoE guide] section "从 Dense FFN 到专家集合" (scores s = W_r x, top-k,
 *   weighted sum); [CS349D L8] section 1.2 (gating variants, noise off at
 *   inference).
 *
 *   logits[t][e] = sum_h x[t][h] * w_router[e][h] + logit_bias[e]   (float32)
 *   If x == NULL and w_router == NULL, `logits` is an INPUT [T][E] and only
 *   the gating runs on it (dt, H, logit_bias are then ignored).
 *   Selection key: logits (modes 0-2) or logits + sel_bias, added in float32
 *   (mode 3).  topk_ids[t][0..k) are the k largest keys ordered by key
 *   descending, equal keys broken towards the lower expert id.
 *   topk_w[t][j] is the gate weight of topk_ids[t][j] per `mode`.
 *
 *   x[T][H], w_router[E][H]: dtype `dt`.  logit_bias[E], sel_bias[E]: float32
 *   or NULL (sel_bias is used by mode 3 only).  Outputs: logits[T][E] float32,
 *   topk_ids[T][k] int32, topk_w[T][k] float32.
 */
int moe_route(const void* x, const void* w_router, int dt, int T, int H, int E, int k,
              int mode, const float* logit_bias, const float* sel_bias,
              float* logits, int32_t* topk_ids, float* topk_w, void* stream);

/*
 * moe_permute -- histogram, prefix sum and stable permutation of token copies.
 *   [MoE guide] section "Dispatch 并不是一次普通 all-to-all" (histogram ->
 *   prefix sum -> permute, e.g. ids [3,1,3,0,6] -> [t3][t1][t0,t2][t4]).
 *
 *   Local experts are [e_begin, e_end), E_loc = e_end - e_begin.
 *   counts[i]   = number of (t, j) with topk_ids[t][j] == e_begin + i.
 *   offsets[0] = 0, offsets[i+1] = offsets[i] + counts[i]  (E_loc + 1 values).
 *   The row of (t, j) is offsets[i] + #{t' < t : e_begin + i in topk_ids[t']}:
 *   rows of one expert keep ascending token order.  dst_row[t][j] is that row,
 *   or -1 when the expert is not local; src_token[row] = t.
 *   If x != NULL, x_perm[row][:] = x[src_token[row]][:] (dtype dt, H columns).
 *
 *   topk_ids[T][k] int32 with values in [0, E) and distinct within a token
 *   (as moe_route produces).  Outputs: counts[E_loc], offsets[E_loc+1],
 *   src_token[T*k] (first offsets[E_loc] entries written), dst_row[T][k]: int32
 *   (topk_ids, src_token and dst_row may be NULL when T = 0).
 *   ws: at least moe_permute_workspace_size(T, k, E_loc) bytes (may be NULL
 *   when T <= 64: a single tile needs no workspace; not with MOE_VALIDATE=1,
 *   whose result word is kept there).
 */
size_t moe_permute_workspace_size(int T, int k, int E_loc);
int moe_permute(const int32_t* topk_ids, int T, int k, int E, int e_begin, int e_end,
                const void* x, int H, int dt,
                int32_t* counts, int32_t* offsets, int32_t* src_token, int32_t* dst_row,
                void* x_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_permute_capacity -- moe_permute with a capacity of `capacity` (token,
 * slot) pairs per local expert.
 *   [MoE guide] section "Capacity、padding 与 token dropping" (C =
 *   ceil(capacity factor * N_a / E); assignments beyond C may be dropped);
 *   [CS349D L8] section 1.4 (a dropped assignment contributes nothing; the
 *   output then depends on the other tokens of the batch, which is why the
 *   default path here is dropless).
 *
 *   An expert keeps its first `capacity` pairs in token order; the others get
 *   dst_row -1 and no row.  counts[i] = kept pairs (<= capacity).  dropped[0]
 *   (int32, may be NULL) = the number of local pairs dropped.  capacity >= 0
 *   (INT_MAX with padded = 0: moe_permute itself).
 *
 *   padded = 0: offsets and src_token as in moe_permute over the kept pairs
 *   (at most min(T*k, E_loc*capacity) rows).
 *   padded = 1: the fixed-shape layout of the same section, every expert
 *   padded to `capacity` rows: offsets[i] = i * capacity, expert i's kept
 *   pairs fill rows i*capacity .. i*capacity + counts[i] - 1 in token order,
 *   and src_token = -1 on the rest of its block.  src_token (and x_perm, whose
 *   padding rows are zero) then hold E_loc * capacity rows, which must fit an
 *   int (else MOE_ERR_INVALID_ARG), and ws is needed for every T > 0.
 *   padded must be 0 or 1.  Other arguments and the workspace as for
 *   moe_permute.
 */
int moe_permute_capacity(const int32_t* topk_ids, int T, int k, int E, int e_begin, int e_end,
                         int capacity, int padded, const void* x, int H, int dt,
                         int32_t* counts, int32_t* offsets, int32_t* src_token, int32_t* dst_row,
                         void* x_perm, int32_t* dropped, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_ffn -- grouped SwiGLU expert MLPs over ragged row counts.
 *   [MoE guide] section "Expert GEMM 为什么经常不够大" (expert i computes
 *   [m_i, hidden] @ W_i in one schedule); [Moebius notes] eq. (2)-(4) and
 *   [Moebius paper] section 3.1 (W13 (E_loc, 2I, H), W2 (E_loc, H, I); the
 *   tensor-parallel share holds I/P of every expert).
 *
 *   For local expert i and every row r in [offsets[i], offsets[i+1]):
 *     a = x_perm[r]            if x_perm != NULL
 *       = x[src_token[r]]      otherwise (gather fused into the GEMM)
 *     g = w13[i][0:I_loc] a,  u = w13[i][I_loc:2I_loc] a,  h = SiLU(g) * u
 *     y_perm[r] = w2[i] h
 *   h is rounded to dtype `dt` between the two GEMMs.  offsets live on the
 *   device: no row count is read back to the host.
 *
 *   max_rows bounds offsets[E_loc] (grid sizing; T*k for a full layer).
 *   x_perm[max_rows][H] or x[*][H] + src_token[max_rows]; w13, w2: dtype dt;
 *   every row in an expert's range is computed, so for the padded layout of
 *   moe_permute_capacity pass its x_perm (padding rows zero, hence outputs
 *   zero); gathering from x, a source of -1 reads row 0 of x and that row's
 *   output is meaningless;
 *   y_perm[max_rows][H] of dtype y_dt.  ws: at least
 *   moe_grouped_ffn_workspace_size(...) bytes.
 */
size_t moe_grouped_ffn_workspace_size(int max_rows, int E_loc, int H, int I_loc, int dt);
int moe_grouped_ffn(const void* x_perm, const void* x, const int32_t* src_token,
                    const int32_t* offsets, int E_loc, int max_rows, int H, int I_loc,
                    const void* w13, const void* w2, int dt,
                    void* y_perm, int y_dt, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine -- inverse permutation with the gate-weighted sum.
 *   [MoE guide] section "Dispatch 并不是一次普通 all-to-all" (combine restores
 *   token order and applies the routing weights); [Moebius notes] eq. (1);
 *   [CS349D L8] section 1.2 (a shared expert every token passes through).
 *
 *   y[t] = sum_{j < k, dst_row[t][j] >= 0} topk_w[t][j] * y_perm[dst_row[t][j]]
 *          (+ y_shared[t] with weight 1 if y_shared != NULL),
 *   accumulated in float32 in slot order and rounded once to dtype dt.
 *   In the tensor-parallel view y is the rank's partial sum.
 *
 *   y_perm[*][H] dtype y_perm_dt; dst_row[T][k] int32; topk_w[T][k] float32;
 *   y_shared[T][H] and y[T][H] dtype dt.
 */
int moe_combine(const void* y_perm, int y_perm_dt, const int32_t* dst_row, const float* topk_w,
                int T, int k, int H, const void* y_shared, void* y, int dt, void* stream);

/*
 * moe_pack_by_rank -- token copies packed by destination rank, the step
 * before the expert-parallel dispatch all-to-all.
 *   [MoE guide] section "一个 token 为什么要跨 GPU" (count / prefix sum /
 *   permute by destination; 8 experts on 4 GPUs, GPU r holding experts 2r,
 *   2r + 1); [CS349D L8] section 3.1 (a token that chose two experts held by
 *   one device is sent there once; its gate weights travel with it).
 *
 *   Rank r holds experts [r*E/P, (r+1)*E/P) (E divisible by P).  A copy is a
 *   (rank r, token t) pair such that some slot of t routes to an expert of r;
 *   copies are ordered by rank, then by token.
 *   send_counts[r]   = copies for rank r;  send_offsets[P + 1] their prefix sum.
 *   send_token[row]  = the token copy `row` carries (first send_offsets[P]).
 *   send_row[t][j]   = the copy carrying slot j of token t (-1 if topk_ids[t][j]
 *                      is outside [0, E): such a slot is not sent).
 *   send_ids[row][:] = topk_ids[t][:], send_w[row][:] = topk_w[t][:] for the
 *                      token of the copy (all k slots: the receiving rank keeps
 *                      the slots of its own experts); both may be NULL.
 *   x_send[row][:]   = x[t][:] when x != NULL (dtype dt, H columns).
 *
 *   topk_ids[T][k] int32 (distinct within a token, as moe_route gives),
 *   topk_w[T][k] float32 (needed only for send_w).  Rows are at most
 *   T * min(k, P); size send_token, send_ids, send_w and x_send for that.
 *   ws: at least moe_pack_workspace_size(T, k, P) bytes (may be NULL when
 *   T <= 64).  Limits: 1 <= P <= 64, k <= 32, E <= 1024.  T = 0 writes zero
 *   counts and offsets.
 */
size_t moe_pack_workspace_size(int T, int k, int P);
int moe_pack_by_rank(const int32_t* topk_ids, const float* topk_w, int T, int k, int E, int P,
                     const void* x, int H, int dt,
                     int32_t* send_counts, int32_t* send_offsets, int32_t* send_token,
                     int32_t* send_row, int32_t* send_ids, float* send_w, void* x_send,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * moe_unpack_sum -- the source rank's sum after the combine all-to-all.
 *   [CS349D L8] section 3.1 (results sent back to the token's device and
 *   added; the gate weights were applied where the experts ran).
 *
 *   y[t] = sum over the distinct rows of send_row[t] (each copy once, in
 *   ascending row = rank order) of y_ret[row], accumulated in float32 and
 *   rounded once to dtype dt.  A token with no copy gets zeros.
 *   y_ret[rows][H] dtype y_ret_dt (the partial outputs returned for the
 *   copies, in the order moe_pack_by_rank sent them); send_row[T][k] as
 *   moe_pack_by_rank wrote it; y[T][H] dtype dt.
 */
int moe_unpack_sum(const void* y_ret, int y_ret_dt, const int32_t* send_row, int T, int k, int H,
                   void* y, int dt, void* stream);

/*
 * moe_reshard_ep_to_tp_pack / moe_reshard_tp_to_ep_interleave -- the two
 * data movements of the EP <-> TP expert-weight reshard on one rank.
 *   [Moebius notes] section 3 (eq. (6)-(8): the two layouts hold the same
 *   volume per rank; Algorithm 1 steps 1-2 pack per peer before the
 *   All-to-All, whose output is already the TP layout; Algorithm 2 step 4
 *   interleaves the received slices into whole experts; Figure 2).
 *
 *   P ranks; E_rank = E/P experts per rank in the EP layout; s = I/P.
 *   EP layout:    w13_ep[E_rank][2I][H] (gate rows [0, I), up rows [I, 2I)),
 *                 w2_ep[E_rank][H][I].
 *   Chunk layout: w13_chunks[P][E_rank][2s][H], w2_chunks[P][E_rank][H][s]:
 *                 chunk p of expert e holds gate rows [p*s, (p+1)*s) then
 *                 up rows I + [p*s, (p+1)*s) (the same intermediate range of
 *                 both halves, so SwiGLU stays local to a TP rank), and the
 *                 same input columns of W2.
 *   pack:        EP layout -> chunks (chunk p goes to peer p).  After the
 *                All-to-All, rank r's received chunks, in peer order, are its
 *                TP layout w13_tp[E][2s][H], w2_tp[E][H][s].
 *   interleave:  chunks received from each peer p (p's TP slice of this
 *                rank's experts; in the TP layout they are rows
 *                [r*E_rank, (r+1)*E_rank) of peer p's w13_tp / w2_tp) ->
 *                EP layout.  The inverse of pack.
 *   dtype dt; either the W13 or the W2 pair may be NULL (both members of a
 *   pair NULL).  Requires I divisible by P, H*elt and s*elt multiples of 16
 *   bytes, and each tensor below 32 GiB.  Source and destination must not
 *   overlap.
 */
int moe_reshard_ep_to_tp_pack(const void* w13_ep, const void* w2_ep, int E_rank, int I, int H,
                              int P, int dt, void* w13_send, void* w2_send, void* stream);
int moe_reshard_tp_to_ep_interleave(const void* w13_recv, const void* w2_recv, int E_rank, int I,
                                    int H, int P, int dt, void* w13_ep, void* w2_ep,
                                    void* stream);

/*
 * moe_layer -- the whole share of the layer in one call:
 *   route -> permute -> grouped SwiGLU GEMMs (gather fused) -> shared expert
 *   -> combine, all enqueued on `stream` without host synchronisation.
 *   [MoE guide] section "一个 token 为什么要跨 GPU" (the data path);
 *   [Moebius notes] eq. (1).
 *
 *   Expert-parallel view: [e_begin, e_end) is the local range and w13/w2 hold
 *   those experts ([Moebius notes] eq. (4)).  Tensor-parallel view: the full
 *   range with I_loc = I/P slices ([Moebius notes] eq. (3)); the output is the
 *   rank's partial sum.  The router always sees all E experts.
 *   I_shared > 0 adds one always-on shared expert (w13_shared[2*I_shared][H],
 *   w2_shared[H][I_shared]) with weight 1.
 */
typedef struct {
  int H, E, k, I_loc, e_begin, e_end, I_shared;
  int mode;                      /* moe_gating */
  int dt;                        /* moe_dtype of x, y and every weight */
  const void* w_router;          /* [E][H] */
  const void* w13;               /* [E_loc][2*I_loc][H] */
  const void* w2;                /* [E_loc][H][I_loc] */
  const void* w13_shared;        /* [2*I_shared][H] or NULL */
  const void* w2_shared;         /* [H][I_shared] or NULL */
  const float* logit_bias;       /* [E] or NULL: added to the logits (selection and weights) */
  const float* sel_bias;         /* [E] or NULL: mode 3 selection only */
} moe_layer_desc;

/* Optional copies of the intermediate results (every field may be NULL);
 * buffers as in moe_route / moe_permute.  stage_events[i], when not NULL, is
 * a hipEvent_t that moe_layer records on `stream` at stage boundary i:
 *   0 before routing, 1 after the routing metadata (route + permute),
 *   2 after the gate/up GEMM, 3 after the down GEMM, 4 after the shared
 *   expert, 5 after the combine.  At a few tokens the shared expert's GEMMs
 *   may run inside the routed GEMMs' launches (stages 2 and 3); stage 4 is
 *   then empty.
 * (Per-stage timing: the time split between router, dispatch metadata,
 * expert GEMMs and combine.) */
#define MOE_STAGE_EVENTS 6
typedef struct {
  float* logits;                 /* [T][E] */
  int32_t* topk_ids;             /* [T][k] */
  float* topk_w;                 /* [T][k] */
  int32_t* counts;               /* [E_loc] */
  int32_t* offsets;              /* [E_loc + 1] */
  int32_t* src_token;            /* [T*k] */
  int32_t* dst_row;              /* [T][k] */
  void* stage_events[MOE_STAGE_EVENTS];
} moe_debug_out;

/* Workspace bytes for moe_layer, moe_layer_decode and moe_layer_staged with
 * up to T_max tokens (0 on invalid desc).
 *
 * The workspace starts with a 132 KiB synchronisation block (4 KiB of
 * counters, then one 128-byte flag line per workgroup) that the single-launch
 * decode path keeps between calls: ZERO IT ONCE (e.g. zero the whole
 * workspace) before the first call that uses the workspace.  Every call
 * leaves it valid for the next; the staged path touches only the result
 * word of the MOE_VALIDATE=1 checks (below).  Calls that
 * share a workspace must be ordered (one stream, or events), as for any
 * scratch buffer.  Bytes 32..35 receive the result of the MOE_VALIDATE=1
 * metadata check.  Bytes 4..7 hold an int32 error word that the decode path
 * sets (bit 0: the router wait, bit 1: an expert wait) if a wait for another
 * workgroup exceeds its bound -- a grid that could not be resident at once;
 * that call's outputs are then undefined.  It stays set until it is read by
 * moe_layer_status (below) or by a call under MOE_VALIDATE=1, which return
 * MOE_ERR_WAIT and clear it.  A caller that runs the decode path without
 * MOE_VALIDATE=1 polls moe_layer_status to learn of such a failure. */
size_t moe_layer_workspace_size(const moe_layer_desc* d, int T_max);

/* The decode path's wait error word of a layer workspace (bytes 4..7 above),
 * read after the work already enqueued on `stream`: MOE_OK if it is zero;
 * otherwise it is cleared and MOE_ERR_WAIT is returned (some decode-path call
 * on this workspace since the last read had undefined outputs).  Waits for the
 * stream, so it cannot be captured in a graph.  MOE_ERR_INVALID_ARG for a null
 * or misaligned ws or ws_bytes below the synchronisation block. */
int moe_layer_status(void* ws, size_t ws_bytes, void* stream);

/* The layer share, choosing the single-launch decode path (moe_layer_decode)
 * for shapes it supports while the expert weights the call can touch
 * (min(E_loc, T*k) routed experts plus the shared one, bf16) are at most
 * 100 MB, and the staged path (moe_layer_staged) otherwise.  Both compute the same function; they
 * differ in rounding only (the staged path rounds each expert's output to
 * dtype dt before the combine, the decode path keeps it in float32). */
int moe_layer(const moe_layer_desc* d, int T, const void* x, void* y,
              void* ws, size_t ws_bytes, moe_debug_out* dbg, void* stream);

/* Which path moe_layer takes for this description and T: 0 staged, 1 the
 * single-launch decode path; negative (a moe_status, negated) for an invalid
 * description or T < 0. */
int moe_layer_path(const moe_layer_desc* d, int T);

/* Staged path: one launch per step (router, gating + metadata, gate/up GEMM,
 * down GEMM, shared expert, combine), any supported shape and T.  When the
 * shared expert and the routed experts take the same small-batch GEMM tiles,
 * the shared expert's two GEMMs ride in the routed GEMMs' launches. */
int moe_layer_staged(const moe_layer_desc* d, int T, const void* x, void* y,
                     void* ws, size_t ws_bytes, moe_debug_out* dbg, void* stream);

/* Staged path with a capacity of `capacity` pairs per local expert, dropping
 * the rest as moe_permute_capacity does (the capacity-factor variant of
 * [MoE guide] section "Capacity、padding 与 token dropping"; not the default,
 * see [CS349D L8] section 1.4).  dropped[0] (int32, may be NULL) receives the
 * number of local pairs dropped; debug copies show the kept counts and -1 for
 * dropped pairs.  capacity >= 0; INT_MAX with padded = 0 gives
 * moe_layer_staged exactly.
 *   padded = 1 lays the expert rows out in fixed blocks of `capacity` rows
 * (moe_permute_capacity's padded layout, debug offsets i * capacity, debug
 * src_token of E_loc * capacity entries with -1 on padding rows); the GEMMs
 * compute the kept rows only, so the output equals that of padded = 0.  The
 * workspace must then be moe_layer_capacity_workspace_size(d, T, capacity, 1)
 * bytes (else MOE_ERR_WORKSPACE), and E_loc * capacity must fit an int (else
 * MOE_ERR_INVALID_ARG). */
int moe_layer_capacity(const moe_layer_desc* d, int T, int capacity, int padded, const void* x,
                       void* y, void* ws, size_t ws_bytes, moe_debug_out* dbg, int32_t* dropped,
                       void* stream);

/* Workspace for moe_layer_capacity with T <= T_max: moe_layer_workspace_size
 * for padded = 0; for padded = 1, h and the expert outputs hold
 * E_loc * capacity rows.  0 for invalid arguments. */
size_t moe_layer_capacity_workspace_size(const moe_layer_desc* d, int T_max, int capacity,
                                         int padded);

/* Single-launch decode path: router, gating, dispatch metadata, both expert
 * GEMMs, the shared expert and the combine in ONE kernel launch whose
 * workgroups hand work to one another through counters in the workspace's
 * synchronisation block ([CS349D L8] section 6: a persistent kernel with
 * device-side dependencies, for the launch and dependency floor of small
 * decode batches).  Same arguments, results and debug copies as moe_layer;
 * stage_events 1-5 are all recorded after the one launch.
 * Supported: dt = MOE_BF16, 1 <= T <= 64, E <= 256, E_loc <= 256, k <= 16,
 * T * k <= 512; otherwise MOE_ERR_UNSUPPORTED.  The grid is sized so that
 * all its workgroups can be resident together (one per CU); a concurrent
 * kernel delays it but cannot deadlock it. */
int moe_layer_decode(const moe_layer_desc* d, int T, const void* x, void* y,
                     void* ws, size_t ws_bytes, moe_debug_out* dbg, void* stream);

/* Bytes of the device array moe_layer_static uses as its workspace. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)

/* moe_layer without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a file-scope device array of
 * MOE_STATIC_SCRATCH_BYTES (64 MiB), one per GPU the library runs on,
 * reserved when the library's code is loaded on that GPU and held until the
 * process ends; the call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine).  Same arguments (less ws, ws_bytes), path
 * choice, results and debug copies as moe_layer.
 *   The first call on a device looks up the array's address and clears its
 * synchronisation block by a small kernel on `stream`, ahead of the call's
 * own launches.  Every later call on that GPU reuses the array, which keeps
 * the last call's contents; calls that may overlap on one GPU (different
 * streams, or several threads) race on it and must be ordered by the caller.
 * Returns MOE_ERR_WORKSPACE, before touching the GPU, when
 * moe_layer_workspace_size(d, T) exceeds MOE_STATIC_SCRATCH_BYTES (it serves
 * decode-sized batches: T up to 400 for the DeepSeek-V3 shape with its shared
 * expert, 737 for the Qwen3-shaped share with all 128 experts, 907 for the
 * Mixtral shape, 966 for the Qwen3 TP share at P = 8); other errors as
 * moe_layer.  The wait error word (see
 * moe_layer_workspace_size) lives in the array too and cannot be read by
 * moe_layer_status: use MOE_VALIDATE=1 to have it checked. */
int moe_layer_static(const moe_layer_desc* d, int T, const void* x, void* y,
                     moe_debug_out* dbg, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
