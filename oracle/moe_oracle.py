"""Plain CPU oracle for one GPU's share of a Mixture-of-Experts layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module: only the tests, the package entry's smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code, table or constant
with the HIP library and imports nothing from it.

Every function is the plain definition of the step it computes, in float64
unless a caller asks for float32 (used only to time a CPU baseline), written
from these pages (cited by title and section):

  [Moebius notes]  Zhongzhu Zhou, reading notes "Moebius：为 MoE 大模型推理服务
                   实现无缝运行时并行策略切换" (zhongzhuzhou.org, 2026-06-28).
  [MoE guide]      "MoE 推理优化全景指南" (charlestar.github.io, 2026-05-13).
  [Moebius paper]  "Moebius: Serving Mixture-of-Expert Models with Seamless
                   Runtime Parallelism Switch" (conceptio.app mirror).
  [CS349D L8]      "Lecture 8 · 混合专家模型的推理" (CS349D notes, semidirectx.com).

Readings taken where the pages are silent (each one is listed, with its reason,
in the design notes of the repository):
  * top-k order: key descending, equal keys -> lower expert id first;
  * rows inside an expert segment: ascending token index (stable);
  * stacked gate/up axis: rows [0, I) are the gate projection, [I, 2I) the up
    projection; SwiGLU is SiLU(gate) * up with SiLU(z) = z / (1 + exp(-z));
  * the tensor-parallel share slices the intermediate index of *both* halves
    of the stacked axis by the same range, and the down projection's input
    dimension by that range;
  * the selection-only bias of the sigmoid gating is added to the logit;
  * a shared expert is added with weight 1 after the routed sum;
  * token copies packed for the expert-parallel dispatch are ordered by
    destination rank, then by token (one copy per token and rank);
  * the EP <-> TP weight reshard cuts the same intermediate range from the
    gate and the up half, as tp_shard does;
  * an expert over capacity keeps its first C (token, slot) pairs in token
    order;
  * in the padded layout expert i owns rows [i*C, (i+1)*C), its kept pairs
    first; a padding row has source -1 and a zero input row.

Parity status: every function below is pinned by the `-m "not gpu"` tests in
tests/test_oracle_pins.py (worked examples printed on the pages, closed forms,
invariants, brute force and library routines on tiny inputs).
"""
from __future__ import annotations

import numpy as np

GATE_TOPK_SOFTMAX = 0          # softmax over the k selected logits
GATE_SOFTMAX_TOPK = 1          # softmax over all E, keep k, no renormalisation
GATE_SOFTMAX_TOPK_RENORM = 2   # softmax over all E, keep k, divide by their sum
GATE_SIGMOID_BIAS_RENORM = 3   # select on logit + bias, weights sigmoid / sum

GATING_MODES = (GATE_TOPK_SOFTMAX, GATE_SOFTMAX_TOPK, GATE_SOFTMAX_TOPK_RENORM,
                GATE_SIGMOID_BIAS_RENORM)


def _as(a, dtype):
    return np.asarray(a, dtype=dtype)


# ---------------------------------------------------------------------------
# Router and gating
# ---------------------------------------------------------------------------

def router_logits(x, w_r, logit_bias=None, dtype=np.float64):
    """Router scores s = W_r x for every token, plus an optional per-expert
    additive bias.

    [MoE guide] section "从 Dense FFN 到专家集合": the router produces expert
    scores s = W_r x.  [CS349D L8] section 1.2: the gate is (x W_g), with the
    noise term turned off at inference.

    x: [T, H], w_r: [E, H]  ->  [T, E]
    """
    s = _as(x, dtype) @ _as(w_r, dtype).T
    if logit_bias is not None:
        s = s + _as(logit_bias, dtype)[None, :]
    return s


def select_topk(key, k):
    """Indices of the k largest keys per row, ordered by key descending and,
    among equal keys, by expert id ascending.

    [CS349D L8] section 1.2: KeepTopK keeps the k largest gate values.  The
    order among equal keys is not given by the pages; lower id first is used.

    key: [T, E] (compared in its own precision)  ->  int64 [T, k]
    """
    key = np.asarray(key)
    T, E = key.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    out = np.empty((T, k), dtype=np.int64)
    ids = np.arange(E)
    for t in range(T):
        # lexsort sorts by the last key first: key descending, then id ascending
        order = np.lexsort((ids, -key[t]))
        out[t] = order[:k]
    return out


def _softmax(v):
    m = np.max(v, axis=-1, keepdims=True)
    e = np.exp(v - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def gate_weights(logits, ids, mode):
    """Gate weights of the selected experts, in float64.

    [CS349D L8] section 1.2 lists the variants:
      mode 0  top-k then softmax (Shazeer, Mixtral): G = Softmax(KeepTopK(H, k)),
              the entries outside the top k are -inf, so the k weights sum to 1;
      mode 1  softmax then top-k without renormalising (DeepSeek-V2): the k
              weights are softmax probabilities over all E and sum to < 1;
      mode 2  mode 1 followed by division by the sum of the k kept weights;
      mode 3  sigmoid affinity, weights renormalised over the k selected; the
              selection bias never enters the weights (DeepSeek-V3).

    logits: [T, E], ids: [T, k]  ->  float64 [T, k]
    """
    s = _as(logits, np.float64)
    sel = np.take_along_axis(s, ids, axis=1)
    if mode == GATE_TOPK_SOFTMAX:
        return _softmax(sel)
    if mode in (GATE_SOFTMAX_TOPK, GATE_SOFTMAX_TOPK_RENORM):
        p = np.take_along_axis(_softmax(s), ids, axis=1)
        if mode == GATE_SOFTMAX_TOPK_RENORM:
            p = p / np.sum(p, axis=1, keepdims=True)
        return p
    if mode == GATE_SIGMOID_BIAS_RENORM:
        a = _sigmoid(sel)
        return a / np.sum(a, axis=1, keepdims=True)
    raise ValueError(f"unknown gating mode {mode}")


def selection_key(logits, mode, sel_bias=None):
    """The value the top-k selection compares.

    Modes 0-2 compare the logits themselves: softmax keeps order, so selecting
    before or after it picks the same experts ([CS349D L8] section 1.2).
    Mode 3 compares logit + bias, the bias changing only which experts are
    picked ([CS349D L8] section 1.2; [MoE guide] section "负载不均会拖慢整个集体
    通信" on DeepSeek-V3's auxiliary-loss-free balancing).  The sum is taken in
    the precision of the logits, so float32 logits give a float32 key.
    """
    s = np.asarray(logits)
    if mode == GATE_SIGMOID_BIAS_RENORM and sel_bias is not None:
        return s + np.asarray(sel_bias, dtype=s.dtype)[None, :]
    return s


def route(logits, k, mode, sel_bias=None):
    """Top-k expert ids and their gate weights for each token.

    logits: [T, E]  ->  (int64 ids [T, k], float64 weights [T, k])
    """
    key = selection_key(logits, mode, sel_bias)
    ids = select_topk(key, k)
    return ids, gate_weights(logits, ids, mode)


# ---------------------------------------------------------------------------
# Dispatch metadata: histogram, prefix sum, permutation
# ---------------------------------------------------------------------------

def expert_histogram(ids, e_begin, e_end):
    """counts[e - e_begin] = number of (token, slot) pairs routed to expert e,
    for the local experts e in [e_begin, e_end).

    [MoE guide] section "Dispatch 并不是一次普通 all-to-all": histogram step.
    """
    counts = np.zeros(e_end - e_begin, dtype=np.int64)
    for e in np.asarray(ids).reshape(-1):
        if e_begin <= e < e_end:
            counts[e - e_begin] += 1
    return counts


def exclusive_offsets(counts):
    """offsets[0] = 0, offsets[i + 1] = offsets[i] + counts[i].

    [MoE guide] section "Dispatch 并不是一次普通 all-to-all": the prefix sum gives
    each expert's output offset.
    """
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    for i, c in enumerate(counts):
        off[i + 1] = off[i] + c
    return off


def permute(ids, e_begin, e_end):
    """Stable grouping of token copies by local expert.

    [MoE guide] section "Dispatch 并不是一次普通 all-to-all": histogram, prefix
    sum, then permute so that each expert's copies are contiguous; its example
    keeps the original token order inside a segment ([t0, t2]).

    Returns counts [E_loc], offsets [E_loc + 1], src_token [rows] (the token
    each permuted row copies) and dst_row [T, k] (the row a (token, slot) pair
    went to, -1 when its expert is not local).
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    counts = expert_histogram(ids, e_begin, e_end)
    offsets = exclusive_offsets(counts)
    cursor = offsets[:-1].copy()
    src_token = np.empty(int(offsets[-1]), dtype=np.int64)
    dst_row = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e_begin <= e < e_end:
                row = cursor[e - e_begin]
                cursor[e - e_begin] += 1
                dst_row[t, j] = row
                src_token[row] = t
    return counts, offsets, src_token, dst_row


def expert_capacity(capacity_factor, n_assign, E):
    """C = ceil(capacity_factor * N_a / E).  [MoE guide] section "Capacity、
    padding 与 token dropping"; [CS349D L8] section 1.4 (N_a = tokens * k)."""
    return int(np.ceil(capacity_factor * n_assign / E))


def permute_capacity(ids, e_begin, e_end, C, padded=False):
    """The permutation with a capacity of C (token, slot) pairs per expert.

    [MoE guide] section "Capacity、padding 与 token dropping" and [CS349D L8]
    section 1.4: an expert over capacity drops the extra assignments, whose
    contribution becomes zero.  Reading (the pages do not say which pairs an
    expert keeps): the first C in the stable order of permute(), i.e. token
    order.

    padded: the same section lets an expert with fewer than C pairs be padded
    to C, so that every expert owns a fixed block of C rows: expert i's rows
    start at i * C, and a padding row has source -1.  Otherwise the kept rows
    are packed as in permute().

    Returns counts [E_loc] (kept pairs), offsets [E_loc + 1], src_token
    [offsets[-1]], dst_row [T, k] (-1 for a pair that is dropped or not
    local) and the number of dropped local pairs.
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    full, _, _, _ = permute(ids, e_begin, e_end)
    counts = np.minimum(full, C)
    if padded:
        offsets = np.arange(e_end - e_begin + 1, dtype=np.int64) * C
    else:
        offsets = exclusive_offsets(counts)
    src_token = np.full(int(offsets[-1]), -1, dtype=np.int64)
    dst_row = np.full((T, k), -1, dtype=np.int64)
    seen = np.zeros(e_end - e_begin, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e_begin <= e < e_end:
                i = e - e_begin
                if seen[i] < C:
                    row = offsets[i] + seen[i]
                    dst_row[t, j] = row
                    src_token[row] = t
                seen[i] += 1
    dropped = int((full - counts).sum())
    return counts, offsets, src_token, dst_row, dropped


# ---------------------------------------------------------------------------
# Expert-parallel dispatch: token copies packed by destination rank
# ---------------------------------------------------------------------------

def owner_rank(e, E, P):
    """Rank holding expert e when E experts are split into P contiguous ranges
    of E/P: [MoE guide] section "一个 token 为什么要跨 GPU" (8 experts on 4 GPUs,
    GPU r holding experts 2r and 2r + 1); [Moebius notes] eq. (4)."""
    if E % P:
        raise ValueError("E must be divisible by P")
    return int(e) // (E // P)


def pack_by_rank(ids, E, P):
    """Token copies packed by destination rank, the step before the dispatch
    all-to-all.

    [MoE guide] section "一个 token 为什么要跨 GPU": count / prefix sum /
    permute by destination, so that each destination's copies are contiguous.
    [CS349D L8] section 3.1: a token that chose two experts held by one
    device is sent there once, its gate weights travelling with it.

    A copy is a (rank r, token t) pair such that some slot j of t has
    owner_rank(ids[t][j]) == r.  Copies are ordered by rank, then by token
    (reading: inside a rank a copy may serve several experts, so the token
    order -- the order the page keeps inside a segment -- is the stable one).

    Returns send_counts [P], send_offsets [P + 1], send_token [rows] (the
    token each copy carries) and send_row [T, k] (the copy carrying slot j).
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    counts = np.zeros(P, dtype=np.int64)
    for t in range(T):
        for r in set(owner_rank(e, E, P) for e in ids[t]):
            counts[r] += 1
    offsets = exclusive_offsets(counts)
    send_token = np.empty(int(offsets[-1]), dtype=np.int64)
    send_row = np.full((T, k), -1, dtype=np.int64)
    row = 0
    for r in range(P):
        for t in range(T):
            slots = [j for j in range(k) if owner_rank(ids[t, j], E, P) == r]
            if slots:
                send_token[row] = t
                for j in slots:
                    send_row[t, j] = row
                row += 1
    return counts, offsets, send_token, send_row


def unpack_sum(y_ret, send_row, dtype=np.float64):
    """The source rank's sum after the combine all-to-all: y[t] is the sum of
    the partial outputs returned for t's copies, in rank order (each copy
    once, however many of t's slots it served).  [CS349D L8] section 3.1
    step 4 (results sent back and added); the gate weights were applied on
    the ranks that computed the experts.

    y_ret: [rows, H]; send_row: [T, k] as from pack_by_rank.  Returns [T, H].
    """
    y_ret = _as(y_ret, dtype)
    send_row = np.asarray(send_row)
    T = send_row.shape[0]
    y = np.zeros((T, y_ret.shape[1]), dtype=dtype)
    for t in range(T):
        for row in sorted(set(int(r) for r in send_row[t] if r >= 0)):
            y[t] += y_ret[row]
    return y


def dispatch_volume_bytes(T, k, D, H, elem_bytes):
    """Bytes one device sends per layer and direction under uniform routing:
    T * k * (D - 1) / D token vectors of H elements.  [CS349D L8] section 3.1
    (communication volume)."""
    return T * k * (D - 1) / D * H * elem_bytes


# ---------------------------------------------------------------------------
# Experts
# ---------------------------------------------------------------------------

def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z)
    return z / (1.0 + np.exp(-z))


def swiglu_expert(x_rows, w13_e, w2_e, dtype=np.float64):
    """One SwiGLU expert applied to a block of rows.

    [Moebius notes] eq. (2) and [Moebius paper] section 3.1: an expert holds a
    gate/up projection of shape (2I, H), the gate and up projections stacked
    on the leading axis, and a down projection of shape (H, I).

    x_rows: [m, H], w13_e: [2I, H], w2_e: [H, I]  ->  [m, H]
    """
    w13_e = _as(w13_e, dtype)
    w2_e = _as(w2_e, dtype)
    i_dim = w13_e.shape[0] // 2
    u = _as(x_rows, dtype) @ w13_e.T
    h = silu(u[:, :i_dim]) * u[:, i_dim:]
    return h @ w2_e.T


def grouped_ffn(x, src_token, offsets, w13, w2, dtype=np.float64):
    """Expert outputs for every permuted row: expert i multiplies its own
    contiguous block of m_i rows.

    [MoE guide] section "Expert GEMM 为什么经常不够大": expert i computes
    [m_i, hidden] @ W_i for its rows.

    x: [T, H]; src_token: [rows]; offsets: [E_loc + 1];
    w13: indexable by local expert -> [2I, H]; w2: -> [H, I]
    ->  y_perm [rows, H]

    A row whose source is -1 is padding (permute_capacity with padded=True):
    its input row is zero.
    """
    x = np.asarray(x)
    H = x.shape[1]
    rows = int(offsets[-1])
    y_perm = np.zeros((rows, H), dtype=dtype)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            src = np.asarray(src_token[r0:r1])
            xin = np.zeros((r1 - r0, H), dtype=x.dtype)
            live = src >= 0
            xin[live] = x[src[live]]
            y_perm[r0:r1] = swiglu_expert(xin, w13[e], w2[e], dtype)
    return y_perm


def combine(y_perm, dst_row, w, y_shared=None, dtype=np.float64):
    """Inverse permutation with the gate-weighted sum:
    y[t] = sum_j w[t, j] * y_perm[dst_row[t, j]] over the local slots, summed
    in slot order, plus the shared expert's output with weight 1.

    [MoE guide] section "Dispatch 并不是一次普通 all-to-all": combine restores
    the original token order and applies the routing weights.  [Moebius notes]
    eq. (1).  [CS349D L8] section 1.2: a shared expert every token passes
    through.
    """
    dst_row = np.asarray(dst_row)
    w = _as(w, dtype)
    T, k = dst_row.shape
    H = y_perm.shape[1]
    y = np.zeros((T, H), dtype=dtype)
    for t in range(T):
        for j in range(k):
            r = dst_row[t, j]
            if r >= 0:
                y[t] += w[t, j] * y_perm[r]
    if y_shared is not None:
        y = y + _as(y_shared, dtype)
    return y


# ---------------------------------------------------------------------------
# The layer
# ---------------------------------------------------------------------------

def moe_layer(x, w_r, w13, w2, k, mode, logit_bias=None, sel_bias=None,
              e_begin=0, e_end=None, w13_shared=None, w2_shared=None,
              logits=None, dtype=np.float64, capacity=None, padded=False):
    """One GPU's share of the MoE layer forward through the permuted data path.

    [MoE guide] section "一个 token 为什么要跨 GPU": router -> top-k ids and
    weights -> count / prefix sum / permute -> experts grouped -> inverse
    permutation + weighted sum.  [Moebius notes] eq. (1) is the result.

    The share: local experts are [e_begin, e_end) (expert-parallel view,
    [Moebius notes] eq. (4)); w13[i], w2[i] are those of expert e_begin + i.
    For the tensor-parallel view pass the rank's slices ([Moebius notes]
    eq. (3); see tp_shard) with the full expert range.

    `logits` may be given (e.g. float32 logits from another implementation) to
    route on exactly those values; otherwise they are computed here.

    `capacity`: C pairs per local expert (permute_capacity); None = dropless.
    `padded`: with a capacity, every expert owns a block of C rows.

    Returns (y [T, H], aux dict with logits, ids, w, counts, offsets,
    src_token, dst_row, dropped).
    """
    x = np.asarray(x)
    E = np.asarray(w_r).shape[0] if logits is None else np.asarray(logits).shape[1]
    if e_end is None:
        e_end = E
    if logits is None:
        logits = router_logits(x, w_r, logit_bias, dtype)
    ids, w = route(logits, k, mode, sel_bias)
    dropped = 0
    if capacity is None:
        counts, offsets, src_token, dst_row = permute(ids, e_begin, e_end)
    else:
        counts, offsets, src_token, dst_row, dropped = permute_capacity(ids, e_begin, e_end,
                                                                         capacity, padded)
    y_perm = grouped_ffn(x, src_token, offsets, w13, w2, dtype)
    y_shared = None
    if w13_shared is not None:
        y_shared = swiglu_expert(x, w13_shared, w2_shared, dtype)
    y = combine(y_perm, dst_row, w, y_shared, dtype)
    aux = dict(logits=logits, ids=ids, w=w, counts=counts, offsets=offsets,
               src_token=src_token, dst_row=dst_row, dropped=dropped)
    return y, aux


def moe_layer_dense(x, w_r, w13, w2, k, mode, logit_bias=None, sel_bias=None,
                    w13_shared=None, w2_shared=None, dtype=np.float64):
    """Brute-force evaluation of the layer with a dense gate vector.

    [CS349D L8] section 1.2: y = sum_{i=1..E} G(x)_i E_i(x), G sparse with k
    non-zeros.  Every expert is evaluated on every token and multiplied by its
    dense gate entry (zero off the top k); no permutation is involved.  Only
    for tiny inputs.
    """
    x = np.asarray(x)
    logits = router_logits(x, w_r, logit_bias, dtype)
    T, E = logits.shape
    ids, w = route(logits, k, mode, sel_bias)
    G = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        G[t, ids[t]] = w[t]
    y = np.zeros((T, x.shape[1]), dtype=dtype)
    for e in range(E):
        y += G[:, e:e + 1] * swiglu_expert(x, w13[e], w2[e], dtype)
    if w13_shared is not None:
        y += swiglu_expert(x, w13_shared, w2_shared, dtype)
    return y


def tp_shard(w13, w2, rank, P):
    """The tensor-parallel share of rank `rank` out of P.

    [Moebius notes] eq. (3) and [Moebius paper] section 3.1: every rank holds
    all E experts with W13 of shape (E, 2I/P, H) and W2 of shape (E, H, I/P).
    Reading: the slice takes intermediate indices [rank*I/P, (rank+1)*I/P) of
    the gate half and the same indices of the up half, so SwiGLU stays local;
    W2 keeps the same input columns.

    w13: [E, 2I, H], w2: [E, H, I]  ->  ([E, 2I/P, H], [E, H, I/P])
    """
    w13 = np.asarray(w13)
    w2 = np.asarray(w2)
    i_dim = w13.shape[1] // 2
    if i_dim % P:
        raise ValueError("I must be divisible by P")
    s = i_dim // P
    lo, hi = rank * s, (rank + 1) * s
    w13_r = np.concatenate([w13[:, lo:hi, :], w13[:, i_dim + lo:i_dim + hi, :]], axis=1)
    w2_r = w2[:, :, lo:hi]
    return w13_r, w2_r


def _tp_rows(I, P, p):
    """Rows of the stacked gate/up axis that TP rank p holds: intermediate
    indices [p*I/P, (p+1)*I/P) of the gate half, then the same of the up half
    (the reading of tp_shard)."""
    s = I // P
    return np.concatenate([np.arange(p * s, (p + 1) * s), I + np.arange(p * s, (p + 1) * s)])


def reshard_ep_to_tp_pack(w13_ep, w2_ep, P):
    """Local pack of the EP -> TP weight reshard: for every peer p the slice of
    this rank's experts that p holds after the switch, grouped by p.

    [Moebius notes] section 3.1, Algorithm 1 steps 1-2 (chunk per peer,
    concatenated into the All-to-All send buffer).  The algorithm writes the
    chunk as a contiguous cut of the stacked 2I axis; read, as for tp_shard,
    as the same intermediate range of the gate and of the up half (so SwiGLU
    stays local), and W2 cut on its input columns by that range.

    w13_ep: [E/P, 2I, H], w2_ep: [E/P, H, I]
    -> send13 [P, E/P, 2I/P, H], send2 [P, E/P, H, I/P]
    """
    w13_ep = np.asarray(w13_ep)
    w2_ep = np.asarray(w2_ep)
    I = w2_ep.shape[2]
    if I % P:
        raise ValueError("I must be divisible by P")
    s = I // P
    send13 = np.stack([w13_ep[:, _tp_rows(I, P, p), :] for p in range(P)])
    send2 = np.stack([w2_ep[:, :, p * s:(p + 1) * s] for p in range(P)])
    return send13, send2


def all_to_all(send):
    """The exchange between P ranks, simulated: send[r][p] is what rank r
    sends to rank p; recv[p][r] = send[r][p].  [Moebius notes] section 3.1,
    Algorithm 1 step 3."""
    P = len(send)
    return [[send[r][p] for r in range(P)] for p in range(P)]


def reshard_ep_to_tp_place(recv13, recv2):
    """Algorithm 1 step 4: rank r's received chunks, in peer order, are its TP
    layout.  recv13[p]: [E/P, 2I/P, H] from peer p -> W_TP [E, 2I/P, H];
    recv2[p]: [E/P, H, I/P] -> W2_TP [E, H, I/P]."""
    return np.concatenate(list(recv13), axis=0), np.concatenate(list(recv2), axis=0)


def reshard_tp_to_ep_split(w13_tp, w2_tp, P):
    """Algorithm 2 steps 1-2: the TP weights split by expert owner (peer p
    receives experts [p*E/P, (p+1)*E/P) of this rank's slice).
    w13_tp: [E, 2I/P, H], w2_tp: [E, H, I/P] -> ([P, E/P, 2I/P, H], [P, E/P, H, I/P])."""
    w13_tp = np.asarray(w13_tp)
    w2_tp = np.asarray(w2_tp)
    E = w13_tp.shape[0]
    n = E // P
    return (np.stack([w13_tp[p * n:(p + 1) * n] for p in range(P)]),
            np.stack([w2_tp[p * n:(p + 1) * n] for p in range(P)]))


def reshard_tp_to_ep_interleave(recv13, recv2):
    """Algorithm 2 step 4: each peer p's slice of every local expert is put
    back at p's rows of the stacked axis (gate and up halves, the reading of
    tp_shard) and p's input columns of W2.
    recv13 [P, E/P, 2I/P, H], recv2 [P, E/P, H, I/P] -> W_EP [E/P, 2I, H],
    W2_EP [E/P, H, I]."""
    recv13 = np.asarray(recv13)
    recv2 = np.asarray(recv2)
    P, n, two_s, H = recv13.shape
    s = two_s // 2
    I = s * P
    w13 = np.empty((n, 2 * I, H), dtype=recv13.dtype)
    w2 = np.empty((n, recv2.shape[2], I), dtype=recv2.dtype)
    for p in range(P):
        w13[:, _tp_rows(I, P, p), :] = recv13[p]
        w2[:, :, p * s:(p + 1) * s] = recv2[p]
    return w13, w2


def touched_experts_expected(E, k, n):
    """Expected number of distinct experts a batch of n tokens touches under
    uniform routing: E * (1 - (1 - k/E)^n).  [CS349D L8] section 2.1."""
    return E * (1.0 - (1.0 - k / E) ** n)


def imbalance_ratio(counts, n_assign=None, E=None):
    """max_i n_i / (N_a / E).  [MoE guide] section "负载不均会拖慢整个集体通信"."""
    counts = np.asarray(counts)
    if n_assign is None:
        n_assign = counts.sum()
    if E is None:
        E = len(counts)
    return float(counts.max()) / (n_assign / E)
