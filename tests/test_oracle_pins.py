"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
example printed on the pages (tests/golden/), a closed form, an invariant the
pages state, a library routine, or brute force on tiny inputs.  A plausible
slip in the oracle (a dropped term, a wrong sign or index, swapped gate/up
halves, a transposed operand, a wrong tie-break) fails at least one of them.
"""
import math

import numpy as np
import pytest

from conftest import golden
from oracle import moe_oracle as O

MODES = O.GATING_MODES


def rng(seed):
    return np.random.default_rng(seed)


def tiny_layer(seed, T=5, H=8, I=16, E=8, shared=False):
    r = rng(seed)
    s = 1.0 / math.sqrt(H)
    d = dict(x=r.standard_normal((T, H)),
             w_r=r.standard_normal((E, H)) * s,
             w13=r.standard_normal((E, 2 * I, H)) * s,
             w2=r.standard_normal((E, H, I)) * s,
             logit_bias=r.standard_normal(E) * 0.3,
             sel_bias=r.standard_normal(E) * 0.5)
    if shared:
        d["w13_shared"] = r.standard_normal((2 * I, H)) * s
        d["w2_shared"] = r.standard_normal((H, I)) * s
    return d


# ---------------------------------------------------------------- selection

def test_topk_worked_example_selects_1_and_4():
    g = golden("topk_worked_example.json")
    scores = np.array([g["scores"]])
    for logits in (scores, np.log(scores)):
        for mode in MODES:
            ids, _ = O.route(logits, g["k"], mode, sel_bias=np.zeros(8))
            assert ids.tolist() == [g["selected_experts"]]


def test_topk_worked_example_weights():
    g = golden("topk_worked_example.json")
    logits = np.log(np.array([g["scores"]]))
    d = g["derived"]
    _, w0 = O.route(logits, 2, O.GATE_TOPK_SOFTMAX)
    _, w1 = O.route(logits, 2, O.GATE_SOFTMAX_TOPK)
    _, w2 = O.route(logits, 2, O.GATE_SOFTMAX_TOPK_RENORM)
    np.testing.assert_allclose(w0[0], d["topk_then_softmax_weights"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(w1[0], d["softmax_then_topk_weights"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(w2[0], d["topk_then_softmax_weights"], rtol=0, atol=1e-15)
    assert w1.sum() < 1.0  # no renormalisation: the kept probabilities sum to 0.77


def test_selection_matches_full_sort_brute_force():
    r = rng(1)
    for E, k in ((8, 2), (16, 5), (64, 8), (9, 9)):
        logits = r.standard_normal((40, E))
        logits[:, 3] = logits[:, 5]          # planted ties: lower id must win
        logits[::3, 0] = logits[::3, E - 1]
        ids = O.select_topk(logits, k)
        for t in range(40):
            ref = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
            assert ids[t].tolist() == ref


def test_tie_break_lower_id_first_and_signed_zero():
    logits = np.array([[0.0, -0.0, 0.0, -1.0, 0.5]], dtype=np.float32)
    assert O.select_topk(logits, 3).tolist() == [[4, 0, 1]]


def test_softmax_keeps_order_modes_0_1_2_select_the_same():
    r = rng(2)
    logits = r.standard_normal((100, 64)).astype(np.float32)
    ids = [O.route(logits, 8, m)[0] for m in (0, 1, 2)]
    assert np.array_equal(ids[0], ids[1]) and np.array_equal(ids[0], ids[2])


def test_weight_sums():
    r = rng(3)
    logits = r.standard_normal((50, 32)) * 3
    for mode in (0, 2, 3):
        _, w = O.route(logits, 4, mode, sel_bias=r.standard_normal(32))
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)
        assert (w > 0).all()
    _, w = O.route(logits, 4, O.GATE_SOFTMAX_TOPK)
    assert (w.sum(1) < 1.0).all()
    _, w = O.route(logits, 32, O.GATE_SOFTMAX_TOPK)   # k = E keeps everything
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)


def test_k_equals_E_selects_every_expert_in_key_order():
    logits = np.array([[0.3, -2.0, 1.5, 0.0]])
    ids, _ = O.route(logits, 4, 0)
    assert ids.tolist() == [[2, 0, 3, 1]]


def test_renormalised_softmax_equals_topk_softmax():
    r = rng(4)
    logits = r.standard_normal((64, 128)) * 2
    _, w0 = O.route(logits, 8, O.GATE_TOPK_SOFTMAX)
    _, w2 = O.route(logits, 8, O.GATE_SOFTMAX_TOPK_RENORM)
    np.testing.assert_allclose(w0, w2, rtol=1e-12, atol=0)


def test_sigmoid_weights_closed_form_and_bias_only_selects():
    # Two experts at logits +a and -a: sigmoid(a) + sigmoid(-a) = 1, so the
    # renormalised weights are sigmoid(a) and sigmoid(-a) exactly.  A softmax
    # over the pair would instead give sigmoid(2a).
    a = 0.7
    logits = np.array([[a, -a, -9.0, -9.0]])
    ids, w = O.route(logits, 2, O.GATE_SIGMOID_BIAS_RENORM, sel_bias=np.zeros(4))
    assert ids.tolist() == [[0, 1]]
    np.testing.assert_allclose(w[0], [1 / (1 + math.exp(-a)), 1 / (1 + math.exp(a))], atol=1e-15)
    # A selection bias changes which experts are picked, never the weights of
    # the picked ones: push expert 3 in with two different bias sizes; the
    # weights must be the same and must not contain the bias.
    got = []
    for b in (20.0, 50.0):
        ids_b, w_b = O.route(logits, 2, O.GATE_SIGMOID_BIAS_RENORM,
                             sel_bias=np.array([0.0, 0.0, 0.0, b]))
        assert ids_b.tolist() == [[3, 0]]
        got.append(w_b[0])
    np.testing.assert_array_equal(got[0], got[1])
    s3, s0 = 1 / (1 + math.exp(9.0)), 1 / (1 + math.exp(-a))
    np.testing.assert_allclose(got[0], [s3 / (s3 + s0), s0 / (s3 + s0)], rtol=1e-14)


def test_selection_bias_key_is_float32_for_float32_logits():
    # Exact sum 1 + 0.875 ulp < 1 + 1 ulp, but float32 rounds it up to 1 + 1 ulp:
    # a tie, broken towards expert 0.  In float64 expert 1 would win.
    logits = np.array([[1.0, 1.0 + 2 ** -23]], dtype=np.float32)
    bias = np.array([2 ** -23 - 2 ** -26, 0.0], dtype=np.float32)
    key = O.selection_key(logits, O.GATE_SIGMOID_BIAS_RENORM, bias)
    assert key.dtype == np.float32
    assert O.select_topk(key, 1).tolist() == [[0]]
    key64 = O.selection_key(logits.astype(np.float64), O.GATE_SIGMOID_BIAS_RENORM, bias)
    assert O.select_topk(key64, 1).tolist() == [[1]]


# ---------------------------------------------------------------- permutation

def test_permute_worked_example():
    g = golden("permute_worked_example.json")
    ids = np.array(g["expert_ids"])[:, None]
    counts, offsets, src, dst = O.permute(ids, 0, g["E"])
    d = g["derived"]
    assert counts.tolist() == d["counts"]
    assert offsets.tolist() == d["offsets"]
    assert src.tolist() == d["src_token"]
    assert dst[:, 0].tolist() == d["dst_row"]
    # the printed segments [t3] [t1] [t0, t2] [t4]
    segs = [[f"t{src[r]}" for r in range(offsets[e], offsets[e + 1])]
            for e in range(g["E"]) if counts[e]]
    assert segs == g["printed_permutation"]
    hist = {str(e): int(c) for e, c in enumerate(counts) if c}
    assert hist == g["printed_histogram"]


def test_permute_equals_library_stable_sort_and_is_a_bijection():
    r = rng(5)
    T, k, E = 300, 4, 16
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)])
    counts, offsets, src, dst = O.permute(ids, 0, E)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")          # library stable sort
    assert np.array_equal(src, order // k)
    assert counts.sum() == T * k
    assert np.array_equal(np.bincount(flat, minlength=E), counts)
    assert sorted(dst.reshape(-1).tolist()) == list(range(T * k))
    for t in range(T):
        for j in range(k):
            assert src[dst[t, j]] == t
            e = ids[t, j]
            assert offsets[e] <= dst[t, j] < offsets[e + 1]


def test_permute_expert_range():
    r = rng(6)
    T, k, E = 100, 3, 12
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)])
    counts, offsets, src, dst = O.permute(ids, 4, 9)
    local = (ids >= 4) & (ids < 9)
    assert counts.sum() == local.sum() == offsets[-1]
    assert (dst[~local] == -1).all()
    flat = ids.reshape(-1)
    sel = np.nonzero((flat >= 4) & (flat < 9))[0]
    order = sel[np.argsort(flat[sel], kind="stable")]
    assert np.array_equal(src, order // k)


# ---------------------------------------------------------------- capacity and dropping

def test_expert_capacity_formula():
    # C = ceil(cf * N_a / E): 4096 tokens, k = 8, E = 128
    assert O.expert_capacity(1.0, 4096 * 8, 128) == 256
    assert O.expert_capacity(1.25, 4096 * 8, 128) == 320
    assert O.expert_capacity(1.0, 10, 3) == 4


def test_capacity_keeps_first_pairs_in_token_order_brute_force():
    r = rng(50)
    T, k, E, C = 120, 3, 8, 20
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)])
    counts, offsets, src, dst, dropped = O.permute_capacity(ids, 0, E, C)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")          # library stable sort
    pos = np.empty_like(order)
    for e in range(E):
        sel = order[flat[order] == e]
        pos[sel] = np.arange(len(sel))              # place in the expert's token order
    kept = pos < C
    assert dropped == int((~kept).sum()) == int(np.maximum(np.bincount(flat, minlength=E) - C, 0).sum())
    assert np.array_equal(counts, np.minimum(np.bincount(flat, minlength=E), C))
    for t in range(T):
        for j in range(k):
            q = t * k + j
            if kept[q]:
                e = ids[t, j]
                assert dst[t, j] == offsets[e] + pos[q] and src[dst[t, j]] == t
            else:
                assert dst[t, j] == -1


def test_padded_layout_brute_force():
    """[MoE guide] "Capacity、padding 与 token dropping": an expert with fewer
    than C pairs is padded to C.  Expert i's block is rows [i*C, (i+1)*C),
    its kept pairs first in token order, then padding (source -1)."""
    r = rng(54)
    T, k, E, C = 90, 3, 8, 30
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)])
    for eb, ee in ((0, E), (2, 7)):
        counts, offsets, src, dst, dropped = O.permute_capacity(ids, eb, ee, C, padded=True)
        E_loc = ee - eb
        assert offsets.tolist() == [i * C for i in range(E_loc + 1)]
        assert len(src) == E_loc * C
        ref_src = -np.ones(E_loc * C, dtype=int)
        ref_dst = -np.ones((T, k), dtype=int)
        n_drop = 0
        for i in range(E_loc):                       # walk each expert's pairs
            pairs = [(t, j) for t in range(T) for j in range(k) if ids[t, j] == eb + i]
            for q, (t, j) in enumerate(pairs):
                if q < C:
                    ref_src[i * C + q] = t
                    ref_dst[t, j] = i * C + q
                else:
                    n_drop += 1
            assert counts[i] == min(len(pairs), C)
        assert np.array_equal(src, ref_src) and np.array_equal(dst, ref_dst)
        assert dropped == n_drop
        # the packed layout holds the same rows, moved to its own offsets
        pc, po, ps, pd, pdrop = O.permute_capacity(ids, eb, ee, C)
        assert np.array_equal(pc, counts) and pdrop == dropped
        for i in range(E_loc):
            assert np.array_equal(src[i * C:i * C + counts[i]], ps[po[i]:po[i + 1]])
        live = pd >= 0
        assert np.array_equal(live, dst >= 0)


def test_padded_rows_are_zero_and_the_layer_is_unchanged():
    """A padding row is a zero input row, so its expert output is exactly
    zero (SwiGLU has no bias: SiLU(0) * 0 = 0); padding changes where rows
    live, not the layer's result."""
    L = tiny_layer(55, T=30)
    k, mode = 2, 2
    for C in (3, 9, 40):
        y0, a0 = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], k, mode, capacity=C)
        y1, a1 = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], k, mode, capacity=C,
                             padded=True)
        assert a1["dropped"] == a0["dropped"]
        assert np.array_equal(y0, y1)
        src = a1["src_token"]
        y_perm = O.grouped_ffn(L["x"], src, a1["offsets"], L["w13"], L["w2"])
        assert np.all(y_perm[src < 0] == 0.0)
        # payload of the fixed-shape buffer: kept pairs over E * C rows
        kept = int((src >= 0).sum())
        assert kept == 30 * k - a1["dropped"] == int(a1["counts"].sum())


def test_large_capacity_is_dropless():
    L = tiny_layer(51, T=20)
    k, mode = 2, 2
    y0, a0 = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], k, mode)
    C = O.expert_capacity(8.0, 20 * k, 8)         # far above any count
    y1, a1 = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], k, mode, capacity=C)
    assert a1["dropped"] == 0
    assert np.array_equal(y0, y1)
    for key in ("counts", "offsets", "src_token", "dst_row"):
        assert np.array_equal(a0[key], a1[key])


def test_dropping_makes_outputs_depend_on_batch_neighbours():
    """[CS349D L8] section 1.4: with a capacity, a token's output depends on
    which other tokens share its batch; dropless it does not."""
    L = tiny_layer(52, T=24)
    k, mode = 2, 0
    y_full, a = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], k, mode, capacity=3)
    assert a["dropped"] > 0
    # the last token alone keeps all its pairs
    t = 23
    y_alone, b = O.moe_layer(L["x"][t:], L["w_r"], L["w13"], L["w2"], k, mode, capacity=3)
    assert b["dropped"] == 0
    dropped_t = (a["dst_row"][t] < 0).any()
    assert dropped_t, "the seed should drop a pair of the last token"
    assert not np.allclose(y_alone[0], y_full[t])
    y_free, _ = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], k, mode)
    np.testing.assert_allclose(y_alone[0], y_free[t], rtol=1e-13, atol=1e-14)


def test_dropped_pair_contributes_zero():
    L = tiny_layer(53, T=10)
    k, mode = 2, 2
    y, a = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], k, mode, capacity=1)
    ids, w = a["ids"], a["w"]
    for t in range(10):
        ref = np.zeros(L["x"].shape[1])
        for j in range(k):
            if a["dst_row"][t, j] >= 0:
                e = ids[t, j]
                ref += w[t, j] * O.swiglu_expert(L["x"][t:t + 1], L["w13"][e], L["w2"][e])[0]
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- dispatch packing by rank

def test_pack_by_rank_worked_example():
    g = golden("dispatch_by_rank_worked_example.json")
    ids = np.array(g["expert_ids"])[:, None]
    counts, offsets, send_token, send_row = O.pack_by_rank(ids, g["E"], g["P"])
    d = g["derived"]
    assert counts.tolist() == d["send_counts"]
    assert offsets.tolist() == d["send_offsets"]
    assert send_token.tolist() == d["send_token"]
    assert send_row[:, 0].tolist() == d["send_row"]
    # grouping the printed expert permutation by owner GPU gives the same copies
    owner = {f"t{t}": g["expert_ids"][t] // (g["E"] // g["P"]) for t in range(len(g["expert_ids"]))}
    by_gpu = [sorted((tok for seg in g["printed_expert_permutation"] for tok in seg
                      if owner[tok] == r), key=lambda s: int(s[1:])) for r in range(g["P"])]
    assert by_gpu == [[f"t{send_token[i]}" for i in range(offsets[r], offsets[r + 1])]
                      for r in range(g["P"])]


def test_pack_sends_a_token_once_per_device():
    # [CS349D L8] section 3.1: two experts of one device -> one copy
    ids = np.array([[0, 1], [0, 2], [7, 6], [5, 3]])
    counts, offsets, send_token, send_row = O.pack_by_rank(ids, 8, 4)
    assert counts.tolist() == [2, 2, 1, 1]
    assert send_token.tolist() == [0, 1, 1, 3, 3, 2]
    assert send_row.tolist() == [[0, 0], [1, 2], [5, 5], [4, 3]]


def test_pack_equals_library_sort_of_deduplicated_pairs():
    r = rng(31)
    T, k, E, P = 200, 6, 32, 8
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)])
    counts, offsets, send_token, send_row = O.pack_by_rank(ids, E, P)
    ranks = ids // (E // P)
    pairs = np.array(sorted({(int(ranks[t, j]), t) for t in range(T) for j in range(k)}))
    order = np.lexsort((pairs[:, 1], pairs[:, 0]))      # library sort: rank, then token
    assert np.array_equal(send_token, pairs[order, 1])
    assert np.array_equal(counts, np.bincount(pairs[:, 0], minlength=P))
    for t in range(T):
        for j in range(k):
            row = send_row[t, j]
            assert send_token[row] == t
            assert offsets[ranks[t, j]] <= row < offsets[ranks[t, j] + 1]


def test_pack_with_one_expert_per_rank_is_the_expert_permutation():
    r = rng(32)
    T, k, E = 150, 4, 16
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)])
    pc, po, ps, pr = O.pack_by_rank(ids, E, E)
    ec, eo, es, er = O.permute(ids, 0, E)
    assert np.array_equal(pc, ec) and np.array_equal(po, eo)
    assert np.array_equal(ps, es) and np.array_equal(pr, er)


def test_dispatch_volume_exercise_and_expectation():
    g = golden("dispatch_volume_exercise.json")
    T, D, k, H = g["T"], g["D"], g["assumed"]["k"], g["assumed"]["H"]
    assert round(O.dispatch_volume_bytes(T, k, D, H, 1) / 1e6, 1) == g["printed_MB"]["dispatch_fp8"]
    assert round(O.dispatch_volume_bytes(T, k, D, H, 2) / 1e6, 1) == g["printed_MB"]["combine_bf16"]
    # with one expert per device no copy is merged, and under uniform routing a
    # device sends k (D - 1) / D copies per token to the others on average
    r = rng(33)
    D, k, T, me = 16, 4, 4000, 5
    ids = np.stack([r.permutation(D)[:k] for _ in range(T)])
    counts, _, _, _ = O.pack_by_rank(ids, D, D)
    assert counts.sum() == T * k
    sent = counts.sum() - counts[me]
    assert abs(sent / (T * k * (D - 1) / D) - 1) < 0.01


@pytest.mark.parametrize("mode", [0, 3])
def test_dispatch_round_trip_equals_the_full_layer(mode):
    """Pack by rank, let every rank run its experts on the copies it received
    (routing travelling with them), return the partial sums and add them at
    the source: the full layer's output."""
    L = tiny_layer(34, T=9, E=8)
    E, P, k = 8, 4, 3
    y_full, aux = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], k, mode,
                              sel_bias=L["sel_bias"])
    ids, w = aux["ids"], aux["w"]
    counts, offsets, send_token, send_row = O.pack_by_rank(ids, E, P)
    y_ret = np.zeros((int(offsets[-1]), L["x"].shape[1]))
    for r in range(P):
        rows = np.arange(offsets[r], offsets[r + 1])
        lo, hi = r * E // P, (r + 1) * E // P
        toks = send_token[rows]
        c, o, src, dst = O.permute(ids[toks], lo, hi)
        y_perm = O.grouped_ffn(L["x"][toks], src, o, L["w13"][lo:hi], L["w2"][lo:hi])
        y_ret[rows] = O.combine(y_perm, dst, w[toks])
    y = O.unpack_sum(y_ret, send_row)
    np.testing.assert_allclose(y, y_full, rtol=0, atol=1e-13 * np.abs(y_full).max())


def test_unpack_sum_adds_each_copy_once_in_rank_order():
    send_row = np.array([[2, 2, 0], [1, -1, 1]])
    y_ret = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    assert O.unpack_sum(y_ret, send_row).tolist() == [[101.0, 202.0], [10.0, 20.0]]


# ---------------------------------------------------------------- EP <-> TP weight reshard

def _ep_weights(seed, P=4, n=2, I=8, H=5):
    r = rng(seed)
    return r.standard_normal((P * n, 2 * I, H)), r.standard_normal((P * n, H, I))


def test_reshard_ep_to_tp_gives_every_rank_its_tp_shard():
    """Algorithm 1 on P simulated ranks: each rank ends with exactly the
    tensor-parallel share of the full weights (tp_shard, pinned above)."""
    P = 4
    w13, w2 = _ep_weights(40, P=P)
    n = w13.shape[0] // P
    sends = [O.reshard_ep_to_tp_pack(w13[r * n:(r + 1) * n], w2[r * n:(r + 1) * n], P)
             for r in range(P)]
    recv13 = O.all_to_all([s[0] for s in sends])
    recv2 = O.all_to_all([s[1] for s in sends])
    for r in range(P):
        t13, t2 = O.reshard_ep_to_tp_place(recv13[r], recv2[r])
        ref13, ref2 = O.tp_shard(w13, w2, r, P)
        assert np.array_equal(t13, ref13) and np.array_equal(t2, ref2)


def test_reshard_tp_to_ep_inverts_ep_to_tp():
    P = 4
    w13, w2 = _ep_weights(41, P=P)
    n = w13.shape[0] // P
    tp = [O.tp_shard(w13, w2, r, P) for r in range(P)]
    splits = [O.reshard_tp_to_ep_split(t13, t2, P) for t13, t2 in tp]
    recv13 = O.all_to_all([sp[0] for sp in splits])
    recv2 = O.all_to_all([sp[1] for sp in splits])
    for r in range(P):
        e13, e2 = O.reshard_tp_to_ep_interleave(recv13[r], recv2[r])
        assert np.array_equal(e13, w13[r * n:(r + 1) * n])
        assert np.array_equal(e2, w2[r * n:(r + 1) * n])


def test_reshard_volume_invariance_and_traffic():
    """[Moebius notes] eq. (6): a rank holds E * 2I * H / P gate/up elements in
    both layouts; section 3.1: it sends (P - 1)/P of them to its peers."""
    P = 4
    w13, w2 = _ep_weights(42, P=P)
    E, twoI, H = w13.shape
    n = E // P
    send13, _ = O.reshard_ep_to_tp_pack(w13[:n], w2[:n], P)
    assert send13.size == w13[:n].size == E * twoI * H // P
    assert O.tp_shard(w13, w2, 0, P)[0].size == E * twoI * H // P
    to_peers = sum(send13[p].size for p in range(P) if p != 0)
    assert to_peers == (P - 1) * send13.size // P


def test_resharded_weights_compute_the_same_layer():
    """The same function over byte-identical weights: the TP shares built by
    the reshard sum to the EP shares' output."""
    L = tiny_layer(43, T=6, E=8, I=8, H=8)
    P, k, mode = 4, 2, 2
    n = 8 // P
    y_full, _ = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], k, mode)
    sends = [O.reshard_ep_to_tp_pack(L["w13"][r * n:(r + 1) * n], L["w2"][r * n:(r + 1) * n], P)
             for r in range(P)]
    recv13 = O.all_to_all([s[0] for s in sends])
    recv2 = O.all_to_all([s[1] for s in sends])
    y_tp = 0
    for r in range(P):
        t13, t2 = O.reshard_ep_to_tp_place(recv13[r], recv2[r])
        y_tp = y_tp + O.moe_layer(L["x"], L["w_r"], t13, t2, k, mode)[0]
    np.testing.assert_allclose(y_tp, y_full, rtol=0, atol=1e-13 * np.abs(y_full).max())


# ---------------------------------------------------------------- experts

def test_silu_identities():
    z = np.linspace(-8, 8, 33)
    np.testing.assert_allclose(O.silu(z) - O.silu(-z), z, atol=1e-14)   # z*(s(z)+s(-z)) = z
    assert O.silu(0.0) == 0.0
    np.testing.assert_allclose(O.silu(math.log(3.0)), 0.75 * math.log(3.0), rtol=1e-15)


def test_swiglu_expert_closed_form_and_gate_up_order():
    # H = 1, I = 1: y = c * SiLU(a x) * (b x)
    x = np.array([[1.0]])
    a, b, c = math.log(3.0), 2.0, -0.5
    y = O.swiglu_expert(x, np.array([[a], [b]]), np.array([[c]]))
    np.testing.assert_allclose(y, [[c * 0.75 * math.log(3.0) * b]], rtol=1e-15)
    # gate half strongly negative kills the output whatever the up half holds;
    # with the halves swapped it would not.
    y = O.swiglu_expert(x, np.array([[-60.0], [3.0]]), np.array([[1.0]]))
    assert abs(y[0, 0]) < 1e-20
    y_sw = O.swiglu_expert(x, np.array([[3.0], [-60.0]]), np.array([[1.0]]))
    assert abs(y_sw[0, 0]) > 1.0


def test_swiglu_is_linear_in_up_and_down_not_gate():
    L = tiny_layer(7)
    x, w13, w2 = L["x"], L["w13"][0], L["w2"][0]
    I = w13.shape[0] // 2
    y = O.swiglu_expert(x, w13, w2)
    up3 = w13.copy(); up3[I:] *= 3
    np.testing.assert_allclose(O.swiglu_expert(x, up3, w2), 3 * y, rtol=1e-12)
    np.testing.assert_allclose(O.swiglu_expert(x, w13, 3 * w2), 3 * y, rtol=1e-12)
    g3 = w13.copy(); g3[:I] *= 3
    assert not np.allclose(O.swiglu_expert(x, g3, w2), 3 * y, rtol=1e-3)


def test_swiglu_expert_elementwise_brute_force():
    L = tiny_layer(8, H=4, I=3)
    x, w13, w2 = L["x"], L["w13"][2], L["w2"][2]
    y = O.swiglu_expert(x, w13, w2)
    for t in range(x.shape[0]):
        h = []
        for i in range(3):
            g = sum(w13[i, q] * x[t, q] for q in range(4))
            u = sum(w13[3 + i, q] * x[t, q] for q in range(4))
            h.append(g / (1 + math.exp(-g)) * u)
        for o in range(4):
            assert abs(y[t, o] - sum(w2[o, i] * h[i] for i in range(3))) < 1e-13


def test_router_logits_brute_force():
    L = tiny_layer(9)
    s = O.router_logits(L["x"], L["w_r"], L["logit_bias"])
    for t in range(5):
        for e in range(8):
            ref = sum(L["w_r"][e, q] * L["x"][t, q] for q in range(8)) + L["logit_bias"][e]
            assert abs(s[t, e] - ref) < 1e-13


# ---------------------------------------------------------------- the layer

@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shared", [False, True])
def test_permuted_path_equals_dense_equation_1(mode, shared):
    L = tiny_layer(10 + mode, shared=shared)
    kw = dict(logit_bias=L["logit_bias"], sel_bias=L["sel_bias"] if mode == 3 else None,
              w13_shared=L.get("w13_shared"), w2_shared=L.get("w2_shared"))
    y, _ = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], 2, mode, **kw)
    y_dense = O.moe_layer_dense(L["x"], L["w_r"], L["w13"], L["w2"], 2, mode, **kw)
    np.testing.assert_allclose(y, y_dense, rtol=0, atol=1e-13 * np.abs(y_dense).max())


def test_single_expert_is_a_dense_ffn():
    L = tiny_layer(11, E=1)
    y, aux = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], 1, 0)
    assert (aux["w"] == 1.0).all()
    np.testing.assert_allclose(y, O.swiglu_expert(L["x"], L["w13"][0], L["w2"][0]), rtol=1e-14)


@pytest.mark.parametrize("mode", MODES)
def test_identical_experts_give_the_expert_output_scaled_by_weight_sum(mode):
    L = tiny_layer(12)
    w13 = np.repeat(L["w13"][:1], 8, axis=0)
    w2 = np.repeat(L["w2"][:1], 8, axis=0)
    y, aux = O.moe_layer(L["x"], L["w_r"], w13, w2, 3, mode, logit_bias=L["logit_bias"],
                         sel_bias=L["sel_bias"])
    f = O.swiglu_expert(L["x"], w13[0], w2[0])
    np.testing.assert_allclose(y, aux["w"].sum(1, keepdims=True) * f, rtol=1e-12, atol=1e-14)
    if mode != O.GATE_SOFTMAX_TOPK:
        np.testing.assert_allclose(y, f, rtol=1e-12, atol=1e-14)


def test_zero_input_gives_zero_output():
    L = tiny_layer(13, shared=True)
    y, _ = O.moe_layer(np.zeros_like(L["x"]), L["w_r"], L["w13"], L["w2"], 2, 0,
                       w13_shared=L["w13_shared"], w2_shared=L["w2_shared"])
    assert (y == 0).all()


def test_tensor_parallel_shares_sum_to_the_full_layer():
    L = tiny_layer(14, I=16)
    P = 4
    y_full, _ = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], 2, 2)
    parts = []
    for r in range(P):
        w13_r, w2_r = O.tp_shard(L["w13"], L["w2"], r, P)
        assert w13_r.shape == (8, 2 * 16 // P, 8) and w2_r.shape == (8, 8, 16 // P)
        parts.append(O.moe_layer(L["x"], L["w_r"], w13_r, w2_r, 2, 2)[0])
    np.testing.assert_allclose(sum(parts), y_full, rtol=0, atol=1e-13 * np.abs(y_full).max())


def test_tp_shard_agrees_with_the_input_generator_layout():
    import torch
    import workloads
    L = tiny_layer(15, I=16)
    for r in range(4):
        a13, a2 = O.tp_shard(L["w13"], L["w2"], r, 4)
        b13, b2 = workloads.share_weights(torch.from_numpy(L["w13"]), torch.from_numpy(L["w2"]),
                                          tp_P=4, tp_rank=r)
        assert np.array_equal(a13, b13.numpy()) and np.array_equal(a2, b2.numpy())


def test_expert_parallel_ranges_sum_to_the_full_layer():
    L = tiny_layer(16)
    y_full, _ = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], 2, 3, sel_bias=L["sel_bias"])
    parts = []
    for lo, hi in ((0, 4), (4, 8)):
        parts.append(O.moe_layer(L["x"], L["w_r"], L["w13"][lo:hi], L["w2"][lo:hi], 2, 3,
                                 sel_bias=L["sel_bias"], e_begin=lo, e_end=hi)[0])
    np.testing.assert_allclose(parts[0] + parts[1], y_full, rtol=0, atol=1e-13 * np.abs(y_full).max())


def test_dropless_outputs_do_not_depend_on_batch_neighbours():
    L = tiny_layer(17, T=24)
    y_full, _ = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], 2, 0)
    sub = np.array([1, 5, 6, 19])
    y_sub, _ = O.moe_layer(L["x"][sub], L["w_r"], L["w13"], L["w2"], 2, 0)
    np.testing.assert_allclose(y_sub, y_full[sub], rtol=1e-14, atol=1e-15)


def test_given_logits_route_exactly_on_them():
    L = tiny_layer(18)
    s32 = O.router_logits(L["x"], L["w_r"]).astype(np.float32)
    _, aux = O.moe_layer(L["x"], L["w_r"], L["w13"], L["w2"], 2, 0, logits=s32)
    assert aux["logits"] is s32
    assert np.array_equal(aux["ids"], O.select_topk(s32, 2))


# ---------------------------------------------------------------- measurement helpers

def test_touched_experts_exercise_values():
    g = golden("touched_experts_exercise.json")
    a = g["exercise_1a"]
    got = [O.touched_experts_expected(a["E"], a["k"], n) for n in a["n"]]
    np.testing.assert_allclose(got, a["expected_touched"], atol=0.05)
    b = g["exercise_1b"]
    assert round(O.touched_experts_expected(b["E"], b["k"], b["n"]), 2) == b["expected_touched"]
    assert round(b["params_per_expert"] * b["bytes_per_param"] / 1e9, 2) == b["gb_per_expert"]


def test_imbalance_ratio():
    assert O.imbalance_ratio([2, 2, 2, 2]) == 1.0
    assert O.imbalance_ratio([5, 1, 1, 1]) == 2.5
