"""Parity of the expert-parallel dispatch packing (moe_pack_by_rank) and the
source-side sum after the return (moe_unpack_sum) with the oracle, and an
expert-parallel round trip simulated on one GPU."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import workloads as W
from conftest import golden
from harness import GpuLayer, to_np, ws_tensor
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _i32(a):
    return torch.as_tensor(np.asarray(a), dtype=torch.int32, device=DEV).contiguous()


def _f32(a):
    return torch.as_tensor(np.asarray(a), dtype=torch.float32, device=DEV).contiguous()


def _routing(T, k, E, seed):
    r = np.random.default_rng(seed)
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), int)
    w = r.random((T, k)).astype(np.float32)
    return ids, w


def run_pack(ids, w, E, P, x=None):
    T, k = ids.shape
    rows = max(T * min(k, P), 1)
    out = dict(
        counts=torch.full((P,), -7, dtype=torch.int32, device=DEV),
        offsets=torch.full((P + 1,), -7, dtype=torch.int32, device=DEV),
        send_token=torch.full((rows,), -7, dtype=torch.int32, device=DEV),
        send_row=torch.full((max(T, 1), k), -7, dtype=torch.int32, device=DEV),
        send_ids=torch.full((rows, k), -7, dtype=torch.int32, device=DEV),
        send_w=torch.full((rows, k), -7.0, dtype=torch.float32, device=DEV))
    ids_d, w_d = _i32(ids if T else np.zeros((1, k))), _f32(w if T else np.zeros((1, k)))
    H, dt, x_send = 0, 0, None
    if x is not None:
        H, dt = x.shape[1], M.dtype_code(x)
        x_send = torch.zeros((rows, H), dtype=x.dtype, device=DEV)
        out["x_send"] = x_send
    nb = M.moe_pack_workspace_size(T, k, P)
    ws = ws_tensor(nb)
    M.moe_pack_by_rank(ids_d, w_d, T, k, E, P, x, H, dt, out["counts"], out["offsets"],
                       out["send_token"], out["send_row"], out["send_ids"], out["send_w"], x_send,
                       ws, nb)
    torch.cuda.synchronize()
    return out


CASES = [
    # (T, k, E, P)
    (1, 8, 256, 8), (5, 2, 8, 4), (63, 8, 128, 8), (64, 8, 128, 8), (65, 8, 256, 8),
    (300, 4, 16, 16), (200, 8, 128, 1), (1000, 8, 256, 64), (4097, 6, 32, 8), (130, 32, 64, 2),
]


@pytest.mark.parametrize("T,k,E,P", CASES)
def test_pack_matches_oracle(T, k, E, P):
    ids, w = _routing(T, k, E, seed=T * 7 + P)
    x = torch.randn((T, 256), device=DEV).to(torch.bfloat16)
    out = run_pack(ids, w, E, P, x)
    counts, offsets, send_token, send_row = O.pack_by_rank(ids, E, P)
    assert np.array_equal(to_np(out["counts"]), counts)
    assert np.array_equal(to_np(out["offsets"]), offsets)
    rows = int(offsets[-1])
    assert np.array_equal(to_np(out["send_token"])[:rows], send_token)
    assert np.array_equal(to_np(out["send_row"]), send_row)
    # the routing travels with every copy, and the rows are exact copies
    assert np.array_equal(to_np(out["send_ids"])[:rows], ids[send_token])
    assert np.array_equal(to_np(out["send_w"])[:rows], w[send_token])
    assert torch.equal(out["x_send"][:rows], x[torch.as_tensor(send_token, device=DEV).long()])


def test_pack_worked_example():
    g = golden("dispatch_by_rank_worked_example.json")
    ids = np.array(g["expert_ids"])[:, None]
    out = run_pack(ids, np.ones_like(ids, dtype=np.float32), g["E"], g["P"])
    d = g["derived"]
    assert to_np(out["counts"]).tolist() == d["send_counts"]
    assert to_np(out["offsets"]).tolist() == d["send_offsets"]
    assert to_np(out["send_token"]).astype(int).tolist()[:5] == d["send_token"]
    assert to_np(out["send_row"])[:, 0].astype(int).tolist() == d["send_row"]


def test_pack_empty_batch_and_unrouted_slots():
    out = run_pack(np.zeros((0, 4), int), np.zeros((0, 4), np.float32), 16, 4)
    assert to_np(out["counts"]).tolist() == [0] * 4
    assert to_np(out["offsets"]).tolist() == [0] * 5
    # ids outside [0, E) are not sent; a token with none sends no copy
    ids = np.array([[3, 16], [-1, 20], [0, 15]])
    out = run_pack(ids, np.ones((3, 2), np.float32), 16, 4)
    assert to_np(out["counts"]).tolist() == [2, 0, 0, 1]
    assert to_np(out["send_token"]).astype(int).tolist()[:3] == [0, 2, 2]
    assert to_np(out["send_row"]).astype(int).tolist() == [[0, -1], [-1, -1], [1, 2]]


@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32"),
                                          ("f32", "bf16")])
@pytest.mark.parametrize("T,k,E,P", [(7, 8, 64, 8), (500, 4, 16, 4)])
def test_unpack_sum_matches_oracle(in_dt, out_dt, T, k, E, P):
    ids, w = _routing(T, k, E, seed=T + k)
    out = run_pack(ids, w, E, P)
    rows = int(to_np(out["offsets"])[-1])
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    H = 96 * 8 // 2
    y_ret = torch.randn((rows, H), device=DEV).to(tdt[in_dt])
    y = torch.empty((T, H), dtype=tdt[out_dt], device=DEV)
    M.moe_unpack_sum(y_ret, M.dtype_code(y_ret), out["send_row"], T, k, H, y, M.dtype_code(y))
    torch.cuda.synchronize()
    ref = O.unpack_sum(to_np(y_ret).astype(np.float64), to_np(out["send_row"]))
    scale = np.abs(ref).max()
    tol = 1e-2 if out_dt == "bf16" else 1e-6
    assert np.abs(to_np(y).astype(np.float64) - ref).max() / scale <= tol


@pytest.mark.parametrize("name,P,T", [("qwen3_ep_all128", 8, 40), ("deepseek_v3", 4, 100),
                                      ("mixtral_8x7b", 4, 70)])
def test_expert_parallel_round_trip_on_one_gpu(name, P, T):
    """Route on the source, pack by rank, let each rank run its experts on the
    copies it received (moe_permute restricted to its range, the grouped FFN
    and the weighted combine), return the partial rows and add them up: the
    layer's output, checked against the oracle and against moe_layer."""
    cfg = W.CONFIGS[name]
    H, I, E = 256, 128, 32
    L = W.make_layer(cfg, device=DEV, seed=9, T_max=T, H=H, I=I, E=E)
    gl = GpuLayer(L)                      # the whole layer on one GPU, for comparison
    full = gl.run(T)
    ids, w = full["ids"], full["w"]
    k = cfg.k
    rows_max = T * min(k, P)
    counts = torch.empty((P,), dtype=torch.int32, device=DEV)
    offsets = torch.empty((P + 1,), dtype=torch.int32, device=DEV)
    send_token = torch.empty((rows_max,), dtype=torch.int32, device=DEV)
    send_row = torch.empty((T, k), dtype=torch.int32, device=DEV)
    send_ids = torch.empty((rows_max, k), dtype=torch.int32, device=DEV)
    send_w = torch.empty((rows_max, k), dtype=torch.float32, device=DEV)
    x = L.x[:T]
    x_send = torch.empty((rows_max, H), dtype=x.dtype, device=DEV)
    nb = M.moe_pack_workspace_size(T, k, P)
    ws = ws_tensor(nb)
    M.moe_pack_by_rank(ids, w, T, k, E, P, x, H, M.dtype_code(x), counts, offsets, send_token,
                       send_row, send_ids, send_w, x_send, ws, nb)
    torch.cuda.synchronize()
    off = to_np(offsets).astype(int)
    y_ret = torch.zeros((max(int(off[-1]), 1), H), dtype=x.dtype, device=DEV)
    dt = M.dtype_code(x)
    for r in range(P):
        n = int(off[r + 1] - off[r])
        if n == 0:
            continue
        lo, hi = r * E // P, (r + 1) * E // P
        E_loc = hi - lo
        seg = slice(int(off[r]), int(off[r + 1]))
        r_ids, r_w, r_x = send_ids[seg].contiguous(), send_w[seg].contiguous(), x_send[seg].contiguous()
        c_r = torch.empty((E_loc,), dtype=torch.int32, device=DEV)
        o_r = torch.empty((E_loc + 1,), dtype=torch.int32, device=DEV)
        src_r = torch.empty((max(n * k, 1),), dtype=torch.int32, device=DEV)
        dst_r = torch.empty((n, k), dtype=torch.int32, device=DEV)
        pnb = M.moe_permute_workspace_size(n, k, E_loc)
        M.moe_permute(r_ids, n, k, E, lo, hi, None, 0, 0, c_r, o_r, src_r, dst_r, None,
                      ws_tensor(pnb), pnb)
        rows = n * min(k, E_loc)
        y_perm = torch.empty((rows, H), dtype=x.dtype, device=DEV)
        fnb = M.moe_grouped_ffn_workspace_size(rows, E_loc, H, I, dt)
        M.moe_grouped_ffn(None, r_x, src_r, o_r, E_loc, rows, H, I, L.w13[lo:hi].contiguous(),
                          L.w2[lo:hi].contiguous(), dt, y_perm, dt, ws_tensor(fnb), fnb)
        M.moe_combine(y_perm, dt, dst_r, r_w, n, k, H, None, y_ret[seg], dt)
    y = torch.empty((T, H), dtype=x.dtype, device=DEV)
    M.moe_unpack_sum(y_ret, dt, send_row, T, k, H, y, dt)
    torch.cuda.synchronize()
    # against the single-GPU layer when it has no shared expert (a shared
    # expert is replicated on every rank and not part of the exchange)
    y_np = to_np(y).astype(np.float64)
    if not gl.I_shared:
        ref_layer = to_np(full["y"]).astype(np.float64)
        assert np.abs(y_np - ref_layer).max() / np.abs(ref_layer).max() <= 2e-2
    # against the oracle's routed experts on the same routing
    ref, _ = O.moe_layer(to_np(x), None, [to_np(L.w13[e]) for e in range(E)],
                         [to_np(L.w2[e]) for e in range(E)], k, cfg.mode,
                         sel_bias=to_np(L.sel_bias), logits=to_np(full["logits"]))
    assert np.abs(y_np - ref).max() / np.abs(ref).max() <= 1e-2
