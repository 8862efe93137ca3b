"""GPU parity: every entry point of the C ABI against the CPU oracle.

Inputs are the seeded synthetic recipe of the `workloads` module; the oracle
and the HIP path see the same values.  Integer results (ids, counts, offsets,
permutations) must match exactly; floating-point results meet the tolerances
of the parity protocol in tests/harness.py.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import workloads as W
from conftest import golden
from harness import GpuLayer, check_layer, to_np, ws_tensor
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.get_lib()


def _i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device=DEV)


def _f32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float32), device=DEV)


def _route_logits_input(logits, k, mode, sel_bias=None):
    T, E = logits.shape
    lg = _f32(logits)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    sb = None if sel_bias is None else _f32(sel_bias)
    M.moe_route(None, None, 0, T, 0, E, k, mode, None, sb, lg, ids, w)
    torch.cuda.synchronize()
    return to_np(ids), to_np(w)


# ---------------------------------------------------------------- route

def test_route_worked_example():
    g = golden("topk_worked_example.json")
    scores = np.array([g["scores"]], dtype=np.float32)
    for mode in range(4):
        ids, w = _route_logits_input(np.log(scores), 2, mode, np.zeros(8))
        assert ids.tolist() == [g["selected_experts"]]
    ids, w = _route_logits_input(np.log(scores), 2, 0)
    np.testing.assert_allclose(w[0], g["derived"]["topk_then_softmax_weights"], atol=1e-6)
    ids, w = _route_logits_input(np.log(scores), 2, 1)
    np.testing.assert_allclose(w[0], g["derived"]["softmax_then_topk_weights"], atol=1e-6)


# E covers every experts-per-lane width of the gating kernel (1 .. 64, staged
# and unstaged logits); k > 16 uses the second choice slot of each lane
@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (128, 8), (256, 8), (300, 5), (8, 8),
                                 (32, 17), (256, 32), (512, 20), (1024, 32)])
@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_route_modes_exact_ids(E, k, mode):
    r = np.random.default_rng(E * 10 + k + mode)
    T = 333
    logits = (r.standard_normal((T, E)) * 2).astype(np.float32)
    logits[::5, 1] = logits[::5, 0]                     # ties -> lower id first
    logits[::7, E - 1] = logits[::7, 2]
    logits[3, :] = 0.5                                  # a fully tied row
    sb = (r.standard_normal(E) * 0.5).astype(np.float32)
    ids, w = _route_logits_input(logits, k, mode, sb)
    ids_ref, w_ref = O.route(logits, k, mode, sb)
    assert np.array_equal(ids, ids_ref)
    np.testing.assert_allclose(w, w_ref, rtol=0, atol=2e-6)


@pytest.mark.parametrize("T", [1, 16, 33, 64, 300])
@pytest.mark.parametrize("E,H", [(8, 512), (128, 4096), (256, 1024), (20, 256), (96, 512),
                                 (10, 256)])
def test_router_logits_bf16(T, E, H):
    g = torch.Generator(device=DEV)
    g.manual_seed(T * 1000 + E)
    x = torch.randn((T, H), generator=g, device=DEV).to(torch.bfloat16)
    wr = (torch.randn((E, H), generator=g, device=DEV) / H ** 0.5).to(torch.bfloat16)
    bias = torch.randn((E,), generator=g, device=DEV) * 0.1
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, 2), dtype=torch.int32, device=DEV)
    w = torch.empty((T, 2), dtype=torch.float32, device=DEV)
    M.moe_route(x, wr, M.MOE_BF16, T, H, E, 2, 0, bias, None, logits, ids, w)
    torch.cuda.synchronize()
    ref = O.router_logits(to_np(x), to_np(wr), to_np(bias))
    err = np.abs(to_np(logits) - ref).max() / np.abs(ref).max()
    assert err <= 1e-5
    assert np.array_equal(to_np(ids), O.route(to_np(logits), 2, 0)[0])


def test_router_logits_f32():
    T, E, H = 70, 8, 256
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    x = torch.randn((T, H), generator=g, device=DEV)
    wr = torch.randn((E, H), generator=g, device=DEV) / 16
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, 2), dtype=torch.int32, device=DEV)
    w = torch.empty((T, 2), dtype=torch.float32, device=DEV)
    M.moe_route(x, wr, M.MOE_F32, T, H, E, 2, 0, None, None, logits, ids, w)
    torch.cuda.synchronize()
    ref = O.router_logits(to_np(x), to_np(wr))
    assert np.abs(to_np(logits) - ref).max() / np.abs(ref).max() <= 1e-6


# ---------------------------------------------------------------- permute

def _permute_gpu(ids_np, E, e_begin, e_end, x=None):
    T, k = ids_np.shape
    E_loc = e_end - e_begin
    ids = _i32(ids_np)
    counts = torch.full((E_loc,), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((E_loc + 1,), -7, dtype=torch.int32, device=DEV)
    src = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device=DEV)
    dst = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    nb = M.moe_permute_workspace_size(T, k, E_loc)
    ws = ws_tensor(nb)
    x_perm = None
    H = 0
    dt = 0
    if x is not None:
        H = x.shape[1]
        dt = M.dtype_code(x)
        x_perm = torch.zeros((max(T * k, 1), H), dtype=x.dtype, device=DEV)
    M.moe_permute(ids, T, k, E, e_begin, e_end, x, H, dt, counts, offsets, src, dst, x_perm, ws, nb)
    torch.cuda.synchronize()
    return counts, offsets, src, dst, x_perm


def test_permute_worked_example():
    g = golden("permute_worked_example.json")
    ids = np.array(g["expert_ids"])[:, None]
    counts, offsets, src, dst, _ = _permute_gpu(ids, g["E"], 0, g["E"])
    d = g["derived"]
    assert to_np(counts).tolist() == d["counts"]
    assert to_np(offsets).tolist() == d["offsets"]
    assert to_np(src).tolist() == d["src_token"]
    assert to_np(dst)[:, 0].tolist() == d["dst_row"]


@pytest.mark.parametrize("T", [1, 7, 63, 64, 65, 130, 1000, 4097])
@pytest.mark.parametrize("E,k,eb,ee", [(16, 4, 0, 16), (128, 8, 0, 128), (128, 8, 16, 32),
                                       (256, 8, 200, 256), (8, 2, 3, 4), (1024, 32, 0, 1024),
                                       (1024, 32, 512, 640)])
def test_permute_exact(T, E, k, eb, ee):
    r = np.random.default_rng(T + E + k + eb)
    # skewed, distinct-per-token ids
    p = np.exp(-0.05 * np.arange(E))
    p /= p.sum()
    ids = np.stack([r.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    x = torch.randn((T, 64), device=DEV).to(torch.bfloat16)
    counts, offsets, src, dst, x_perm = _permute_gpu(ids, E, eb, ee, x)
    c_ref, o_ref, s_ref, d_ref = O.permute(ids, eb, ee)
    assert np.array_equal(to_np(counts), c_ref)
    assert np.array_equal(to_np(offsets), o_ref)
    rows = int(o_ref[-1])
    assert np.array_equal(to_np(src)[:rows], s_ref)
    assert np.array_equal(to_np(dst), d_ref)
    assert torch.equal(x_perm[:rows], x[torch.as_tensor(s_ref, device=DEV)])


def test_permute_empty_batch():
    counts, offsets, src, dst, _ = _permute_gpu(np.zeros((0, 2), dtype=np.int32), 8, 0, 8)
    assert to_np(counts).tolist() == [0] * 8
    assert to_np(offsets).tolist() == [0] * 9


# ---------------------------------------------------------------- grouped FFN + combine

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,E,k", [(3, 8, 2), (40, 16, 4), (300, 16, 2), (700, 8, 2), (1500, 4, 2)])
def test_grouped_ffn_and_combine(dt, T, E, k):
    H, I = 256, 128
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    g = torch.Generator(device=DEV)
    g.manual_seed(T + E)
    x = torch.randn((T, H), generator=g, device=DEV).to(tdt)
    w13 = (torch.randn((E, 2 * I, H), generator=g, device=DEV) / H ** 0.5).to(tdt)
    w2 = (torch.randn((E, H, I), generator=g, device=DEV) / H ** 0.5).to(tdt)
    r = np.random.default_rng(T)
    ids = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)])
    wts = r.random((T, k)).astype(np.float32)
    counts, offsets, src, dst = O.permute(ids, 0, E)
    rows = T * k
    dtc = M.dtype_code(tdt)
    y_perm = torch.empty((rows, H), dtype=tdt, device=DEV)
    nb = M.moe_grouped_ffn_workspace_size(rows, E, H, I, dtc)
    ws = ws_tensor(nb)
    # gather fused into the GEMM
    M.moe_grouped_ffn(None, x, _i32(src), _i32(offsets), E, rows, H, I, w13, w2, dtc, y_perm, dtc,
                      ws, nb)
    # pre-permuted rows
    x_perm = x[torch.as_tensor(src, device=DEV)].contiguous()
    y_perm2 = torch.empty_like(y_perm)
    M.moe_grouped_ffn(x_perm, None, None, _i32(offsets), E, rows, H, I, w13, w2, dtc, y_perm2, dtc,
                      ws, nb)
    y = torch.empty((T, H), dtype=tdt, device=DEV)
    M.moe_combine(y_perm, dtc, _i32(dst), _f32(wts), T, k, H, None, y, dtc)
    torch.cuda.synchronize()
    assert torch.equal(y_perm, y_perm2)
    ref = O.grouped_ffn(to_np(x), src, offsets, to_np(w13), to_np(w2))
    tol = 1e-2 if dt == "bf16" else 1e-5
    assert np.abs(to_np(y_perm) - ref).max() / np.abs(ref).max() <= tol
    y_ref = O.combine(ref, dst, wts)
    assert np.abs(to_np(y) - y_ref).max() / np.abs(y_ref).max() <= tol


# Expert segments crafted around the 256-row tile of the prefill GEMMs (mean
# rows per expert >= 384): exact multiples of 256, one row, tails of at most
# 128 rows (which run two N-tiles wide, or as a plain half tile on the last
# N-tile of an odd count: 1 and 3 N-tiles below), tails of 129-255 rows, an
# empty expert; contractions of 2 to 16 LDS stages (K = 128 ... 1024).
BIG_TILE_COUNTS = [767, 1, 128, 385, 256, 640, 0, 903]


@pytest.mark.parametrize("H,I", [(512, 256), (1024, 128), (256, 512), (768, 384)])
def test_grouped_ffn_big_tiles_ragged(H, I):
    counts = np.array(BIG_TILE_COUNTS)
    E, rows, T = len(counts), int(counts.sum()), 1000
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    g = torch.Generator(device=DEV)
    g.manual_seed(H + I)
    x = torch.randn((T, H), generator=g, device=DEV).to(torch.bfloat16)
    w13 = (torch.randn((E, 2 * I, H), generator=g, device=DEV) / H ** 0.5).to(torch.bfloat16)
    w2 = (torch.randn((E, H, I), generator=g, device=DEV) / H ** 0.5).to(torch.bfloat16)
    src = np.random.default_rng(H + I).integers(0, T, rows).astype(np.int32)
    y_perm = torch.empty((rows, H), dtype=torch.bfloat16, device=DEV)
    nb = M.moe_grouped_ffn_workspace_size(rows, E, H, I, 1)
    ws = ws_tensor(nb)
    M.moe_grouped_ffn(None, x, _i32(src), _i32(offsets), E, rows, H, I, w13, w2, 1, y_perm, 1,
                      ws, nb)
    y32 = torch.empty((rows, H), dtype=torch.float32, device=DEV)
    M.moe_grouped_ffn(None, x, _i32(src), _i32(offsets), E, rows, H, I, w13, w2, 1, y32, 0,
                      ws, nb)
    torch.cuda.synchronize()
    ref = O.grouped_ffn(to_np(x), src, offsets, to_np(w13), to_np(w2))
    scale = np.abs(ref).max()
    for out in (y_perm, y32):
        got = to_np(out).astype(np.float64)
        # every row, and each expert's rows on their own (a wrong tile would
        # show at its expert's scale)
        assert np.abs(got - ref).max() / scale <= 1e-2
        for e in range(E):
            r0, r1 = offsets[e], offsets[e + 1]
            if r1 > r0:
                assert np.abs(got[r0:r1] - ref[r0:r1]).max() / scale <= 1e-2, e


def test_combine_skips_nonlocal_and_adds_shared():
    T, k, H = 5, 3, 64
    y_perm = torch.randn((6, H), device=DEV)
    dst = np.array([[0, -1, 1], [-1, -1, -1], [2, 3, -1], [4, 5, -1], [-1, -1, -1]])
    wts = np.random.default_rng(0).random((T, k)).astype(np.float32)
    ysh = torch.randn((T, H), device=DEV)
    y = torch.empty((T, H), device=DEV)
    M.moe_combine(y_perm, 0, _i32(dst), _f32(wts), T, k, H, ysh, y, 0)
    torch.cuda.synchronize()
    ref = O.combine(to_np(y_perm).astype(np.float64), dst, wts, to_np(ysh))
    np.testing.assert_allclose(to_np(y), ref, rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------- whole layer, reduced sizes

SMALL = [
    # (config, H, I, E)   -- same k / mode / skew / shared expert as the config
    ("mixtral_8x7b", 256, 448, 8),
    ("qwen3_ep_all128", 256, 192, 128),
    ("deepseek_v3", 256, 128, 256),
]


@pytest.mark.parametrize("name,H,I,E", SMALL)
@pytest.mark.parametrize("T", [1, 5, 64, 65, 300])
def test_layer_small(name, H, I, E, T):
    cfg = W.CONFIGS[name]
    L = W.make_layer(cfg, device=DEV, seed=1, T_max=T, H=H, I=I, E=E)
    if cfg.I_shared:
        s = 1.0 / H ** 0.5
        L.w13_shared = (torch.randn((2 * I, H), device=DEV) * s).to(torch.bfloat16)
        L.w2_shared = (torch.randn((H, I), device=DEV) * s).to(torch.bfloat16)
    gl = GpuLayer(L)
    check_layer(gl, gl.run(T), T)
    # where moe_layer takes the single-launch path, the staged one as well
    if M.moe_layer_path(gl.desc, T) == "decode":
        check_layer(gl, gl.run(T, path="staged"), T)


# the ABI's limits: many experts and k > 16 (gating with 4-wave tiles and
# unstaged logits, two choice slots per lane)
@pytest.mark.parametrize("E,k,T", [(512, 20, 1), (512, 20, 70), (1024, 32, 64), (1024, 32, 129)])
def test_layer_many_experts(E, k, T):
    import dataclasses
    cfg = dataclasses.replace(W.CONFIGS["qwen3_ep_all128"], E=E, k=k)
    L = W.make_layer(cfg, device=DEV, seed=7, T_max=T, H=256, I=64, E=E)
    gl = GpuLayer(L)
    check_layer(gl, gl.run(T), T)


# shapes that take the LDS-tiled prefill kernel (>= 64 rows per expert,
# I_loc a multiple of 128, H a multiple of 256), with ragged expert tails
TILE = [
    ("mixtral_8x7b", 512, 256, 8, 2000),        # 256-row tiles (500 rows per expert)
    ("qwen3_ep_all128", 256, 128, 16, 1500),    # 256-row tiles, skewed
    ("mixtral_8x7b", 256, 256, 8, 300),
    ("mixtral_8x7b", 512, 384, 8, 1000),
    ("qwen3_ep_all128", 256, 128, 16, 1111),
    ("deepseek_v3", 512, 256, 32, 700),
    ("qwen3_ep_all128", 512, 192, 16, 700),     # gate/up width 192: 64-column tiles
    ("mixtral_8x7b", 512, 256, 8, 200),         # 50 rows per expert: 128-column down tiles
]


@pytest.mark.parametrize("name,H,I,E,T", TILE)
def test_layer_tile_path(name, H, I, E, T):
    cfg = W.CONFIGS[name]
    L = W.make_layer(cfg, device=DEV, seed=5, T_max=T, H=H, I=I, E=E)
    if cfg.I_shared:
        s = 1.0 / H ** 0.5
        L.w13_shared = (torch.randn((2 * I, H), device=DEV) * s).to(torch.bfloat16)
        L.w2_shared = (torch.randn((H, I), device=DEV) * s).to(torch.bfloat16)
    gl = GpuLayer(L)
    check_layer(gl, gl.run(T), T)
    gl2 = GpuLayer(L, e_begin=E // 4, e_end=E // 2)
    check_layer(gl2, gl2.run(T), T)


@pytest.mark.parametrize("name,T,H,I,E", [("mixtral_8x7b", 200, 512, 256, 8),
                                           ("qwen3_tp8_rank0", 8, 1024, 1536, 128),
                                           ("qwen3_tp8_rank0", 3, 1024, 1536, 128)])
def test_narrower_tiles_match_the_grouped_ffn_bit_for_bit(name, T, H, I, E):
    """Where plan_layer_gemms narrows a GEMM's column tiles, moe_layer and
    moe_grouped_ffn (which keeps the wide ones) give the same bits on the
    layer's own routing, since each output's sum over K runs in the same
    order either way.  Mixtral shape, a few experts of one 128-row tile each:
    the down projection on 128-column LDS tiles instead of 256.  TP share
    (I/P = 192) at a few tokens: the direct gate/up GEMM on 8-column tiles,
    8 gate and 8 up rows in one MFMA operand, instead of 16 columns."""
    cfg = W.CONFIGS[name]
    L = W.make_layer(cfg, device=DEV, seed=11, T_max=T, H=H, I=I, E=E)
    gl = GpuLayer(L)
    out = gl.run(T, path="staged")
    rows = T * gl.k
    dtc = gl.dt
    y_perm = torch.empty((rows, gl.H), dtype=L.x.dtype, device=DEV)
    nb = M.moe_grouped_ffn_workspace_size(rows, gl.E, gl.H, gl.I_loc, dtc)
    ws = ws_tensor(nb)
    M.moe_grouped_ffn(None, L.x[:T], out["src_token"], out["offsets"], gl.E, rows, gl.H, gl.I_loc,
                      gl.w13, gl.w2, dtc, y_perm, dtc, ws, nb)
    y = torch.empty((T, gl.H), dtype=L.x.dtype, device=DEV)
    M.moe_combine(y_perm, dtc, out["dst_row"], out["w"], T, gl.k, gl.H, None, y, dtc)
    torch.cuda.synchronize()
    assert torch.equal(y, out["y"])


# The shared expert's GEMMs ride in the routed GEMMs' launches or run in
# launches of their own, each GEMM by its own choice (plan_layer_gemms; the
# host test test_host_tile_choice.py asserts these plans).  Always through
# the staged path, which is the one that makes these launches (moe_layer
# would take the single-launch path at the smaller T here).  At H = 1024,
# I = 256, E = 64, k = 8:
#   I_shared = 256: both GEMMs ride in the direct launches (T = 1), both take
#     the routed 16-row tile in place of their own LDS tile (T = 16), both ride
#     in the LDS-tiled launches (T = 64), both take the routed 128-row tile in
#     place of their own 256-row one (T = 600);
#   I_shared = 512: both ride as with 256 (the down projections in the
#     kernel that shares its rows' activations through LDS);
#   I_shared = 4096: the gate/up GEMM rides in the routed launch and the down
#     projection has its own (T = 1: its 4096-long contraction takes the plain
#     direct kernel, with more waves per block than the routed one; T = 16:
#     the gate/up GEMM switched to the routed tile, the down projection on its
#     own 128-row tile).
# The opposite mix -- the gate/up GEMM in its own launch, the down projection
# riding -- needs a long contraction: H = 6144, I = 2048, I_shared = 4096,
# E = 32, k = 8, T = 4 (routed gate/up on LDS tiles, its down projection
# direct, the shared expert's direct 16-row tile fitting only the latter).
SHARED_CASES = [(1024, 256, 64, 256, 1), (1024, 256, 64, 256, 16), (1024, 256, 64, 256, 64),
                (1024, 256, 64, 256, 600), (1024, 256, 64, 512, 1), (1024, 256, 64, 512, 16),
                (1024, 256, 64, 512, 64), (1024, 256, 64, 4096, 1), (1024, 256, 64, 4096, 16),
                (6144, 2048, 32, 4096, 4),
                # 256-row tiles for the routed experts (about 409 rows each) and
                # 1636 dense shared-expert rows: six full tiles and a 100-row
                # tail that runs two N-tiles wide
                (512, 256, 32, 256, 1636)]


@pytest.mark.parametrize("H,I,E,I_shared,T", SHARED_CASES)
def test_shared_expert_with_the_routed_launches(H, I, E, I_shared, T):
    cfg = W.CONFIGS["deepseek_v3"]
    L = W.make_layer(cfg, device=DEV, seed=8, T_max=T, H=H, I=I, E=E)
    s = 1.0 / H ** 0.5
    g = torch.Generator(device=DEV).manual_seed(8)
    L.w13_shared = (torch.randn((2 * I_shared, H), device=DEV, generator=g) * s).to(torch.bfloat16)
    L.w2_shared = (torch.randn((H, I_shared), device=DEV, generator=g) * s).to(torch.bfloat16)
    ranges = (dict(), dict(e_begin=8, e_end=24)) if E <= 32 else (dict(), dict(e_begin=8, e_end=40))
    for kw in ranges:
        gl = GpuLayer(L, **kw)
        check_layer(gl, gl.run(T, path="staged"), T)
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1, 9, 64, 200])
def test_layer_small_tp_and_ep_shares(T):
    cfg = W.CONFIGS["qwen3_ep_all128"]
    L = W.make_layer(cfg, device=DEV, seed=2, T_max=T, H=256, I=256, E=32)
    for kw in (dict(tp_P=4, tp_rank=1), dict(tp_P=8, tp_rank=7), dict(e_begin=8, e_end=24)):
        gl = GpuLayer(L, **kw)
        check_layer(gl, gl.run(T), T)


def test_layer_toy_f32_full():
    cfg = W.CONFIGS["toy_f32"]
    L = W.make_layer(cfg, device=DEV, seed=0)
    gl = GpuLayer(L)
    res = check_layer(gl, gl.run(64), 64)
    assert res["y_rel"] <= 1e-5


def test_layer_is_bitwise_repeatable():
    cfg = W.CONFIGS["deepseek_v3"]
    L = W.make_layer(cfg, device=DEV, seed=3, T_max=200, H=256, I=128, E=64)
    L.w13_shared = L.w13[0].clone()
    L.w2_shared = L.w2[0].clone()
    gl = GpuLayer(L)
    a = gl.run(200)
    b = gl.run(200)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_shares_sum_to_full_layer():
    cfg = W.CONFIGS["qwen3_ep_all128"]
    T = 50
    L = W.make_layer(cfg, device=DEV, seed=4, T_max=T, H=256, I=256, E=16)
    full = GpuLayer(L).run(T)["y"].double()
    tp = sum(GpuLayer(L, tp_P=4, tp_rank=r).run(T)["y"].double() for r in range(4))
    ep = sum(GpuLayer(L, e_begin=a, e_end=b).run(T)["y"].double() for a, b in ((0, 5), (5, 16)))
    torch.cuda.synchronize()
    scale = full.abs().max().item()
    assert (tp - full).abs().max().item() / scale <= 2e-2
    assert (ep - full).abs().max().item() / scale <= 2e-2


def test_rejects_bad_arguments():
    cfg = W.CONFIGS["qwen3_ep_all128"]
    L = W.make_layer(cfg, device=DEV, seed=0, T_max=4, H=256, I=192, E=16)
    gl = GpuLayer(L)
    y = torch.empty((4, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(M.MoEError) as e:
        M.moe_layer(gl.desc, 4, L.x, y, gl.ws, 16)
    assert e.value.status == 3
    with pytest.raises(M.MoEError) as e:
        M.moe_layer(gl.desc, -1, L.x, y, gl.ws, gl.ws_bytes)
    assert e.value.status == 1
