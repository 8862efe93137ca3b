"""The capacity-factor variant on the GPU: moe_permute_capacity and
moe_layer_capacity, packed and padded, against the oracle's permute_capacity
/ moe_layer(capacity=C), and the properties the pages state for it."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import workloads as W
from harness import GpuLayer, to_np, ws_tensor
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"
BIG = 2 ** 31 - 1


def _skewed_ids(T, k, E, seed):
    """Distinct experts per token drawn with a Zipf-like skew, so that some
    experts overflow a capacity near the mean."""
    r = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** 0.8
    p = p / p.sum()
    if T == 0:
        return np.zeros((0, k), int)
    return np.stack([r.choice(E, size=k, replace=False, p=p) for _ in range(T)])


def _permute(ids, E, eb, ee, C, padded, x=None):
    T, k = ids.shape
    E_loc = ee - eb
    rows = E_loc * C if padded else max(T * k, 1)
    out = dict(counts=torch.empty((E_loc,), dtype=torch.int32, device=DEV),
               offsets=torch.empty((E_loc + 1,), dtype=torch.int32, device=DEV),
               src=torch.full((max(rows, 1),), -7, dtype=torch.int32, device=DEV),
               dst=torch.empty((max(T, 1), k), dtype=torch.int32, device=DEV),
               dropped=torch.full((4,), -7, dtype=torch.int32, device=DEV))
    H, dt, x_perm = 0, 0, None
    if x is not None:
        H, dt = x.shape[1], M.dtype_code(x)
        x_perm = torch.full((max(rows, 1), H), 3.0, dtype=x.dtype, device=DEV)
        out["x_perm"] = x_perm
    nb = M.moe_permute_workspace_size(T, k, E_loc)
    ids_d = torch.as_tensor(ids if T else np.zeros((1, k)), dtype=torch.int32,
                            device=DEV).contiguous()
    M.moe_permute_capacity(ids_d, T, k, E, eb, ee, C, padded, x, H, dt, out["counts"],
                           out["offsets"], out["src"], out["dst"], x_perm, out["dropped"],
                           ws_tensor(nb), nb)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("T", [5, 64, 65, 1000, 4097])
@pytest.mark.parametrize("cap", ["zero", "one", "cf1", "cf1.25", "big"])
@pytest.mark.parametrize("eb,ee", [(0, 16), (4, 12)])
@pytest.mark.parametrize("padded", [0, 1])
def test_permute_capacity_matches_oracle(T, cap, eb, ee, padded):
    E, k = 16, 4
    ids = _skewed_ids(T, k, E, seed=T + eb)
    C = {"zero": 0, "one": 1, "cf1": O.expert_capacity(1.0, T * k, E),
         "cf1.25": O.expert_capacity(1.25, T * k, E), "big": BIG}[cap]
    if padded and cap == "big":
        pytest.skip("E_loc * capacity does not fit an int (rejected on the host, see test_abi)")
    x = torch.randn((T, 64), device=DEV).to(torch.bfloat16) if padded else None
    out = _permute(ids, E, eb, ee, C, padded, x)
    rc, ro, rs, rd, rdrop = O.permute_capacity(ids, eb, ee, C, padded=bool(padded))
    assert np.array_equal(to_np(out["counts"]), rc)
    assert np.array_equal(to_np(out["offsets"]), ro)
    rows = int(ro[-1])
    assert np.array_equal(to_np(out["src"])[:rows], rs)
    assert np.array_equal(to_np(out["dst"])[:T], rd)
    assert int(out["dropped"][0]) == rdrop
    if cap == "cf1":
        assert rdrop > 0, "the skew should overflow a capacity at the mean"
    if x is not None and rows:
        # the fixed-shape token buffer: kept rows are copies, padding rows zero
        xp = out["x_perm"][:rows]
        live = torch.as_tensor(rs >= 0, device=DEV)
        src_l = torch.as_tensor(np.maximum(rs, 0), device=DEV).long()
        assert torch.equal(xp[live], x[src_l[live]])
        assert torch.count_nonzero(xp[~live]).item() == 0


# More than 256 local experts: the scan block finishes counts, offsets and
# the dropped total with block-wide scans instead of one wave (T = 40: the
# gating kernel's own single-tile finish; T = 1000: the scan kernel).
@pytest.mark.parametrize("T", [40, 1000])
@pytest.mark.parametrize("cap", ["cf1", "big"])
@pytest.mark.parametrize("eb,ee", [(0, 300), (10, 290)])
@pytest.mark.parametrize("padded", [0, 1])
def test_permute_capacity_many_local_experts(T, cap, eb, ee, padded):
    E, k = 300, 8
    ids = _skewed_ids(T, k, E, seed=3 * T + eb)
    C = O.expert_capacity(1.0, T * k, E) if cap == "cf1" else BIG
    if padded and cap == "big":
        pytest.skip("E_loc * capacity does not fit an int (rejected on the host, see test_abi)")
    out = _permute(ids, E, eb, ee, C, padded)
    rc, ro, rs, rd, rdrop = O.permute_capacity(ids, eb, ee, C, padded=bool(padded))
    assert np.array_equal(to_np(out["counts"]), rc)
    assert np.array_equal(to_np(out["offsets"]), ro)
    rows = int(ro[-1])
    assert np.array_equal(to_np(out["src"])[:rows], rs)
    assert np.array_equal(to_np(out["dst"])[:T], rd)
    assert int(out["dropped"][0]) == rdrop
    if cap == "cf1":
        assert rdrop > 0, "the skew should overflow a capacity at the mean"


def test_padded_permute_of_an_empty_batch():
    out = _permute(np.zeros((0, 4), int), 16, 2, 10, 5, 1)
    assert to_np(out["counts"]).tolist() == [0] * 8
    assert to_np(out["offsets"]).tolist() == [5 * i for i in range(9)]
    assert to_np(out["src"]).tolist() == [-1] * 40
    assert int(out["dropped"][0]) == 0


def _layer(name, T, seed, H=256, I=192, E=32):
    cfg = W.CONFIGS[name]
    L = W.make_layer(cfg, device=DEV, seed=seed, T_max=T, H=H, I=I, E=E)
    L.w13_shared = L.w2_shared = None
    return L


def _run_capacity(gl, T, C, x=None, padded=0):
    x = gl.L.x[:T] if x is None else x
    E_loc = gl.e_end - gl.e_begin
    rows = E_loc * C if padded else max(T * gl.k, 1)
    out = dict(y=torch.empty((T, gl.H), dtype=x.dtype, device=DEV),
               logits=torch.empty((T, gl.E), dtype=torch.float32, device=DEV),
               counts=torch.empty((E_loc,), dtype=torch.int32, device=DEV),
               offsets=torch.empty((E_loc + 1,), dtype=torch.int32, device=DEV),
               src_token=torch.full((max(rows, 1),), -7, dtype=torch.int32, device=DEV),
               dst_row=torch.empty((T, gl.k), dtype=torch.int32, device=DEV),
               dropped=torch.full((4,), -7, dtype=torch.int32, device=DEV))
    dbg = M.debug_out(logits=out["logits"], counts=out["counts"], offsets=out["offsets"],
                      src_token=out["src_token"], dst_row=out["dst_row"])
    if padded:
        nb = M.moe_layer_capacity_workspace_size(gl.desc, T, C, 1)
        assert nb > 0
        ws = ws_tensor(nb)
    else:
        ws, nb = gl.ws, gl.ws_bytes
    M.moe_layer_capacity(gl.desc, T, C, padded, x, out["y"], ws, nb, dbg, out["dropped"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["qwen3_ep_all128", "deepseek_v3", "mixtral_8x7b"])
@pytest.mark.parametrize("T,cf", [(64, 1.0), (300, 1.0), (300, 1.25)])
@pytest.mark.parametrize("padded", [0, 1])
def test_layer_capacity_matches_oracle(name, T, cf, padded):
    L = _layer(name, T, seed=31)
    gl = GpuLayer(L)
    C = O.expert_capacity(cf, T * gl.k, gl.E)
    out = _run_capacity(gl, T, C, padded=padded)
    lg = to_np(out["logits"])
    x = to_np(L.x[:T])
    ref, aux = O.moe_layer(x, None, [to_np(L.w13[e]) for e in range(gl.E)],
                           [to_np(L.w2[e]) for e in range(gl.E)], gl.k, gl.mode,
                           sel_bias=to_np(L.sel_bias), logits=lg, capacity=C,
                           padded=bool(padded))
    assert np.array_equal(to_np(out["counts"]), aux["counts"])
    assert np.array_equal(to_np(out["offsets"]), aux["offsets"])
    assert np.array_equal(to_np(out["dst_row"]), aux["dst_row"])
    rows = int(aux["offsets"][-1])
    assert np.array_equal(to_np(out["src_token"])[:rows], aux["src_token"])
    assert int(out["dropped"][0]) == aux["dropped"]
    y = to_np(out["y"]).astype(np.float64)
    assert np.abs(y - ref).max() / np.abs(ref).max() <= 1e-2
    if padded:
        # the layout moves rows, not results: every row is computed the same
        packed = _run_capacity(gl, T, C, padded=0)
        assert torch.equal(out["y"], packed["y"])


def test_padded_layer_on_an_expert_range():
    """An EP share (experts 8..23 of 32) with the padded layout: blocks of C
    rows for the local experts only."""
    T = 200
    L = _layer("qwen3_ep_all128", T, seed=34)
    gl = GpuLayer(L, e_begin=8, e_end=24)
    C = O.expert_capacity(1.0, T * gl.k, gl.E)
    out = _run_capacity(gl, T, C, padded=1)
    lg = to_np(out["logits"])
    ref, aux = O.moe_layer(to_np(L.x[:T]), None, [to_np(L.w13[e]) for e in range(8, 24)],
                           [to_np(L.w2[e]) for e in range(8, 24)], gl.k, gl.mode,
                           sel_bias=to_np(L.sel_bias), e_begin=8, e_end=24, logits=lg,
                           capacity=C, padded=True)
    assert to_np(out["offsets"]).tolist() == [C * i for i in range(17)]
    assert np.array_equal(to_np(out["src_token"])[:16 * C], aux["src_token"])
    assert np.array_equal(to_np(out["dst_row"]), aux["dst_row"])
    y = to_np(out["y"]).astype(np.float64)
    assert np.abs(y - ref).max() / np.abs(ref).max() <= 1e-2


def test_fixed_shape_chain_computes_padding_as_zero():
    """The fixed-shape form of the padded variant: moe_permute_capacity gathers
    x into E_loc blocks of C rows (padding zero), moe_grouped_ffn runs every
    block in full, and the combine reads the kept rows.  Padding rows come out
    exactly zero, and the result equals the oracle's layer."""
    name, T = "mixtral_8x7b", 300
    L = _layer(name, T, seed=35)
    gl = GpuLayer(L)
    full = gl.run(T)
    ids, w = to_np(full["ids"]), full["w"]
    E, k, H, I = gl.E, gl.k, gl.H, gl.I_loc
    C = O.expert_capacity(1.25, T * k, E)
    x = L.x[:T]
    pm = _permute(ids, E, 0, E, C, 1, x)
    rows = E * C
    dt = M.dtype_code(x)
    y_perm = torch.full((rows, H), 5.0, dtype=x.dtype, device=DEV)
    nb = M.moe_grouped_ffn_workspace_size(rows, E, H, I, dt)
    M.moe_grouped_ffn(pm["x_perm"], None, None, pm["offsets"], E, rows, H, I, L.w13, L.w2, dt,
                      y_perm, dt, ws_tensor(nb), nb)
    y = torch.empty((T, H), dtype=x.dtype, device=DEV)
    M.moe_combine(y_perm, dt, pm["dst"], w, T, k, H, None, y, dt)
    torch.cuda.synchronize()
    src = to_np(pm["src"])
    pad = torch.as_tensor(src < 0, device=DEV)
    assert pad.any()
    assert torch.count_nonzero(y_perm[pad]).item() == 0
    ref, aux = O.moe_layer(to_np(x), None, [to_np(L.w13[e]) for e in range(E)],
                           [to_np(L.w2[e]) for e in range(E)], k, gl.mode,
                           sel_bias=to_np(L.sel_bias), logits=to_np(full["logits"]), capacity=C,
                           padded=True)
    assert np.array_equal(src, aux["src_token"])
    y_np = to_np(y).astype(np.float64)
    assert np.abs(y_np - ref).max() / np.abs(ref).max() <= 1e-2


def test_large_capacity_is_the_dropless_staged_path():
    L = _layer("qwen3_ep_all128", 300, seed=32)
    gl = GpuLayer(L)
    a = _run_capacity(gl, 300, BIG)
    b = gl.run(300, path="staged")
    torch.cuda.synchronize()
    assert int(a["dropped"][0]) == 0
    assert torch.equal(a["y"], b["y"]) and torch.equal(a["dst_row"], b["dst_row"])


def test_dropping_makes_outputs_depend_on_batch_neighbours():
    """[CS349D L8] section 1.4, on the GPU: with a capacity a token's output
    changes with the tokens batched before it; alone it gets all its
    experts and equals the dropless output."""
    T = 200
    L = _layer("qwen3_ep_all128", T, seed=33)
    gl = GpuLayer(L)
    C = O.expert_capacity(1.0, T * gl.k, gl.E)
    out = _run_capacity(gl, T, C)
    dst = to_np(out["dst_row"])
    dropped_tokens = np.nonzero((dst < 0).any(axis=1))[0]
    assert len(dropped_tokens) > 0
    t = int(dropped_tokens[-1])
    alone = _run_capacity(gl, 1, C, x=L.x[t:t + 1].contiguous())
    free = gl.run(1, x=L.x[t:t + 1].contiguous(), path="staged")
    torch.cuda.synchronize()
    assert int(alone["dropped"][0]) == 0
    assert torch.equal(alone["y"], free["y"])
    assert not torch.allclose(alone["y"][0].float(), out["y"][t].float(), rtol=1e-2, atol=1e-3)
