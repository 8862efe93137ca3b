"""The capacity-factor variant on the GPU: moe_permute_capacity and
moe_layer_capacity against the oracle's permute_capacity / moe_layer
(capacity=C), and the properties the pages state for it."""
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


@pytest.mark.parametrize("T", [5, 64, 65, 1000, 4097])
@pytest.mark.parametrize("cap", ["zero", "one", "cf1", "cf1.25", "big"])
@pytest.mark.parametrize("eb,ee", [(0, 16), (4, 12)])
def test_permute_capacity_matches_oracle(T, cap, eb, ee):
    E, k = 16, 4
    ids = _skewed_ids(T, k, E, seed=T + eb)
    C = {"zero": 0, "one": 1, "cf1": O.expert_capacity(1.0, T * k, E),
         "cf1.25": O.expert_capacity(1.25, T * k, E), "big": BIG}[cap]
    E_loc = ee - eb
    counts = torch.empty((E_loc,), dtype=torch.int32, device=DEV)
    offsets = torch.empty((E_loc + 1,), dtype=torch.int32, device=DEV)
    src = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    dst = torch.empty((T, k), dtype=torch.int32, device=DEV)
    dropped = torch.full((4,), -7, dtype=torch.int32, device=DEV)
    nb = M.moe_permute_workspace_size(T, k, E_loc)
    ids_d = torch.as_tensor(ids, dtype=torch.int32, device=DEV).contiguous()
    M.moe_permute_capacity(ids_d, T, k, E, eb, ee, C, None, 0, 0, counts, offsets, src, dst, None,
                           dropped, ws_tensor(nb), nb)
    torch.cuda.synchronize()
    rc, ro, rs, rd, rdrop = O.permute_capacity(ids, eb, ee, C)
    assert np.array_equal(to_np(counts), rc)
    assert np.array_equal(to_np(offsets), ro)
    rows = int(ro[-1])
    assert np.array_equal(to_np(src)[:rows], rs)
    assert np.array_equal(to_np(dst), rd)
    assert int(dropped[0]) == rdrop
    if cap == "cf1":
        assert rdrop > 0, "the skew should overflow a capacity at the mean"


def _layer(name, T, seed, H=256, I=192, E=32):
    cfg = W.CONFIGS[name]
    L = W.make_layer(cfg, device=DEV, seed=seed, T_max=T, H=H, I=I, E=E)
    L.w13_shared = L.w2_shared = None
    return L


def _run_capacity(gl, T, C, x=None):
    x = gl.L.x[:T] if x is None else x
    out = dict(y=torch.empty((T, gl.H), dtype=x.dtype, device=DEV),
               logits=torch.empty((T, gl.E), dtype=torch.float32, device=DEV),
               counts=torch.empty((gl.E,), dtype=torch.int32, device=DEV),
               dst_row=torch.empty((T, gl.k), dtype=torch.int32, device=DEV),
               dropped=torch.full((4,), -7, dtype=torch.int32, device=DEV))
    dbg = M.debug_out(logits=out["logits"], counts=out["counts"], dst_row=out["dst_row"])
    M.moe_layer_capacity(gl.desc, T, C, x, out["y"], gl.ws, gl.ws_bytes, dbg, out["dropped"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["qwen3_ep_all128", "deepseek_v3", "mixtral_8x7b"])
@pytest.mark.parametrize("T,cf", [(64, 1.0), (300, 1.0), (300, 1.25)])
def test_layer_capacity_matches_oracle(name, T, cf):
    L = _layer(name, T, seed=31)
    gl = GpuLayer(L)
    C = O.expert_capacity(cf, T * gl.k, gl.E)
    out = _run_capacity(gl, T, C)
    lg = to_np(out["logits"])
    x = to_np(L.x[:T])
    ref, aux = O.moe_layer(x, None, [to_np(L.w13[e]) for e in range(gl.E)],
                           [to_np(L.w2[e]) for e in range(gl.E)], gl.k, gl.mode,
                           sel_bias=to_np(L.sel_bias), logits=lg, capacity=C)
    assert np.array_equal(to_np(out["counts"]), aux["counts"])
    assert np.array_equal(to_np(out["dst_row"]), aux["dst_row"])
    assert int(out["dropped"][0]) == aux["dropped"]
    y = to_np(out["y"]).astype(np.float64)
    assert np.abs(y - ref).max() / np.abs(ref).max() <= 1e-2


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
