"""Degenerate inputs on the GPU: empty batches through every entry point that
takes one (a no-op that leaves the outputs untouched), a grouped FFN with no
rows, and a capacity of zero, which drops every pair (the layer's output is
then the shared expert alone, or zero)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import workloads as W
from harness import GpuLayer, to_np, ws_tensor
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINEL = -5.0


def _full(shape, dtype=torch.float32, value=SENTINEL):
    return torch.full(shape, value, dtype=dtype, device=DEV)


def test_empty_batch_is_a_no_op_everywhere():
    E, k, H = 16, 4, 256
    x = _full((1, H), torch.bfloat16, 1.0)
    w_r = _full((E, H), torch.bfloat16, 0.5)
    logits, ids, w = _full((1, E)), _full((1, k), torch.int32, -5), _full((1, k))
    M.moe_route(x, w_r, 1, 0, H, E, k, 2, None, None, logits, ids, w)
    y_perm, dst = _full((1, H), torch.bfloat16), _full((1, k), torch.int32, -1)
    y = _full((1, H), torch.bfloat16)
    M.moe_combine(y_perm, 1, dst, w, 0, k, H, None, y, 1)
    M.moe_unpack_sum(y_perm, 1, dst, 0, k, H, y, 1)
    torch.cuda.synchronize()
    assert (logits == SENTINEL).all() and (ids == -5).all() and (w == SENTINEL).all()
    assert (y == SENTINEL).all()
    # the layer entry points, on real buffers
    L = W.make_layer(W.CONFIGS["qwen3_ep_all128"], device=DEV, seed=41, T_max=4, H=256, I=128,
                     E=32)
    gl = GpuLayer(L)
    y = _full((4, gl.H), torch.bfloat16)
    for fn in (M.moe_layer, M.moe_layer_staged, M.moe_layer_decode):
        fn(gl.desc, 0, L.x, y, gl.ws, gl.ws_bytes)
    M.moe_layer_capacity(gl.desc, 0, 3, 1, L.x, y, gl.ws, gl.ws_bytes)
    torch.cuda.synchronize()
    assert (y == SENTINEL).all()


def test_grouped_ffn_with_no_rows_writes_nothing():
    E, H, I, max_rows = 8, 256, 128, 64
    g = torch.Generator(device=DEV).manual_seed(5)
    w13 = torch.randn((E, 2 * I, H), generator=g, device=DEV).to(torch.bfloat16)
    w2 = torch.randn((E, H, I), generator=g, device=DEV).to(torch.bfloat16)
    x_perm = torch.randn((max_rows, H), generator=g, device=DEV).to(torch.bfloat16)
    offsets = torch.zeros((E + 1,), dtype=torch.int32, device=DEV)
    y_perm = _full((max_rows, H), torch.bfloat16)
    nb = M.moe_grouped_ffn_workspace_size(max_rows, E, H, I, 1)
    M.moe_grouped_ffn(x_perm, None, None, offsets, E, max_rows, H, I, w13, w2, 1, y_perm, 1,
                      ws_tensor(nb), nb)
    torch.cuda.synchronize()
    assert (y_perm == SENTINEL).all()


@pytest.mark.parametrize("padded", [0, 1])
@pytest.mark.parametrize("shared", [False, True])
def test_zero_capacity_drops_every_pair(padded, shared):
    T = 70
    cfg = W.CONFIGS["deepseek_v3"]
    L = W.make_layer(cfg, device=DEV, seed=42, T_max=T, H=256, I=128, E=32)
    if shared:
        s = 1.0 / 16
        L.w13_shared = (torch.randn((2 * 256, 256), device=DEV) * s).to(torch.bfloat16)
        L.w2_shared = (torch.randn((256, 256), device=DEV) * s).to(torch.bfloat16)
    else:
        L.w13_shared = L.w2_shared = None
    gl = GpuLayer(L)
    nb = M.moe_layer_capacity_workspace_size(gl.desc, T, 0, padded)
    y = _full((T, gl.H), torch.bfloat16)
    logits = torch.empty((T, gl.E), dtype=torch.float32, device=DEV)
    dst = torch.empty((T, gl.k), dtype=torch.int32, device=DEV)
    dropped = torch.zeros((4,), dtype=torch.int32, device=DEV)
    dbg = M.debug_out(logits=logits, dst_row=dst)
    M.moe_layer_capacity(gl.desc, T, 0, padded, L.x[:T], y, ws_tensor(nb), nb, dbg, dropped)
    torch.cuda.synchronize()
    assert int(dropped[0]) == T * gl.k
    assert (dst == -1).all()
    ref, aux = O.moe_layer(to_np(L.x[:T]), None, [to_np(L.w13[e]) for e in range(gl.E)],
                           [to_np(L.w2[e]) for e in range(gl.E)], gl.k, gl.mode,
                           sel_bias=to_np(L.sel_bias), logits=to_np(logits), capacity=0,
                           padded=bool(padded),
                           w13_shared=None if not shared else to_np(L.w13_shared),
                           w2_shared=None if not shared else to_np(L.w2_shared))
    assert aux["dropped"] == T * gl.k
    y_np = to_np(y).astype(np.float64)
    if shared:
        assert np.abs(y_np - ref).max() / np.abs(ref).max() <= 1e-2
    else:
        assert np.all(ref == 0.0) and np.all(y_np == 0.0)
