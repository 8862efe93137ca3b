"""Parity of the single-launch decode path (moe_layer_decode) with the oracle,
its agreement with the staged path, and the synchronisation block it keeps
in the workspace across calls, including HIP-graph replays."""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import workloads as W
from harness import GpuLayer, check_layer, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"

SMALL = [
    # (config, H, I, E): the configs' k, gating mode, skew and shared expert
    ("mixtral_8x7b", 256, 448, 8),
    ("qwen3_ep_all128", 256, 192, 128),
    ("qwen3_ep_all128", 512, 96, 100),      # E not a multiple of 16
    ("deepseek_v3", 256, 128, 256),
]


def _layer(name, H, I, E, T, seed):
    cfg = W.CONFIGS[name]
    L = W.make_layer(cfg, device=DEV, seed=seed, T_max=T, H=H, I=I, E=E)
    if cfg.I_shared:
        s = 1.0 / H ** 0.5
        L.w13_shared = (torch.randn((2 * 2 * I, H), device=DEV) * s).to(torch.bfloat16)
        L.w2_shared = (torch.randn((H, 2 * I), device=DEV) * s).to(torch.bfloat16)
    return L


@pytest.mark.parametrize("name,H,I,E", SMALL)
@pytest.mark.parametrize("T", [1, 5, 16, 33, 64])
def test_decode_small(name, H, I, E, T):
    L = _layer(name, H, I, E, T, seed=21)
    gl = GpuLayer(L)
    check_layer(gl, gl.run(T, path="decode"), T)
    assert gl.sync_error() == 0


@pytest.mark.parametrize("T", [1, 9, 64])
def test_decode_tp_and_ep_shares(T):
    cfg = W.CONFIGS["qwen3_ep_all128"]
    L = W.make_layer(cfg, device=DEV, seed=22, T_max=T, H=256, I=256, E=32)
    for kw in (dict(tp_P=4, tp_rank=1), dict(tp_P=8, tp_rank=7), dict(e_begin=8, e_end=24),
               dict(e_begin=31, e_end=32)):
        gl = GpuLayer(L, **kw)
        check_layer(gl, gl.run(T, path="decode"), T)
        assert gl.sync_error() == 0


def test_decode_k_16_and_top_e():
    # k = 16 (one choice per lane of a gating row) and k = E
    for E, k, T in ((64, 16, 32), (16, 16, 8)):
        cfg = dataclasses.replace(W.CONFIGS["qwen3_ep_all128"], E=E, k=k)
        L = W.make_layer(cfg, device=DEV, seed=23, T_max=T, H=256, I=64, E=E)
        gl = GpuLayer(L)
        check_layer(gl, gl.run(T, path="decode"), T)


def test_decode_matches_staged():
    L = _layer("deepseek_v3", 512, 128, 64, 48, seed=24)
    gl = GpuLayer(L)
    a = gl.run(48, path="decode")
    b = gl.run(48, path="staged")
    torch.cuda.synchronize()
    for key in ("logits", "ids", "w", "counts", "offsets", "dst_row"):
        assert torch.equal(a[key], b[key]), key
    rows = int(a["offsets"][-1])
    assert torch.equal(a["src_token"][:rows], b["src_token"][:rows])
    ya, yb = a["y"].double(), b["y"].double()
    assert (ya - yb).abs().max().item() <= 1e-2 * yb.abs().max().item()


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("E", [8, 100, 256])
def test_whole_wave_gating_matches_row_gating_bitwise(mode, E):
    """A batch (or tile) of at most 16 tokens is gated a whole wave per token
    (a quarter of the keys per lane), a larger one a 16-lane row per token.
    Gating is per token, so the first 16 tokens of a 17-token batch (row
    gating) must get the logits, ids and weights of a 16-token batch
    (whole-wave gating) bit for bit, on both paths and in every gating mode;
    at 16 tokens the two paths also agree on the routing metadata."""
    cfg = dataclasses.replace(W.CONFIGS["deepseek_v3"], mode=mode, I_shared=0)
    L = W.make_layer(cfg, device=DEV, seed=26 + mode, T_max=17, H=256, I=128, E=E)
    gl = GpuLayer(L)
    rows = gl.run(17, path="staged")
    wave = {path: gl.run(16, path=path) for path in ("staged", "decode")}
    torch.cuda.synchronize()
    for path, a in wave.items():
        for key in ("logits", "ids", "w"):
            assert torch.equal(a[key], rows[key][:16]), (path, key)
    for key in ("counts", "offsets", "dst_row"):
        assert torch.equal(wave["staged"][key], wave["decode"][key]), key


def test_decode_repeated_calls_and_sync_block():
    """Many calls in a row on one workspace (the counter sets alternate), with
    changing T: every call matches the first call at its T bit for bit."""
    L = _layer("qwen3_ep_all128", 256, 192, 128, 64, seed=25)
    gl = GpuLayer(L, T_max=64)
    first = {}
    for i, T in enumerate([3, 64, 3, 17, 64, 1, 17, 3, 64, 1, 1]):
        out = gl.run(T, path="decode")
        torch.cuda.synchronize()
        if T not in first:
            first[T] = {k: v.clone() for k, v in out.items()}
            check_layer(gl, out, T)
        else:
            for key, v in out.items():
                assert torch.equal(v, first[T][key]), (i, T, key)
    ws = gl.ws.view(torch.int32)
    assert int(ws[1]) == 0           # error word
    assert int(ws[0]) in (0, 1)      # parity of the counter set in use


def test_decode_and_staged_share_a_workspace():
    L = _layer("mixtral_8x7b", 256, 448, 8, 200, seed=26)
    gl = GpuLayer(L, T_max=200)
    for T, path in ((4, "decode"), (200, "staged"), (7, "decode"), (64, "staged"),
                    (7, "decode"), (16, "auto")):
        check_layer(gl, gl.run(T, path=path), T)
    assert gl.sync_error() == 0


def test_decode_in_hip_graph():
    """Replays of a captured decode call, with eager work between replays,
    each checked against the eager result."""
    L = _layer("deepseek_v3", 256, 128, 256, 24, seed=27)
    gl = GpuLayer(L)
    T = 24
    x = L.x[:T]
    y = torch.empty((T, gl.H), dtype=x.dtype, device=DEV)
    M.moe_layer_decode(gl.desc, T, x, y, gl.ws, gl.ws_bytes)
    torch.cuda.synchronize()
    ref = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        y.zero_()
        with torch.cuda.graph(g, stream=s):
            M.moe_layer_decode(gl.desc, T, x, y, gl.ws, gl.ws_bytes, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for i in range(5):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {i}"
        gl.run(T, path="staged")     # eager work on the same workspace between replays
        torch.cuda.synchronize()
    assert gl.sync_error() == 0


def test_decode_rejects_unsupported():
    L = _layer("qwen3_ep_all128", 256, 192, 128, 65, seed=28)
    gl = GpuLayer(L)
    y = torch.empty((65, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(M.MoEError) as e:
        M.moe_layer_decode(gl.desc, 65, L.x[:65], y, gl.ws, gl.ws_bytes)
    assert e.value.status == 2
    # moe_layer takes the staged path for the same call
    M.moe_layer(gl.desc, 65, L.x[:65], y, gl.ws, gl.ws_bytes)
    torch.cuda.synchronize()


def test_decode_bitwise_repeatable_and_no_local_rows():
    L = _layer("qwen3_ep_all128", 256, 192, 128, 2, seed=29)
    ids = None
    gl = GpuLayer(L)
    a = gl.run(2, path="decode")
    b = gl.run(2, path="decode")
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
    ids = set(to_np(a["ids"]).astype(int).ravel().tolist())
    # an expert range no token routes to: zero rows, output all zeros
    free = [e for e in range(128) if e not in ids]
    gl2 = GpuLayer(L, e_begin=free[0], e_end=free[0] + 1)
    out = gl2.run(2, path="decode")
    torch.cuda.synchronize()
    assert int(out["counts"][0]) == 0 and int(out["offsets"][1]) == 0
    assert torch.count_nonzero(out["y"]).item() == 0
    assert np.all(to_np(out["dst_row"]) == -1)
