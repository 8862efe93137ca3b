"""Parity of the local halves of the EP <-> TP weight reshard
(moe_reshard_ep_to_tp_pack, moe_reshard_tp_to_ep_interleave) with the oracle,
and the whole reshard with P ranks simulated in one GPU's memory (the
All-to-All done by plain copies between their buffers)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import workloads as W
from harness import GpuLayer, to_np
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _weights(n_total, I, H, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    w13 = torch.randn((n_total, 2 * I, H), generator=g, device=DEV).to(dtype)
    w2 = torch.randn((n_total, H, I), generator=g, device=DEV).to(dtype)
    return w13, w2


def _pack(w13_ep, w2_ep, P):
    n, twoI, H = w13_ep.shape
    I = twoI // 2
    s13 = torch.empty((P, n, 2 * I // P, H), dtype=w13_ep.dtype, device=DEV)
    s2 = torch.empty((P, n, H, I // P), dtype=w2_ep.dtype, device=DEV)
    M.moe_reshard_ep_to_tp_pack(w13_ep, w2_ep, n, I, H, P, M.dtype_code(w13_ep), s13, s2)
    return s13, s2


def _interleave(r13, r2, P):
    _, n, two_s, H = r13.shape
    I = two_s // 2 * P
    w13 = torch.empty((n, 2 * I, H), dtype=r13.dtype, device=DEV)
    w2 = torch.empty((n, H, I), dtype=r2.dtype, device=DEV)
    M.moe_reshard_tp_to_ep_interleave(r13, r2, n, I, H, P, M.dtype_code(r13), w13, w2)
    return w13, w2


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n,I,H,P", [(2, 64, 32, 4), (3, 256, 512, 8), (1, 96, 64, 1), (5, 128, 96, 2)])
def test_pack_and_interleave_match_oracle(dtype, n, I, H, P):
    w13, w2 = _weights(n, I, H, dtype, seed=n * 100 + P)
    s13, s2 = _pack(w13, w2, P)
    torch.cuda.synchronize()
    ref13, ref2 = O.reshard_ep_to_tp_pack(to_np(w13), to_np(w2), P)
    assert np.array_equal(to_np(s13), ref13) and np.array_equal(to_np(s2), ref2)
    # interleave on arbitrary chunks against the oracle, and as pack's inverse
    c13 = torch.randn_like(s13.float()).to(dtype)
    c2 = torch.randn_like(s2.float()).to(dtype)
    e13, e2 = _interleave(c13, c2, P)
    torch.cuda.synchronize()
    o13, o2 = O.reshard_tp_to_ep_interleave(to_np(c13), to_np(c2))
    assert np.array_equal(to_np(e13), o13) and np.array_equal(to_np(e2), o2)
    b13, b2 = _interleave(s13, s2, P)
    torch.cuda.synchronize()
    assert torch.equal(b13, w13) and torch.equal(b2, w2)


def test_reshard_round_trip_on_simulated_ranks():
    """EP -> TP -> EP for P = 4 ranks of the Figure 2 configuration scaled
    up: every rank ends with exactly its tensor-parallel share, and back."""
    P, n, I, H = 4, 3, 256, 256
    w13, w2 = _weights(P * n, I, H, torch.bfloat16, seed=7)
    # EP -> TP: pack on every rank, exchange, and the received chunks in
    # peer order are the TP layout
    sends = [_pack(w13[r * n:(r + 1) * n].contiguous(), w2[r * n:(r + 1) * n].contiguous(), P)
             for r in range(P)]
    tp = []
    for r in range(P):
        t13 = torch.cat([sends[p][0][r] for p in range(P)], dim=0)   # the All-to-All
        t2 = torch.cat([sends[p][1][r] for p in range(P)], dim=0)
        ref13, ref2 = O.tp_shard(to_np(w13), to_np(w2), r, P)
        assert np.array_equal(to_np(t13), ref13) and np.array_equal(to_np(t2), ref2)
        tp.append((t13, t2))
    # TP -> EP: split by expert owner (contiguous rows), exchange, interleave
    for r in range(P):
        r13 = torch.stack([tp[p][0][r * n:(r + 1) * n] for p in range(P)])
        r2 = torch.stack([tp[p][1][r * n:(r + 1) * n] for p in range(P)])
        e13, e2 = _interleave(r13.contiguous(), r2.contiguous(), P)
        torch.cuda.synchronize()
        assert torch.equal(e13, w13[r * n:(r + 1) * n]) and torch.equal(e2, w2[r * n:(r + 1) * n])


def test_resharded_weights_compute_the_same_layer():
    """The same function over byte-identical weights: the TP shares the
    reshard builds, run through moe_layer and summed over ranks, equal the EP
    shares' sum."""
    cfg = W.CONFIGS["qwen3_ep_all128"]
    P, E, I, H, T = 4, 16, 256, 256, 48
    L = W.make_layer(cfg, device=DEV, seed=11, T_max=T, H=H, I=I, E=E)
    n = E // P
    sends = [_pack(L.w13[r * n:(r + 1) * n].contiguous(), L.w2[r * n:(r + 1) * n].contiguous(), P)
             for r in range(P)]
    y_tp = 0
    for r in range(P):
        t13 = torch.cat([sends[p][0][r] for p in range(P)], dim=0).contiguous()
        t2 = torch.cat([sends[p][1][r] for p in range(P)], dim=0).contiguous()
        Lr = W.LayerInputs(cfg=L.cfg, x=L.x, w_r=L.w_r, w13=t13, w2=t2, logit_bias=L.logit_bias,
                           sel_bias=L.sel_bias)
        y_tp = y_tp + GpuLayer(Lr).run(T)["y"].double()
    y_ep = sum(GpuLayer(L, e_begin=r * n, e_end=(r + 1) * n).run(T)["y"].double()
               for r in range(P))
    torch.cuda.synchronize()
    scale = y_ep.abs().max().item()
    assert (y_tp - y_ep).abs().max().item() / scale <= 2e-2


def test_full_size_rank_share_sampled():
    """One rank of the Qwen3-235B-A22B-shaped layer at P = 8 (16 experts,
    I = 1536, H = 4096): sampled chunk rows against their EP rows, and the
    exact inverse."""
    P, n, I, H = 8, 16, 1536, 4096
    w13, w2 = _weights(n, I, H, torch.bfloat16, seed=3)
    s13, s2 = _pack(w13, w2, P)
    torch.cuda.synchronize()
    r = np.random.default_rng(5)
    s = I // P
    for _ in range(64):
        p, e, j = int(r.integers(P)), int(r.integers(n)), int(r.integers(2 * s))
        row = p * s + j if j < s else I + p * s + (j - s)
        assert torch.equal(s13[p, e, j], w13[e, row])
        h = int(r.integers(H))
        assert torch.equal(s2[p, e, h], w2[e, h, p * s:(p + 1) * s])
    b13, b2 = _interleave(s13, s2, P)
    torch.cuda.synchronize()
    assert torch.equal(b13, w13) and torch.equal(b2, w2)
