"""The seeded input recipe: determinism, layout of a share, routing skew."""
import numpy as np
import torch

import workloads as W
from oracle import moe_oracle as O


def test_inputs_are_deterministic_and_prefix_stable():
    cfg = W.CONFIGS["toy_f32"]
    a = W.make_layer(cfg, seed=3)
    b = W.make_layer(cfg, seed=3)
    c = W.make_layer(cfg, seed=4)
    assert torch.equal(a.x, b.x) and torch.equal(a.w13, b.w13) and torch.equal(a.w2, b.w2)
    assert not torch.equal(a.x, c.x)
    assert a.x.shape == (64, 256) and a.w13.shape == (8, 1024, 256) and a.w2.shape == (8, 256, 512)
    assert a.x.dtype == torch.float32


def test_bf16_inputs_are_bf16():
    cfg = W.CONFIGS["qwen3_ep_all128"]
    L = W.make_layer(cfg, seed=0, T_max=8, H=64, I=32, E=16)
    assert L.x.dtype == torch.bfloat16 and L.w13.dtype == torch.bfloat16
    assert L.logit_bias.dtype == torch.float32 and L.logit_bias.shape == (16,)


def test_zipf_bias_is_a_permuted_log_rank():
    b = W.zipf_logit_bias(128, 0.15, seed=0).double().numpy()
    ranks = np.sort(np.exp(-b / 0.15))
    np.testing.assert_allclose(ranks, np.arange(1, 129), rtol=1e-5)


def test_expert_parallel_share_is_a_range():
    w13 = torch.arange(4 * 6 * 2, dtype=torch.float32).reshape(4, 6, 2)
    w2 = torch.arange(4 * 2 * 3, dtype=torch.float32).reshape(4, 2, 3)
    a, b = W.share_weights(w13, w2, e_begin=1, e_end=3)
    assert torch.equal(a, w13[1:3]) and torch.equal(b, w2[1:3])


def _routing_counts(name, T):
    cfg = W.CONFIGS[name]
    L = W.make_layer(cfg, seed=0, T_max=T, experts=False)
    s = O.router_logits(L.x.float().numpy(), L.w_r.float().numpy(),
                        None if L.logit_bias is None else L.logit_bias.numpy(), dtype=np.float32)
    sb = None if L.sel_bias is None else L.sel_bias.numpy()
    ids, _ = O.route(s, cfg.k, cfg.mode, sb)
    return np.bincount(ids.reshape(-1), minlength=cfg.E), cfg


def test_qwen3_skew_gives_imbalance_two_to_three():
    counts, cfg = _routing_counts("qwen3_ep_all128", 8192)
    assert 2.0 <= O.imbalance_ratio(counts) <= 3.0


def test_deepseek_skew_top_five_percent_take_about_thirty_percent():
    counts, cfg = _routing_counts("deepseek_v3", 4096)
    top = np.sort(counts)[::-1][:round(0.05 * cfg.E)].sum() / (4096 * cfg.k)
    assert 0.26 <= top <= 0.34
