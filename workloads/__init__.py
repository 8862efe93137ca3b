"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws numbers and lays them out; it computes nothing the
layer computes (no router, no gating, no expert math), so the CPU oracle and
the HIP path can both be fed from it without sharing arithmetic.

Shapes follow the models the pages name: Mixtral-8x7B (8 experts choose 2),
Qwen3-235B-A22B (128 choose 8), DeepSeek-V3 (256 choose 8 plus one shared
expert) -- "Lecture 8 · 混合专家模型的推理" (CS349D notes) section 1.2 and the
Moebius reading notes' background section.  There is no dataset: every tensor
is drawn from torch's generator with a per-tensor seed, so a (config, seed)
pair fixes every value on a given device type.

Recipe (all per-tensor generators are torch.Generator seeded with
seed * 1000 + tag):
  x           ~ N(0, 1)                      [T_max, H]   tag 0
  W_r         ~ N(0, 1) / sqrt(H)            [E, H]       tag 1
  W13, W2     ~ N(0, 1) / sqrt(H)            per expert   tags 2, 3
  Zipf bias   logit_bias[e] = -beta * ln(rho[e]), rho a seeded permutation of
              1..E (Zipf s = 1 popularity ranks)           tag 4
  sel_bias    ~ N(0, 1) * sel_bias_std       [E]          tag 5
  shared W13, W2 ~ N(0, 1) / sqrt(H)                       tags 6, 7
bf16 tensors are drawn in float32 and rounded to nearest even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

MODE_TOPK_SOFTMAX = 0
MODE_SOFTMAX_TOPK = 1
MODE_SOFTMAX_TOPK_RENORM = 2
MODE_SIGMOID_BIAS_RENORM = 3


@dataclass(frozen=True)
class MoEConfig:
    name: str
    H: int
    I: int
    E: int
    k: int
    mode: int
    dtype: str                      # "f32" or "bf16"
    T_list: tuple
    tp_P: int = 1                   # tensor-parallel degree of the share
    tp_rank: int = 0
    e_begin: int = 0                # expert-parallel range of the share
    e_end: int | None = None
    I_shared: int = 0               # 0 = no shared expert
    zipf_beta: float = 0.0          # skew of the logit bias (0 = none)
    sel_bias_std: float = 0.0       # selection-only bias (mode 3)
    describe: str = ""

    @property
    def I_loc(self):
        return self.I // self.tp_P

    @property
    def E_loc(self):
        return (self.e_end if self.e_end is not None else self.E) - self.e_begin

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def T_max(self):
        return max(self.T_list)


CONFIGS = {
    "toy_f32": MoEConfig(
        "toy_f32", H=256, I=512, E=8, k=2, mode=MODE_TOPK_SOFTMAX, dtype="f32",
        T_list=(64,), describe="toy fp32 layer, top-k then softmax"),
    "mixtral_8x7b": MoEConfig(
        "mixtral_8x7b", H=4096, I=14336, E=8, k=2, mode=MODE_TOPK_SOFTMAX, dtype="bf16",
        T_list=(1, 16, 256, 4096), describe="Mixtral-8x7B-shaped layer, bf16"),
    "qwen3_ep_all128": MoEConfig(
        "qwen3_ep_all128", H=4096, I=1536, E=128, k=8, mode=MODE_SOFTMAX_TOPK_RENORM,
        dtype="bf16", T_list=(16, 64, 128, 256, 1024, 8192), zipf_beta=0.15,
        describe="Qwen3-235B-A22B-shaped layer, all 128 experts resident, Zipf-skewed"),
    "qwen3_tp8_rank0": MoEConfig(
        "qwen3_tp8_rank0", H=4096, I=1536, E=128, k=8, mode=MODE_SOFTMAX_TOPK_RENORM,
        dtype="bf16", T_list=(1, 8, 32, 64), tp_P=8, tp_rank=0,
        describe="Qwen3-shaped layer, tensor-parallel share of rank 0 of 8 (I/P = 192)"),
    "deepseek_v3": MoEConfig(
        "deepseek_v3", H=7168, I=2048, E=256, k=8, mode=MODE_SIGMOID_BIAS_RENORM,
        dtype="bf16", T_list=(1, 16, 64, 4096), I_shared=2048, zipf_beta=0.30, sel_bias_std=0.5,
        describe="DeepSeek-V3-shaped layer, sigmoid + selection bias, 1 shared expert"),
}


def _gen(seed, tag, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(tag))
    return g


def _normal(shape, seed, tag, device, scale, dtype):
    g = _gen(seed, tag, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(dtype)


def _normal_experts(n_exp, shape, seed, tag, device, scale, dtype):
    """Draw per-expert blocks one at a time (bounded float32 scratch)."""
    out = torch.empty((n_exp,) + tuple(shape), device=device, dtype=dtype)
    g = _gen(seed, tag, device)
    for e in range(n_exp):
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        t.mul_(scale)
        out[e].copy_(t.to(dtype))
    return out


def zipf_logit_bias(E, beta, seed, device="cpu"):
    """logit_bias[e] = -beta * ln(rank[e]) with rank a seeded permutation of
    1..E: Zipf(s = 1) popularity ranks turned into a log-probability offset."""
    g = _gen(seed, 4, "cpu")
    rank = torch.randperm(E, generator=g).to(torch.float64) + 1.0
    return (-beta * torch.log(rank)).to(torch.float32).to(device)


@dataclass
class LayerInputs:
    cfg: MoEConfig
    x: torch.Tensor                  # [T_max, H]
    w_r: torch.Tensor                # [E, H]
    w13: torch.Tensor                # [E_full, 2I, H]  (full experts, unsliced)
    w2: torch.Tensor                 # [E_full, H, I]
    logit_bias: torch.Tensor | None  # [E] fp32
    sel_bias: torch.Tensor | None    # [E] fp32
    w13_shared: torch.Tensor | None = None
    w2_shared: torch.Tensor | None = None
    extra: dict = field(default_factory=dict)


def make_layer(cfg: MoEConfig, device="cpu", seed=0, T_max=None, H=None, I=None, E=None,
               experts=True):
    """Draw every input of a layer.  Optional H/I/E/T_max override the config's
    sizes (small cases of the same recipe).  The expert tensors are the FULL
    experts; share_weights() cuts one GPU's share from them.  experts=False
    draws only the router-side inputs (x, W_r, biases)."""
    H = H or cfg.H
    I = I or cfg.I
    E = E or cfg.E
    T_max = T_max or cfg.T_max
    dt = cfg.torch_dtype
    s = 1.0 / math.sqrt(H)
    x = _normal((T_max, H), seed, 0, device, 1.0, dt)
    w_r = _normal((E, H), seed, 1, device, s, dt)
    w13 = w2 = None
    if experts:
        w13 = _normal_experts(E, (2 * I, H), seed, 2, device, s, dt)
        w2 = _normal_experts(E, (H, I), seed, 3, device, s, dt)
    logit_bias = zipf_logit_bias(E, cfg.zipf_beta, seed, device) if cfg.zipf_beta else None
    sel_bias = None
    if cfg.sel_bias_std:
        sel_bias = _normal((E,), seed, 5, device, cfg.sel_bias_std, torch.float32)
    w13_s = w2_s = None
    if cfg.I_shared and experts:
        w13_s = _normal((2 * cfg.I_shared, H), seed, 6, device, s, dt)
        w2_s = _normal((H, cfg.I_shared), seed, 7, device, s, dt)
    return LayerInputs(cfg, x, w_r, w13, w2, logit_bias, sel_bias, w13_s, w2_s)


def share_weights(w13, w2, tp_P=1, tp_rank=0, e_begin=0, e_end=None):
    """One GPU's share of the expert weights, as the caller hands it to the
    library: experts [e_begin, e_end) and, for a tensor-parallel share, the
    intermediate indices [rank*I/P, (rank+1)*I/P) of the gate half and of the
    up half of the stacked gate/up axis (down projection: the same input
    columns).  Layout only; returns contiguous tensors."""
    E = w13.shape[0]
    e_end = E if e_end is None else e_end
    w13 = w13[e_begin:e_end]
    w2 = w2[e_begin:e_end]
    if tp_P == 1:
        return w13.contiguous(), w2.contiguous()
    I = w13.shape[1] // 2
    sl = I // tp_P
    lo, hi = tp_rank * sl, (tp_rank + 1) * sl
    w13_r = torch.cat([w13[:, lo:hi], w13[:, I + lo:I + hi]], dim=1).contiguous()
    w2_r = w2[:, :, lo:hi].contiguous()
    return w13_r, w2_r


def sample_rows(T, n, seed=0):
    """A seeded sorted subset of n distinct token indices out of T."""
    if n >= T:
        return torch.arange(T)
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) * 1000 + 99)
    return torch.sort(torch.randperm(T, generator=g)[:n]).values
