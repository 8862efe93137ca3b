"""Full-size parity: every workload shape at every token count it names, run
through moe_layer exactly as the benchmark calls it.

Routing metadata (ids, counts, offsets, src_token, dst_row) is checked for the
whole batch; layer outputs are checked on a seeded sample of tokens, which is
exact because the layer is dropless (a token's output depends on that token
alone).  The oracle widens only the experts the sampled tokens use.
"""
import gc

import pytest
import torch

import mixture_experts_layer_amd as M
import workloads as W
from harness import GpuLayer, check_layer

pytestmark = pytest.mark.gpu

CASES = [(name, T) for name in ("mixtral_8x7b", "qwen3_ep_all128", "qwen3_tp8_rank0",
                                "deepseek_v3") for T in W.CONFIGS[name].T_list]
N_SAMPLE = {"mixtral_8x7b": 12, "qwen3_ep_all128": 24, "qwen3_tp8_rank0": 32, "deepseek_v3": 12}

_cache = {}


def _layer(name):
    if name not in _cache:
        _cache.clear()
        gc.collect()
        torch.cuda.empty_cache()
        cfg = W.CONFIGS[name]
        L = W.make_layer(cfg, device="cuda", seed=0)
        _cache[name] = GpuLayer(L, tp_P=cfg.tp_P, tp_rank=cfg.tp_rank)
    return _cache[name]


@pytest.mark.parametrize("name,T", CASES)
def test_full_size_layer(name, T):
    gl = _layer(name)
    out = gl.run(T)
    sample = W.sample_rows(T, N_SAMPLE[name], seed=T).numpy()
    res = check_layer(gl, out, T, sample=sample)
    print(f"{name} T={T} ({M.moe_layer_path(gl.desc, T)}): {res}", flush=True)


# decode-sized batches also through the path moe_layer does not take, so
# both the staged and the single-launch path are checked at full size
ALT = [(name, T) for name, T in CASES if T <= 64 and W.CONFIGS[name].dtype == "bf16"]


@pytest.mark.parametrize("name,T", ALT)
def test_full_size_layer_other_path(name, T):
    gl = _layer(name)
    path = "staged" if M.moe_layer_path(gl.desc, T) == "decode" else "decode"
    out = gl.run(T, path=path)
    sample = W.sample_rows(T, N_SAMPLE[name], seed=T + 1).numpy()
    res = check_layer(gl, out, T, sample=sample)
    if path == "decode":
        assert gl.sync_error() == 0
    print(f"{name} T={T} ({path}): {res}", flush=True)


def teardown_module():
    _cache.clear()
    gc.collect()
    torch.cuda.empty_cache()
