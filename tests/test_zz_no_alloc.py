"""moe_layer_static, the entry point that allocates nothing: its workspace is
the library's own device array.  Two calls in a row (the second with fewer
tokens, so it runs on what the first left in the array) must equal
moe_layer on a caller workspace bit for bit, and meet the oracle's
tolerance.  Sizes past the array are rejected on the host (test_abi.py)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import workloads as W
from harness import GpuLayer, check_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _static_run(gl, T):
    out = gl.run(T, debug=True)            # the same call shape, on the caller workspace
    y_ws = out["y"].clone()
    y = torch.empty_like(y_ws)
    dbg_ids = torch.empty_like(out["ids"])
    dbg = M.debug_out(topk_ids=dbg_ids)
    M.moe_layer_static(gl.desc, T, gl.L.x[:T], y, dbg)
    torch.cuda.synchronize()
    return out, y_ws, y, dbg_ids


# (workload, reduced sizes or None, T first, T second): the two calls take the
# staged path then the single-launch one (Qwen3 TP share), or both the
# staged path with a shared expert (DeepSeek-V3-shaped, reduced)
CASES = [("qwen3_tp8_rank0", None, 64, 2),
         ("deepseek_v3", dict(H=1024, I=256, E=64), 300, 37)]


@pytest.mark.parametrize("name,small,T1,T2", CASES)
def test_static_entry_point_equals_moe_layer(name, small, T1, T2):
    cfg = W.CONFIGS[name]
    kw = small or {}
    L = W.make_layer(cfg, device=DEV, seed=21, T_max=T1, **kw)
    if cfg.I_shared and small:
        s = 1.0 / kw["H"] ** 0.5
        g = torch.Generator(device=DEV).manual_seed(21)
        L.w13_shared = (torch.randn((2 * kw["I"], kw["H"]), device=DEV, generator=g) * s
                        ).to(torch.bfloat16)
        L.w2_shared = (torch.randn((kw["H"], kw["I"]), device=DEV, generator=g) * s
                       ).to(torch.bfloat16)
    gl = GpuLayer(L, tp_P=cfg.tp_P, tp_rank=cfg.tp_rank)
    for T in (T1, T2):
        assert M.moe_layer_workspace_size(gl.desc, T) <= M.STATIC_SCRATCH_BYTES
        out, y_ws, y, ids = _static_run(gl, T)
        print(f"{name} T={T} ({M.moe_layer_path(gl.desc, T)})", flush=True)
        assert torch.equal(ids, out["ids"])
        assert torch.equal(y, y_ws), "moe_layer_static differs from moe_layer"
        out["y"] = y
        check_layer(gl, out, T)
