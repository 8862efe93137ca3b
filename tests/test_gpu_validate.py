"""The MOE_VALIDATE=1 metadata checks on the GPU: consistent metadata from
every path passes (and the outputs are those of an unchecked call), and ids
outside [0, E) are reported as MOE_ERR_METADATA.  The permute kernels treat
such ids as not local, so the failing call itself stays in bounds."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_amd as M
import workloads as W
from harness import GpuLayer, ws_tensor
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"
METADATA = 5


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("MOE_VALIDATE", "1")


def _permute(ids, E, eb, ee, C=None, padded=0):
    T, k = ids.shape
    E_loc = ee - eb
    rows = E_loc * C if padded else max(T * k, 1)
    counts = torch.empty((E_loc,), dtype=torch.int32, device=DEV)
    offsets = torch.empty((E_loc + 1,), dtype=torch.int32, device=DEV)
    src = torch.empty((max(rows, 1),), dtype=torch.int32, device=DEV)
    dst = torch.empty((max(T, 1), k), dtype=torch.int32, device=DEV)
    dropped = torch.zeros((4,), dtype=torch.int32, device=DEV)
    nb = M.moe_permute_workspace_size(T, k, E_loc)
    ids_d = torch.as_tensor(ids, dtype=torch.int32, device=DEV).contiguous()
    if C is None:
        M.moe_permute(ids_d, T, k, E, eb, ee, None, 0, 0, counts, offsets, src, dst, None,
                      ws_tensor(nb), nb)
    else:
        M.moe_permute_capacity(ids_d, T, k, E, eb, ee, C, padded, None, 0, 0, counts, offsets, src,
                               dst, None, dropped, ws_tensor(nb), nb)
    torch.cuda.synchronize()
    return counts


def _ids(T, k, E, seed):
    r = np.random.default_rng(seed)
    return np.stack([r.permutation(E)[:k] for _ in range(T)])


@pytest.mark.parametrize("T", [1, 64, 65, 1000])
@pytest.mark.parametrize("eb,ee", [(0, 16), (4, 12)])
def test_consistent_permutations_pass(validate, T, eb, ee):
    ids = _ids(T, 4, 16, seed=T)
    counts = _permute(ids, 16, eb, ee)
    ref, _, _, _ = O.permute(ids, eb, ee)
    assert np.array_equal(counts.cpu().numpy(), ref)
    C = O.expert_capacity(1.0, T * 4, 16)
    for padded in (0, 1):
        _permute(ids, 16, eb, ee, C, padded)


@pytest.mark.parametrize("T", [5, 64, 1000])
@pytest.mark.parametrize("bad", [16, -1, 99])
def test_ids_out_of_range_are_reported(validate, T, bad):
    ids = _ids(T, 4, 16, seed=T + 1)
    ids[T // 2, 1] = bad
    with pytest.raises(M.MoEError) as e:
        _permute(ids, 16, 0, 16)
    assert e.value.status == METADATA
    with pytest.raises(M.MoEError) as e:
        _permute(ids, 16, 0, 16, C=O.expert_capacity(1.25, T * 4, 16), padded=1)
    assert e.value.status == METADATA


def test_without_the_variable_nothing_is_checked(monkeypatch):
    monkeypatch.delenv("MOE_VALIDATE", raising=False)
    ids = _ids(64, 4, 16, seed=3)
    ids[0, 0] = 16
    _permute(ids, 16, 0, 16)       # the id is simply not local


@pytest.mark.parametrize("name,T,path", [("qwen3_ep_all128", 300, "staged"),
                                         ("deepseek_v3", 40, "staged"),
                                         ("qwen3_ep_all128", 5, "decode"),
                                         ("mixtral_8x7b", 1, "decode")])
def test_layer_paths_pass_and_match_unchecked_calls(monkeypatch, name, T, path):
    L = W.make_layer(W.CONFIGS[name], device=DEV, seed=21, T_max=T, H=256, I=192, E=32)
    gl = GpuLayer(L)
    monkeypatch.delenv("MOE_VALIDATE", raising=False)
    ref = gl.run(T, path=path)
    monkeypatch.setenv("MOE_VALIDATE", "1")
    out = gl.run(T, path=path)
    out_nodbg = gl.run(T, path=path, debug=False)
    torch.cuda.synchronize()
    assert torch.equal(out["y"], ref["y"]) and torch.equal(out_nodbg["y"], ref["y"])
    assert torch.equal(out["dst_row"], ref["dst_row"])


def test_capacity_layer_passes(validate):
    T = 300
    L = W.make_layer(W.CONFIGS["qwen3_ep_all128"], device=DEV, seed=22, T_max=T, H=256, I=192,
                     E=32)
    gl = GpuLayer(L)
    C = O.expert_capacity(1.0, T * gl.k, gl.E)
    for padded in (0, 1):
        nb = M.moe_layer_capacity_workspace_size(gl.desc, T, C, padded)
        y = torch.empty((T, gl.H), dtype=L.x.dtype, device=DEV)
        dropped = torch.zeros((4,), dtype=torch.int32, device=DEV)
        M.moe_layer_capacity(gl.desc, T, C, padded, L.x[:T], y, ws_tensor(nb), nb, None, dropped)
        torch.cuda.synchronize()
        assert int(dropped[0]) > 0


WAIT = 6


def _decode_layer():
    cfg = W.CONFIGS["qwen3_tp8_rank0"]
    L = W.make_layer(cfg, device=DEV, seed=12, T_max=8, H=512, I=256, E=32)
    return GpuLayer(L)


def test_wait_error_word_is_reported_by_a_validated_call(validate):
    """A wait error word left in the workspace (written here from the host;
    no kernel is made to wait) makes the next validated decode-path call
    return MOE_ERR_WAIT, and that call clears it."""
    gl = _decode_layer()
    assert M.moe_layer_path(gl.desc, 8) == "decode"
    gl.run(8)                                   # a clean validated call passes
    gl.ws[4:8].view(torch.int32).fill_(2)       # bit 1: an expert wait ran out
    with pytest.raises(M.MoEError) as e:
        gl.run(8)
    assert e.value.status == WAIT
    assert gl.sync_error() == 0                 # read and cleared
    gl.run(8)


def test_layer_status_reads_and_clears_the_wait_word():
    gl = _decode_layer()
    gl.run(8)
    M.moe_layer_status(gl.ws, gl.ws_bytes)      # clean
    gl.ws[4:8].view(torch.int32).fill_(1)       # bit 0: the router wait ran out
    with pytest.raises(M.MoEError) as e:
        M.moe_layer_status(gl.ws, gl.ws_bytes)
    assert e.value.status == WAIT
    assert gl.sync_error() == 0
    M.moe_layer_status(gl.ws, gl.ws_bytes)
