"""The C ABI on the host: the library loads, exports every entry point the
header declares, and rejects bad arguments before touching a GPU.  No call
here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

import mixture_experts_layer_amd as M
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 24
    out = subprocess.run(["nm", "-D", "--defined-only", M.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(moe_\w+)", out))
    assert set(names) <= exported
    assert set(names) == set(M.EXPORTED_SYMBOLS)
    lib = M.get_lib()
    for n in names:
        assert getattr(lib, n) is not None


def test_version_and_status_strings():
    assert M.moe_abi_version() == 1
    for s in range(7):
        assert M.moe_status_str(s)
    assert M.moe_status_str(99) == "unknown status"


def test_workspace_queries():
    assert M.moe_permute_workspace_size(8192, 8, 128) > 8192 * 8 * 4
    assert M.moe_permute_workspace_size(-1, 8, 128) == 0
    assert M.moe_grouped_ffn_workspace_size(65536, 128, 4096, 1536, 1) >= 65536 * 1536 * 2
    d = M.MoELayerDesc(H=4096, E=128, k=8, I_loc=1536, e_begin=0, e_end=128, I_shared=0, mode=2,
                       dt=1, w_router=256, w13=512, w2=768)
    n = M.moe_layer_workspace_size(d, 8192)
    assert n >= 8192 * 8 * (1536 + 4096) * 2
    assert M.moe_layer_workspace_size(d, 16) < n
    # the device counts T * E logits in int: one token past that is rejected
    assert M.moe_layer_workspace_size(d, (2 ** 31 - 1) // 128) > 0
    assert M.moe_layer_workspace_size(d, (2 ** 31 - 1) // 128 + 1) == 0
    assert M.moe_permute_workspace_size(2 ** 31 - 1, 2, 8) == 0
    assert M.moe_permute_workspace_size(2 ** 31 - 1, 1, 8) > 0
    d.k = 200
    assert M.moe_layer_workspace_size(d, 16) == 0


class _FakePtr:
    """Stands in for a device tensor: argument checks read only the address."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


P = _FakePtr(1 << 20)
MIS = _FakePtr((1 << 20) + 4)


@pytest.mark.parametrize("kw,status", [
    (dict(k=9, E=8), 1),            # k > E
    (dict(k=0), 1),
    (dict(T=-1), 1),
    (dict(mode=7), 1),
    (dict(E=2000, k=2), 2),         # beyond the supported E
    (dict(k=40, E=64), 2),          # beyond the supported k
    (dict(H=100), 2),               # H not a multiple of 32
    (dict(H=0), 1),
])
def test_route_rejects(kw, status):
    a = dict(T=4, H=256, E=8, k=2, mode=0)
    a.update(kw)
    with pytest.raises(M.MoEError) as e:
        M.moe_route(P, P, 1, a["T"], a["H"], a["E"], a["k"], a["mode"], None, None, P, P, P,
                    stream=0)
    assert e.value.status == status


def test_route_rejects_misaligned_and_null():
    with pytest.raises(M.MoEError) as e:
        M.moe_route(MIS, P, 1, 4, 256, 8, 2, 0, None, None, P, P, P, stream=0)
    assert e.value.status == 1
    with pytest.raises(M.MoEError) as e:
        M.moe_route(P, P, 1, 4, 256, 8, 2, 0, None, None, None, P, P, stream=0)
    assert e.value.status == 1


def test_permute_rejects():
    with pytest.raises(M.MoEError) as e:   # bad expert range
        M.moe_permute(P, 4, 2, 8, 5, 3, None, 0, 0, P, P, P, P, None, P, 1 << 20, stream=0)
    assert e.value.status == 1
    with pytest.raises(M.MoEError) as e:   # multi-tile batch without workspace
        M.moe_permute(P, 1000, 2, 8, 0, 8, None, 0, 0, P, P, P, P, None, None, 0, stream=0)
    assert e.value.status == 3


def test_grouped_ffn_and_combine_reject():
    with pytest.raises(M.MoEError) as e:   # I_loc not a multiple of 32
        M.moe_grouped_ffn(P, None, None, P, 8, 16, 256, 100, P, P, 1, P, 1, P, 1 << 20, stream=0)
    assert e.value.status == 2
    with pytest.raises(M.MoEError) as e:   # no workspace
        M.moe_grouped_ffn(P, None, None, P, 8, 16, 256, 128, P, P, 1, P, 1, None, 0, stream=0)
    assert e.value.status == 3
    with pytest.raises(M.MoEError) as e:   # fp32 layer cannot emit bf16 rows
        M.moe_grouped_ffn(P, None, None, P, 8, 16, 256, 128, P, P, 0, P, 1, P, 1 << 20, stream=0)
    assert e.value.status == 2
    with pytest.raises(M.MoEError) as e:
        M.moe_combine(P, 1, P, P, 4, 2, 256, None, MIS, 1, stream=0)
    assert e.value.status == 1


def test_layer_rejects_bad_descriptors():
    base = dict(H=256, E=8, k=2, I_loc=128, e_begin=0, e_end=8, I_shared=0, mode=0, dt=1,
                w_router=1 << 20, w13=1 << 21, w2=1 << 22)
    for change, status in ((dict(e_end=9), 1), (dict(e_begin=8), 1), (dict(I_loc=100), 2),
                           (dict(dt=5), 1), (dict(w13=(1 << 21) + 8), 1), (dict(I_shared=64), 1)):
        d = M.MoELayerDesc(**{**base, **change})
        with pytest.raises(M.MoEError) as e:
            M.moe_layer(d, 4, P, P, P, 1 << 30, stream=0)
        assert e.value.status == status, change
    d = M.MoELayerDesc(**base)
    with pytest.raises(M.MoEError) as e:
        M.moe_layer(d, 4, P, P, P, 10, stream=0)
    assert e.value.status == 3
    M.moe_layer(d, 0, P, P, P, 0, stream=0)   # T = 0 is a no-op


def test_layer_paths_reject_before_launch():
    base = dict(H=256, E=8, k=2, I_loc=128, e_begin=0, e_end=8, I_shared=0, mode=0, dt=1,
                w_router=1 << 20, w13=1 << 21, w2=1 << 22)
    d = M.MoELayerDesc(**base)
    # shapes outside the single-launch path's limits
    for change, T in ((dict(dt=0), 4), ({}, 65), (dict(E=300, e_end=300, k=2), 4),
                      (dict(E=64, e_end=64, k=17), 4), (dict(E=16, e_end=16, k=9), 60)):
        dd = M.MoELayerDesc(**{**base, **change})
        with pytest.raises(M.MoEError) as e:
            M.moe_layer_decode(dd, T, P, P, P, 1 << 30, stream=0)
        assert e.value.status == 2, (change, T)
    for fn in (M.moe_layer_decode, M.moe_layer_staged):
        with pytest.raises(M.MoEError) as e:      # workspace too small
            fn(d, 4, P, P, P, 10, stream=0)
        assert e.value.status == 3
        with pytest.raises(M.MoEError) as e:      # misaligned output
            fn(d, 4, P, MIS, P, 1 << 30, stream=0)
        assert e.value.status == 1
        fn(d, 0, P, P, P, 0, stream=0)            # T = 0 is a no-op


def test_layer_workspace_starts_with_sync_block():
    d = M.MoELayerDesc(H=256, E=8, k=2, I_loc=128, e_begin=0, e_end=8, I_shared=0, mode=0, dt=1,
                       w_router=1 << 20, w13=1 << 21, w2=1 << 22)
    n1 = M.moe_layer_workspace_size(d, 1)
    # logits, ids, weights, metadata, h and the expert outputs of one token follow the block
    assert n1 >= M.LAYER_SYNC_BYTES + 8 * 4 + 2 * 128 * 2 + 2 * 256 * 2


def test_layer_path_choice():
    def desc(**kw):
        base = dict(H=4096, E=128, k=8, I_loc=192, e_begin=0, e_end=128, I_shared=0, mode=2, dt=1,
                    w_router=1 << 20, w13=1 << 21, w2=1 << 22)
        base.update(kw)
        return M.MoELayerDesc(**base)
    tp = desc()                                   # tensor-parallel share: 4.7 MB per expert
    # 2 * 8 experts * 4.72 MB = 75.5 MB; 3 * 8 * 4.72 MB = 113 MB (limit 100 MB)
    assert [M.moe_layer_path(tp, T) for T in (1, 2, 3, 8, 64, 65)] == \
        ["decode", "decode", "staged", "staged", "staged", "staged"]
    ep = desc(I_loc=1536)                         # whole experts: 37.7 MB each
    assert [M.moe_layer_path(ep, T) for T in (1, 2)] == ["staged", "staged"]
    small = desc(I_loc=1536, H=1024)              # 9.4 MB per expert: 8 experts = 75.5 MB
    assert [M.moe_layer_path(small, T) for T in (1, 2)] == ["decode", "staged"]
    assert M.moe_layer_path(desc(dt=0), 1) == "staged"        # float32 layers
    assert M.moe_layer_path(tp, 0) == "staged"
    with pytest.raises(M.MoEError):
        M.moe_layer_path(tp, -1)
    with pytest.raises(M.MoEError):
        M.moe_layer_path(desc(k=0), 1)


def test_pack_and_unpack_reject_before_launch():
    with pytest.raises(M.MoEError) as e:     # E not divisible by P
        M.moe_pack_by_rank(P, None, 4, 2, 10, 4, None, 0, 0, P, P, P, P, None, None, None, None, 0,
                           stream=0)
    assert e.value.status == 1
    with pytest.raises(M.MoEError) as e:     # more than 64 ranks
        M.moe_pack_by_rank(P, None, 4, 2, 128, 128, None, 0, 0, P, P, P, P, None, None, None,
                           None, 0, stream=0)
    assert e.value.status == 2
    with pytest.raises(M.MoEError) as e:     # weights requested without topk_w
        M.moe_pack_by_rank(P, None, 4, 2, 8, 4, None, 0, 0, P, P, P, P, None, P, None, None, 0,
                           stream=0)
    assert e.value.status == 1
    with pytest.raises(M.MoEError) as e:     # multi-tile batch without workspace
        M.moe_pack_by_rank(P, None, 100, 2, 8, 4, None, 0, 0, P, P, P, P, None, None, None, None,
                           0, stream=0)
    assert e.value.status == 3
    assert M.moe_pack_workspace_size(100, 2, 4) >= 100 * 8
    assert M.moe_pack_workspace_size(10, 2, 65) == 0
    with pytest.raises(M.MoEError) as e:
        M.moe_unpack_sum(P, 1, P, 4, 2, 100, P, 1, stream=0)   # H not a multiple of 32
    assert e.value.status == 2
    M.moe_unpack_sum(P, 1, P, 0, 2, 256, P, 1, stream=0)      # T = 0 is a no-op


def test_reshard_rejects_before_launch():
    for args, status in (((P, P, 2, 100, 256, 8, 1, P, P), 1),       # I not divisible by P
                         ((P, P, 2, 96, 256, 8, 1, P, P), 2),        # I/P * 2 bytes not 16-aligned
                         ((P, None, 2, 128, 256, 8, 1, P, P), 1),    # half a W2 pair
                         ((None, None, 2, 128, 256, 8, 1, None, None), 1),
                         ((MIS, P, 2, 128, 256, 8, 1, P, P), 1)):
        for fn in (M.moe_reshard_ep_to_tp_pack, M.moe_reshard_tp_to_ep_interleave):
            with pytest.raises(M.MoEError) as e:
                fn(*args, stream=0)
            assert e.value.status == status, args


def test_capacity_entries_reject_before_launch():
    for cap, padded, dropped, ws, status in [
            (-1, 0, None, None, 1),            # negative capacity
            (3, 0, MIS, None, 1),              # misaligned dropped counter
            (3, 2, None, None, 1),             # padded is 0 or 1
            (2 ** 31 - 1, 1, None, P, 1),      # E_loc * capacity does not fit an int
            (3, 1, None, None, 3)]:            # the padded layout needs a workspace at any T
        with pytest.raises(M.MoEError) as e:
            M.moe_permute_capacity(P, 4, 2, 8, 0, 8, cap, padded, None, 0, 0, P, P, P, P, None,
                                   dropped, ws, 0 if ws is None else 1 << 20, stream=0)
        assert e.value.status == status, (cap, padded)
    d = M.MoELayerDesc(H=256, E=8, k=2, I_loc=128, e_begin=0, e_end=8, I_shared=0, mode=0, dt=1,
                       w_router=1 << 20, w13=1 << 21, w2=1 << 22)
    with pytest.raises(M.MoEError) as e:
        M.moe_layer_capacity(d, 4, -5, 0, P, P, P, 1 << 30, stream=0)
    assert e.value.status == 1
    with pytest.raises(M.MoEError) as e:
        M.moe_layer_capacity(d, 4, 3, 3, P, P, P, 1 << 30, stream=0)
    assert e.value.status == 1
    with pytest.raises(M.MoEError) as e:
        M.moe_layer_capacity(d, 4, 2 ** 31 - 1, 1, P, P, P, 1 << 40, stream=0)
    assert e.value.status == 1
    with pytest.raises(M.MoEError) as e:      # workspace too small
        M.moe_layer_capacity(d, 4, 3, 0, P, P, P, 10, stream=0)
    assert e.value.status == 3
    # the padded layout needs E_loc * capacity rows of h and y_perm: the
    # dropless workspace is too small for a large capacity
    n = M.moe_layer_workspace_size(d, 4)
    with pytest.raises(M.MoEError) as e:
        M.moe_layer_capacity(d, 4, 1000, 1, P, P, P, n, stream=0)
    assert e.value.status == 3


def test_capacity_workspace_sizes():
    d = M.MoELayerDesc(H=256, E=8, k=2, I_loc=128, e_begin=0, e_end=8, I_shared=0, mode=0, dt=1,
                       w_router=1 << 20, w13=1 << 21, w2=1 << 22)
    T = 100
    assert M.moe_layer_capacity_workspace_size(d, T, 7, 0) == M.moe_layer_workspace_size(d, T)
    small = M.moe_layer_capacity_workspace_size(d, T, 0, 1)
    big = M.moe_layer_capacity_workspace_size(d, T, 1000, 1)
    # 8 experts x 1000 rows of h (128) and y_perm (256) in bf16, and src_token
    assert big - small >= 8 * 1000 * (128 + 256) * 2
    assert M.moe_layer_capacity_workspace_size(d, T, -1, 1) == 0
    assert M.moe_layer_capacity_workspace_size(d, T, 3, 2) == 0
    assert M.moe_layer_capacity_workspace_size(d, T, 2 ** 31 - 1, 1) == 0


def test_validate_mode_keeps_its_result_word_in_the_workspace(monkeypatch):
    monkeypatch.delenv("MOE_VALIDATE", raising=False)
    base = M.moe_permute_workspace_size(100, 4, 16)
    monkeypatch.setenv("MOE_VALIDATE", "1")
    assert M.moe_permute_workspace_size(100, 4, 16) == base + 256
    # a single-tile batch needs a workspace in this mode
    with pytest.raises(M.MoEError) as e:
        M.moe_permute(P, 4, 2, 8, 0, 8, None, 0, 0, P, P, P, P, None, None, 0, stream=0)
    assert e.value.status == 3
    assert M.moe_status_str(5) == "routing metadata check failed"


def test_library_stamp_matches_the_sources():
    """The loader refuses a library built from other sources (a stale
    binary); the loaded one carries the tree's stamp."""
    from mixture_experts_layer_amd import build as B
    assert M.moe_source_sha256() == B.source_sha256()


def test_layer_status_rejects_bad_workspace():
    assert M.lib.moe_layer_status(None, 1 << 20, None) == 1
    assert M.lib.moe_layer_status(ctypes.c_void_p(MIS.addr), 1 << 20, None) == 1
    assert M.lib.moe_layer_status(ctypes.c_void_p(P.addr), 4096, None) == 1


def test_static_entry_rejects_sizes_past_its_array():
    """moe_layer_static refuses, on the host, a call whose workspace would
    exceed its fixed device array (and an invalid description)."""
    d = M.MoELayerDesc(H=4096, E=128, k=8, I_loc=1536, e_begin=0, e_end=128, I_shared=0, mode=2,
                       dt=1, w_router=P.addr, w13=P.addr, w2=P.addr)
    assert M.moe_layer_workspace_size(d, 8192) > M.STATIC_SCRATCH_BYTES
    assert M.lib.moe_layer_static(ctypes.byref(d), 8192, ctypes.c_void_p(P.addr),
                                  ctypes.c_void_p(P.addr), None, None) == 3
    assert M.lib.moe_layer_static(ctypes.byref(d), 0, None, None, None, None) == 0
    assert M.lib.moe_layer_static(ctypes.byref(d), -1, None, None, None, None) == 1
    d.k = 200
    assert M.lib.moe_layer_static(ctypes.byref(d), 16, ctypes.c_void_p(P.addr),
                                  ctypes.c_void_p(P.addr), None, None) == 1
