"""Python binding of the MI355X MoE layer library (ctypes, marshalling only).

Every function here has the name and the argument order of the C entry point
it wraps (include/moe.h).  Arguments are torch tensors on the GPU (or None for
NULL); the binding passes their data pointers and the current HIP stream,
checks the returned status and raises MoEError on failure.  No step of the
layer is computed in Python: if the HIP library is not built, the first call
raises ImportError (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

from ._abi import (MOE_F32, MOE_BF16, MOE_OK, GATE_TOPK_SOFTMAX, GATE_SOFTMAX_TOPK,  # noqa: F401
                   GATE_SOFTMAX_TOPK_RENORM, GATE_SIGMOID_BIAS_RENORM, MoELayerDesc, MoEDebugOut,
                   EXPORTED_SYMBOLS, LAYER_SYNC_BYTES, STATIC_SCRATCH_BYTES, lib_path,
                   load_library)

__all__ = [
    "MoEError", "lib", "get_lib", "moe_abi_version", "moe_status_str", "moe_route", "moe_permute",
    "moe_permute_workspace_size", "moe_permute_capacity", "moe_grouped_ffn",
    "moe_grouped_ffn_workspace_size", "moe_layer_capacity", "moe_layer_capacity_workspace_size",
    "moe_combine", "moe_pack_by_rank", "moe_pack_workspace_size", "moe_unpack_sum",
    "moe_reshard_ep_to_tp_pack", "moe_reshard_tp_to_ep_interleave", "moe_layer",
    "moe_layer_path", "moe_layer_staged", "moe_layer_decode", "moe_layer_static",
    "STATIC_SCRATCH_BYTES",
    "moe_layer_workspace_size", "moe_layer_status", "moe_source_sha256", "MOE_ERR_WAIT",
    "layer_workspace", "layer_desc", "dtype_code", "LAYER_SYNC_BYTES",
    "MoELayerDesc", "MoEDebugOut",
]

_LIB = None


def get_lib():
    """The loaded HIP library; raises ImportError if it has not been built."""
    global _LIB
    if _LIB is None:
        _LIB = load_library()
    return _LIB


class _LazyLib:
    def __getattr__(self, name):
        return getattr(get_lib(), name)


lib = _LazyLib()


class MoEError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({moe_status_str(status)})")


def moe_abi_version() -> int:
    return lib.moe_abi_version()


def moe_status_str(status: int) -> str:
    return lib.moe_status_str(status).decode()


def moe_source_sha256() -> str:
    return lib.moe_source_sha256().decode()


MOE_ERR_WAIT = 6


def dtype_code(t) -> int:
    import torch
    dt = t if isinstance(t, torch.dtype) else t.dtype
    if dt == torch.float32:
        return MOE_F32
    if dt == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, status):
    if status != MOE_OK:
        raise MoEError(fn, status)


def moe_route(x, w_router, dt, T, H, E, k, mode, logit_bias, sel_bias, logits, topk_ids, topk_w,
              stream=None):
    _check("moe_route", lib.moe_route(_p(x), _p(w_router), dt, T, H, E, k, mode, _p(logit_bias),
                                      _p(sel_bias), _p(logits), _p(topk_ids), _p(topk_w),
                                      _stream(stream)))


def moe_permute_workspace_size(T, k, E_loc) -> int:
    return lib.moe_permute_workspace_size(T, k, E_loc)


def moe_permute(topk_ids, T, k, E, e_begin, e_end, x, H, dt, counts, offsets, src_token, dst_row,
                x_perm, ws, ws_bytes, stream=None):
    _check("moe_permute", lib.moe_permute(_p(topk_ids), T, k, E, e_begin, e_end, _p(x), H, dt,
                                          _p(counts), _p(offsets), _p(src_token), _p(dst_row),
                                          _p(x_perm), _p(ws), ws_bytes, _stream(stream)))


def moe_permute_capacity(topk_ids, T, k, E, e_begin, e_end, capacity, padded, x, H, dt, counts,
                         offsets, src_token, dst_row, x_perm, dropped, ws, ws_bytes, stream=None):
    _check("moe_permute_capacity",
           lib.moe_permute_capacity(_p(topk_ids), T, k, E, e_begin, e_end, capacity, int(padded),
                                    _p(x), H, dt,
                                    _p(counts), _p(offsets), _p(src_token), _p(dst_row),
                                    _p(x_perm), _p(dropped), _p(ws), ws_bytes, _stream(stream)))


def moe_grouped_ffn_workspace_size(max_rows, E_loc, H, I_loc, dt) -> int:
    return lib.moe_grouped_ffn_workspace_size(max_rows, E_loc, H, I_loc, dt)


def moe_grouped_ffn(x_perm, x, src_token, offsets, E_loc, max_rows, H, I_loc, w13, w2, dt,
                    y_perm, y_dt, ws, ws_bytes, stream=None):
    _check("moe_grouped_ffn",
           lib.moe_grouped_ffn(_p(x_perm), _p(x), _p(src_token), _p(offsets), E_loc, max_rows, H,
                               I_loc, _p(w13), _p(w2), dt, _p(y_perm), y_dt, _p(ws), ws_bytes,
                               _stream(stream)))


def moe_combine(y_perm, y_perm_dt, dst_row, topk_w, T, k, H, y_shared, y, dt, stream=None):
    _check("moe_combine", lib.moe_combine(_p(y_perm), y_perm_dt, _p(dst_row), _p(topk_w), T, k, H,
                                          _p(y_shared), _p(y), dt, _stream(stream)))


def moe_pack_workspace_size(T, k, P) -> int:
    return lib.moe_pack_workspace_size(T, k, P)


def moe_pack_by_rank(topk_ids, topk_w, T, k, E, P, x, H, dt, send_counts, send_offsets, send_token,
                     send_row, send_ids, send_w, x_send, ws, ws_bytes, stream=None):
    _check("moe_pack_by_rank",
           lib.moe_pack_by_rank(_p(topk_ids), _p(topk_w), T, k, E, P, _p(x), H, dt,
                                _p(send_counts), _p(send_offsets), _p(send_token), _p(send_row),
                                _p(send_ids), _p(send_w), _p(x_send), _p(ws), ws_bytes,
                                _stream(stream)))


def moe_unpack_sum(y_ret, y_ret_dt, send_row, T, k, H, y, dt, stream=None):
    _check("moe_unpack_sum", lib.moe_unpack_sum(_p(y_ret), y_ret_dt, _p(send_row), T, k, H, _p(y),
                                                dt, _stream(stream)))


def moe_reshard_ep_to_tp_pack(w13_ep, w2_ep, E_rank, I, H, P, dt, w13_send, w2_send,
                              stream=None):
    _check("moe_reshard_ep_to_tp_pack",
           lib.moe_reshard_ep_to_tp_pack(_p(w13_ep), _p(w2_ep), E_rank, I, H, P, dt, _p(w13_send),
                                         _p(w2_send), _stream(stream)))


def moe_reshard_tp_to_ep_interleave(w13_recv, w2_recv, E_rank, I, H, P, dt, w13_ep, w2_ep,
                                    stream=None):
    _check("moe_reshard_tp_to_ep_interleave",
           lib.moe_reshard_tp_to_ep_interleave(_p(w13_recv), _p(w2_recv), E_rank, I, H, P, dt,
                                               _p(w13_ep), _p(w2_ep), _stream(stream)))


def layer_desc(H, E, k, I_loc, mode, dt, w_router, w13, w2, e_begin=0, e_end=None, I_shared=0,
               w13_shared=None, w2_shared=None, logit_bias=None, sel_bias=None) -> MoELayerDesc:
    """Fill the moe_layer_desc struct from tensors (pointers only)."""
    d = MoELayerDesc()
    d.H, d.E, d.k, d.I_loc = H, E, k, I_loc
    d.e_begin = e_begin
    d.e_end = E if e_end is None else e_end
    d.I_shared = I_shared
    d.mode, d.dt = mode, dt
    d.w_router, d.w13, d.w2 = _p(w_router), _p(w13), _p(w2)
    d.w13_shared, d.w2_shared = _p(w13_shared), _p(w2_shared)
    d.logit_bias, d.sel_bias = _p(logit_bias), _p(sel_bias)
    return d


def moe_layer_workspace_size(desc: MoELayerDesc, T_max: int) -> int:
    return lib.moe_layer_workspace_size(ctypes.byref(desc), T_max)


def moe_layer(desc: MoELayerDesc, T, x, y, ws, ws_bytes, dbg: MoEDebugOut | None = None,
              stream=None):
    _check("moe_layer", lib.moe_layer(ctypes.byref(desc), T, _p(x), _p(y), _p(ws), ws_bytes,
                                      None if dbg is None else ctypes.byref(dbg),
                                      _stream(stream)))


def moe_layer_path(desc: MoELayerDesc, T: int) -> str:
    """"decode" or "staged": the path moe_layer takes for this call."""
    r = lib.moe_layer_path(ctypes.byref(desc), T)
    if r < 0:
        raise MoEError("moe_layer_path", -r)
    return "decode" if r == 1 else "staged"


def moe_layer_staged(desc: MoELayerDesc, T, x, y, ws, ws_bytes, dbg: MoEDebugOut | None = None,
                     stream=None):
    _check("moe_layer_staged",
           lib.moe_layer_staged(ctypes.byref(desc), T, _p(x), _p(y), _p(ws), ws_bytes,
                                None if dbg is None else ctypes.byref(dbg), _stream(stream)))


def moe_layer_capacity(desc: MoELayerDesc, T, capacity, padded, x, y, ws, ws_bytes,
                       dbg: MoEDebugOut | None = None, dropped=None, stream=None):
    _check("moe_layer_capacity",
           lib.moe_layer_capacity(ctypes.byref(desc), T, capacity, int(padded), _p(x), _p(y),
                                  _p(ws), ws_bytes, None if dbg is None else ctypes.byref(dbg),
                                  _p(dropped), _stream(stream)))


def moe_layer_capacity_workspace_size(desc: MoELayerDesc, T_max: int, capacity: int,
                                      padded: int) -> int:
    return lib.moe_layer_capacity_workspace_size(ctypes.byref(desc), T_max, capacity, int(padded))


def moe_layer_decode(desc: MoELayerDesc, T, x, y, ws, ws_bytes, dbg: MoEDebugOut | None = None,
                     stream=None):
    _check("moe_layer_decode",
           lib.moe_layer_decode(ctypes.byref(desc), T, _p(x), _p(y), _p(ws), ws_bytes,
                                None if dbg is None else ctypes.byref(dbg), _stream(stream)))


def moe_layer_status(ws, ws_bytes, stream=None):
    """Read (and clear) the decode path's wait error word of a layer
    workspace; raises MoEError(MOE_ERR_WAIT) if it was set."""
    _check("moe_layer_status", lib.moe_layer_status(_p(ws), ws_bytes, _stream(stream)))


def moe_layer_static(desc: MoELayerDesc, T, x, y, dbg: MoEDebugOut | None = None, stream=None):
    _check("moe_layer_static",
           lib.moe_layer_static(ctypes.byref(desc), T, _p(x), _p(y),
                                None if dbg is None else ctypes.byref(dbg), _stream(stream)))


def layer_workspace(desc: MoELayerDesc, T_max: int, device="cuda", capacity=None, padded=0):
    """A zeroed workspace tensor for the layer entry points (the decode path's
    synchronisation block must start zeroed); with capacity and padded = 1,
    sized for moe_layer_capacity's padded layout."""
    import torch
    if capacity is None:
        n = moe_layer_workspace_size(desc, T_max)
    else:
        n = moe_layer_capacity_workspace_size(desc, T_max, capacity, padded)
    if n == 0:
        raise ValueError("invalid layer description")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def debug_out(logits=None, topk_ids=None, topk_w=None, counts=None, offsets=None, src_token=None,
              dst_row=None, stage_events=None) -> MoEDebugOut:
    """Fill moe_debug_out; stage_events: up to 6 raw hipEvent_t handles (ints) or None."""
    o = MoEDebugOut()
    o.logits, o.topk_ids, o.topk_w = _p(logits), _p(topk_ids), _p(topk_w)
    o.counts, o.offsets, o.src_token, o.dst_row = _p(counts), _p(offsets), _p(src_token), _p(dst_row)
    for i, ev in enumerate(stage_events or ()):
        o.stage_events[i] = ev
    return o
