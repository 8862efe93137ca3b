"""ctypes declarations of the C ABI in include/moe.h."""
from __future__ import annotations

import ctypes
import os

MOE_OK = 0
MOE_F32 = 0
MOE_BF16 = 1
GATE_TOPK_SOFTMAX = 0
GATE_SOFTMAX_TOPK = 1
GATE_SOFTMAX_TOPK_RENORM = 2
GATE_SIGMOID_BIAS_RENORM = 3

_PKG = os.path.dirname(os.path.abspath(__file__))

c_int, c_size_t, c_void_p, c_char_p = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_char_p


class MoELayerDesc(ctypes.Structure):
    _fields_ = [("H", c_int), ("E", c_int), ("k", c_int), ("I_loc", c_int), ("e_begin", c_int),
                ("e_end", c_int), ("I_shared", c_int), ("mode", c_int), ("dt", c_int),
                ("w_router", c_void_p), ("w13", c_void_p), ("w2", c_void_p),
                ("w13_shared", c_void_p), ("w2_shared", c_void_p),
                ("logit_bias", c_void_p), ("sel_bias", c_void_p)]


class MoEDebugOut(ctypes.Structure):
    _fields_ = [("logits", c_void_p), ("topk_ids", c_void_p), ("topk_w", c_void_p),
                ("counts", c_void_p), ("offsets", c_void_p), ("src_token", c_void_p),
                ("dst_row", c_void_p), ("stage_events", c_void_p * 6)]


# name -> (restype, argtypes)
_SIGS = {
    "moe_abi_version": (c_int, []),
    "moe_source_sha256": (c_char_p, []),
    "moe_status_str": (c_char_p, [c_int]),
    "moe_route": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_int, c_void_p,
                          c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_permute_workspace_size": (c_size_t, [c_int, c_int, c_int]),
    "moe_permute": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int, c_void_p, c_int, c_int,
                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                            c_void_p]),
    "moe_permute_capacity": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                     c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_grouped_ffn_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
    "moe_grouped_ffn": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                                c_void_p, c_void_p, c_int, c_void_p, c_int, c_void_p, c_size_t,
                                c_void_p]),
    "moe_combine": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p,
                            c_void_p, c_int, c_void_p]),
    "moe_pack_workspace_size": (c_size_t, [c_int, c_int, c_int]),
    "moe_pack_by_rank": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_int,
                                 c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_unpack_sum": (c_int, [c_void_p, c_int, c_void_p, c_int, c_int, c_int, c_void_p, c_int,
                               c_void_p]),
    "moe_reshard_ep_to_tp_pack": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                          c_void_p, c_void_p, c_void_p]),
    "moe_reshard_tp_to_ep_interleave": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                                                c_int, c_void_p, c_void_p, c_void_p]),
    "moe_layer_workspace_size": (c_size_t, [ctypes.POINTER(MoELayerDesc), c_int]),
    "moe_layer": (c_int, [ctypes.POINTER(MoELayerDesc), c_int, c_void_p, c_void_p, c_void_p,
                          c_size_t, ctypes.POINTER(MoEDebugOut), c_void_p]),
    "moe_layer_path": (c_int, [ctypes.POINTER(MoELayerDesc), c_int]),
    "moe_layer_status": (c_int, [c_void_p, c_size_t, c_void_p]),
    "moe_layer_staged": (c_int, [ctypes.POINTER(MoELayerDesc), c_int, c_void_p, c_void_p,
                                 c_void_p, c_size_t, ctypes.POINTER(MoEDebugOut), c_void_p]),
    "moe_layer_capacity": (c_int, [ctypes.POINTER(MoELayerDesc), c_int, c_int, c_int, c_void_p,
                                   c_void_p, c_void_p, c_size_t, ctypes.POINTER(MoEDebugOut),
                                   c_void_p, c_void_p]),
    "moe_layer_capacity_workspace_size": (c_size_t, [ctypes.POINTER(MoELayerDesc), c_int, c_int,
                                                     c_int]),
    "moe_layer_decode": (c_int, [ctypes.POINTER(MoELayerDesc), c_int, c_void_p, c_void_p,
                                 c_void_p, c_size_t, ctypes.POINTER(MoEDebugOut), c_void_p]),
    "moe_layer_static": (c_int, [ctypes.POINTER(MoELayerDesc), c_int, c_void_p, c_void_p,
                                 ctypes.POINTER(MoEDebugOut), c_void_p]),
}
# bytes of the device array moe_layer_static uses as its workspace
STATIC_SCRATCH_BYTES = 64 << 20
# bytes at the start of a layer workspace that the decode path keeps between calls
LAYER_SYNC_BYTES = 4096 + 1024 * 128
EXPORTED_SYMBOLS = tuple(_SIGS)


def lib_path():
    return os.environ.get("MOE_MI355X_LIB", os.path.join(_PKG, "lib", "libmoe_mi355x.so"))


def load_library():
    """Load the built library.  Raises ImportError if it is missing, or if it
    was built from other sources than those in the tree (a stale binary);
    MOE_MI355X_LIB names another library explicitly and skips that check."""
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"HIP library not built: {path} is missing "
                          "(run `python -m mixture_experts_layer_amd.build`)")
    # torch first: its HIP runtime (soname libamdhip64.so.7) is then the one
    # the library binds to.  Loaded the other way round, torch would load a
    # second runtime beside the library's, and the stream handles the binding
    # takes from torch would be foreign to the runtime that launches the
    # kernels.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if "MOE_MI355X_LIB" not in os.environ:
        from .build import source_sha256
        built, want = lib.moe_source_sha256().decode(), source_sha256()
        if built != want:
            raise ImportError(f"stale HIP library {path}: built from sources {built[:12]}, the "
                              f"tree holds {want[:12]} (run `python -m "
                              "mixture_experts_layer_amd.build`)")
    return lib
