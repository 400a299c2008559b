"""ctypes loader for libw4a16moe.so (the C ABI declared in include/w4a16_moe.h).

Argument marshalling only.  The library must have been built in-tree
(``w4a16_grouped_expert_amd._build.build()``); a missing library is an error,
never a fallback.
"""
import ctypes
import os

from ._build import LIBDIR, LIBNAME

LIB_PATH = os.path.join(LIBDIR, LIBNAME)

c_int, c_i64, c_vp, c_double = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
c_i32p = ctypes.POINTER(ctypes.c_int32)
c_i64p = ctypes.POINTER(ctypes.c_int64)
c_u64p = ctypes.POINTER(ctypes.c_uint64)

MOE_OK = 0
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED_SHAPE", 3: "MOE_ERR_WORKSPACE",
          4: "MOE_ERR_CAPACITY", 5: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with {STATUS.get(status, status)}: {msg}")
        self.status = status


class ExpertLayout(ctypes.Structure):
    _fields_ = [("w13_codes", c_i64), ("w13_scales", c_i64), ("w2_codes", c_i64), ("w2_scales", c_i64),
                ("blob_bytes", c_i64)]


class MatLayout(ctypes.Structure):
    _fields_ = [("w13_hi", c_i64), ("w13_lo", c_i64), ("w13_scales", c_i64), ("w2_hi", c_i64), ("w2_lo", c_i64),
                ("w2_scales", c_i64), ("blob_bytes", c_i64), ("two_bit_bytes", c_i64)]


class FfnArgs(ctypes.Structure):
    _fields_ = [
        ("x", c_vp), ("T", c_int), ("d", c_int), ("I", c_int), ("E", c_int), ("k", c_int),
        ("topk_ids", c_vp), ("topk_weights", c_vp),
        ("expert_offsets", c_vp), ("sorted_pairs", c_vp), ("pair_pos", c_vp), ("active_experts", c_vp),
        ("tile_offsets", c_vp),
        ("bank", c_vp), ("bank_stride", c_i64), ("slot_of_expert", c_vp),
        ("mode", c_int), ("combine", c_int), ("out", c_vp),
        ("workspace", c_vp), ("workspace_bytes", c_i64),
    ]


class LayerArgs(ctypes.Structure):
    _fields_ = [
        ("x", c_vp), ("w_router", c_vp), ("T", c_int), ("d", c_int), ("I", c_int), ("E", c_int), ("k", c_int),
        ("renormalize", c_int), ("bank", c_vp), ("bank_stride", c_i64),
        ("logits", c_vp), ("topk_ids", c_vp), ("topk_weights", c_vp), ("out", c_vp),
        ("workspace", c_vp), ("workspace_bytes", c_i64), ("counters", c_vp),
    ]


# name -> (restype, argtypes)
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_abi_version": (c_int, []),
    "moe_expert_layout_get": (c_int, [c_int, c_int, ctypes.POINTER(ExpertLayout)]),
    "pack_w4_g128": (c_int, [c_vp, c_int, c_int, c_int, c_int, c_vp, c_i64, c_vp, c_i64, c_vp]),
    "moe_route": (c_int, [c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp]),
    "moe_align": (c_int, [c_vp, c_int, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_route_align": (c_int, [c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp,
                                c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_ffn_workspace_bytes": (c_i64, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "moe_w4a16_grouped_ffn": (c_int, [ctypes.POINTER(FfnArgs), c_vp]),
    "moe_w4a16_grouped_ffn_noalloc": (c_int, [ctypes.POINTER(FfnArgs), c_vp]),
    "moe_bf16_expert_bytes": (c_i64, [c_int, c_int]),
    "moe_bf16_pack": (c_int, [c_vp, c_vp, c_int, c_int, c_int, c_vp, c_i64, c_vp]),
    "moe_bf16_grouped_ffn": (c_int, [ctypes.POINTER(FfnArgs), c_vp]),
    "moe_mat_layout_get": (c_int, [c_int, c_int, ctypes.POINTER(MatLayout)]),
    "moe_mat_from_w4": (c_int, [c_vp, c_i64, c_int, c_int, c_int, c_vp, c_i64, c_vp]),
    "moe_mat_grouped_ffn": (c_int, [ctypes.POINTER(FfnArgs), ctypes.c_float, c_vp]),
    "moe_decode_layer_workspace_bytes": (c_i64, [c_int, c_int, c_int, c_int, c_int]),
    "moe_decode_layer": (c_int, [ctypes.POINTER(LayerArgs), c_vp]),
    "moe_mat_decode_layer": (c_int, [ctypes.POINTER(LayerArgs), ctypes.c_float, c_vp]),
    "moe_slot_cache_create": (c_int, [c_int, c_int, c_i64, c_vp, c_vp, ctypes.POINTER(c_vp)]),
    "moe_slot_cache_destroy": (c_int, [c_vp]),
    "slot_cache_load": (c_int, [c_vp, c_u64p, c_u64p, c_vp, c_i32p, c_i32p, c_vp, c_vp, c_vp]),
    "moe_slot_cache_state": (c_int, [c_vp, c_i32p, c_i64p, c_i64p]),
    "slot_cache_prefetch": (c_int, [c_vp, c_u64p, c_int, c_i32p, c_vp, c_vp]),
    "moe_slot_cache_configure": (c_int, [c_vp, c_int, c_double, c_int]),
    "slot_cache_begin_step": (c_int, [c_vp, c_u64p]),
    "moe_slot_cache_set_prefix": (c_int, [c_vp, c_i64]),
    "slot_cache_load_precision": (c_int, [c_vp, c_u64p, c_u64p, c_u64p, c_vp, c_i32p, c_i32p, c_i64p, c_vp, c_vp,
                                          c_vp]),
    "moe_slot_cache_planes": (c_int, [c_vp, c_i32p, c_i64p, c_i64p]),
    "moe_timing_enable": (c_int, [c_int]),
    "moe_timing_reset": (c_int, []),
    "moe_timing_read": (c_int, [c_int, ctypes.POINTER(c_double), c_i64p]),
}

_lib = None


def lib():
    """The loaded library (loads on first use; raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it first with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype, fn.argtypes = res, args
        _lib = l
    return _lib


def check(fn_name, status):
    if status != MOE_OK:
        msg = lib().moe_last_error().decode(errors="replace")
        raise MoeError(fn_name, status, msg)
    return status
