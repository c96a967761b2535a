"""ctypes declarations of libmoedecode's C ABI (include/moedecode.h).

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoedecode.so")

c_status = C.c_int32
vp = C.c_void_p


class moe_shape(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("inter", C.c_int32), ("shared_inter", C.c_int32), ("group", C.c_int32)]


class moe_q4(C.Structure):
    _fields_ = [("q", vp), ("s", vp)]


class moe_blob_layout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s", "total")]


class moe_cache_event(C.Structure):
    _fields_ = [("expert", C.c_int32), ("slot", C.c_int32), ("hit", C.c_int32), ("evicted", C.c_int32)]


class moe_attn_shape(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("max_ctx", C.c_int32), ("rope_theta", C.c_float), ("eps", C.c_float)]


class moe_attn_weights(C.Structure):
    _fields_ = [("norm_w", vp), ("qkv_q", vp), ("qkv_s", vp), ("o_q", vp), ("o_s", vp)]


class moe_layer_desc(C.Structure):
    _fields_ = [("router", vp), ("bias", vp), ("shared_blob", vp), ("experts_dev", vp),
                ("experts_host", vp), ("slot_pool", vp), ("n_slots", C.c_int32),
                ("copy_stream", vp), ("workspace", vp), ("workspace_bytes", C.c_size_t),
                ("store", vp), ("store_layer", C.c_int32), ("cache_policy", C.c_int32),
                ("cache_on_device", C.c_int32)]


class moe_decode_stats(C.Structure):
    _fields_ = [("hits", C.c_int64), ("misses", C.c_int64), ("h2d_bytes", C.c_int64), ("calls", C.c_int64),
                ("ms_route", C.c_float), ("ms_fill", C.c_float), ("ms_wait_fill", C.c_float),
                ("ms_total", C.c_float)]


class moe_kernel_time(C.Structure):
    _fields_ = [("launches", C.c_int64), ("ms_total", C.c_double)]


P = C.POINTER

# name -> (restype, argtypes); every symbol declared in include/moedecode.h
SIGNATURES = {
    "moe_last_error": (C.c_char_p, []),
    "moe_abi_version": (C.c_int32, []),
    "moe_expert_bytes": (C.c_size_t, [C.c_int32, C.c_int32]),
    "moe_blob_layout_of": (c_status, [C.c_int32, C.c_int32, P(moe_blob_layout)]),
    "moe_route_workspace_bytes": (C.c_size_t, [P(moe_shape), C.c_int32]),
    "moe_route": (c_status, [P(moe_shape), vp, vp, vp, vp, C.c_int32, vp, vp, vp, C.c_size_t, vp]),
    "moe_route_noalloc": (c_status, [P(moe_shape), vp, vp, vp, vp, C.c_int32, vp, vp, vp]),
    "moe_cache_create": (c_status, [C.c_int32, C.c_int32, P(vp)]),
    "moe_cache_create_policy": (c_status, [C.c_int32, C.c_int32, C.c_int32, P(vp)]),
    "moe_cache_destroy": (None, [vp]),
    "moe_cache_step": (c_status, [vp, P(C.c_int32), C.c_int32, P(moe_cache_event), P(C.c_int32)]),
    "moe_cache_reset": (c_status, [vp]),
    "moe_cache_slots": (c_status, [vp, P(C.c_int32), P(C.c_int32), P(C.c_int64), C.c_int32]),
    "moe_cache_counters": (c_status, [vp, P(C.c_int64), P(C.c_int64), P(C.c_int64)]),
    "moe_expert_gemv_q4": (c_status, [P(moe_q4), C.c_int32, C.c_int32, vp, C.c_int32, vp, vp]),
    "moe_layer_workspace_bytes": (c_status, [P(moe_shape), C.c_int32, C.c_int32, P(C.c_size_t)]),
    "moe_layer_create": (c_status, [P(moe_shape), P(moe_layer_desc), C.c_int32, C.c_int32, P(vp)]),
    "moe_layer_destroy": (None, [vp]),
    "moe_layer_set_experts": (c_status, [vp, vp]),
    "moe_layer_cache": (vp, [vp]),
    "moe_layer_decode": (c_status, [vp, vp, vp, C.c_int32, C.c_uint32, vp, vp, vp, vp,
                                    P(moe_cache_event), P(moe_decode_stats), vp]),
    "moe_layer_prefill": (c_status, [vp, vp, vp, C.c_int32, vp, vp, vp, vp]),
    "moe_layer_prefill_chunk": (c_status, [vp, C.c_int32]),
    "moe_debug_fail_copy": (c_status, [vp, C.c_int32]),
    "moe_layer_profile": (c_status, [vp, C.c_int32]),
    "moe_layer_profile_kinds": (c_status, [vp, C.c_uint32, C.c_int32, C.c_int32]),
    "moe_layer_profile_read": (c_status, [vp, C.c_int32, P(moe_kernel_time)]),
    "moe_debug_unpack_q4": (c_status, [P(moe_q4), C.c_int32, C.c_int32, vp, vp]),
    "moe_layer_cache_state": (c_status, [vp, vp, vp, vp, C.c_int32, vp, vp, vp, vp]),
    "moe_attn_workspace_bytes": (c_status, [P(moe_attn_shape), P(C.c_size_t)]),
    "moe_attn_decode": (c_status, [P(moe_attn_shape), P(moe_attn_weights), vp, vp, C.c_int32, vp, vp, vp,
                                   C.c_size_t, vp]),
    "moe_debug_read_floor": (c_status, [vp, C.c_int64, C.c_int64, C.c_int32, C.c_int32, C.c_int32, vp,
                                        P(C.c_double), vp]),
    "moe_store_stride": (C.c_int64, [C.c_int64]),
    "moe_store_open": (c_status, [C.c_char_p, C.c_int32, C.c_int32, C.c_int64, C.c_int32, C.c_int32, P(vp)]),
    "moe_store_is_direct": (C.c_int32, [vp]),
    "moe_store_close": (None, [vp]),
    "moe_store_read": (c_status, [vp, C.c_int32, P(C.c_int32), C.c_int32, P(vp)]),
}

_lib = None


def load():
    """Loads libmoedecode.so and declares every entry point; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; build it with `python -m bit_quantized_expert_softmax_amd.build`")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
