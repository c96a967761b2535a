"""Python binding of libmoedecode: same names as the C ABI, marshalling only.

Device buffers are torch tensors (their ``data_ptr()`` is passed), host
buffers are numpy arrays or pinned torch tensors, streams are
``torch.cuda.Stream`` objects (or raw hipStream_t ints; None means torch's
current stream). Every step of the layer runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import _lib as L

MOE_F_RMSNORM_IN = 1
MOE_F_RESIDUAL = 2
MOE_F_FILL_KERNEL = 4
MOE_F_STAGE_TIMES = 16
MOE_POLICY_LFU = 0
MOE_POLICY_LRU = 1
STATUS = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_ESHAPE", -3: "MOE_EALIGN", -4: "MOE_EHIP",
          -5: "MOE_ENOMEM", -6: "MOE_ESTATE"}

moe_decode_stats = L.moe_decode_stats
moe_cache_event = L.moe_cache_event


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str, text: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {text}")
        self.status = status


def lib():
    return L.load()


def _check(st: int, fn: str) -> None:
    if st != 0:
        raise MoeError(st, fn, lib().moe_last_error().decode())


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def make_shape(sh) -> L.moe_shape:
    return L.moe_shape(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter,
                       getattr(sh, "group", 32))


# ------------------------------------------------------------------ misc
def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_expert_bytes(hidden: int, inter: int) -> int:
    return lib().moe_expert_bytes(hidden, inter)


def moe_blob_layout_of(hidden: int, inter: int) -> dict:
    out = L.moe_blob_layout()
    _check(lib().moe_blob_layout_of(hidden, inter, C.byref(out)), "moe_blob_layout_of")
    return {n: getattr(out, n) for n, _ in L.moe_blob_layout._fields_}


# ------------------------------------------------------------------ routing
def moe_route_workspace_bytes(sh, B: int) -> int:
    s = make_shape(sh)
    return lib().moe_route_workspace_bytes(C.byref(s), B)


def moe_route(sh, x, wr, bias, logits_in, B, ids, w, workspace=None, stream=None):
    s = make_shape(sh)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_route(C.byref(s), _p(x), _p(wr), _p(bias), _p(logits_in), B, _p(ids), _p(w),
                           _p(workspace), ws_bytes, _stream(stream)), "moe_route")


MOE_ROUTE_NOALLOC_MAX = 131072


def moe_route_noalloc(sh, x, wr, bias, logits_in, B, ids, w, stream=None):
    s = make_shape(sh)
    _check(lib().moe_route_noalloc(C.byref(s), _p(x), _p(wr), _p(bias), _p(logits_in), B, _p(ids), _p(w),
                                   _stream(stream)), "moe_route_noalloc")


# ------------------------------------------------------------------ LFU cache
def moe_cache_create(n_slots: int, n_experts: int, policy: int = 0) -> int:
    h = C.c_void_p()
    if policy == MOE_POLICY_LFU:
        _check(lib().moe_cache_create(n_slots, n_experts, C.byref(h)), "moe_cache_create")
    else:
        _check(lib().moe_cache_create_policy(n_slots, n_experts, policy, C.byref(h)), "moe_cache_create_policy")
    return h.value


def moe_cache_destroy(h) -> None:
    lib().moe_cache_destroy(h)


def moe_cache_step(h, ids):
    """Returns (events int32 [k][4] = expert, slot, hit, evicted; n_miss)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    k = ids.size
    ev = (L.moe_cache_event * max(k, 1))()
    n = C.c_int32(0)
    _check(lib().moe_cache_step(h, ids.ctypes.data_as(C.POINTER(C.c_int32)), k, ev, C.byref(n)),
           "moe_cache_step")
    return events_to_array(ev, k), n.value


def events_to_array(ev, k: int) -> np.ndarray:
    return np.array([[e.expert, e.slot, e.hit, e.evicted] for e in ev[:k]], dtype=np.int32).reshape(k, 4)


def moe_cache_reset(h) -> None:
    _check(lib().moe_cache_reset(h), "moe_cache_reset")


def moe_cache_slots(h, n_slots: int):
    ex = np.zeros(n_slots, np.int32)
    fr = np.zeros(n_slots, np.int32)
    la = np.zeros(n_slots, np.int64)
    _check(lib().moe_cache_slots(h, ex.ctypes.data_as(C.POINTER(C.c_int32)),
                                 fr.ctypes.data_as(C.POINTER(C.c_int32)),
                                 la.ctypes.data_as(C.POINTER(C.c_int64)), n_slots), "moe_cache_slots")
    return ex, fr, la


def moe_cache_counters(h):
    a, b, c = C.c_int64(), C.c_int64(), C.c_int64()
    _check(lib().moe_cache_counters(h, C.byref(a), C.byref(b), C.byref(c)), "moe_cache_counters")
    return a.value, b.value, c.value


# ------------------------------------------------------------------ GEMV
def moe_expert_gemv_q4(q, s, N, K, x, M, y, stream=None):
    W = L.moe_q4(_p(q), _p(s))
    _check(lib().moe_expert_gemv_q4(C.byref(W), N, K, _p(x), M, _p(y), _stream(stream)),
           "moe_expert_gemv_q4")


def moe_debug_unpack_q4(q, N, K, out, stream=None):
    W = L.moe_q4(_p(q), None)
    _check(lib().moe_debug_unpack_q4(C.byref(W), N, K, _p(out), _stream(stream)), "moe_debug_unpack_q4")


def moe_debug_read_floor(src, nbytes, blocks, out, *, region_stride=0, regions=1, reps=1, timed=False,
                         stream=None):
    """Streams nbytes per launch (reps launches rotating over regions); returns
    the mean µs per launch when timed, else None (launches only enqueued)."""
    us = C.c_double(0.0)
    _check(lib().moe_debug_read_floor(_p(src), nbytes, region_stride, regions, blocks, reps, _p(out),
                                      C.byref(us) if timed else None, _stream(stream)),
           "moe_debug_read_floor")
    return us.value if timed else None


# ------------------------------------------------------------------ attention step
def make_attn_shape(a) -> L.moe_attn_shape:
    return L.moe_attn_shape(a.hidden, a.n_heads, a.n_kv_heads, a.head_dim, a.max_ctx, a.rope_theta, a.eps)


def moe_attn_workspace_bytes(a) -> int:
    s = make_attn_shape(a)
    out = C.c_size_t(0)
    _check(lib().moe_attn_workspace_bytes(C.byref(s), C.byref(out)), "moe_attn_workspace_bytes")
    return out.value


def moe_attn_decode(a, w, k_cache, v_cache, pos, x, y, workspace, stream=None):
    """One token at position pos through the attention step. w: mapping with
    device tensors norm_w, qkv_q, qkv_s, o_q, o_s; caches fp16 (as int16)
    [n_kv_heads][max_ctx][d]; x, y fp32 [H]; workspace a uint8 tensor of at
    least moe_attn_workspace_bytes bytes."""
    s = make_attn_shape(a)
    W = L.moe_attn_weights(_p(w["norm_w"]), _p(w["qkv_q"]), _p(w["qkv_s"]), _p(w["o_q"]), _p(w["o_s"]))
    nbytes = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    _check(lib().moe_attn_decode(C.byref(s), C.byref(W), _p(k_cache), _p(v_cache), pos, _p(x), _p(y),
                                 _p(workspace), nbytes, _stream(stream)), "moe_attn_decode")


# ------------------------------------------------------------------ layer
def moe_layer_workspace_bytes(sh, max_B: int, max_T: int = 0) -> int:
    s = make_shape(sh)
    out = C.c_size_t(0)
    _check(lib().moe_layer_workspace_bytes(C.byref(s), max_B, max_T, C.byref(out)),
           "moe_layer_workspace_bytes")
    return out.value


def moe_layer_create(sh, *, router, shared_blob, workspace, bias=None, experts_dev=None,
                     experts_host=None, slot_pool=None, n_slots=0, copy_stream=None, max_B=1,
                     max_T=0, store=None, store_layer=0, cache_policy=0, cache_on_device=False) -> int:
    s = make_shape(sh)
    d = L.moe_layer_desc(_p(router), _p(bias), _p(shared_blob), _p(experts_dev), _p(experts_host),
                         _p(slot_pool), n_slots,
                         None if copy_stream is None else _stream(copy_stream),
                         _p(workspace), workspace.numel() * workspace.element_size(), store, store_layer,
                         cache_policy, 1 if cache_on_device else 0)
    h = C.c_void_p()
    _check(lib().moe_layer_create(C.byref(s), C.byref(d), max_B, max_T, C.byref(h)), "moe_layer_create")
    return h.value


def moe_layer_destroy(h) -> None:
    lib().moe_layer_destroy(h)


def moe_layer_set_experts(h, experts_dev) -> None:
    _check(lib().moe_layer_set_experts(h, _p(experts_dev)), "moe_layer_set_experts")


def moe_layer_cache(h):
    return lib().moe_layer_cache(h)


def moe_layer_cache_state(h, n_slots, stream=None):
    """(expert, freq, last, hits, misses, steps) of the handle's slot cache."""
    ex = np.zeros(n_slots, np.int32)
    fr = np.zeros(n_slots, np.int32)
    la = np.zeros(n_slots, np.int64)
    hits, misses, steps = C.c_int64(), C.c_int64(), C.c_int64()
    _check(lib().moe_layer_cache_state(h, ex.ctypes.data, fr.ctypes.data, la.ctypes.data, n_slots,
                                       C.byref(hits), C.byref(misses), C.byref(steps), _stream(stream)),
           "moe_layer_cache_state")
    return ex, fr, la, hits.value, misses.value, steps.value


def moe_layer_decode(h, x, add_in, B, flags, y, ids_out=None, w_out=None, u_out=None,
                     trace_k: int = 0, stats=None, stream=None):
    """Returns the cache events as int32 [B*k][4] when trace_k > 0 (cache mode), else None."""
    ev = (L.moe_cache_event * (B * trace_k))() if trace_k else None
    st = lib().moe_layer_decode(h, _p(x), _p(add_in), B, flags, _p(y), _p(ids_out), _p(w_out),
                                _p(u_out), ev, None if stats is None else C.byref(stats),
                                _stream(stream))
    _check(st, "moe_layer_decode")
    return events_to_array(ev, B * trace_k) if trace_k else None


def moe_layer_prefill_chunk(h, tokens: int) -> None:
    _check(lib().moe_layer_prefill_chunk(h, tokens), "moe_layer_prefill_chunk")


def moe_debug_fail_copy(h, nth: int) -> None:
    _check(lib().moe_debug_fail_copy(h, nth), "moe_debug_fail_copy")


def moe_layer_prefill(h, x_bf16, logits_in, T, y, ids_out=None, w_out=None, stream=None):
    _check(lib().moe_layer_prefill(h, _p(x_bf16), _p(logits_in), T, _p(y), _p(ids_out), _p(w_out),
                                   _stream(stream)), "moe_layer_prefill")


def moe_layer_profile(h, enable: bool) -> None:
    _check(lib().moe_layer_profile(h, 1 if enable else 0), "moe_layer_profile")


def moe_layer_profile_kinds(h, mask: int, every: int = 1, reserve_events: int = 0) -> None:
    _check(lib().moe_layer_profile_kinds(h, mask, every, reserve_events), "moe_layer_profile_kinds")


def moe_layer_profile_read(h, kind: int):
    out = L.moe_kernel_time()
    _check(lib().moe_layer_profile_read(h, kind, C.byref(out)), "moe_layer_profile_read")
    return out.launches, out.ms_total


# ---------------------------------------------------------------- expert file store
def moe_store_stride(blob_bytes: int) -> int:
    return int(lib().moe_store_stride(blob_bytes))


def moe_store_open(path: str, n_layers: int, n_experts: int, blob_bytes: int, threads: int = 8,
                   direct: bool = True) -> int:
    h = C.c_void_p()
    _check(lib().moe_store_open(path.encode(), n_layers, n_experts, blob_bytes, threads, 1 if direct else 0,
                                C.byref(h)), "moe_store_open")
    return h.value


def moe_store_is_direct(h) -> bool:
    return bool(lib().moe_store_is_direct(h))


def moe_store_close(h) -> None:
    lib().moe_store_close(h)


def moe_store_read(h, layer: int, experts, dst_ptrs) -> None:
    """Reads the padded blobs of `experts` (ints) of `layer` into host buffers
    at the addresses dst_ptrs (one stride each)."""
    n = len(experts)
    ids = (C.c_int32 * max(n, 1))(*experts)
    ptrs = (C.c_void_p * max(n, 1))(*dst_ptrs)
    _check(lib().moe_store_read(h, layer, ids, n, ptrs), "moe_store_read")
