"""Python binding of libeo (the MoE expert-offload layer for MI355X).

Argument marshalling only: every call goes straight to the C ABI declared in
``include/eo.h`` under the same name. Pointers may be passed as ints or as
objects with ``data_ptr()`` (torch tensors); streams as ints or
``torch.cuda.Stream``. Raises RuntimeError when the HIP library is not built —
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libeo.so")

EO_OK, EO_ERR_INVALID_ARG, EO_ERR_OOM, EO_ERR_HIP, EO_ERR_STATE, EO_ERR_UNSUPPORTED = \
    0, -1, -2, -3, -4, -5
EO_W_FP32, EO_W_BF16, EO_W_MXFP4, EO_W_NVFP4, EO_W_FP8 = 0, 1, 2, 3, 4
EO_MAX_EXPERTS = 1024

STATUS_NAMES = {0: "EO_OK", -1: "EO_ERR_INVALID_ARG", -2: "EO_ERR_OOM", -3: "EO_ERR_HIP",
                -4: "EO_ERR_STATE", -5: "EO_ERR_UNSUPPORTED"}


class eo_config(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("shared_experts", ctypes.c_int32),
                ("wfmt", ctypes.c_int32), ("act_bf16", ctypes.c_int32),
                ("cache_slots", ctypes.c_int64), ("max_tokens", ctypes.c_int32),
                ("host_threads", ctypes.c_int32), ("device", ctypes.c_int32)]


_A = ctypes.c_int32 * EO_MAX_EXPERTS


class eo_plan_host(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32), ("m", ctypes.c_int32), ("q", ctypes.c_int32),
                ("q_fill", ctypes.c_int32), ("n_hit", ctypes.c_int32),
                ("n_host", ctypes.c_int32), ("n_evict", ctypes.c_int32),
                ("pad_", ctypes.c_int32), ("clock", ctypes.c_int64),
                ("credit", ctypes.c_int64), ("hit_expert", _A), ("hit_slot", _A),
                ("fill_expert", _A), ("fill_slot", _A), ("host_expert", _A),
                ("evicted_key", _A)]


class eo_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("lookups", "hits", "misses", "fills",
                                               "host_experts", "pcie_bytes", "host_bytes",
                                               "prefill_layers", "device_expert_bytes",
                                               "host_wait_ns", "host_routine_ns")]


class EOError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I32, _I64, _U32, _U64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64
_SIGS = {
    "eo_create": [ctypes.POINTER(eo_config), ctypes.POINTER(_P)],
    "eo_destroy": [_P],
    "eo_pool_expert": [_P, _I32, _I32, ctypes.POINTER(_P), ctypes.POINTER(_U64)],
    "eo_set_shared_expert": [_P, _I32, _P, _U64],
    "eo_set_router": [_P, _I32, _P],
    "eo_measure_bandwidth": [_P, ctypes.POINTER(_U32), ctypes.POINTER(_U32)],
    "eo_remeasure_bandwidth": [_P, ctypes.POINTER(_U32), ctypes.POINTER(_U32)],
    "eo_set_bandwidth": [_P, _U32, _U32],
    "eo_route": [_P, _I32, _P, _I32, _P, _P, _P, _P],
    "eo_route_noalloc": [_P, _I32, _P, _I32, _P, _P, _P, _P],
    "eo_lookup_plan": [_P, _I32, _P, _I32, _P],
    "eo_fill": [_P, _P],
    "eo_host_execute": [_P, _P, _P, _P, _P],
    "eo_expert_ffn_combine": [_P, _I32, _P, _P, _P, _P, _P],
    "eo_moe_layer": [_P, _I32, _P, _P, _I32, _P, _P],
    "eo_decode_step": [_P, _P, _I32, _P, _P],
    "eo_prefill": [_P, _P, _I32, _I32, _P],
    "eo_set_capture": [_P, _P, _P, _P, _P, _I32],
    "eo_cache_snapshot": [_P, _P, _P, ctypes.POINTER(_I64), ctypes.POINTER(_I64)],
    "eo_last_plan": [_P, ctypes.POINTER(eo_plan_host)],
    "eo_dequant": [_P, _I32, _I32, _P],
    "eo_dequant_with": [_P, _I32, _I32, _I32, _P],
    "eo_stats_get": [_P, ctypes.POINTER(eo_stats)],
    "eo_resize_cache": [_P, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64)],
    "eo_set_static_placement": [_P, _P, _I32],
    "eo_clear_static_placement": [_P],
    "eo_kernel_times": [_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64), _I32],
    "eo_set_timing": [_P, _I32],
    "eo_stream_times": [_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64), _I32],
    "eo_set_plan_log": [_P, _I32],
    "eo_get_plan_log": [_P, _P, _I64, ctypes.POINTER(_I64)],
    "eo_expert_bytes": [_I32, _I32, _I32],
    "eo_sync": [_P],
    "eo_last_error": [],
}
EXPORTED = tuple(_SIGS)


def lib():
    """The loaded libeo.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is not built "
                               "(python -m expert_offload_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.eo_expert_bytes.restype = _U64
        L.eo_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError(f"cannot take a pointer of {type(x)}")


def _stream(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int):
    if status != EO_OK:
        raise EOError(status, lib().eo_last_error().decode())


def eo_last_error() -> str:
    return lib().eo_last_error().decode()


def eo_expert_bytes(hidden: int, inter: int, wfmt: int) -> int:
    return int(lib().eo_expert_bytes(hidden, inter, wfmt))


def eo_create(layers, experts, top_k, hidden, inter, wfmt, act_bf16, cache_slots, max_tokens,
              shared_experts=0, host_threads=0, device=0) -> int:
    cfg = eo_config(layers, experts, top_k, hidden, inter, shared_experts, wfmt, act_bf16,
                    cache_slots, max_tokens, host_threads, device)
    out = _P()
    _check(lib().eo_create(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def eo_destroy(e: int) -> None:
    _check(lib().eo_destroy(e))


def eo_pool_expert(e: int, layer: int, expert: int):
    p, n = _P(), _U64()
    _check(lib().eo_pool_expert(e, layer, expert, ctypes.byref(p), ctypes.byref(n)))
    return p.value, n.value


def eo_set_shared_expert(e: int, layer: int, host_block, nbytes: int) -> None:
    _check(lib().eo_set_shared_expert(e, layer, _ptr(host_block), nbytes))


def eo_set_router(e: int, layer: int, host_w) -> None:
    _check(lib().eo_set_router(e, layer, _ptr(host_w)))


def eo_measure_bandwidth(e: int):
    bp, bh = _U32(), _U32()
    _check(lib().eo_measure_bandwidth(e, ctypes.byref(bp), ctypes.byref(bh)))
    return bp.value, bh.value


def eo_remeasure_bandwidth(e: int):
    bp, bh = _U32(), _U32()
    _check(lib().eo_remeasure_bandwidth(e, ctypes.byref(bp), ctypes.byref(bh)))
    return bp.value, bh.value


def eo_set_bandwidth(e: int, bp_mbps: int, bh_mbps: int) -> None:
    _check(lib().eo_set_bandwidth(e, bp_mbps, bh_mbps))


def eo_route(e, layer, x, T, forced_ids, ids, w, stream=None) -> None:
    _check(lib().eo_route(e, layer, _ptr(x), T, _ptr(forced_ids), _ptr(ids), _ptr(w),
                          _stream(stream)))


def eo_route_noalloc(e, layer, x, T, forced_ids, ids, w, stream=None) -> None:
    _check(lib().eo_route_noalloc(e, layer, _ptr(x), T, _ptr(forced_ids), _ptr(ids), _ptr(w),
                                  _stream(stream)))


def eo_lookup_plan(e, layer, ids, T, stream=None) -> None:
    _check(lib().eo_lookup_plan(e, layer, _ptr(ids), T, _stream(stream)))


def eo_fill(e, stream=None) -> None:
    _check(lib().eo_fill(e, _stream(stream)))


def eo_host_execute(e, x, ids, w, stream=None) -> None:
    _check(lib().eo_host_execute(e, _ptr(x), _ptr(ids), _ptr(w), _stream(stream)))


def eo_expert_ffn_combine(e, layer, x, ids, w, y, stream=None) -> None:
    _check(lib().eo_expert_ffn_combine(e, layer, _ptr(x), _ptr(ids), _ptr(w), _ptr(y),
                                       _stream(stream)))


def eo_moe_layer(e, layer, x, y, T, forced_ids=None, stream=None) -> None:
    _check(lib().eo_moe_layer(e, layer, _ptr(x), _ptr(y), T, _ptr(forced_ids), _stream(stream)))


def eo_decode_step(e, x_inout, T, forced_ids=None, stream=None) -> None:
    _check(lib().eo_decode_step(e, _ptr(x_inout), T, _ptr(forced_ids), _stream(stream)))


EO_PREFILL_DOUBLE_BUFFER, EO_PREFILL_SKIP_RESIDENT = 1, 2


def eo_prefill(e, x_inout, T, flags=EO_PREFILL_DOUBLE_BUFFER, stream=None) -> None:
    _check(lib().eo_prefill(e, _ptr(x_inout), T, flags, _stream(stream)))


def eo_set_capture(e, x_in, y, ids, w, tokens_per_layer) -> None:
    _check(lib().eo_set_capture(e, _ptr(x_in), _ptr(y), _ptr(ids), _ptr(w), tokens_per_layer))


def eo_cache_snapshot(e, slot_key, slot_stamp):
    clock, credit = _I64(), _I64()
    _check(lib().eo_cache_snapshot(e, _ptr(slot_key), _ptr(slot_stamp), ctypes.byref(clock),
                                   ctypes.byref(credit)))
    return clock.value, credit.value


def eo_last_plan(e) -> dict:
    p = eo_plan_host()
    _check(lib().eo_last_plan(e, ctypes.byref(p)))
    return {"layer": p.layer, "m": p.m, "q": p.q, "q_fill": p.q_fill, "clock": p.clock,
            "credit": p.credit,
            "hits": [(p.hit_expert[i], p.hit_slot[i]) for i in range(p.n_hit)],
            "fills": [(p.fill_expert[i], p.fill_slot[i]) for i in range(p.q_fill)],
            "host": [p.host_expert[i] for i in range(p.n_host)],
            "evicted": [p.evicted_key[i] for i in range(p.n_evict)]}


def eo_dequant(e, layer, expert, out_host) -> None:
    _check(lib().eo_dequant(e, layer, expert, _ptr(out_host)))


EO_DECODER_SCALAR, EO_DECODER_GEMM, EO_DECODER_GEMV = 0, 1, 2


def eo_dequant_with(e, layer, expert, decoder, out_host) -> None:
    _check(lib().eo_dequant_with(e, layer, expert, decoder, _ptr(out_host)))


def eo_resize_cache(e, slots: int):
    """Elastic resize between steps; returns (evicted, moved)."""
    ne, nm = _I64(0), _I64(0)
    _check(lib().eo_resize_cache(e, slots, ctypes.byref(ne), ctypes.byref(nm)))
    return ne.value, nm.value


def eo_set_static_placement(e, keys) -> None:
    """keys: int32 host array of layer*E + expert (numpy)."""
    import numpy as np
    k = np.ascontiguousarray(keys, dtype=np.int32)
    _check(lib().eo_set_static_placement(e, k.ctypes.data if k.size else None, int(k.size)))


def eo_clear_static_placement(e) -> None:
    _check(lib().eo_clear_static_placement(e))


def eo_stats_get(e) -> dict:
    s = eo_stats()
    _check(lib().eo_stats_get(e, ctypes.byref(s)))
    return {n: getattr(s, n) for n, _ in eo_stats._fields_}


def eo_set_plan_log(e, enable: bool) -> None:
    _check(lib().eo_set_plan_log(e, 1 if enable else 0))


def eo_get_plan_log(e):
    """int32 numpy array [n, 4]: {layer, hits, fills, host experts} per lookup."""
    import numpy as np
    n = _I64(0)
    _check(lib().eo_get_plan_log(e, None, 0, ctypes.byref(n)))
    out = np.zeros((n.value, 4), dtype=np.int32)
    if n.value:
        _check(lib().eo_get_plan_log(e, out.ctypes.data, n.value, ctypes.byref(n)))
    return out


def eo_set_timing(e, enable: bool) -> None:
    _check(lib().eo_set_timing(e, 1 if enable else 0))


def eo_kernel_times(e, reset: bool = False) -> dict:
    ms = (ctypes.c_double * 5)()
    n = (_I64 * 3)()
    _check(lib().eo_kernel_times(e, ms, n, 1 if reset else 0))
    return {"gemv_gate_up_ms": ms[0], "gemv_down_ms": ms[1], "gemm_gate_up_ms": ms[2],
            "gemm_down_ms": ms[3], "fill_ms": ms[4], "gemv_launches": n[0],
            "gemm_launches": n[1], "fill_launches": n[2]}


def eo_stream_times(e, reset: bool = False) -> dict:
    ms = (ctypes.c_double * 2)()
    n = (_I64 * 2)()
    _check(lib().eo_stream_times(e, ms, n, 1 if reset else 0))
    return {"copy_ms": ms[0], "compute_ms": ms[1], "copy_layers": n[0], "compute_layers": n[1]}


def eo_sync(e) -> None:
    _check(lib().eo_sync(e))
