"""Seeded synthetic inputs shared by the HIP path and the CPU oracle.

Nothing here computes any part of the MoE layer: it draws random numbers and
writes them in the storage formats the layer consumes (see ``gen.c`` for the
expert-block layout and the quantisers). The weights stand in for trained
experts, the sticky-Zipf trace for a real routing trace.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "_gen.so")

FMT_FP32, FMT_BF16, FMT_MXFP4, FMT_NVFP4, FMT_FP8 = 0, 1, 2, 3, 4
FMT_NAMES = {"fp32": FMT_FP32, "bf16": FMT_BF16, "mxfp4": FMT_MXFP4, "nvfp4": FMT_NVFP4,
             "fp8": FMT_FP8}

# Philox key word 1: one sub-stream per purpose.
P_EXPERT, P_SHARED, P_ROUTER, P_ACT, P_TRACE = 1, 2, 3, 4, 5


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        u32, i32, i64, u64, dbl = (ctypes.c_uint32, ctypes.c_int32, ctypes.c_int64,
                                   ctypes.c_uint64, ctypes.c_double)
        vp = ctypes.c_void_p
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        L.synth_normal_f32.argtypes = [u32, u32, u32, u32, u32, dbl, i64, vp]
        L.synth_f32_to_bf16.argtypes = [vp, vp, i64]
        L.synth_expert_bytes.argtypes = [i32, i32, i32]
        L.synth_expert_bytes.restype = u64
        L.synth_pack_expert.argtypes = [vp, vp, vp, i32, i32, i32, vp, u64]
        L.synth_expert_block.argtypes = [u32, u32, i32, i32, i32, i32, i32, dbl, vp, u64]
        L.synth_expert_block_f32.argtypes = [u32, u32, i32, i32, i32, i32, i32, dbl, vp, u64, vp]
        L.synth_e2m1_encode.argtypes = [dbl]
        L.synth_e2m1_encode.restype = ctypes.c_uint8
        L.synth_e4m3_encode.argtypes = [dbl]
        L.synth_e4m3_encode.restype = ctypes.c_uint8
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
    return o


def normal_f32(seed: int, purpose: int, c1: int, c2: int, c3: int, sigma: float, n: int):
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(seed, purpose, c1, c2, c3, sigma, n, _ptr(out))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().synth_f32_to_bf16(_ptr(x), _ptr(out), x.size)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening (storage conversion, used to hand bf16 inputs to fp32 code)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def expert_bytes(H: int, I: int, fmt: int) -> int:
    return int(lib().synth_expert_bytes(H, I, fmt))


def pack_expert(wg, wu, wd, fmt: int) -> np.ndarray:
    wg = np.ascontiguousarray(wg, dtype=np.float32)
    wu = np.ascontiguousarray(wu, dtype=np.float32)
    wd = np.ascontiguousarray(wd, dtype=np.float32)
    I, H = wg.shape
    out = np.zeros(expert_bytes(H, I, fmt), dtype=np.uint8)
    rc = lib().synth_pack_expert(_ptr(wg), _ptr(wu), _ptr(wd), H, I, fmt, _ptr(out), out.size)
    if rc:
        raise ValueError(f"pack_expert failed ({rc})")
    return out


def expert_block_into(ptr: int, nbytes: int, seed: int, layer: int, expert: int, H: int, I: int,
                      fmt: int, sigma: float = 0.02, purpose: int = P_EXPERT) -> None:
    rc = lib().synth_expert_block(seed, purpose, layer, expert, H, I, fmt, sigma, ptr, nbytes)
    if rc:
        raise ValueError(f"expert_block failed ({rc})")


def expert_block(seed: int, layer: int, expert: int, H: int, I: int, fmt: int,
                 sigma: float = 0.02, purpose: int = P_EXPERT) -> np.ndarray:
    out = np.zeros(expert_bytes(H, I, fmt), dtype=np.uint8)
    expert_block_into(_ptr(out), out.size, seed, layer, expert, H, I, fmt, sigma, purpose)
    return out


def expert_block_with_f32(seed: int, layer: int, expert: int, H: int, I: int, fmt: int,
                          sigma: float = 0.02, purpose: int = P_EXPERT):
    """Packed block plus the fp32 weights it was quantised from (gate, up, down)."""
    out = np.zeros(expert_bytes(H, I, fmt), dtype=np.uint8)
    w = np.empty(3 * I * H, dtype=np.float32)
    rc = lib().synth_expert_block_f32(seed, purpose, layer, expert, H, I, fmt, sigma, _ptr(out),
                                      out.size, _ptr(w))
    if rc:
        raise ValueError(f"expert_block failed ({rc})")
    return out, w[:I * H].reshape(I, H), w[I * H:2 * I * H].reshape(I, H), \
        w[2 * I * H:].reshape(H, I)


def router_weights(seed: int, layer: int, E: int, H: int, sigma: float = 0.02) -> np.ndarray:
    """Router matrix R_l, fp32 [E, H]."""
    return normal_f32(seed, P_ROUTER, 0, layer, 0, sigma, E * H).reshape(E, H)


def activations(seed: int, index: int, T: int, H: int, sigma: float, bf16: bool) -> np.ndarray:
    """Layer input, [T, H]: fp32 values, or bf16 bit patterns (uint16) when bf16."""
    x = normal_f32(seed, P_ACT, 0, index, 0, sigma, T * H).reshape(T, H)
    return f32_to_bf16_bits(x) if bf16 else x


def sticky_zipf_trace(seed: int, steps: int, L: int, E: int, k: int, alpha: float = 1.1,
                      p_keep: float = 0.6) -> np.ndarray:
    """Routing trace int32 [steps, L, k] with temporal locality.

    Per layer: a seeded permutation maps Zipf rank r (popularity ~ r^-alpha) to
    an expert id. Step 0 draws k distinct experts by popularity; each later step
    keeps every expert of the previous step with probability p_keep and refills
    to k by popularity-weighted draws without replacement from the experts not
    yet chosen. Each row lists its k distinct experts, kept ones first.
    """
    rng = np.random.Generator(np.random.Philox(key=[seed, P_TRACE]))
    out = np.zeros((steps, L, k), dtype=np.int32)
    ranks = np.arange(1, E + 1, dtype=np.float64)
    pop_rank = ranks ** (-alpha)
    for l in range(L):
        perm = rng.permutation(E)
        pop = np.empty(E)
        pop[perm] = pop_rank  # expert perm[r] has rank r+1
        prev: list[int] = []
        for s in range(steps):
            kept = [e for e in prev if rng.random() < p_keep]
            chosen = list(kept)
            avail = np.ones(E, dtype=bool)
            avail[chosen] = False
            while len(chosen) < k:
                p = np.where(avail, pop, 0.0)
                e = int(rng.choice(E, p=p / p.sum()))
                chosen.append(e)
                avail[e] = False
            out[s, l] = chosen
            prev = chosen
    return out


@dataclass(frozen=True)
class LayerShape:
    name: str
    mode: str
    hidden: int
    experts: int
    top_k: int
    inter: int
    layers: int
    fmt: int
    tokens: int
    cache_slots: int
    shared: int = 0
    steps: int = 0


# The five workloads, by what they are (synth/workloads.json: shapes, formats,
# cache sizes and the generators' parameters, one file for every consumer).
WORKLOADS_JSON = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workloads.json")


def _load_shapes(path: str = WORKLOADS_JSON) -> dict:
    import json
    with open(path) as f:
        doc = json.load(f)
    out = {}
    for w in doc["workloads"]:
        slots = w["cache_slots"] if "cache_slots" in w else \
            int(w["cache_fraction"] * w["layers"] * w["experts"])
        out[w["name"]] = LayerShape(w["name"], w["mode"], w["hidden"], w["experts"], w["top_k"],
                                    w["inter"], w["layers"], FMT_NAMES[w["format"]], w["tokens"],
                                    slots, shared=w["shared"], steps=w["steps"])
    return out


SHAPES = _load_shapes()
