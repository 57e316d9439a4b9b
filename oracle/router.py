"""ORACLE (test infrastructure only) — router: logits, top-k, weights.

Routing is named on the pages only as one axis on which MoE architectures
differ (papers.ananclaw.com explainer, "core method" section 4), and the decode
paragraph of the zhichai.net article (section 2) takes "which routed experts a
token activates" as its input. The reading used here:

* logits z = x . R_l^T in fp32, accumulated in the fixed order described in
  ``corder.c`` (64 strided fused-multiply-add chains, then an xor butterfly);
  bf16 inputs are widened exactly to fp32 first;
* top-k: the k largest logits, ties to the lower expert id, listed in
  (logit descending, id ascending) order;
* weights: softmax over the k selected logits, which equals a softmax over all
  E logits restricted to the top-k and renormalised. Computed in fp64.
* When a routing trace fixes the ids (decode workloads), the ids are taken as
  given, in trace order, and the weights are the softmax of the logits at them.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "corder.c")
_LIB = os.path.join(_HERE, "_corder.so")
_lib = None


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", tmp,
                               _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.oracle_router_logits.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        _lib = L
    return _lib


def logits(x: np.ndarray, R: np.ndarray) -> np.ndarray:
    """z [T, E] fp32 from x [T, H] fp32 and R [E, H] fp32, in the fixed order."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R = np.ascontiguousarray(R, dtype=np.float32)
    T, H = x.shape
    E, H2 = R.shape
    assert H == H2
    z = np.empty((T, E), dtype=np.float32)
    _load().oracle_router_logits(x.ctypes.data, R.ctypes.data, T, E, H, z.ctypes.data)
    return z


def topk(z: np.ndarray, k: int) -> np.ndarray:
    """ids [T, k] int32: for each row, experts sorted by (z descending, id ascending)."""
    T, E = z.shape
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        row = [float(v) for v in z[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))
        out[t] = order[:k]
    return out


def weights(z: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w [T, k] fp64: softmax of z over each row's selected ids."""
    T, k = ids.shape
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        sel = [float(z[t, e]) for e in ids[t]]
        zmax = max(sel)
        ex = [math.exp(v - zmax) for v in sel]
        s = math.fsum(ex)
        w[t] = [v / s for v in ex]
    return w


def route(x: np.ndarray, R: np.ndarray, k: int, forced_ids: np.ndarray | None = None):
    """(ids [T,k] int32, w [T,k] fp64, z [T,E] fp32) for layer input x."""
    z = logits(x, R)
    ids = topk(z, k) if forced_ids is None else np.ascontiguousarray(forced_ids, dtype=np.int32)
    return ids, weights(z, ids), z
