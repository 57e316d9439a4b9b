"""ORACLE (test infrastructure only) — the MoE layer's value.

The MoE layer forward (zhichai.net article, section 2, Decode paragraph: tokens
activate a few routed experts; the layer's value does not depend on where an
expert runs) is, for input X [T, H]:

    Y[t] = sum_j w[t, j] * FFN_{e_j}(X[t])  (+ FFN_shared(X[t]) when the model
           has an always-on shared expert, weight 1 — the explainer names the
           shared expert as an architecture axis, "core method" section 4)

    FFN_e(x) = W_down ( silu(W_gate x) * (W_up x) ),  silu(u) = u / (1 + e^-u)

SwiGLU is the reading of "activation" for these workloads. Caching, filling,
host execution, permutation and streaming change where and when this is
computed, never what: the oracle evaluates it directly in fp64 on the
dequantised fp32 weights, with no intermediate rounding.

Between MoE layers (the pages are silent; reading): a pre-norm residual stream.
The residual r_l (activation dtype) feeds layer l through a parameter-free RMS
normalisation, u_l = r_l / sqrt(mean(r_l^2) + 1e-6) rounded to the activation
dtype, and r_{l+1} = r_l + Y_l(u_l), rounded to the activation dtype. Without
the normalisation a SwiGLU stack grows without bound (the FFN is quadratic in
its input).
"""
from __future__ import annotations

import numpy as np

from . import router as _router


RMS_EPS = 1e-6


def rmsnorm(r: np.ndarray) -> np.ndarray:
    """r / sqrt(mean(r^2) + eps) per row, fp64 (rounding to the activation dtype
    is the caller's)."""
    r = np.asarray(r, dtype=np.float64)
    return r / np.sqrt(np.mean(r * r, axis=-1, keepdims=True) + RMS_EPS)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round fp64 to the nearest bfloat16 (8 significant bits), ties to even,
    directly from fp64 (normal range; returned as fp64)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)  # v = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)  # rint: half to even


def round_act(v: np.ndarray, act_bf16: bool) -> np.ndarray:
    """Storage rounding of the activation dtype (bf16, else fp32), as fp64."""
    v = np.asarray(v, dtype=np.float64)
    return round_bf16(v) if act_bf16 else v.astype(np.float32).astype(np.float64)


def layer_input(r: np.ndarray, act_bf16: bool) -> np.ndarray:
    """The MoE layer's input from the residual stream: RMS-normalised, stored."""
    return round_act(rmsnorm(r), act_bf16)


def silu(u: np.ndarray) -> np.ndarray:
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):  # e^-u -> inf gives the limit silu(u) -> -0
        return u / (1.0 + np.exp(-u))


def ffn(wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, x: np.ndarray) -> np.ndarray:
    """SwiGLU expert on one token or a batch (x [H] or [n, H]); fp64 result."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ np.asarray(wg, dtype=np.float64).T
    u = x @ np.asarray(wu, dtype=np.float64).T
    return (silu(g) * u) @ np.asarray(wd, dtype=np.float64).T


def layer_output(X: np.ndarray, ids: np.ndarray, w: np.ndarray, expert, shared=None):
    """Y [T, H] fp64 (without the residual).

    expert(e) -> (W_gate, W_up, W_down) fp32; shared: that triple or None.
    Every (token, slot) pair is evaluated separately.
    """
    X = np.asarray(X, dtype=np.float64)
    T, H = X.shape
    k = ids.shape[1]
    Y = np.zeros((T, H), dtype=np.float64)
    cache = {}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = expert(e)
            Y[t] += w[t, j] * ffn(*cache[e], X[t])
        if shared is not None:
            Y[t] += ffn(*shared, X[t])
    return Y


def dense_layer_output(X: np.ndarray, ids: np.ndarray, w: np.ndarray, expert, E: int,
                       shared=None):
    """Brute force: evaluate every expert on every token, weight by a dense gate
    G [T, E] that holds w on the selected ids and 0 elsewhere."""
    X = np.asarray(X, dtype=np.float64)
    T, H = X.shape
    G = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        for j in range(ids.shape[1]):
            G[t, int(ids[t, j])] += w[t, j]
    Y = np.zeros((T, H), dtype=np.float64)
    for e in range(E):
        Y += G[:, e:e + 1] * ffn(*expert(e), X)
    if shared is not None:
        Y += ffn(*shared, X)
    return Y


def moe_layer(X: np.ndarray, R: np.ndarray, k: int, expert, shared=None,
              forced_ids: np.ndarray | None = None):
    """Route, then evaluate: returns (Y fp64 [T,H], ids, w fp64, z fp32)."""
    ids, w, z = _router.route(np.asarray(X, dtype=np.float32), R, k, forced_ids)
    return layer_output(X, ids, w, expert, shared), ids, w, z


def stack_forward(X0: np.ndarray, layers, act_bf16: bool):
    """Several MoE layers on the residual stream, from the stored input X0 [T,H].

    layers: per layer (R, k, expert, shared, forced_ids or None). Per layer
    u = layer_input(r), (Y, ids, w) = moe_layer(u, ...), r <- round_act(r + Y).
    Returns r after the last layer and the per-layer (u, ids, w, Y).
    """
    r = np.asarray(X0, dtype=np.float64)
    trace = []
    for R, k, expert, shared, forced in layers:
        u = layer_input(r, act_bf16)
        Y, ids, w, _ = moe_layer(u, R, k, expert, shared, forced)
        trace.append((u, ids, w, Y))
        r = round_act(r + Y, act_bf16)
    return r, trace
