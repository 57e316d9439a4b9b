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
dequantised fp32 weights, with no intermediate rounding. The residual
X_{l+1} = X_l + Y_l links layers (nothing else sits between MoE layers here).
"""
from __future__ import annotations

import numpy as np

from . import router as _router


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
