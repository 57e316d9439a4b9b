"""Pins for the oracle's layer value (SwiGLU FFN, weighting, shared expert) — CPU only."""
import math

import numpy as np
import torch

import synth
from oracle import formats as F
from oracle import moe, router


def test_silu_matches_torch_fp64():
    u = np.linspace(-30, 30, 2001)
    ref = torch.nn.functional.silu(torch.from_numpy(u)).numpy()
    assert np.allclose(moe.silu(u), ref, rtol=1e-15, atol=1e-300)


def test_ffn_hand_worked():
    # H = 2, I = 1: gate reads x0, up reads x1, down writes (h, 2h)
    wg = np.array([[1.0, 0.0]])
    wu = np.array([[0.0, 1.0]])
    wd = np.array([[1.0], [2.0]])
    a, b = math.log(3.0), 5.0
    h = a / (1.0 + 1.0 / 3.0) * b  # silu(ln 3) = ln 3 / (1 + 1/3)
    out = moe.ffn(wg, wu, wd, np.array([a, b]))
    assert np.allclose(out, [h, 2 * h], rtol=1e-15, atol=0)
    assert np.array_equal(moe.ffn(wg, wu, wd, np.array([0.0, 7.0])), [0.0, 0.0])


def test_ffn_matches_torch_linear_fp64():
    rng = np.random.default_rng(0)
    H, I = 48, 24
    wg, wu = rng.standard_normal((I, H)), rng.standard_normal((I, H))
    wd, x = rng.standard_normal((H, I)), rng.standard_normal((5, H))
    t = [torch.from_numpy(v) for v in (wg, wu, wd, x)]
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(t[3], t[0]))
        * torch.nn.functional.linear(t[3], t[1]), t[2]).numpy()
    assert np.allclose(moe.ffn(wg, wu, wd, x), ref, rtol=1e-12, atol=1e-12)


def _tiny_experts(H, I, E, fmt, seed=3, layer=0):
    blocks = [synth.expert_block(seed, layer, e, H, I, fmt) for e in range(E)]
    return lambda e: F.dequant_expert(blocks[e], H, I, fmt)


def test_sparse_layer_matches_dense_brute_force():
    H, I, E, k, T = 64, 32, 16, 2, 24
    expert = _tiny_experts(H, I, E, F.FP32)
    R = synth.router_weights(0, 0, E, H)
    X = synth.activations(0, 0, T, H, 0.02, False)
    Y, ids, w, _ = moe.moe_layer(X, R, k, expert)
    Yd = moe.dense_layer_output(X, ids, w, expert, E)
    assert np.max(np.abs(Y - Yd)) <= 1e-12 * np.max(np.abs(Yd))


def test_shared_expert_and_k_equals_e():
    H, I, E, T = 64, 32, 4, 6
    expert = _tiny_experts(H, I, E, F.BF16)
    shared = F.dequant_expert(synth.expert_block(3, 0, 0, H, I, F.BF16, purpose=synth.P_SHARED),
                              H, I, F.BF16)
    R = synth.router_weights(1, 0, E, H)
    X = synth.activations(1, 0, T, H, 1.0, False)
    # k = E: every expert is chosen, so the gate is the full softmax
    Y, ids, w, z = moe.moe_layer(X, R, E, expert, shared)
    full = np.exp(z - z.max(axis=1, keepdims=True)).astype(np.float64)
    full /= full.sum(axis=1, keepdims=True)
    ref = moe.ffn(*shared, X)
    for e in range(E):
        ref += full[:, e:e + 1] * moe.ffn(*expert(e), X)
    assert np.max(np.abs(Y - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_layer_output_invariant_to_slot_order():
    H, I, E, k, T = 64, 32, 8, 3, 10
    expert = _tiny_experts(H, I, E, F.FP32)
    R = synth.router_weights(2, 0, E, H)
    X = synth.activations(2, 0, T, H, 0.02, False)
    ids, w, _ = router.route(X, R, k)
    perm = [2, 0, 1]
    Y1 = moe.layer_output(X, ids, w, expert)
    Y2 = moe.layer_output(X, ids[:, perm], w[:, perm], expert)
    assert np.max(np.abs(Y1 - Y2)) <= 1e-13 * np.max(np.abs(Y1))
