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


def test_rmsnorm_pins():
    rng = np.random.default_rng(9)
    r = rng.standard_normal((5, 256)) * np.array([[0.01], [1.0], [7.0], [300.0], [2.0]])
    u = moe.rmsnorm(r)
    # unit mean square (up to eps), direction kept, scale invariant
    assert np.allclose(np.mean(u * u, axis=1), 1.0 / (1.0 + moe.RMS_EPS / np.mean(r * r, axis=1)))
    assert np.allclose(u / np.linalg.norm(u, axis=1, keepdims=True),
                       r / np.linalg.norm(r, axis=1, keepdims=True), rtol=1e-14)
    # scale invariant once eps is negligible (mean square 1 vs 9: eps/ms = 1e-6)
    assert np.allclose(moe.rmsnorm(3.0 * r[1:2]), moe.rmsnorm(r[1:2]), rtol=1e-6, atol=0)
    # hand-worked: (3, 4) has mean square 12.5
    assert np.allclose(moe.rmsnorm(np.array([3.0, 4.0])), np.array([3.0, 4.0]) / np.sqrt(12.5 + 1e-6))
    assert np.array_equal(moe.rmsnorm(np.zeros(4)), np.zeros(4))


def test_round_bf16_against_torch_and_ties():
    rng = np.random.default_rng(4)
    # fp32-representable inputs: torch's fp32 -> bf16 conversion rounds once
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(moe.round_bf16(v.astype(np.float64)), ref)
    # ties go to even: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7
    assert moe.round_bf16(np.array([1 + 2.0**-8]))[0] == 1.0
    assert moe.round_bf16(np.array([1 + 3 * 2.0**-8]))[0] == 1 + 2.0**-6
    # just above a tie rounds up (fp64 input, no intermediate fp32 rounding)
    assert moe.round_bf16(np.array([1 + 2.0**-8 + 2.0**-40]))[0] == 1 + 2.0**-7
    assert moe.round_bf16(np.array([-1.5, 0.0]))[1] == 0.0


def test_stack_forward_matches_explicit_chain():
    # two layers written out by hand from the primitives, forced and routed ids
    H, I, E, k, T = 64, 32, 8, 2, 5
    ex = [_tiny_experts(H, I, E, F.BF16, seed=11, layer=l) for l in range(2)]
    R = [synth.router_weights(11, l, E, H) for l in range(2)]
    X0 = synth.bf16_bits_to_f32(synth.activations(11, 0, T, H, 3.0, True)).astype(np.float64)
    forced = np.array([[1, 4]] * T, dtype=np.int32)
    rL, tr = moe.stack_forward(X0, [(R[0], k, ex[0], None, None), (R[1], k, ex[1], None, forced)],
                               True)
    u0 = moe.round_bf16(X0 / np.sqrt(np.mean(X0 ** 2, axis=1, keepdims=True) + 1e-6))
    assert np.array_equal(tr[0][0], u0)
    ids0, w0, _ = router.route(u0.astype(np.float32), R[0], k)
    assert np.array_equal(tr[0][1], ids0)
    r1 = moe.round_bf16(X0 + moe.layer_output(u0, ids0, w0, ex[0]))
    u1 = moe.round_bf16(r1 / np.sqrt(np.mean(r1 ** 2, axis=1, keepdims=True) + 1e-6))
    assert np.array_equal(tr[1][0], u1) and np.array_equal(tr[1][1], forced)
    _, w1, _ = router.route(u1.astype(np.float32), R[1], k, forced)
    assert np.array_equal(rL, moe.round_bf16(r1 + moe.layer_output(u1, forced, w1, ex[1])))
    # every stored value is a bf16 value; the inputs are normalised
    assert np.array_equal(moe.round_bf16(rL), rL)
    assert np.allclose(np.mean(tr[1][0] ** 2, axis=1), 1.0, rtol=1e-2)
