"""Helpers for the GPU parity tests: device tensors and oracle references."""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import formats as OF
from oracle import moe as OM


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def act_f32(x: np.ndarray, bf16: bool) -> np.ndarray:
    return synth.bf16_bits_to_f32(x) if bf16 else np.asarray(x, dtype=np.float32)


def oracle_expert_fn(shape: synth.LayerShape, seed: int, layer: int):
    cache = {}

    def f(e):
        if e not in cache:
            blk = synth.expert_block(seed, layer, e, shape.hidden, shape.inter, shape.fmt)
            cache[e] = OF.dequant_expert(blk, shape.hidden, shape.inter, shape.fmt)
        return cache[e]
    return f


def oracle_shared(shape: synth.LayerShape, seed: int, layer: int):
    if not shape.shared:
        return None
    blk = synth.expert_block(seed, layer, 0, shape.hidden, shape.inter, shape.fmt,
                             purpose=synth.P_SHARED)
    return OF.dequant_expert(blk, shape.hidden, shape.inter, shape.fmt)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def oracle_layer(shape, seed, layer, x_f32, ids, w):
    return OM.layer_output(x_f32, ids, w, oracle_expert_fn(shape, seed, layer),
                           oracle_shared(shape, seed, layer))


def check_residual_stream(x0_bits: np.ndarray, xin_bits: np.ndarray, ys: np.ndarray) -> np.ndarray:
    """Multi-layer calls with bf16 activations: x0 [T,H] is the residual stream's
    start, xin [L,T,H] the captured layer inputs, ys [L,T,H] the captured fp32
    layer outputs. The stream is stored in bf16 after each layer (the device adds
    in fp32, then rounds to nearest even, replayed here exactly); each layer input
    must be the oracle's RMS-normalised stream within one bf16 unit in the last
    place (the device normalises in fp32, the oracle in fp64).
    Returns the expected bf16 bits of the stream after the last layer."""
    r = np.asarray(x0_bits, dtype=np.uint16)
    for l in range(xin_bits.shape[0]):
        rf = synth.bf16_bits_to_f32(r)
        ref = OM.layer_input(rf, True)
        got = synth.bf16_bits_to_f32(xin_bits[l]).astype(np.float64)
        ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), 1e-30))[1] - 8)
        assert np.all(np.abs(got - ref) <= ulp), f"layer {l}: normalised input off by > 1 ulp"
        assert np.mean(got == ref) >= 0.98, f"layer {l}: too many 1-ulp differences"
        r = synth.f32_to_bf16_bits(rf + ys[l])
    return r
