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
