"""Set up an engine of the HIP library with the seeded synthetic weights.

Input plumbing only: the pool, routers and shared experts are written with the
generator's bytes through the library's C ABI (via the Python binding). The
oracle never imports this module.
"""
from __future__ import annotations

import concurrent.futures as cf
import ctypes
import os

import numpy as np

import expert_offload_amd as eo

from . import (FMT_FP32, P_SHARED, LayerShape, expert_block, expert_block_into, expert_bytes,
               router_weights)


def make_engine(shape: LayerShape, seed: int = 0, cache_slots: int | None = None,
                max_tokens: int | None = None, layers: int | None = None, host_threads: int = 0,
                fill_pool: bool = True, device: int = 0) -> int:
    L = shape.layers if layers is None else layers
    C = shape.cache_slots if cache_slots is None else cache_slots
    T = shape.tokens if max_tokens is None else max_tokens
    e = eo.eo_create(L, shape.experts, shape.top_k, shape.hidden, shape.inter, shape.fmt,
                     0 if shape.fmt == FMT_FP32 else 1, C, T, shape.shared, host_threads,
                     device)
    try:
        for l in range(L):
            eo.eo_set_router(e, l, router_weights(seed, l, shape.experts, shape.hidden))
            if shape.shared:
                blk = expert_block(seed, l, 0, shape.hidden, shape.inter, shape.fmt,
                                   purpose=P_SHARED)
                eo.eo_set_shared_expert(e, l, blk, blk.size)
        if fill_pool:
            write_pool(e, shape, seed, L)
    except Exception:
        eo.eo_destroy(e)
        raise
    return e


def write_pool(e: int, shape: LayerShape, seed: int, layers: int, workers: int = 0) -> None:
    """All pool entries, generated in parallel (one expert per task)."""
    workers = workers or min(16, os.cpu_count() or 1)
    jobs = [(l, x) for l in range(layers) for x in range(shape.experts)]
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda lx: write_pool_expert(e, shape, seed, *lx), jobs))


def write_pool_expert(e: int, shape: LayerShape, seed: int, layer: int, expert: int) -> None:
    ptr, nbytes = eo.eo_pool_expert(e, layer, expert)
    assert nbytes == expert_bytes(shape.hidden, shape.inter, shape.fmt)
    expert_block_into(ptr, nbytes, seed, layer, expert, shape.hidden, shape.inter, shape.fmt)


def pool_block(e: int, layer: int, expert: int) -> np.ndarray:
    """Copy of a pool entry's bytes (host memory)."""
    ptr, nbytes = eo.eo_pool_expert(e, layer, expert)
    return np.ctypeslib.as_array((ctypes.c_uint8 * nbytes).from_address(ptr)).copy()
