"""GPU: eo_route_noalloc (the router with its scratch in a fixed device array,
for callers that cannot allocate) against eo_route, through the C ABI.

Two calls in a row on each engine, the second with fewer tokens, so the second
runs on whatever the first left in the shared array: ids must match eo_route's
bit for bit and the weights within 1e-6 (the router's bar), and the oracle's
ids bit for bit. Sizes past the array are refused before any launch.
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expert_offload_amd as eo  # noqa: E402
import synth  # noqa: E402
from oracle import router as OR  # noqa: E402
from synth.workload import make_engine  # noqa: E402
from tests.gpu_util import dev  # noqa: E402

pytestmark = pytest.mark.gpu


def _s():
    return torch.cuda.current_stream().cuda_stream


def _compare(e, shape, seed, layer, T, bf16, forced=None):
    H, E, k = shape.hidden, shape.experts, shape.top_k
    x = synth.activations(seed, 500 + T, T, H, 1.0 if bf16 else 0.02, bf16)
    xd = dev(x.view(np.int16) if bf16 else x)
    fd = dev(forced) if forced is not None else None
    out = []
    for fn in (eo.eo_route, eo.eo_route_noalloc):
        ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
        w = torch.full((T, k), -1.0, dtype=torch.float32, device="cuda")
        fn(e, layer, xd, T, fd, ids, w, _s())
        torch.cuda.synchronize()
        out.append((ids.cpu().numpy(), w.cpu().numpy()))
    (i0, w0), (i1, w1) = out
    assert np.array_equal(i0, i1), (shape.name, T)
    assert np.max(np.abs(w0 - w1)) <= 1e-6, (shape.name, T)
    xf = synth.bf16_bits_to_f32(x) if bf16 else x
    rids, rw, _ = OR.route(xf, synth.router_weights(seed, layer, E, H), k, forced_ids=forced)
    assert np.array_equal(i1, rids), (shape.name, T)
    assert np.max(np.abs(w1 - rw)) <= 1e-6, (shape.name, T)


def test_route_noalloc_matches_route_bf16():
    # H 2048, 128 experts, top-8: the chain-interleaved kernel at T >= 32 (its
    # xT scratch in the array too), the direct kernel below
    shape = dataclasses.replace(synth.SHAPES["decode_bf16_48L"], layers=2, cache_slots=0)
    seed = 31
    e = make_engine(shape, seed, max_tokens=4096, fill_pool=False)
    try:
        _compare(e, shape, seed, 1, 300, True)
        _compare(e, shape, seed, 0, 37, True)   # smaller, after the larger
        _compare(e, shape, seed, 0, 5, True)
        tr = synth.sticky_zipf_trace(seed, 3, 1, shape.experts, shape.top_k)[:, 0, :]
        _compare(e, shape, seed, 1, 3, True, forced=np.ascontiguousarray(tr, dtype=np.int32))
        # 3641 tokens need 3641 * (4 * 128 + 2 * 2048) bytes > 16 MiB: refused
        x = torch.zeros((4096, shape.hidden), dtype=torch.int16, device="cuda")
        ids = torch.zeros((4096, shape.top_k), dtype=torch.int32, device="cuda")
        w = torch.zeros((4096, shape.top_k), dtype=torch.float32, device="cuda")
        with pytest.raises(eo.EOError) as ex:
            eo.eo_route_noalloc(e, 0, x, 3641, None, ids, w, _s())
        assert ex.value.status == eo.EO_ERR_INVALID_ARG
        eo.eo_route_noalloc(e, 0, x, 3640, None, ids, w, _s())  # fits exactly
        torch.cuda.synchronize()
        eo.eo_sync(e)
    finally:
        eo.eo_destroy(e)


def test_route_noalloc_matches_route_fp32():
    shape = synth.SHAPES["tiny_fp32"]
    seed = 32
    e = make_engine(shape, seed, fill_pool=False)
    try:
        _compare(e, shape, seed, 0, 64, False)
        _compare(e, shape, seed, 0, 9, False)
    finally:
        eo.eo_destroy(e)
