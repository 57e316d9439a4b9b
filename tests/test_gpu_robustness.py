"""GPU: failure handling and the debugging mode.

* EO_DEBUG_SYNC=1 waits for the device after every stage and names the stage of
  any asynchronous error; the kernels and their order are unchanged, so decode
  steps, layer calls and streamed prefill give the same bits as without it.
* A device allocation that cannot succeed (an elastic resize to 8192 slots of a
  75.5 MB expert, 618 GB) returns EO_ERR_OOM and leaves the engine as it was:
  the slot table is unchanged and the next layer call matches the oracle. An
  engine whose cache cannot be allocated is not created, and the next one is.
* An empty batch (T = 0) or one above max_tokens is rejected by every step call
  with EO_ERR_INVALID_ARG before any launch: buffers untouched, cache, clock,
  credit and statistics unchanged, and the next calls match the oracle.
* A filled expert's gate/up rows wait, bounded, for the fill workgroups of the
  same launch. With the bound forced to one tick from the host
  (EO_TEST_FILL_WAIT_TICKS) the wait runs out at once; no kernel faults or
  hangs, the launch records it, and the next one-token plan returns EO_ERR_HIP
  and changes nothing (the clock stays at the last plan read); the record is
  cleared and the next layer call matches the oracle.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expert_offload_amd as eo  # noqa: E402
import synth  # noqa: E402
from oracle import router as OR  # noqa: E402
from synth.workload import make_engine  # noqa: E402
from tests.gpu_util import dev, oracle_layer, rel_err  # noqa: E402

pytestmark = pytest.mark.gpu


def _s():
    return torch.cuda.current_stream().cuda_stream


def _run_all(shape, seed, trace):
    """Decode steps, a 40-token layer call and a 300-token prefill; all outputs."""
    L, k, H = shape.layers, shape.top_k, shape.hidden
    e = make_engine(shape, seed, cache_slots=10, max_tokens=300)
    out = []
    try:
        eo.eo_set_bandwidth(e, 2, 3)
        for st in range(trace.shape[0]):
            x = dev(synth.activations(seed, 700 + st, 1, H, 1.0, True).view(np.int16))
            eo.eo_decode_step(e, x, 1, dev(trace[st].reshape(L, 1, k)), _s())
            torch.cuda.synchronize()
            out.append(x.cpu().numpy().copy())
        x = dev(synth.activations(seed, 710, 40, H, 1.0, True).view(np.int16))
        y = torch.zeros((40, H), dtype=torch.float32, device="cuda")
        eo.eo_moe_layer(e, 1, x, y, 40, None, _s())
        torch.cuda.synchronize()
        out.append(y.cpu().numpy().copy())
        x = dev(synth.activations(seed, 711, 300, H, 1.0, True).view(np.int16))
        eo.eo_prefill(e, x, 300, eo.EO_PREFILL_DOUBLE_BUFFER, _s())
        torch.cuda.synchronize()
        out.append(x.cpu().numpy().copy())
        eo.eo_sync(e)
    finally:
        eo.eo_destroy(e)
    return out


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4"])
def test_debug_sync_gives_the_same_bits(fmt, monkeypatch):
    shape = synth.LayerShape(f"dbg_{fmt}", "test", 512, 16, 4, 256, 3, synth.FMT_NAMES[fmt], 300,
                             10, shared=1)
    seed = 41
    trace = synth.sticky_zipf_trace(seed, 5, shape.layers, shape.experts, shape.top_k)
    monkeypatch.setenv("EO_DEBUG_SYNC", "1")
    dbg = _run_all(shape, seed, trace)
    monkeypatch.delenv("EO_DEBUG_SYNC")
    plain = _run_all(shape, seed, trace)
    assert len(dbg) == len(plain)
    for i, (a, b) in enumerate(zip(dbg, plain)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), i


def test_failed_device_allocation_leaves_the_engine_usable():
    # bf16 expert of H 6144, I 2048: 75.5 MB; 8192 slots need 618 GB of HBM
    shape = synth.LayerShape("oom_bf16", "test", 6144, 4, 2, 2048, 1, synth.FMT_BF16, 3, 2)
    seed = 42
    with pytest.raises(eo.EOError) as ex:
        eo.eo_create(1, 4, 2, 6144, 2048, synth.FMT_BF16, 1, 8192, 3)
    assert ex.value.status == eo.EO_ERR_OOM
    e = make_engine(shape, seed)
    try:
        eo.eo_set_bandwidth(e, 100, 100)
        H, T = shape.hidden, 3
        x = synth.activations(seed, 1, T, H, 1.0, True)
        xd = dev(x.view(np.int16))
        y = torch.zeros((T, H), dtype=torch.float32, device="cuda")
        eo.eo_moe_layer(e, 0, xd, y, T, None, _s())  # fills the two slots
        torch.cuda.synchronize()
        keys0 = np.zeros(2, dtype=np.int32)
        stamps0 = np.zeros(2, dtype=np.int64)
        c0 = eo.eo_cache_snapshot(e, keys0, stamps0)
        with pytest.raises(eo.EOError) as ex:
            eo.eo_resize_cache(e, 8192)
        assert ex.value.status == eo.EO_ERR_OOM
        keys1 = np.zeros(2, dtype=np.int32)
        stamps1 = np.zeros(2, dtype=np.int64)
        assert eo.eo_cache_snapshot(e, keys1, stamps1) == c0
        assert np.array_equal(keys0, keys1) and np.array_equal(stamps0, stamps1)
        # the engine still serves a layer call, with the cache it had
        x2 = synth.activations(seed, 2, T, H, 1.0, True)
        eo.eo_moe_layer(e, 0, dev(x2.view(np.int16)), y, T, None, _s())
        torch.cuda.synchronize()
        xf = synth.bf16_bits_to_f32(x2)
        rids, rw, _ = OR.route(xf, synth.router_weights(seed, 0, shape.experts, H), shape.top_k)
        assert rel_err(y.cpu().numpy(), oracle_layer(shape, seed, 0, xf, rids, rw)) <= 2e-2
        eo.eo_sync(e)
    finally:
        eo.eo_destroy(e)


def test_empty_and_oversized_batches_are_rejected():
    shape = synth.LayerShape("edge_bf16", "test", 512, 16, 4, 256, 2, synth.FMT_BF16, 8, 6,
                             shared=1)
    seed = 43
    H, k, C, L = shape.hidden, shape.top_k, shape.cache_slots, shape.layers
    e = make_engine(shape, seed, max_tokens=8)
    try:
        eo.eo_set_bandwidth(e, 1, 2)
        x = synth.activations(seed, 1, 3, H, 1.0, True)
        xd = dev(x.view(np.int16))
        y = torch.zeros((3, H), dtype=torch.float32, device="cuda")
        eo.eo_moe_layer(e, 0, xd, y, 3, None, _s())  # some state first
        torch.cuda.synchronize()
        keys0 = np.zeros(C, dtype=np.int32)
        stamps0 = np.zeros(C, dtype=np.int64)
        snap0 = eo.eo_cache_snapshot(e, keys0, stamps0)
        st0 = {n: v for n, v in eo.eo_stats_get(e).items() if not n.endswith("_ns")}
        big = dev(synth.activations(seed, 2, 9, H, 1.0, True).view(np.int16))
        before = big.clone()
        ids = torch.full((9, k), -7, dtype=torch.int32, device="cuda")
        w = torch.full((9, k), -7.0, dtype=torch.float32, device="cuda")
        yb = torch.full((9, H), -7.0, dtype=torch.float32, device="cuda")
        calls = [
            lambda T: eo.eo_route(e, 0, big, T, None, ids, w, _s()),
            lambda T: eo.eo_route_noalloc(e, 0, big, T, None, ids, w, _s()),
            lambda T: eo.eo_lookup_plan(e, 0, ids, T, _s()),
            lambda T: eo.eo_moe_layer(e, 1, big, yb, T, None, _s()),
            lambda T: eo.eo_decode_step(e, big, T, None, _s()),
            lambda T: eo.eo_prefill(e, big, T, eo.EO_PREFILL_DOUBLE_BUFFER, _s()),
        ]
        for n, call in enumerate(calls):
            for T in (0, 9):
                with pytest.raises(eo.EOError) as ex:
                    call(T)
                assert ex.value.status == eo.EO_ERR_INVALID_ARG, (n, T)
        torch.cuda.synchronize()
        assert torch.equal(big, before)
        assert bool((ids == -7).all()) and bool((w == -7.0).all()) and bool((yb == -7.0).all())
        keys1 = np.zeros(C, dtype=np.int32)
        stamps1 = np.zeros(C, dtype=np.int64)
        assert eo.eo_cache_snapshot(e, keys1, stamps1) == snap0
        assert np.array_equal(keys0, keys1) and np.array_equal(stamps0, stamps1)
        assert {n: v for n, v in eo.eo_stats_get(e).items() if not n.endswith("_ns")} == st0
        # no plan is pending: the per-stage calls still refuse, the layer call serves
        with pytest.raises(eo.EOError) as ex:
            eo.eo_fill(e, _s())
        assert ex.value.status == eo.EO_ERR_STATE
        x2 = synth.activations(seed, 3, 8, H, 1.0, True)
        y2 = torch.zeros((8, H), dtype=torch.float32, device="cuda")
        eo.eo_moe_layer(e, 1, dev(x2.view(np.int16)), y2, 8, None, _s())
        torch.cuda.synchronize()
        xf = synth.bf16_bits_to_f32(x2)
        rids, rw, _ = OR.route(xf, synth.router_weights(seed, 1, shape.experts, H), k)
        assert rel_err(y2.cpu().numpy(), oracle_layer(shape, seed, 1, xf, rids, rw)) <= 2e-2
        assert eo.eo_last_plan(e)["clock"] == snap0[0] + 1
        eo.eo_sync(e)
    finally:
        eo.eo_destroy(e)


def test_fill_wait_that_runs_out_fails_the_next_plan(monkeypatch):
    shape = synth.LayerShape("fw_bf16", "test", 512, 16, 4, 256, 3, synth.FMT_BF16, 8, 6,
                             shared=1)
    seed = 49
    H, k, C = shape.hidden, shape.top_k, shape.cache_slots
    monkeypatch.setenv("EO_TEST_FILL_WAIT_TICKS", "1")
    e = make_engine(shape, seed, max_tokens=8)
    monkeypatch.delenv("EO_TEST_FILL_WAIT_TICKS")
    try:
        eo.eo_set_bandwidth(e, 1, 1)  # every miss filled: layer 0 of the first step fills k
        x = dev(synth.activations(seed, 100, 1, H, 1.0, True).view(np.int16))
        with pytest.raises(eo.EOError) as ex:
            eo.eo_decode_step(e, x, 1, None, _s())
        assert ex.value.status == eo.EO_ERR_HIP and "gave up waiting for its fills" in str(ex.value)
        torch.cuda.synchronize()
        keys = np.zeros(C, dtype=np.int32)
        stamps = np.zeros(C, dtype=np.int64)
        snap = eo.eo_cache_snapshot(e, keys, stamps)
        st = eo.eo_stats_get(e)
        # layer 0's plan was read (k fills); layer 1's plan reported the error and ticked nothing
        assert snap[0] == 1 == eo.eo_last_plan(e)["clock"] == st["lookups"]
        assert st["fills"] == k and int((keys >= 0).sum()) == k
        x2 = synth.activations(seed, 3, 8, H, 1.0, True)
        y2 = torch.zeros((8, H), dtype=torch.float32, device="cuda")
        eo.eo_moe_layer(e, 1, dev(x2.view(np.int16)), y2, 8, None, _s())
        torch.cuda.synchronize()
        xf = synth.bf16_bits_to_f32(x2)
        rids, rw, _ = OR.route(xf, synth.router_weights(seed, 1, shape.experts, H), k)
        assert rel_err(y2.cpu().numpy(), oracle_layer(shape, seed, 1, xf, rids, rw)) <= 2e-2
        assert eo.eo_last_plan(e)["clock"] == 2
        eo.eo_sync(e)
    finally:
        eo.eo_destroy(e)
