"""GPU parity of whole layers, decode steps and prefill for every weight format.

Layer outputs are compared with the oracle within 2e-2 * max|ref| (bf16 / fp4 / fp8
weights, bf16 activations); router ids must match bit for bit. Multi-layer calls
capture each layer's input on the device and are checked per layer on that input;
the residual stream linking the layers is replayed from the captured outputs and
each captured input checked against the oracle's normalisation of it.
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expert_offload_amd as eo  # noqa: E402
import synth  # noqa: E402
from oracle import router as OR  # noqa: E402
from oracle.residency import Residency  # noqa: E402
from synth.workload import make_engine  # noqa: E402
from tests.gpu_util import check_residual_stream, dev, oracle_layer, rel_err  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 2e-2
FMTS = ["bf16", "fp8", "mxfp4", "nvfp4"]


def _stream():
    return torch.cuda.current_stream().cuda_stream


def small_shape(fmt, shared=1, layers=2):
    return synth.LayerShape(f"small_{fmt}", "test", 512, 16, 4, 256, layers,
                            synth.FMT_NAMES[fmt], 300, 16 * layers, shared=shared)


def bf16_to_f32(t):
    return synth.bf16_bits_to_f32(t.cpu().numpy().view(np.uint16))


def check_layer(shape, seed, layer, x_bits, y_dev, ids_dev=None, rows=None):
    """Oracle on the given bf16 layer input; compare y (and ids) on `rows`."""
    xf = synth.bf16_bits_to_f32(x_bits)
    if rows is not None:
        xf = xf[rows]
    R = synth.router_weights(seed, layer, shape.experts, shape.hidden)
    ids, w, _ = OR.route(xf, R, shape.top_k)
    if ids_dev is not None:
        got_ids = ids_dev if rows is None else ids_dev[rows]
        assert np.array_equal(got_ids, ids), f"layer {layer}: router ids differ"
    ref = oracle_layer(shape, seed, layer, xf, ids, w)
    got = y_dev if rows is None else y_dev[rows]
    err = rel_err(got, ref)
    assert err <= TOL, f"layer {layer}: rel err {err:.3e}"
    return err


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [300, 1])
def test_moe_layer_formats(fmt, T):
    shape = small_shape(fmt)
    seed = 3
    e = make_engine(shape, seed)
    try:
        eo.eo_set_bandwidth(e, 100, 100)
        x = synth.activations(seed, 40 + T, T, shape.hidden, 1.0, True)
        y = torch.zeros((T, shape.hidden), dtype=torch.float32, device="cuda")
        for layer in range(shape.layers):
            eo.eo_moe_layer(e, layer, dev(x.view(np.int16)), y, T, None, _stream())
            torch.cuda.synchronize()
            check_layer(shape, seed, layer, x, y.cpu().numpy())
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "nvfp4", "fp8"])
def test_moe_layer_with_host_execution(fmt):
    # small cache and B_P << B_H: most misses run in the host routine
    shape = small_shape(fmt)
    seed = 4
    e = make_engine(shape, seed, cache_slots=3)
    try:
        eo.eo_set_bandwidth(e, 1, 5)
        for T in (1, 37):
            x = synth.activations(seed, 60 + T, T, shape.hidden, 1.0, True)
            y = torch.zeros((T, shape.hidden), dtype=torch.float32, device="cuda")
            eo.eo_moe_layer(e, 1, dev(x.view(np.int16)), y, T, None, _stream())
            torch.cuda.synchronize()
            check_layer(shape, seed, 1, x, y.cpu().numpy())
        assert eo.eo_stats_get(e)["host_experts"] > 0
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_steps_per_layer(fmt):
    shape = small_shape(fmt, layers=3)
    seed = 5
    L, k, H = shape.layers, shape.top_k, shape.hidden
    steps = 6
    e = make_engine(shape, seed, cache_slots=10, max_tokens=1)
    try:
        eo.eo_set_bandwidth(e, 2, 3)
        trace = synth.sticky_zipf_trace(seed, steps, L, shape.experts, k)
        cx = torch.zeros((L, 1, H), dtype=torch.int16, device="cuda")
        cy = torch.zeros((L, 1, H), dtype=torch.float32, device="cuda")
        ci = torch.zeros((L, 1, k), dtype=torch.int32, device="cuda")
        cw = torch.zeros((L, 1, k), dtype=torch.float32, device="cuda")
        eo.eo_set_capture(e, cx, cy, ci, cw, 1)
        res = Residency(10, L, shape.experts, 2, 3)
        for s in range(steps):
            x = synth.activations(seed, 100 + s, 1, H, 1.0, True)
            xd = dev(x.view(np.int16))
            eo.eo_decode_step(e, xd, 1, dev(trace[s].reshape(L, 1, k)), _stream())
            torch.cuda.synchronize()
            xin = cx.cpu().numpy().view(np.uint16)
            rL = check_residual_stream(x, xin, cy.cpu().numpy())
            assert np.array_equal(xd.cpu().numpy().view(np.uint16), rL)
            for l in range(L):
                assert np.array_equal(ci.cpu().numpy()[l, 0], trace[s, l])
                xf = synth.bf16_bits_to_f32(xin[l])
                R = synth.router_weights(seed, l, shape.experts, H)
                ids, w, _ = OR.route(xf, R, k, trace[s, l][None, :])
                assert np.max(np.abs(cw.cpu().numpy()[l] - w)) <= 1e-6
                ref = oracle_layer(shape, seed, l, xf, ids, w)
                assert rel_err(cy.cpu().numpy()[l], ref) <= TOL, (s, l)
                res.lookup_plan(l, ids)
        keys = np.zeros(10, dtype=np.int32)
        stamps = np.zeros(10, dtype=np.int64)
        eo.eo_cache_snapshot(e, keys, stamps)
        assert list(keys) == res.snapshot()[0] and list(stamps) == res.snapshot()[1]
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("db", [1, 0])
def test_prefill_per_layer(fmt, db):
    shape = small_shape(fmt, layers=3)
    seed = 6
    L, k, H, T = shape.layers, shape.top_k, shape.hidden, 300
    e = make_engine(shape, seed, cache_slots=0, max_tokens=T)
    try:
        x = synth.activations(seed, 200, T, H, 1.0, True)
        xd = dev(x.view(np.int16))
        cx = torch.zeros((L, T, H), dtype=torch.int16, device="cuda")
        cy = torch.zeros((L, T, H), dtype=torch.float32, device="cuda")
        ci = torch.zeros((L, T, k), dtype=torch.int32, device="cuda")
        cw = torch.zeros((L, T, k), dtype=torch.float32, device="cuda")
        eo.eo_set_capture(e, cx, cy, ci, cw, T)
        eo.eo_prefill(e, xd, T, db, _stream())
        torch.cuda.synchronize()
        xin = cx.cpu().numpy().view(np.uint16)
        ys = cy.cpu().numpy()
        ids = ci.cpu().numpy()
        rL = check_residual_stream(x, xin, ys)
        for l in range(L):
            check_layer(shape, seed, l, xin[l], ys[l], ids[l])
        assert np.array_equal(xd.cpu().numpy().view(np.uint16), rL)
        st = eo.eo_stats_get(e)
        assert st["prefill_layers"] == L and st["lookups"] == 0
    finally:
        eo.eo_destroy(e)


def test_prefill_stream_times():
    # per-layer copy and compute stamps of a streamed prefill: every layer
    # stamped on both streams; with double buffering the chunk is at least the
    # longer of the two sums, without it at least their sum (the copy of layer
    # l + 1 then waits for layer l's kernels); the events change no bits
    import time
    shape = small_shape("bf16", layers=4)
    seed = 8
    L, H, T = shape.layers, shape.hidden, 300
    e = make_engine(shape, seed, cache_slots=0, max_tokens=T)
    try:
        x = dev(synth.activations(seed, 310, T, H, 1.0, True).view(np.int16))
        outs, walls, times = [], [], []
        for timing, db in ((False, 1), (True, 1), (True, 0)):
            xd = x.clone()
            eo.eo_set_timing(e, timing)
            eo.eo_stream_times(e, reset=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            eo.eo_prefill(e, xd, T, db, _stream())
            torch.cuda.synchronize()
            walls.append(1e3 * (time.perf_counter() - t0))
            times.append(eo.eo_stream_times(e, reset=True))
            outs.append(xd.cpu().numpy())
        eo.eo_set_timing(e, False)
        assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
        assert times[0] == {"copy_ms": 0.0, "compute_ms": 0.0, "copy_layers": 0,
                            "compute_layers": 0}
        for st in times[1:]:
            assert st["copy_layers"] == L and st["compute_layers"] == L
            assert st["copy_ms"] > 0 and st["compute_ms"] > 0
        layer_bytes = shape.experts * ((synth.expert_bytes(H, shape.inter, shape.fmt) + 4095)
                                       // 4096 * 4096)
        assert L * layer_bytes / (times[1]["copy_ms"] * 1e-3) > 1e9  # over 1 GB/s
        assert max(times[1]["copy_ms"], times[1]["compute_ms"]) <= walls[1]
        assert times[2]["copy_ms"] + times[2]["compute_ms"] <= walls[2]
    finally:
        eo.eo_destroy(e)


def test_prefill_streaming_matches_cache_path():
    # streaming must not change the arithmetic: same layer through the cache path
    shape = small_shape("bf16", layers=1, shared=0)
    seed = 7
    T = 300
    e = make_engine(shape, seed, cache_slots=shape.experts, max_tokens=T)
    try:
        eo.eo_set_bandwidth(e, 9, 9)
        x = synth.activations(seed, 300, T, shape.hidden, 1.0, True)
        cx = torch.zeros((1, T, shape.hidden), dtype=torch.int16, device="cuda")
        cy = torch.zeros((1, T, shape.hidden), dtype=torch.float32, device="cuda")
        ci = torch.zeros((1, T, shape.top_k), dtype=torch.int32, device="cuda")
        cw = torch.zeros((1, T, shape.top_k), dtype=torch.float32, device="cuda")
        eo.eo_set_capture(e, cx, cy, ci, cw, T)
        eo.eo_prefill(e, dev(x.view(np.int16)), T, 1, _stream())
        # the layer's own input (the normalised stream) through the cache path
        y1 = torch.zeros((T, shape.hidden), dtype=torch.float32, device="cuda")
        eo.eo_moe_layer(e, 0, cx[0].clone(), y1, T, None, _stream())
        torch.cuda.synchronize()
        assert torch.equal(y1, cy[0])
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4"])
def test_decode_stack_against_oracle_chain(fmt):
    # three layers on forced expert ids: the oracle runs the whole residual
    # stream itself (normalise, route weights, layer, residual) from x0 alone
    shape = small_shape(fmt, layers=3)
    seed = 12
    L, k, H = shape.layers, shape.top_k, shape.hidden
    e = make_engine(shape, seed, cache_slots=20, max_tokens=1)
    try:
        eo.eo_set_bandwidth(e, 5, 7)
        trace = synth.sticky_zipf_trace(seed, 3, L, shape.experts, k)
        from oracle import moe as OM
        from tests.gpu_util import oracle_expert_fn, oracle_shared
        layers = None
        for s in range(3):
            x = synth.activations(seed, 700 + s, 1, H, 2.0, True)
            xd = dev(x.view(np.int16))
            eo.eo_decode_step(e, xd, 1, dev(trace[s].reshape(L, 1, k)), _stream())
            torch.cuda.synchronize()
            if layers is None:
                layers = [[synth.router_weights(seed, l, shape.experts, H), k,
                           oracle_expert_fn(shape, seed, l), oracle_shared(shape, seed, l), None]
                          for l in range(L)]
            for l in range(L):
                layers[l][4] = trace[s, l][None, :]
            rL, _ = OM.stack_forward(synth.bf16_bits_to_f32(x), [tuple(v) for v in layers], True)
            got = synth.bf16_bits_to_f32(xd.cpu().numpy().view(np.uint16))
            err = rel_err(got, rL)
            assert err <= TOL, f"step {s}: rel err {err:.3e}"
    finally:
        eo.eo_destroy(e)


def _decode_capture(shape, seed, steps, forced, env, cache_slots=7, bw=(3, 5)):
    """Decode `steps` tokens on a fresh engine with EO_FUSED_ENTRY=env (a string)
    or with the variables of env (a dict) set throughout; returns the final
    streams, every capture as bytes, the statistics and the cache snapshot."""
    import os
    L, k, H = shape.layers, shape.top_k, shape.hidden
    env = {"EO_FUSED_ENTRY": env} if isinstance(env, str) else env
    saved = {v: os.environ.get(v) for v in env}
    os.environ.update(env)
    try:
        return _decode_capture_run(shape, seed, steps, forced, cache_slots, bw)
    finally:
        for v, old in saved.items():
            if old is None:
                del os.environ[v]
            else:
                os.environ[v] = old


def _decode_capture_run(shape, seed, steps, forced, cache_slots, bw):
    L, k, H = shape.layers, shape.top_k, shape.hidden
    e = make_engine(shape, seed, cache_slots=cache_slots, max_tokens=1)
    out = []
    try:
        eo.eo_set_bandwidth(e, *bw)
        tr = synth.sticky_zipf_trace(seed, steps, L, shape.experts, k)
        cx = torch.zeros((L, 1, H), dtype=torch.int16, device="cuda")
        cy = torch.zeros((L, 1, H), dtype=torch.float32, device="cuda")
        ci = torch.zeros((L, 1, k), dtype=torch.int32, device="cuda")
        cw = torch.zeros((L, 1, k), dtype=torch.float32, device="cuda")
        eo.eo_set_capture(e, cx, cy, ci, cw, 1)
        for s in range(steps):
            x = synth.activations(seed, 900 + s, 1, H, 1.0, True)
            xd = dev(x.view(np.int16))
            eo.eo_decode_step(e, xd, 1, dev(tr[s].reshape(L, 1, k)) if forced else None,
                              _stream())
            torch.cuda.synchronize()
            out.append((x, xd.cpu().numpy().view(np.uint16).copy(),
                        cx.cpu().numpy().view(np.uint16).copy(), cy.cpu().numpy().copy(),
                        ci.cpu().numpy().copy(), cw.cpu().numpy().copy()))
        # the counters (the host timers differ from run to run)
        out.append({n: v for n, v in eo.eo_stats_get(e).items() if not n.endswith("_ns")})
        keys = np.zeros(max(cache_slots, 1), dtype=np.int32)
        stamps = np.zeros(max(cache_slots, 1), dtype=np.int64)
        out.append((eo.eo_cache_snapshot(e, keys, stamps), keys.tolist(), stamps.tolist()))
    finally:
        eo.eo_destroy(e)
    return out


@pytest.mark.parametrize("forced", [True, False])
def test_decode_fused_entry_matches_separate_kernels(forced):
    # the fused one-token layer entry (residual + norm + logits, top-k in the
    # plan kernel) does the same arithmetic in the same order as the separate
    # residual, normalisation, router and top-k kernels: results are identical
    shape = small_shape("bf16", layers=3)
    a = _decode_capture(shape, 13, 4, forced, "1")
    b = _decode_capture(shape, 13, 4, forced, "0")
    for s in range(4):
        for i in range(1, 6):
            assert np.array_equal(a[s][i], b[s][i]), (s, i)
    assert a[-2:] == b[-2:]


def test_decode_entry_and_plan_in_one_launch_long_run():
    # the one-launch entry + plan at the benchmark's layer shape (H 2048, 128
    # experts: 32 workgroups store their logits at device scope for the last
    # one to plan from) over 1200 launches, the router choosing the experts:
    # every capture, the statistics and the slot table equal the separate
    # entry and plan launches, whose logits cross a kernel boundary
    base = synth.SHAPES["decode_bf16_48L"]
    shape = dataclasses.replace(base, layers=8, cache_slots=int(0.37 * 8 * base.experts))
    steps = 150
    a = _decode_capture(shape, 31, steps, False, {"EO_ENTRY_PLAN": "1"}, shape.cache_slots)
    b = _decode_capture(shape, 31, steps, False, {"EO_ENTRY_PLAN": "0"}, shape.cache_slots)
    for s in range(steps):
        for i in range(1, 6):
            assert np.array_equal(a[s][i], b[s][i]), (s, i)
    assert a[-2:] == b[-2:]
    assert a[-2]["fills"] > 0 and a[-2]["host_experts"] > 0


@pytest.mark.parametrize("bw", [(3, 5), (1, 1)])
@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4", "nvfp4"])
def test_decode_fill_and_gate_up_in_one_launch(fmt, bw):
    # the one launch that copies a call's fills while the other experts'
    # gate/up rows run (a filled expert's rows once the bytes they read are in)
    # gives the bits of the fill kernel followed by the GEMV kernels: every
    # capture, the counters and the slot table; B_P = B_H fills every miss the
    # capacity allows (several fills per call)
    shape = small_shape(fmt, layers=3)
    a = _decode_capture(shape, 17, 8, False, {"EO_FILL_GEMV": "1"}, 7, bw)
    b = _decode_capture(shape, 17, 8, False, {"EO_FILL_GEMV": "0"}, 7, bw)
    for s in range(8):
        for i in range(1, 6):
            assert np.array_equal(a[s][i], b[s][i]), (s, i)
    assert a[-2:] == b[-2:]
    assert a[-2]["fills"] > 0 and (a[-2]["host_experts"] > 0) == (bw != (1, 1))


def test_decode_fill_and_gate_up_in_one_launch_long_run():
    # the same at the benchmark's layer shape over 1200 layer calls
    base = synth.SHAPES["decode_bf16_48L"]
    shape = dataclasses.replace(base, layers=8, cache_slots=int(0.37 * 8 * base.experts))
    steps = 150
    a = _decode_capture(shape, 33, steps, False, {"EO_FILL_GEMV": "1"}, shape.cache_slots)
    b = _decode_capture(shape, 33, steps, False, {"EO_FILL_GEMV": "0"}, shape.cache_slots)
    for s in range(steps):
        for i in range(1, 6):
            assert np.array_equal(a[s][i], b[s][i]), (s, i)
    assert a[-2:] == b[-2:]
    assert a[-2]["fills"] > 0 and a[-2]["host_experts"] > 0


@pytest.mark.parametrize("experts,top_k,slots", [(16, 4, 7), (128, 8, 90), (128, 8, 0)])
@pytest.mark.parametrize("forced", [True, False])
def test_decode_entry_and_plan_in_one_launch(experts, top_k, slots, forced):
    # the layer entry and the one-token plan in one launch (the last workgroup
    # to finish its logits plans) against separate entry and plan launches:
    # streams, captures, routed ids, statistics and the slot table identical
    shape = dataclasses.replace(small_shape("bf16", layers=3), experts=experts, top_k=top_k)
    a = _decode_capture(shape, 15, 5, forced, {"EO_ENTRY_PLAN": "1"}, slots)
    b = _decode_capture(shape, 15, 5, forced, {"EO_ENTRY_PLAN": "0"}, slots)
    for s in range(5):
        for i in range(1, 6):
            assert np.array_equal(a[s][i], b[s][i]), (s, i)
    assert a[-2:] == b[-2:]


def test_decode_routed_ids_bit_exact():
    # no forced ids: the top-k taken inside the plan kernel against the oracle
    shape = small_shape("bf16", layers=3)
    seed = 14
    res = _decode_capture(shape, seed, 5, False, "1")
    for s in range(5):
        x, xout, xin, ys, ids, ws = res[s]
        rL = check_residual_stream(x, xin, ys)
        assert np.array_equal(xout, rL)
        for l in range(shape.layers):
            R = synth.router_weights(seed, l, shape.experts, shape.hidden)
            rid, rw, _ = OR.route(synth.bf16_bits_to_f32(xin[l]), R, shape.top_k)
            assert np.array_equal(ids[l], rid), (s, l)
            assert np.max(np.abs(ws[l] - rw)) <= 1e-6
            check_layer(shape, seed, l, xin[l], ys[l], ids[l])


def test_elastic_resize_between_steps():
    # shrink and grow the cache between decode steps: the slot table must follow
    # the oracle's resize bit for bit and the moved experts must still compute
    shape = small_shape("mxfp4", layers=3)
    seed = 15
    L, k, H = shape.layers, shape.top_k, shape.hidden
    C0 = 20
    e = make_engine(shape, seed, cache_slots=C0, max_tokens=1)
    try:
        eo.eo_set_bandwidth(e, 7, 7)  # every miss filled: the cache churns
        res = Residency(C0, L, shape.experts, 7, 7)
        trace = synth.sticky_zipf_trace(seed, 12, L, shape.experts, k)
        cx = torch.zeros((L, 1, H), dtype=torch.int16, device="cuda")
        cy = torch.zeros((L, 1, H), dtype=torch.float32, device="cuda")
        ci = torch.zeros((L, 1, k), dtype=torch.int32, device="cuda")
        cw = torch.zeros((L, 1, k), dtype=torch.float32, device="cuda")
        eo.eo_set_capture(e, cx, cy, ci, cw, 1)

        def check_state(C):
            keys = np.zeros(max(C, 1), dtype=np.int32)
            stamps = np.zeros(max(C, 1), dtype=np.int64)
            clock, credit = eo.eo_cache_snapshot(e, keys, stamps)
            rk, rs, rc, rcr = res.snapshot()
            assert list(keys[:C]) == rk and list(stamps[:C]) == rs and (clock, credit) == (rc, rcr)

        for s, C in enumerate([None, None, None, 8, None, None, 3, None, 30, None, None, 0]):
            if C is not None:
                ne, nm = eo.eo_resize_cache(e, C)
                ev, mv = res.resize(C)
                assert (ne, nm) == (len(ev), len(mv)), s
                check_state(C)
            x = synth.activations(seed, 800 + s, 1, H, 1.0, True)
            eo.eo_decode_step(e, dev(x.view(np.int16)), 1, dev(trace[s].reshape(L, 1, k)), _stream())
            torch.cuda.synchronize()
            for l in range(L):
                res.lookup_plan(l, trace[s, l][None, :])
            check_state(res.C)
            xin = cx.cpu().numpy().view(np.uint16)
            ys, ws = cy.cpu().numpy(), cw.cpu().numpy()
            for l in range(L):
                xf = synth.bf16_bits_to_f32(xin[l])
                R = synth.router_weights(seed, l, shape.experts, H)
                ids, w, _ = OR.route(xf, R, k, trace[s, l][None, :])
                assert rel_err(ys[l], oracle_layer(shape, seed, l, xf, ids, w)) <= TOL, (s, l)
        # not between steps: a pending plan blocks the resize
        eo.eo_lookup_plan(e, 0, dev(trace[0, 0][None, :].astype(np.int32)), 1, _stream())
        with pytest.raises(eo.EOError) as ei:
            eo.eo_resize_cache(e, 4)
        assert ei.value.status == eo.EO_ERR_STATE
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4"])
def test_prefill_skipping_resident_experts(fmt):
    # resident-aware streaming reads cached experts from their slots and streams
    # only the rest: the same result bit for bit, fewer bytes over PCIe, and the
    # cache untouched
    shape = small_shape(fmt, layers=3)
    seed = 16
    L, k, H, T = shape.layers, shape.top_k, shape.hidden, 300
    e = make_engine(shape, seed, cache_slots=22, max_tokens=T)
    try:
        eo.eo_set_bandwidth(e, 5, 5)
        tr = synth.sticky_zipf_trace(seed, 6, L, shape.experts, k)
        for s in range(6):
            xd = dev(synth.activations(seed, 900 + s, 1, H, 1.0, True).view(np.int16))
            eo.eo_decode_step(e, xd, 1, dev(tr[s].reshape(L, 1, k)), _stream())
        torch.cuda.synchronize()
        keys = np.zeros(22, dtype=np.int32)
        stamps = np.zeros(22, dtype=np.int64)
        before = eo.eo_cache_snapshot(e, keys, stamps), keys.copy(), stamps.copy()
        n_res = int((keys >= 0).sum())
        assert n_res > 0
        S_pad = (synth.expert_bytes(H, shape.inter, shape.fmt) + 4095) // 4096 * 4096
        x = synth.activations(seed, 950, T, H, 1.0, True)
        outs = []
        for flags in (1, 3, 2):
            xd = dev(x.view(np.int16))
            b0 = eo.eo_stats_get(e)["pcie_bytes"]
            eo.eo_prefill(e, xd, T, flags, _stream())
            torch.cuda.synchronize()
            outs.append((xd.cpu().numpy().tobytes(), eo.eo_stats_get(e)["pcie_bytes"] - b0))
        assert outs[0][0] == outs[1][0] == outs[2][0]
        assert outs[0][1] == L * shape.experts * S_pad
        assert outs[1][1] == outs[2][1] == (L * shape.experts - n_res) * S_pad
        keys2 = np.zeros(22, dtype=np.int32)
        stamps2 = np.zeros(22, dtype=np.int64)
        after = eo.eo_cache_snapshot(e, keys2, stamps2)
        assert after == before[0] and np.array_equal(keys2, before[1]) and \
            np.array_equal(stamps2, before[2])
        with pytest.raises(eo.EOError):
            eo.eo_prefill(e, dev(x.view(np.int16)), T, 4, _stream())
    finally:
        eo.eo_destroy(e)


def test_remeasure_bandwidth_keeps_the_cache():
    # online re-measurement between steps: residency, stamps and clock kept,
    # credit clamped, and the following plans use the new split
    shape = small_shape("bf16", layers=2)
    seed = 17
    L, k, H = shape.layers, shape.top_k, shape.hidden
    e = make_engine(shape, seed, cache_slots=9, max_tokens=1)
    try:
        eo.eo_set_bandwidth(e, 3, 11)
        res = Residency(9, L, shape.experts, 3, 11)
        tr = synth.sticky_zipf_trace(seed, 8, L, shape.experts, k)
        for s in range(8):
            if s == 4:
                keys0 = np.zeros(9, dtype=np.int32)
                stamps0 = np.zeros(9, dtype=np.int64)
                clock0, _ = eo.eo_cache_snapshot(e, keys0, stamps0)
                bp, bh = eo.eo_remeasure_bandwidth(e)
                assert bp > 0 and bh > 0
                res.set_bandwidth(bp, bh)
                keys = np.zeros(9, dtype=np.int32)
                stamps = np.zeros(9, dtype=np.int64)
                clock, credit = eo.eo_cache_snapshot(e, keys, stamps)
                assert np.array_equal(keys, keys0) and np.array_equal(stamps, stamps0)
                assert clock == clock0 and credit == res.credit < bh
            xd = dev(synth.activations(seed, 990 + s, 1, H, 1.0, True).view(np.int16))
            eo.eo_decode_step(e, xd, 1, dev(tr[s].reshape(L, 1, k)), _stream())
            torch.cuda.synchronize()
            for l in range(L):
                res.lookup_plan(l, tr[s, l][None, :])
            keys = np.zeros(9, dtype=np.int32)
            stamps = np.zeros(9, dtype=np.int64)
            assert eo.eo_cache_snapshot(e, keys, stamps) == (res.clock, res.credit)
            assert list(keys) == res.snapshot()[0] and list(stamps) == res.snapshot()[1]
    finally:
        eo.eo_destroy(e)


def test_static_placement_then_lru():
    # a frozen placement: hits only on the placed keys, nothing filled or
    # evicted, every miss on the host; then back to the LRU from that state
    shape = small_shape("fp8", layers=3)
    seed = 18
    L, k, H, E = shape.layers, shape.top_k, shape.hidden, shape.experts
    C = 14
    e = make_engine(shape, seed, cache_slots=C, max_tokens=1)
    try:
        eo.eo_set_bandwidth(e, 9, 9)
        res = Residency(C, L, E, 9, 9)
        keys = np.random.default_rng(seed).choice(L * E, size=11, replace=False).astype(np.int32)
        eo.eo_set_static_placement(e, keys)
        res.set_static(keys)
        tr = synth.sticky_zipf_trace(seed, 8, L, E, k)
        cx = torch.zeros((L, 1, H), dtype=torch.int16, device="cuda")
        cy = torch.zeros((L, 1, H), dtype=torch.float32, device="cuda")
        ci = torch.zeros((L, 1, k), dtype=torch.int32, device="cuda")
        cw = torch.zeros((L, 1, k), dtype=torch.float32, device="cuda")
        eo.eo_set_capture(e, cx, cy, ci, cw, 1)
        st0 = eo.eo_stats_get(e)
        for s in range(8):
            if s == 5:
                eo.eo_clear_static_placement(e)
                res.clear_static()
            xd = dev(synth.activations(seed, 970 + s, 1, H, 1.0, True).view(np.int16))
            eo.eo_decode_step(e, xd, 1, dev(tr[s].reshape(L, 1, k)), _stream())
            torch.cuda.synchronize()
            for l in range(L):
                res.lookup_plan(l, tr[s, l][None, :])
            kk = np.zeros(C, dtype=np.int32)
            ss = np.zeros(C, dtype=np.int64)
            assert eo.eo_cache_snapshot(e, kk, ss) == (res.clock, res.credit)
            assert list(kk) == res.snapshot()[0] and list(ss) == res.snapshot()[1], s
            if s == 4:
                st = eo.eo_stats_get(e)
                assert st["fills"] == st0["fills"]  # frozen: no fills at all
            xin = cx.cpu().numpy().view(np.uint16)
            ys = cy.cpu().numpy()
            for l in range(L):
                xf = synth.bf16_bits_to_f32(xin[l])
                R = synth.router_weights(seed, l, E, H)
                ids, w, _ = OR.route(xf, R, k, tr[s, l][None, :])
                assert rel_err(ys[l], oracle_layer(shape, seed, l, xf, ids, w)) <= TOL, (s, l)
        assert eo.eo_stats_get(e)["fills"] > st0["fills"]  # the LRU filled again
        with pytest.raises(eo.EOError):
            eo.eo_set_static_placement(e, np.array([1, 1], dtype=np.int32))
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4", "nvfp4"])
def test_grouped_gemm_at_its_shortest_contraction(fmt, monkeypatch):
    # H 256, I 128: the down projection's K of 128 is a single four-tile fp4 span
    # (two FP8 spans), so the async-ring kernel's prologue span is its only one
    # and every span request past it is clamped; gate/up has K 256. Every kernel
    # path, ragged groups (197 tokens over 8 experts, top-2, one shared expert).
    shape = synth.LayerShape(f"short_k_{fmt}", "test", 256, 8, 2, 128, 1,
                             synth.FMT_NAMES[fmt], 197, 8, shared=1)
    seed = 23
    x = synth.activations(seed, 91, 197, shape.hidden, 1.0, True)
    for path in ("0", "1", "2", "3"):
        monkeypatch.setenv("EO_GEMM_PATH", path)
        e = make_engine(shape, seed, max_tokens=197)
        try:
            eo.eo_set_bandwidth(e, 50, 50)
            y = torch.zeros((197, shape.hidden), dtype=torch.float32, device="cuda")
            eo.eo_moe_layer(e, 0, dev(x.view(np.int16)), y, 197, None, _stream())
            torch.cuda.synchronize()
            check_layer(shape, seed, 0, x, y.cpu().numpy())
        finally:
            eo.eo_destroy(e)
    monkeypatch.delenv("EO_GEMM_PATH")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4", "nvfp4"])
def test_grouped_gemm_falls_back_on_shapes_the_tiled_kernels_reject(fmt):
    # H 384, I 192: neither dimension fits the 128 x 256 tiles (I % 128, H % 256),
    # so the default path must hand both projections to the plain 128 x 128 kernel.
    # H 384 is also an odd multiple of 128: setting the router once wrote its
    # chain-interleaved copy past the end of the host buffer at such sizes.
    shape = synth.LayerShape(f"odd_{fmt}", "test", 384, 8, 2, 192, 1,
                             synth.FMT_NAMES[fmt], 150, 8, shared=1)
    seed = 29
    x = synth.activations(seed, 93, 150, shape.hidden, 1.0, True)
    e = make_engine(shape, seed, max_tokens=150)
    try:
        eo.eo_set_bandwidth(e, 50, 50)
        y = torch.zeros((150, shape.hidden), dtype=torch.float32, device="cuda")
        eo.eo_moe_layer(e, 0, dev(x.view(np.int16)), y, 150, None, _stream())
        torch.cuda.synchronize()
        check_layer(shape, seed, 0, x, y.cpu().numpy())
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("T", [1, 40])
@pytest.mark.parametrize("experts,top_k", [(5, 1), (6, 6), (12, 3)])
@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
def test_expert_counts_and_top_k_edges(fmt, experts, top_k, T):
    # expert counts that are not a multiple of 4 (the routers' 4- and 8-wide
    # groups run past E), top-1, and top-k = E (every token routes to every
    # expert), no shared expert; cache of 3 slots, half the misses on the host
    shape = synth.LayerShape(f"edge_{fmt}_{experts}_{top_k}", "test", 256, experts, top_k, 128,
                             1, synth.FMT_NAMES[fmt], T, 3, shared=0)
    seed = 37
    e = make_engine(shape, seed, max_tokens=T)
    try:
        eo.eo_set_bandwidth(e, 50, 100)
        for c in range(3):
            x = synth.activations(seed, 300 + c, T, shape.hidden, 1.0, True)
            y = torch.zeros((T, shape.hidden), dtype=torch.float32, device="cuda")
            eo.eo_moe_layer(e, 0, dev(x.view(np.int16)), y, T, None, _stream())
            torch.cuda.synchronize()
            check_layer(shape, seed, 0, x, y.cpu().numpy())
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("lane", ["fill", "host"])
@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4", "nvfp4"])
def test_one_token_calls_at_an_odd_multiple_of_128(fmt, lane):
    # H 384, I 192 at T = 1: no tuned GEMV instantiation fits, so the generic
    # GEMV runs; B_P = B_H fills every miss, B_P << B_H sends every miss to the
    # host routine (its vector route needs H % 128 and I % 64 only)
    shape = synth.LayerShape(f"odd1_{fmt}", "test", 384, 8, 2, 192, 1,
                             synth.FMT_NAMES[fmt], 1, 4, shared=1)
    seed = 31
    e = make_engine(shape, seed, max_tokens=1)
    try:
        eo.eo_set_bandwidth(e, 50, 50) if lane == "fill" else eo.eo_set_bandwidth(e, 1, 100000)
        st0 = eo.eo_stats_get(e)
        for t in range(6):
            x = synth.activations(seed, 200 + t, 1, shape.hidden, 1.0, True)
            y = torch.zeros((1, shape.hidden), dtype=torch.float32, device="cuda")
            eo.eo_moe_layer(e, 0, dev(x.view(np.int16)), y, 1, None, _stream())
            torch.cuda.synchronize()
            check_layer(shape, seed, 0, x, y.cpu().numpy())
        st1 = eo.eo_stats_get(e)
        if lane == "host":
            assert st1["host_experts"] > st0["host_experts"] and st1["fills"] == st0["fills"]
        else:
            assert st1["fills"] > st0["fills"] and st1["host_experts"] == st0["host_experts"]
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4", "nvfp4"])
def test_every_gemm_and_gemv_kernel_against_the_oracle(fmt, monkeypatch):
    # the grouped GEMM's kernels (plain 128x128, register-prefetch 128x256,
    # async-ring 128x256: v4 for bf16, v4q for quantised weights; bf16 with
    # 128-byte weight rows, v5) and both decode GEMV families on one shape,
    # each against the oracle
    shape = small_shape(fmt)
    seed = 19
    x = synth.activations(seed, 77, 300, shape.hidden, 1.0, True)
    for path in ("0", "1", "2", "3"):
        monkeypatch.setenv("EO_GEMM_PATH", path)
        e = make_engine(shape, seed, max_tokens=300)
        try:
            eo.eo_set_bandwidth(e, 50, 50)
            y = torch.zeros((300, shape.hidden), dtype=torch.float32, device="cuda")
            eo.eo_moe_layer(e, 1, dev(x.view(np.int16)), y, 300, None, _stream())
            torch.cuda.synchronize()
            check_layer(shape, seed, 1, x, y.cpu().numpy())
        finally:
            eo.eo_destroy(e)
    monkeypatch.delenv("EO_GEMM_PATH")
    x1 = x[:1]
    for fast in ("1", "0"):
        monkeypatch.setenv("EO_GEMV_FAST", fast)
        e = make_engine(shape, seed, max_tokens=1)
        try:
            eo.eo_set_bandwidth(e, 50, 50)
            y = torch.zeros((1, shape.hidden), dtype=torch.float32, device="cuda")
            eo.eo_moe_layer(e, 1, dev(x1.view(np.int16)), y, 1, None, _stream())
            torch.cuda.synchronize()
            check_layer(shape, seed, 1, x1, y.cpu().numpy())
        finally:
            eo.eo_destroy(e)


def test_fills_by_kernel_and_by_copy_engine_agree():
    # EO_FILL_SDMA=1 fills with hipMemcpyAsync after a host wait; same results
    shape = small_shape("mxfp4", layers=3)
    a = _decode_capture(shape, 20, 4, True, "1")
    import os
    os.environ["EO_FILL_SDMA"] = "1"
    try:
        b = _decode_capture(shape, 20, 4, True, "1")
    finally:
        del os.environ["EO_FILL_SDMA"]
    for s in range(4):
        for i in range(1, 6):
            assert np.array_equal(a[s][i], b[s][i]), (s, i)
    assert a[-1] == b[-1]


def test_decode_determinism():
    shape = small_shape("bf16", layers=2)
    outs = []
    for _ in range(2):
        e = make_engine(shape, 8, cache_slots=5, max_tokens=1)
        try:
            eo.eo_set_bandwidth(e, 3, 4)
            tr = synth.sticky_zipf_trace(8, 4, 2, shape.experts, shape.top_k)
            xd = dev(synth.activations(8, 1, 1, shape.hidden, 1.0, True).view(np.int16))
            for s in range(4):
                eo.eo_decode_step(e, xd, 1, dev(tr[s].reshape(2, 1, -1)), _stream())
            torch.cuda.synchronize()
            keys = np.zeros(5, dtype=np.int32)
            stamps = np.zeros(5, dtype=np.int64)
            st = eo.eo_cache_snapshot(e, keys, stamps)
            outs.append((xd.cpu().numpy().tobytes(), keys.tobytes(), stamps.tobytes(), st))
        finally:
            eo.eo_destroy(e)
    assert outs[0] == outs[1]


def test_invalid_forced_ids_rejected():
    shape = small_shape("bf16", layers=1)
    e = make_engine(shape, 9, max_tokens=2, fill_pool=False)
    try:
        xd = dev(synth.activations(9, 1, 1, shape.hidden, 1.0, True).view(np.int16))
        y = torch.zeros((1, shape.hidden), dtype=torch.float32, device="cuda")
        bad = dev(np.array([[0, 0, 1, 2]], dtype=np.int32))  # repeated id
        with pytest.raises(eo.EOError) as ei:
            eo.eo_moe_layer(e, 0, xd, y, 1, bad, _stream())
        assert ei.value.status == eo.EO_ERR_INVALID_ARG
        bad = dev(np.array([[0, 99, 1, 2]], dtype=np.int32))  # out of range
        with pytest.raises(eo.EOError):
            eo.eo_moe_layer(e, 0, xd, y, 1, bad, _stream())
        # the engine stays usable
        good = dev(np.array([[3, 0, 1, 2]], dtype=np.int32))
        eo.eo_moe_layer(e, 0, xd, y, 1, good, _stream())
        torch.cuda.synchronize()
        with pytest.raises(eo.EOError):
            eo.eo_fill(e, _stream())  # no pending plan
    finally:
        eo.eo_destroy(e)


@pytest.mark.timeout(600)
def test_bf16_gemm_with_128_byte_weight_rows_matches_the_ring_kernel():
    # v5 (EO_GEMM_PATH=3) runs the same MFMAs in the same K order as v4, so a
    # prefill through either gives the same bits; the per-layer shape of the
    # 48-layer bf16 model (H 2048, 128 experts, top-8, I 768), two layers, one
    # 4096-token chunk (K 2048 and 768: 32 and 12 K-64 tiles), plus the oracle
    # on sampled tokens
    import os
    shape = synth.LayerShape("v5_bf16", "test", 2048, 128, 8, 768, 2, synth.FMT_NAMES["bf16"],
                             4096, 94)
    T, L, H, k, seed = 4096, 2, 2048, 8, 5
    x = synth.activations(seed, 5000, T, H, 1.0, True)
    outs = {}
    for path in ("2", "3"):
        os.environ["EO_GEMM_PATH"] = path
        try:
            e = make_engine(shape, seed, max_tokens=T)
            try:
                cy = torch.zeros((L, T, H), dtype=torch.float32, device="cuda")
                cx = torch.zeros((L, T, H), dtype=torch.int16, device="cuda")
                ci = torch.zeros((L, T, k), dtype=torch.int32, device="cuda")
                cw = torch.zeros((L, T, k), dtype=torch.float32, device="cuda")
                eo.eo_set_capture(e, cx, cy, ci, cw, T)
                eo.eo_prefill(e, dev(x.view(np.int16)), T, 1, _stream())
                torch.cuda.synchronize()
                outs[path] = (cx.cpu().numpy(), cy.cpu().numpy())
            finally:
                eo.eo_destroy(e)
        finally:
            del os.environ["EO_GEMM_PATH"]
    assert np.array_equal(outs["2"][0], outs["3"][0])
    assert np.array_equal(outs["2"][1].view(np.uint32), outs["3"][1].view(np.uint32))
    rows = np.sort(np.random.default_rng(seed).choice(T, size=12, replace=False))
    for l in range(L):
        check_layer(shape, seed, l, outs["3"][0][l][rows].view(np.uint16), outs["3"][1][l][rows])


def test_bf16_gemm_split_ragged_tiles_at_their_boundary():
    # Forced routing gives the experts groups of exactly 0, 1, 24, 30..33, 63, 64,
    # 65, 128 and 129 rows (150 tokens, top-4, 16 experts, plus the shared expert's
    # 150 rows), so the grouped GEMM meets tiles of at most 64 rows, which the
    # 128-byte-row kernel splits over its wavefronts by columns, right beside
    # tiles of 65 rows, which it does not. Its layer output must be the bits of
    # the three-stage ring kernel's and within the bar of the oracle's.
    import os
    shape = small_shape("bf16")
    seed, T, k, E = 41, 150, shape.top_k, shape.experts
    counts = [64, 65, 1, 128, 129, 63, 0, 32, 33, 31, 30, 24, 0, 0, 0, 0]
    assert sum(counts) == T * k and max(counts) <= T
    pool = np.repeat(np.arange(E, dtype=np.int32), counts)
    ids = np.stack([pool[j * T:(j + 1) * T] for j in range(k)], axis=1)  # token t: pool[t + jT]
    assert all(len(set(r)) == k for r in ids)
    x = synth.activations(seed, 93, T, shape.hidden, 1.0, True)
    ys = {}
    for path in ("2", "3"):
        os.environ["EO_GEMM_PATH"] = path
        try:
            e = make_engine(shape, seed, max_tokens=T)
            try:
                eo.eo_set_bandwidth(e, 50, 50)
                y = torch.zeros((T, shape.hidden), dtype=torch.float32, device="cuda")
                eo.eo_moe_layer(e, 0, dev(x.view(np.int16)), y, T, dev(ids), _stream())
                torch.cuda.synchronize()
                ys[path] = y.cpu().numpy()
            finally:
                eo.eo_destroy(e)
        finally:
            del os.environ["EO_GEMM_PATH"]
    assert np.array_equal(ys["2"].view(np.uint32), ys["3"].view(np.uint32))
    xf = synth.bf16_bits_to_f32(x)
    R = synth.router_weights(seed, 0, E, shape.hidden)
    ids_o, w_o, _ = OR.route(xf, R, k, ids)
    assert np.array_equal(ids_o, ids)
    err = rel_err(ys["3"], oracle_layer(shape, seed, 0, xf, ids_o, w_o))
    assert err <= TOL, f"rel err {err:.3e}"
