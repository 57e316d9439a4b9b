"""GPU parity: the HIP path (through the C ABI) against the CPU oracle."""
import ctypes
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expert_offload_amd as eo  # noqa: E402
import synth  # noqa: E402
from oracle import formats as OF  # noqa: E402
from oracle import router as OR  # noqa: E402
from oracle.residency import Residency  # noqa: E402
from synth.workload import make_engine  # noqa: E402
from tests.gpu_util import act_f32, dev, oracle_layer, rel_err  # noqa: E402

pytestmark = pytest.mark.gpu

TINY = synth.SHAPES["tiny_fp32"]
SEED = 0


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.fixture
def tiny_engine():
    e = make_engine(TINY, SEED)
    eo.eo_set_bandwidth(e, 1000, 1000)
    yield e
    eo.eo_destroy(e)


def _route_case(shape, T, seed, forced=None):
    bf16 = shape.fmt != synth.FMT_FP32
    e = make_engine(shape, seed, cache_slots=0, max_tokens=T, layers=1, fill_pool=False)
    try:
        sigma = 1.0 if bf16 else 0.02
        x = synth.activations(seed, 7, T, shape.hidden, sigma, bf16)
        ids = torch.zeros((T, shape.top_k), dtype=torch.int32, device="cuda")
        w = torch.zeros((T, shape.top_k), dtype=torch.float32, device="cuda")
        fx = None if forced is None else dev(forced)
        eo.eo_route(e, 0, dev(x), T, fx, ids, w, _stream())
        torch.cuda.synchronize()
        R = synth.router_weights(seed, 0, shape.experts, shape.hidden)
        rids, rw, _ = OR.route(act_f32(x, bf16), R, shape.top_k, forced)
        return ids.cpu().numpy(), w.cpu().numpy(), rids, rw
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("name,T", [("tiny_fp32", 64), ("tiny_fp32", 1),
                                    ("decode_bf16_48L", 300), ("decode_mxfp4_43L", 37)])
def test_router_topk_bit_exact(name, T):
    ids, w, rids, rw = _route_case(synth.SHAPES[name], T, SEED + T)
    assert np.array_equal(ids, rids)
    assert np.max(np.abs(w - rw)) <= 1e-6
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)


def test_router_forced_ids():
    shape = synth.SHAPES["decode_bf16_48L"]
    tr = synth.sticky_zipf_trace(3, 5, 1, shape.experts, shape.top_k)[:, 0, :]
    ids, w, rids, rw = _route_case(shape, 5, 11, forced=tr)
    assert np.array_equal(ids, tr)
    assert np.max(np.abs(w - rw)) <= 1e-6


@pytest.mark.parametrize("case", range(4))
def test_plan_and_cache_state_bit_exact(case):
    rng = np.random.default_rng(case)
    L, E, k = 3, 16, int(rng.integers(1, 5))
    C = [8, 3, 20, 0][case]
    bp, bh = [(5, 5), (1, 3), (11800, 47500), (7, 2)][case]
    shape = dataclasses.replace(TINY, layers=L, experts=E, top_k=k, cache_slots=C)
    e = make_engine(shape, 0, max_tokens=8, fill_pool=False)
    try:
        eo.eo_set_bandwidth(e, bp, bh)
        ref = Residency(C, L, E, bp, bh)
        for call in range(60):
            l = int(rng.integers(0, L))
            T = int(rng.integers(1, 9))
            ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
            eo.eo_lookup_plan(e, l, dev(ids), T, _stream())
            got = eo.eo_last_plan(e)
            p = ref.lookup_plan(l, ids)
            assert got["hits"] == p.hits, call
            assert got["fills"] == p.fills, call
            assert got["host"] == p.host, call
            assert got["evicted"] == p.evicted, call
            assert (got["m"], got["q"], got["q_fill"], got["clock"], got["credit"]) == \
                (p.m, p.q, p.q_fill, p.clock, p.credit)
            keys = np.zeros(max(C, 1), dtype=np.int32)
            stamps = np.zeros(max(C, 1), dtype=np.int64)
            clock, credit = eo.eo_cache_snapshot(e, keys, stamps)
            sk, ss, sc, scr = ref.snapshot()
            assert list(keys[:C]) == sk and list(stamps[:C]) == ss
            assert (clock, credit) == (sc, scr)
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("case", range(5))
def test_one_token_plan_bit_exact(case, monkeypatch):
    # one-token lookups go to their own kernel; both kernels against the oracle
    rng = np.random.default_rng(100 + case)
    L, E, k = 3, 24, int(rng.integers(1, 9))
    C = [9, 2, 30, 0, 72][case]
    bp, bh = [(5, 5), (1, 3), (11800, 47500), (7, 2), (3, 4)][case]
    shape = dataclasses.replace(TINY, layers=L, experts=E, top_k=k, cache_slots=C)
    for plan1 in ("1", "0"):
        monkeypatch.setenv("EO_PLAN1", plan1)
        e = make_engine(shape, 0, max_tokens=1, fill_pool=False)
        try:
            eo.eo_set_bandwidth(e, bp, bh)
            ref = Residency(C, L, E, bp, bh)
            for call in range(80):
                l = int(rng.integers(0, L))
                ids = rng.choice(E, size=(1, k), replace=False).astype(np.int32)
                eo.eo_lookup_plan(e, l, dev(ids), 1, _stream())
                got = eo.eo_last_plan(e)
                p = ref.lookup_plan(l, ids)
                assert got["hits"] == p.hits and got["fills"] == p.fills, (plan1, call)
                assert got["host"] == p.host and got["evicted"] == p.evicted, (plan1, call)
                assert (got["m"], got["q"], got["q_fill"], got["clock"], got["credit"]) == \
                    (p.m, p.q, p.q_fill, p.clock, p.credit)
            keys = np.zeros(max(C, 1), dtype=np.int32)
            stamps = np.zeros(max(C, 1), dtype=np.int64)
            assert eo.eo_cache_snapshot(e, keys, stamps) == (ref.clock, ref.credit)
            assert list(keys[:C]) == ref.snapshot()[0] and list(stamps[:C]) == ref.snapshot()[1]
            bad = dev(np.array([[0] * k], dtype=np.int32)) if k > 1 else \
                dev(np.array([[E]], dtype=np.int32))
            with pytest.raises(eo.EOError):
                eo.eo_lookup_plan(e, 0, bad, 1, _stream())
                eo.eo_last_plan(e)
        finally:
            eo.eo_destroy(e)


@pytest.mark.parametrize("fmt", ["fp32", "bf16", "mxfp4", "nvfp4", "fp8"])
def test_device_dequant_bit_exact(fmt):
    f = synth.FMT_NAMES[fmt]
    H, I = 256, 128
    shape = dataclasses.replace(TINY, hidden=H, inter=I, fmt=f, experts=2, layers=1)
    e = make_engine(shape, 5, cache_slots=0, fill_pool=False)
    try:
        ptr, nbytes = eo.eo_pool_expert(e, 0, 1)
        blk = synth.expert_block(5, 0, 1, H, I, f)
        lay_data_end = {0: nbytes, 1: nbytes, 2: 3 * H * I // 2, 3: 3 * H * I // 2,
                        4: 3 * H * I}[f]
        if f in (synth.FMT_MXFP4, synth.FMT_NVFP4, synth.FMT_FP8):
            # every element code, scales as generated
            rng = np.random.default_rng(1)
            blk[:lay_data_end] = rng.integers(0, 256, size=lay_data_end, dtype=np.uint8)
        np.ctypeslib.as_array((ctypes.c_uint8 * nbytes).from_address(ptr))[:] = blk
        out = np.zeros(3 * H * I, dtype=np.float32)
        eo.eo_dequant(e, 0, 1, out)
        wg, wu, wd = OF.dequant_expert(blk, H, I, f)
        ref = np.concatenate([wg.ravel(), wu.ravel(), wd.ravel()])
        assert np.array_equal(out, ref, equal_nan=True)
    finally:
        eo.eo_destroy(e)


def _tiny_inputs(T, index):
    return synth.activations(SEED, index, T, TINY.hidden, 0.02, False)


def test_tiny_layer_64_tokens(tiny_engine):
    e = tiny_engine
    T = 64
    x = _tiny_inputs(T, 0)
    y = torch.zeros((T, TINY.hidden), dtype=torch.float32, device="cuda")
    eo.eo_moe_layer(e, 0, dev(x), y, T, None, _stream())
    torch.cuda.synchronize()
    R = synth.router_weights(SEED, 0, TINY.experts, TINY.hidden)
    ids, w, _ = OR.route(x, R, TINY.top_k)
    ref = oracle_layer(TINY, SEED, 0, x, ids, w)
    assert rel_err(y.cpu().numpy(), ref) <= 1e-4


@pytest.mark.parametrize("bw", [(1000, 1000), (1, 4), (3, 1)])
def test_tiny_one_token_calls_and_state(bw):
    e = make_engine(TINY, SEED)
    try:
        eo.eo_set_bandwidth(e, *bw)
        ref = Residency(TINY.cache_slots, 1, TINY.experts, *bw)
        R = synth.router_weights(SEED, 0, TINY.experts, TINY.hidden)
        X = _tiny_inputs(64, 1)
        worst = 0.0
        for t in range(64):
            x = X[t:t + 1]
            y = torch.zeros((1, TINY.hidden), dtype=torch.float32, device="cuda")
            eo.eo_moe_layer(e, 0, dev(x), y, 1, None, _stream())
            torch.cuda.synchronize()
            ids, w, _ = OR.route(x, R, TINY.top_k)
            ref.lookup_plan(0, ids)
            out = oracle_layer(TINY, SEED, 0, x, ids, w)
            worst = max(worst, rel_err(y.cpu().numpy(), out))
        assert worst <= 1e-4
        keys = np.zeros(TINY.cache_slots, dtype=np.int32)
        stamps = np.zeros(TINY.cache_slots, dtype=np.int64)
        clock, credit = eo.eo_cache_snapshot(e, keys, stamps)
        assert (list(keys), list(stamps), clock, credit) == tuple(ref.snapshot())
        st = eo.eo_stats_get(e)
        assert st["lookups"] == 64
        if bw == (1, 4):
            assert st["host_experts"] > 0
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("C,bw", [(0, (5, 5)), (8, (1, 50)), (16, (9, 9)), (1, (9, 9))])
def test_tiny_placement_invariance(C, bw):
    e = make_engine(TINY, SEED, cache_slots=C)
    try:
        eo.eo_set_bandwidth(e, *bw)
        T = 64
        x = _tiny_inputs(T, 2)
        y = torch.zeros((T, TINY.hidden), dtype=torch.float32, device="cuda")
        for _ in range(2):  # second call sees a warm cache
            eo.eo_moe_layer(e, 0, dev(x), y, T, None, _stream())
            torch.cuda.synchronize()
            R = synth.router_weights(SEED, 0, TINY.experts, TINY.hidden)
            ids, w, _ = OR.route(x, R, TINY.top_k)
            assert rel_err(y.cpu().numpy(), oracle_layer(TINY, SEED, 0, x, ids, w)) <= 1e-4
    finally:
        eo.eo_destroy(e)
