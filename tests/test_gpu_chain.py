"""GPU: the per-stage calls of the C ABI run as a chain, one layer at a time,
in the method's order (zhichai.net article, section 2, Decode paragraph):

    eo_route -> eo_lookup_plan -> eo_fill -> eo_host_execute -> eo_expert_ffn_combine

checked three ways on the same seeded inputs:
* against eo_moe_layer on a twin engine that sees the same calls: the plans,
  the cache state and the layer outputs are the same bit for bit (the chain's
  lookup does not mirror ids, w and x to the host, so the host routine takes
  them by device-to-host copies and the one-token GEMV takes its weight bases
  from the plan: paths eo_moe_layer does not use);
* against the oracle: router ids bit-exact, the plan and the slot table after
  every call bit-exact (oracle.residency), y within 2e-2 * max|ref|;
* out-of-order calls return EO_ERR_STATE and leave the engine usable.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expert_offload_amd as eo  # noqa: E402
import synth  # noqa: E402
from oracle import router as OR  # noqa: E402
from oracle.residency import Residency  # noqa: E402
from synth.workload import make_engine  # noqa: E402
from tests.gpu_util import dev, oracle_layer, rel_err  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _s():
    return torch.cuda.current_stream().cuda_stream


def _shape(fmt):
    return synth.LayerShape(f"chain_{fmt}", "test", 512, 16, 4, 256, 2, synth.FMT_NAMES[fmt],
                            300, 6, shared=1)


def _snapshot(e, C):
    keys = np.zeros(max(C, 1), dtype=np.int32)
    stamps = np.zeros(max(C, 1), dtype=np.int64)
    clock, credit = eo.eo_cache_snapshot(e, keys, stamps)
    return list(keys[:C]), list(stamps[:C]), clock, credit


def _plan_matches(got, p, what):
    assert got["hits"] == p.hits, what
    assert got["fills"] == p.fills, what
    assert got["host"] == p.host, what
    assert got["evicted"] == p.evicted, what
    assert (got["m"], got["q"], got["q_fill"], got["clock"], got["credit"]) == \
        (p.m, p.q, p.q_fill, p.clock, p.credit), what


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4"])
def test_per_stage_chain(fmt):
    shape = _shape(fmt)
    seed = 21
    H, E, k, C, L = shape.hidden, shape.experts, shape.top_k, shape.cache_slots, shape.layers
    bp, bh = 1, 2  # half of the misses filled, half on the host routine
    chain = make_engine(shape, seed)
    twin = make_engine(shape, seed)
    try:
        for e in (chain, twin):
            eo.eo_set_bandwidth(e, bp, bh)
        ref = Residency(C, L, E, bp, bh)
        fills = hosts = 0
        calls = [(T, l) for T in (1, 300, 1, 40, 1) for l in range(L)]
        for n, (T, layer) in enumerate(calls):
            x = synth.activations(seed, 200 + n, T, H, 1.0, True)
            xd = dev(x.view(np.int16))
            ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
            w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
            y = torch.zeros((T, H), dtype=torch.float32, device="cuda")
            eo.eo_route(chain, layer, xd, T, None, ids, w, _s())
            eo.eo_lookup_plan(chain, layer, ids, T, _s())
            eo.eo_fill(chain, _s())
            eo.eo_host_execute(chain, xd, ids, w, _s())
            eo.eo_expert_ffn_combine(chain, layer, xd, ids, w, y, _s())
            torch.cuda.synchronize()
            plan = eo.eo_last_plan(chain)
            snap = _snapshot(chain, C)

            y2 = torch.zeros((T, H), dtype=torch.float32, device="cuda")
            eo.eo_moe_layer(twin, layer, xd, y2, T, None, _s())
            torch.cuda.synchronize()
            what = (fmt, n, T, layer)
            assert eo.eo_last_plan(twin) == plan, what
            assert _snapshot(twin, C) == snap, what
            got = y.cpu().numpy()
            assert np.array_equal(got.view(np.uint32), y2.cpu().numpy().view(np.uint32)), what

            xf = synth.bf16_bits_to_f32(x)
            R = synth.router_weights(seed, layer, E, H)
            rids, rw, _ = OR.route(xf, R, k)
            assert np.array_equal(ids.cpu().numpy(), rids), what
            assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-6, what
            p = ref.lookup_plan(layer, rids)
            _plan_matches(plan, p, what)
            sk, ss, sc, scr = ref.snapshot()
            assert snap == (sk, ss, sc, scr), what
            err = rel_err(got, oracle_layer(shape, seed, layer, xf, rids, rw))
            assert err <= TOL, (what, err)
            fills += len(p.fills)
            hosts += len(p.host)
        assert fills > 0 and hosts > 0, "both miss lanes must be exercised"
    finally:
        eo.eo_destroy(chain)
        eo.eo_destroy(twin)


def test_per_stage_calls_out_of_order():
    shape = _shape("bf16")
    seed = 22
    H, k = shape.hidden, shape.top_k
    e = make_engine(shape, seed)
    try:
        eo.eo_set_bandwidth(e, 1, 2)
        T = 3
        x = synth.activations(seed, 1, T, H, 1.0, True)
        xd = dev(x.view(np.int16))
        ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
        w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
        y = torch.zeros((T, H), dtype=torch.float32, device="cuda")

        def status(fn, *a):
            try:
                fn(*a)
            except eo.EOError as err:
                return err.status
            return eo.EO_OK

        # nothing planned yet
        assert status(eo.eo_fill, e, _s()) == eo.EO_ERR_STATE
        assert status(eo.eo_host_execute, e, xd, ids, w, _s()) == eo.EO_ERR_STATE
        assert status(eo.eo_expert_ffn_combine, e, 0, xd, ids, w, y, _s()) == eo.EO_ERR_STATE
        eo.eo_route(e, 0, xd, T, None, ids, w, _s())
        eo.eo_lookup_plan(e, 0, ids, T, _s())
        # the plan is layer 0's
        assert status(eo.eo_expert_ffn_combine, e, 1, xd, ids, w, y, _s()) == eo.EO_ERR_STATE
        eo.eo_fill(e, _s())
        eo.eo_host_execute(e, xd, ids, w, _s())
        eo.eo_expert_ffn_combine(e, 0, xd, ids, w, y, _s())
        torch.cuda.synchronize()
        # the combine consumed the plan
        assert status(eo.eo_fill, e, _s()) == eo.EO_ERR_STATE
        assert status(eo.eo_expert_ffn_combine, e, 0, xd, ids, w, y, _s()) == eo.EO_ERR_STATE
        # and the engine still serves the next layer call
        rids, rw, _ = OR.route(synth.bf16_bits_to_f32(x), synth.router_weights(seed, 1, shape.experts, H), k)
        eo.eo_moe_layer(e, 1, xd, y, T, None, _s())
        torch.cuda.synchronize()
        err = rel_err(y.cpu().numpy(),
                      oracle_layer(shape, seed, 1, synth.bf16_bits_to_f32(x), rids, rw))
        assert err <= TOL
        eo.eo_sync(e)
    finally:
        eo.eo_destroy(e)


def test_plan_log_matches_the_oracle_plans():
    """eo_set_plan_log / eo_get_plan_log over decode steps: one entry per layer
    call, {layer, hits, fills, host experts}, equal to the oracle's plans."""
    shape = _shape("bf16")
    seed = 23
    L, E, k, H = shape.layers, shape.experts, shape.top_k, shape.hidden
    e = make_engine(shape, seed, max_tokens=1)
    try:
        eo.eo_set_bandwidth(e, 2, 5)
        ref = Residency(shape.cache_slots, L, E, 2, 5)
        trace = synth.sticky_zipf_trace(seed, 12, L, E, k)
        eo.eo_set_plan_log(e, True)
        for st in range(12):
            x = dev(synth.activations(seed, 900 + st, 1, H, 1.0, True).view(np.int16))
            eo.eo_decode_step(e, x, 1, dev(trace[st].reshape(L, 1, k)), _s())
        torch.cuda.synchronize()
        eo.eo_set_plan_log(e, False)
        log = eo.eo_get_plan_log(e)
        want = []
        for st in range(12):
            for l in range(L):
                p = ref.lookup_plan(l, trace[st, l][None, :])
                want.append([l, len(p.hits), len(p.fills), len(p.host)])
        assert log.shape == (12 * L, 4)
        assert np.array_equal(log, np.array(want, dtype=np.int32))
        assert log[:, 2].sum() > 0 and log[:, 3].sum() > 0
        # stopped: further calls are not logged; re-enabling clears
        x = dev(synth.activations(seed, 999, 1, H, 1.0, True).view(np.int16))
        eo.eo_decode_step(e, x, 1, dev(trace[0].reshape(L, 1, k)), _s())
        torch.cuda.synchronize()
        assert eo.eo_get_plan_log(e).shape == (12 * L, 4)
        eo.eo_set_plan_log(e, True)
        assert eo.eo_get_plan_log(e).shape == (0, 4)
    finally:
        eo.eo_destroy(e)
