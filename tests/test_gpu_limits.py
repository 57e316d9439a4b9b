"""GPU parity at the engine's limits: 1024 experts, top-16, 8192 cache slots,
T at max_tokens, k = E, and the argument checks at the boundaries."""
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
WIDE = synth.LayerShape("wide_bf16", "test", 512, 1024, 16, 64, 8, synth.FMT_BF16, 300, 8192)


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("T", [300, 1])
def test_router_1024_experts_top16(T):
    e = make_engine(WIDE, 21, cache_slots=0, max_tokens=T, layers=1, fill_pool=False)
    try:
        x = synth.activations(21, 3, T, WIDE.hidden, 1.0, True)
        ids = torch.zeros((T, 16), dtype=torch.int32, device="cuda")
        w = torch.zeros((T, 16), dtype=torch.float32, device="cuda")
        eo.eo_route(e, 0, dev(x.view(np.int16)), T, None, ids, w, _stream())
        torch.cuda.synchronize()
        R = synth.router_weights(21, 0, WIDE.experts, WIDE.hidden)
        rids, rw, _ = OR.route(synth.bf16_bits_to_f32(x), R, 16)
        assert np.array_equal(ids.cpu().numpy(), rids)
        assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-6
    finally:
        eo.eo_destroy(e)


def test_plan_8192_slots_1024_experts():
    L, E, k, C = 8, 1024, 16, 8192
    e = make_engine(WIDE, 0, cache_slots=C, max_tokens=8, fill_pool=False)
    try:
        rng = np.random.default_rng(3)
        ref = Residency(C, L, E, 9, 9)
        for bp, bh in ((9, 9), (2, 7)):
            eo.eo_set_bandwidth(e, bp, bh)
            ref.set_bandwidth(bp, bh)
            for call in range(40):
                l = int(rng.integers(0, L))
                T = int(rng.integers(1, 9))
                ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
                eo.eo_lookup_plan(e, l, dev(ids), T, _stream())
                got = eo.eo_last_plan(e)
                p = ref.lookup_plan(l, ids)
                assert (got["hits"], got["fills"], got["host"], got["evicted"]) == \
                    (p.hits, p.fills, p.host, p.evicted), call
            keys = np.zeros(C, dtype=np.int32)
            stamps = np.zeros(C, dtype=np.int64)
            assert eo.eo_cache_snapshot(e, keys, stamps) == (ref.clock, ref.credit)
            assert list(keys) == ref.snapshot()[0] and list(stamps) == ref.snapshot()[1]
    finally:
        eo.eo_destroy(e)


@pytest.mark.timeout(600)
def test_decode_1024_experts_top16_full_cache():
    # every key fits (C = L*E): after the first visits everything hits; the
    # one-token entry spans 256 workgroups and the plan's top-k 16 rounds
    shape = synth.LayerShape("wide2", "test", 512, 1024, 16, 64, 2, synth.FMT_BF16, 1, 2048)
    L, E, k, H = shape.layers, shape.experts, shape.top_k, shape.hidden
    e = make_engine(shape, 22, max_tokens=1)
    try:
        eo.eo_set_bandwidth(e, 4, 4)
        res = Residency(2048, L, E, 4, 4)
        cx = torch.zeros((L, 1, H), dtype=torch.int16, device="cuda")
        cy = torch.zeros((L, 1, H), dtype=torch.float32, device="cuda")
        ci = torch.zeros((L, 1, k), dtype=torch.int32, device="cuda")
        cw = torch.zeros((L, 1, k), dtype=torch.float32, device="cuda")
        eo.eo_set_capture(e, cx, cy, ci, cw, 1)
        for s in range(3):
            x = synth.activations(22, 40 + s, 1, H, 1.0, True)
            xd = dev(x.view(np.int16))
            eo.eo_decode_step(e, xd, 1, None, _stream())
            torch.cuda.synchronize()
            xin = cx.cpu().numpy().view(np.uint16)
            ys = cy.cpu().numpy()
            rL = check_residual_stream(x, xin, ys)
            assert np.array_equal(xd.cpu().numpy().view(np.uint16), rL)
            for l in range(L):
                xf = synth.bf16_bits_to_f32(xin[l])
                ids, w, _ = OR.route(xf, synth.router_weights(22, l, E, H), k)
                assert np.array_equal(ci.cpu().numpy()[l], ids), (s, l)
                res.lookup_plan(l, ids)
                assert rel_err(ys[l], oracle_layer(shape, 22, l, xf, ids, w)) <= TOL, (s, l)
            keys = np.zeros(2048, dtype=np.int32)
            stamps = np.zeros(2048, dtype=np.int64)
            assert eo.eo_cache_snapshot(e, keys, stamps) == (res.clock, res.credit)
            assert list(keys) == res.snapshot()[0]
    finally:
        eo.eo_destroy(e)


def test_k_equals_e_and_t_at_max_tokens():
    shape = synth.LayerShape("k_eq_e", "test", 512, 4, 4, 64, 1, synth.FMT_BF16, 77, 4)
    T = 77
    e = make_engine(shape, 23, max_tokens=T)
    try:
        eo.eo_set_bandwidth(e, 3, 3)
        x = synth.activations(23, 1, T, shape.hidden, 1.0, True)
        y = torch.zeros((T, shape.hidden), dtype=torch.float32, device="cuda")
        eo.eo_moe_layer(e, 0, dev(x.view(np.int16)), y, T, None, _stream())
        torch.cuda.synchronize()
        xf = synth.bf16_bits_to_f32(x)
        ids, w, _ = OR.route(xf, synth.router_weights(23, 0, 4, shape.hidden), 4)
        assert rel_err(y.cpu().numpy(), oracle_layer(shape, 23, 0, xf, ids, w)) <= TOL
        for bad_T in (0, T + 1):
            with pytest.raises(eo.EOError) as ei:
                eo.eo_moe_layer(e, 0, dev(x.view(np.int16)), y, bad_T, None, _stream())
            assert ei.value.status == eo.EO_ERR_INVALID_ARG
    finally:
        eo.eo_destroy(e)


def test_create_rejects_out_of_range_configs():
    base = dict(layers=1, experts=8, top_k=2, hidden=256, inter=128, wfmt=synth.FMT_BF16,
                act_bf16=1, cache_slots=4, max_tokens=4, shared=0, host_threads=1, device=0)
    bad = [dict(experts=1025), dict(top_k=17, experts=32), dict(top_k=9, experts=8),
           dict(hidden=200), dict(inter=100), dict(cache_slots=8193), dict(max_tokens=0),
           dict(wfmt=synth.FMT_FP32), dict(shared=2)]
    for b in bad:
        cfg = dict(base, **b)
        with pytest.raises(eo.EOError) as ei:
            eo.eo_create(cfg["layers"], cfg["experts"], cfg["top_k"], cfg["hidden"], cfg["inter"],
                         cfg["wfmt"], cfg["act_bf16"], cfg["cache_slots"], cfg["max_tokens"],
                         cfg["shared"], cfg["host_threads"], cfg["device"])
        assert ei.value.status in (eo.EO_ERR_INVALID_ARG, eo.EO_ERR_UNSUPPORTED), b
