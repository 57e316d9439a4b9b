"""GPU parity at the workloads' full per-layer sizes, in the launch configuration
bench.py times, on outputs the oracle can compute one by one.

* bf16, 48 layers, hidden 2048, 128 experts, top-8, inter 768, 37% cache,
  16384-token prefill capacity (the engine bench.py builds): decode steps of the
  bench's trace with every layer captured, the cache state bit-exact against
  the oracle's replay after each step, and sampled layers checked; then an
  8192-token and a 16384-token prefill, sampled tokens of sampled layers checked.
* MXFP4 decode (hidden 4096, 256 experts + shared, inter 2048, 11% cache) and
  NVFP4 prefill + decode (hidden 6144, 256 experts + shared, inter 2048) at full
  per-layer shape with fewer layers.
* The same decode and prefill checks on a small two-layer model whose hidden size
  is an odd multiple of 128 (the kernels' generic paths).
"""
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
BP, BH = 52000, 155000  # MB/s, the order of the box's measured B_P and B_H


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _capture(e, L, T, H, k):
    bufs = (torch.zeros((L, T, H), dtype=torch.int16, device="cuda"),
            torch.zeros((L, T, H), dtype=torch.float32, device="cuda"),
            torch.zeros((L, T, k), dtype=torch.int32, device="cuda"),
            torch.zeros((L, T, k), dtype=torch.float32, device="cuda"))
    eo.eo_set_capture(e, *bufs, T)
    return bufs


def _decode_and_check(e, shape, seed, steps, layers_checked, C, trace_seed=None):
    L, E, k, H = shape.layers, shape.experts, shape.top_k, shape.hidden
    trace = synth.sticky_zipf_trace(seed if trace_seed is None else trace_seed, 512, L, E, k)[:steps]
    cx, cy, ci, cw = _capture(e, L, 1, H, k)
    res = Residency(C, L, E, BP, BH)
    routers = {}
    for s in range(steps):
        x = synth.activations(seed, 1000 + s, 1, H, 1.0, True)
        xd = dev(x.view(np.int16))
        eo.eo_decode_step(e, xd, 1, dev(trace[s].reshape(L, 1, k)), _stream())
        torch.cuda.synchronize()
        for l in range(L):
            res.lookup_plan(l, trace[s, l][None, :])
        keys = np.zeros(C, dtype=np.int32)
        stamps = np.zeros(C, dtype=np.int64)
        clock, credit = eo.eo_cache_snapshot(e, keys, stamps)
        ref_keys, ref_stamps, ref_clock, ref_credit = res.snapshot()
        assert list(keys) == ref_keys and list(stamps) == ref_stamps, f"step {s}: slot table"
        assert (clock, credit) == (ref_clock, ref_credit)
        xin = cx.cpu().numpy().view(np.uint16)
        ys, ws = cy.cpu().numpy(), cw.cpu().numpy()
        assert np.all(np.isfinite(ys)), f"step {s}: non-finite layer output"
        rL = check_residual_stream(x, xin, ys)
        assert np.array_equal(xd.cpu().numpy().view(np.uint16), rL), f"step {s}: residual stream"
        for l in layers_checked(s):
            xf = synth.bf16_bits_to_f32(xin[l])
            if l not in routers:
                routers[l] = synth.router_weights(seed, l, E, H)
            ids, w, _ = OR.route(xf, routers[l], k, trace[s, l][None, :])
            assert np.max(np.abs(ws[l] - w)) <= 1e-6
            err = rel_err(ys[l], oracle_layer(shape, seed, l, xf, ids, w))
            assert err <= TOL, f"step {s} layer {l}: rel err {err:.3e}"


def _prefill_and_check(e, shape, seed, T, layers, ntok):
    L, E, k, H = shape.layers, shape.experts, shape.top_k, shape.hidden
    x = synth.activations(seed, 5000, T, H, 1.0, True)
    xd = dev(x.view(np.int16))
    cx, cy, ci, cw = _capture(e, L, T, H, k)
    eo.eo_prefill(e, xd, T, 1, _stream())
    torch.cuda.synchronize()
    assert bool(torch.isfinite(cy).all()), "non-finite layer output"
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(T, size=ntok, replace=False))
    rows_d = torch.from_numpy(rows).cuda()
    # the residual stream on the sampled rows, every layer
    xs = cx.index_select(1, rows_d).cpu().numpy().view(np.uint16)
    rL = check_residual_stream(x[rows], xs, cy.index_select(1, rows_d).cpu().numpy())
    assert np.array_equal(xd.index_select(0, rows_d).cpu().numpy().view(np.uint16), rL)
    for l in layers:
        xin = cx[l].index_select(0, rows_d).cpu().numpy().view(np.uint16)
        y = cy[l].index_select(0, rows_d).cpu().numpy()
        ids_got = ci[l].index_select(0, rows_d).cpu().numpy()
        xf = synth.bf16_bits_to_f32(xin)
        ids, w, _ = OR.route(xf, synth.router_weights(seed, l, E, H), k)
        assert np.array_equal(ids_got, ids), f"layer {l}: router ids"
        err = rel_err(y, oracle_layer(shape, seed, l, xf, ids, w))
        assert err <= TOL, f"layer {l}: rel err {err:.3e}"
    return xd


@pytest.mark.timeout(900)
def test_bf16_48_layers_as_benchmarked():
    shape = synth.SHAPES["decode_bf16_48L"]
    pshape = synth.SHAPES["prefill_bf16_48L"]
    e = make_engine(shape, 0, max_tokens=2 * pshape.tokens)
    try:
        eo.eo_set_bandwidth(e, BP, BH)
        _decode_and_check(e, shape, 0, 6, lambda s: (0, 23, 47) if s < 5 else range(48),
                          shape.cache_slots)
        st = eo.eo_stats_get(e)
        assert st["fills"] > 0 and st["host_experts"] > 0  # both miss lanes exercised
        _prefill_and_check(e, pshape, 0, pshape.tokens, (0, 31, 47), 24)
        # the prefill configuration's other chunk size
        _prefill_and_check(e, pshape, 0, 2 * pshape.tokens, (0, 47), 16)
    finally:
        eo.eo_destroy(e)


@pytest.mark.timeout(900)
def test_mxfp4_decode_full_layer_shape():
    base = synth.SHAPES["decode_mxfp4_43L"]
    L = 3
    shape = synth.LayerShape("mxfp4_3L", "decode", base.hidden, base.experts, base.top_k,
                             base.inter, L, base.fmt, 1, int(0.11 * L * base.experts), shared=1)
    e = make_engine(shape, 1, max_tokens=1)
    try:
        eo.eo_set_bandwidth(e, BP, BH)
        _decode_and_check(e, shape, 1, 4, lambda s: range(L), shape.cache_slots)
    finally:
        eo.eo_destroy(e)


@pytest.mark.timeout(900)
def test_nvfp4_prefill_and_decode_full_layer_shape():
    base = synth.SHAPES["prefill_decode_nvfp4_8L"]
    L = 2
    shape = synth.LayerShape("nvfp4_2L", "prefill+decode", base.hidden, base.experts,
                             base.top_k, base.inter, L, base.fmt, base.tokens, 128, shared=1)
    e = make_engine(shape, 2, max_tokens=base.tokens)
    try:
        eo.eo_set_bandwidth(e, BP, BH)
        _prefill_and_check(e, shape, 2, base.tokens, range(L), 4)
        _decode_and_check(e, shape, 2, 2, lambda s: range(L), 128)
    finally:
        eo.eo_destroy(e)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4", "nvfp4"])
def test_decode_steps_and_prefill_at_an_odd_multiple_of_128(fmt):
    # two layers with H 384, I 192: the separate norm / router / plan kernels
    # (the fused layer entry needs H % 512), the generic GEMV, and a streamed
    # prefill through the plain grouped GEMM; the cache state is replayed by the
    # oracle after every decode step
    shape = synth.LayerShape(f"odd_{fmt}", "prefill+decode", 384, 8, 2, 192, 2,
                             synth.FMT_NAMES[fmt], 96, 6, shared=1)
    e = make_engine(shape, 3, max_tokens=96)
    try:
        eo.eo_set_bandwidth(e, BP, BH)
        _decode_and_check(e, shape, 3, 5, lambda s: range(2), shape.cache_slots)
        _prefill_and_check(e, shape, 3, 96, range(2), 12)
    finally:
        eo.eo_destroy(e)
