"""Host-core expert routine (C++, CPU) against the oracle, and its thread pool.

The routine is built from its own sources with g++ into a small driver; no GPU
is involved.
"""
import os
import subprocess

import numpy as np
import pytest

import synth
from oracle import formats as OF
from oracle import moe as OM
from oracle import router as OR

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "expert_offload_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("drv") / "host_driver")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-mavx2", "-mfma", "-pthread",
                           "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "cpp", "host_driver.cpp"),
                           os.path.join(CSRC, "host_ffn.cpp"), os.path.join(CSRC, "layout.cpp"),
                           "-o", out])
    return out


def test_pool_runs_right_after_creation(driver):
    r = subprocess.run([driver, "pool"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr


def _cpu_has_avx512bf16():
    try:
        return "avx512_bf16" in open("/proc/cpuinfo").read()
    except OSError:
        return False


@pytest.mark.parametrize("isa", ["avx2", "native"])
@pytest.mark.parametrize("fmt", ["fp32", "bf16", "mxfp4", "nvfp4", "fp8"])
def test_host_ffn_matches_oracle(driver, tmp_path, fmt, isa):
    # avx2: fp32 route (h kept in fp32), within 1e-5 of the oracle. native: on a
    # CPU with AVX512_BF16, bf16, MXFP4, NVFP4 and FP8 experts take the bf16
    # pair-dot route (fp4 codes looked up as bf16 with block scales on the partial
    # sums, fp8 codes converted through fp16), which rounds h to bf16 as the
    # device does (bound: the layer tolerance, 2e-2)
    pair_route = fmt in ("bf16", "mxfp4", "nvfp4", "fp8")
    if isa == "native" and pair_route and not _cpu_has_avx512bf16():
        pytest.skip("CPU without AVX512_BF16")
    f = synth.FMT_NAMES[fmt]
    H, I, E, k, T = 256, 128, 6, 2, 9
    blocks = [synth.expert_block(2, 0, e, H, I, f) for e in range(E)]
    x = synth.activations(2, 0, T, H, 1.0, f != synth.FMT_FP32)
    xf = synth.bf16_bits_to_f32(x) if f != synth.FMT_FP32 else x
    R = synth.router_weights(2, 0, E, H)
    ids, w, _ = OR.route(xf, R, k)
    d = str(tmp_path)
    open(os.path.join(d, "meta.txt"), "w").write(f"{f} {H} {I} {T} {k} {E} 3\n")
    np.concatenate(blocks).tofile(os.path.join(d, "blocks.bin"))
    xf.astype(np.float32).tofile(os.path.join(d, "x.bin"))
    ids.astype(np.int32).tofile(os.path.join(d, "ids.bin"))
    w.astype(np.float32).tofile(os.path.join(d, "w.bin"))
    env = dict(os.environ, EO_HOST_ISA=isa)
    subprocess.check_call([driver, "ffn", d], timeout=120, env=env)
    y = np.fromfile(os.path.join(d, "y.bin"), dtype=np.float32).reshape(T, H)
    ref = OM.layer_output(xf, ids, w, lambda e: OF.dequant_expert(blocks[e], H, I, f))
    err = np.max(np.abs(y - ref)) / np.max(np.abs(ref))
    bf16_route = isa == "native" and pair_route
    assert err <= (2e-2 if bf16_route else 1e-5), err
    if bf16_route:
        assert err > 1e-7  # the bf16 route did run (h is rounded)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
def test_host_route_weight_decode_is_exact(driver, fmt):
    # the AVX512-BF16 route's decode of every code against the oracle's tables:
    # fp8 codes 0..255 give value / 256 (the dot is rescaled by 256 afterwards),
    # fp4 bytes 0..255 give their two e2m1 values (low nibble first), unscaled;
    # bit-exact, signed zeros included; e4m3fn's NaN codes are never stored
    if not _cpu_has_avx512bf16():
        pytest.skip("CPU without AVX512_BF16")
    f = synth.FMT_NAMES[fmt]
    r = subprocess.run([driver, "decode", str(f)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    bits = np.array([int(v) for v in r.stdout.split()], dtype=np.uint32)
    got = (bits << 16).view(np.float32).astype(np.float64)
    if f == synth.FMT_FP8:
        assert got.size == 256
        want = OF.E4M3 / 256.0
        ok = ~np.isnan(want)
        assert ok.sum() == 254
    else:
        assert got.size == 512
        byte = np.arange(256)
        want = np.stack([OF.E2M1[byte & 0xF], OF.E2M1[byte >> 4]], axis=1).reshape(-1)
        ok = np.ones(512, dtype=bool)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))
