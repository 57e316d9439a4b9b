"""Host code and the oracle's C under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

The host-side C++ of the library (the host-core expert routine, its thread
pool, the expert-block layout and the router's chain-interleaved layout) is
built from its own sources with g++ -fsanitize=address,undefined into the test
driver and run across hidden sizes that are and are not multiples of the
layouts' block sizes: H in {256, 384, 512, 2048, 6144}, every weight format,
both instruction routes. Any out-of-bounds access, use after free or
undefined behaviour aborts the driver. The router layout at H = 384 is the
shape whose index arithmetic once overran its buffer: it must be refused with
the output untouched. The oracle's fixed-order router logits (its only C code)
run under the same sanitizers at hidden sizes around the 64 chains, against
exact integer dot products.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth
from oracle import formats as OF
from oracle import moe as OM
from oracle import router as OR

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "expert_offload_amd", "csrc")
HS = [256, 384, 512, 2048, 6144]
SAN_ENV = {"ASAN_OPTIONS": "halt_on_error=1:abort_on_error=1:detect_leaks=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


@pytest.fixture(scope="module")
def san_driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("san") / "host_driver_san")
    subprocess.check_call(["g++", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-mavx2", "-mfma", "-pthread", "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "cpp", "host_driver.cpp"),
                           os.path.join(CSRC, "host_ffn.cpp"), os.path.join(CSRC, "layout.cpp"),
                           "-o", out])
    return out


def _run(driver, args, extra_env=None):
    env = dict(os.environ, **SAN_ENV, **(extra_env or {}))
    return subprocess.run([driver, *args], capture_output=True, text=True, timeout=300, env=env)


def test_thread_pool_under_sanitizers(san_driver):
    r = _run(san_driver, ["pool"])
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr[-3000:]


@pytest.mark.parametrize("E", [1, 3, 16])
@pytest.mark.parametrize("H", HS)
def test_router_chain_layout_under_sanitizers(san_driver, E, H):
    r = _run(san_driver, ["chains", str(E), str(H)])
    want = "refused" if H % 256 else "ok"
    assert r.returncode == 0 and r.stdout.strip() == want, r.stdout + r.stderr[-3000:]


def _cpu_has_avx512bf16():
    try:
        return "avx512_bf16" in open("/proc/cpuinfo").read()
    except OSError:
        return False


@pytest.mark.parametrize("isa", ["avx2", "native"])
@pytest.mark.parametrize("fmt", ["fp32", "bf16", "mxfp4", "nvfp4", "fp8"])
@pytest.mark.parametrize("H", HS)
def test_host_ffn_under_sanitizers(san_driver, tmp_path, H, fmt, isa):
    pair_route = fmt in ("bf16", "mxfp4", "nvfp4", "fp8")
    if isa == "native" and pair_route and not _cpu_has_avx512bf16():
        pytest.skip("CPU without AVX512_BF16")
    f = synth.FMT_NAMES[fmt]
    I, E, k, T = 192 if H == 384 else 256, 3, 2, 3
    blocks = [synth.expert_block(5, 0, e, H, I, f) for e in range(E)]
    x = synth.activations(5, H, T, H, 1.0, f != synth.FMT_FP32)
    xf = synth.bf16_bits_to_f32(x) if f != synth.FMT_FP32 else x
    ids, w, _ = OR.route(xf, synth.router_weights(5, 0, E, H), k)
    d = str(tmp_path)
    open(os.path.join(d, "meta.txt"), "w").write(f"{f} {H} {I} {T} {k} {E} 3\n")
    np.concatenate(blocks).tofile(os.path.join(d, "blocks.bin"))
    xf.astype(np.float32).tofile(os.path.join(d, "x.bin"))
    ids.astype(np.int32).tofile(os.path.join(d, "ids.bin"))
    w.astype(np.float32).tofile(os.path.join(d, "w.bin"))
    r = _run(san_driver, ["ffn", d], {"EO_HOST_ISA": isa})
    assert r.returncode == 0, r.stderr[-3000:]
    y = np.fromfile(os.path.join(d, "y.bin"), dtype=np.float32).reshape(T, H)
    ref = OM.layer_output(xf, ids, w, lambda e: OF.dequant_expert(blocks[e], H, I, f))
    err = np.max(np.abs(y - ref)) / np.max(np.abs(ref))
    assert err <= (2e-2 if (isa == "native" and pair_route) else 1e-5), err


@pytest.fixture(scope="module")
def corder_driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("san") / "corder_driver_san")
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           os.path.join(ROOT, "tests", "cpp", "corder_driver.c"),
                           os.path.join(ROOT, "oracle", "corder.c"), "-lm", "-o", out])
    return out


@pytest.mark.parametrize("T,E,H", [(1, 1, 1), (2, 3, 63), (1, 5, 64), (3, 2, 65), (2, 7, 130),
                                   (1, 128, 2048), (2, 16, 6144)])
def test_oracle_router_logits_under_sanitizers(corder_driver, T, E, H):
    r = _run(corder_driver, [str(T), str(E), str(H)])
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr[-3000:]
