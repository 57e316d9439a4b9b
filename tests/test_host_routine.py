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


@pytest.mark.parametrize("fmt", ["fp32", "bf16", "mxfp4", "nvfp4", "fp8"])
def test_host_ffn_matches_oracle(driver, tmp_path, fmt):
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
    subprocess.check_call([driver, "ffn", d], timeout=120)
    y = np.fromfile(os.path.join(d, "y.bin"), dtype=np.float32).reshape(T, H)
    ref = OM.layer_output(xf, ids, w, lambda e: OF.dequant_expert(blocks[e], H, I, f))
    err = np.max(np.abs(y - ref)) / np.max(np.abs(ref))
    assert err <= 1e-5, err
