"""The C-ABI library loads and exports every entry point include/eo.h declares (no GPU calls)."""
import ctypes
import os
import re

import expert_offload_amd as eo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "eo.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(eo_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(eo.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(eo.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name


def test_pure_calls_without_device():
    # calls that touch no device: sizes, argument checks, error text
    assert eo.eo_expert_bytes(2048, 768, eo.EO_W_BF16) == 9437184
    assert eo.eo_expert_bytes(4096, 2048, eo.EO_W_MXFP4) == 13369344
    assert eo.eo_expert_bytes(6144, 2048, eo.EO_W_NVFP4) == 21233676
    assert eo.eo_expert_bytes(256, 128, eo.EO_W_FP32) == 393216
    assert eo.eo_expert_bytes(0, 128, eo.EO_W_FP32) == 0
    cfg = eo.eo_config(1, 2000, 2, 256, 128, 0, 0, 0, 8, 64, 1, 0)  # too many experts
    out = ctypes.c_void_p()
    st = eo.lib().eo_create(ctypes.byref(cfg), ctypes.byref(out))
    assert st == eo.EO_ERR_INVALID_ARG and "experts" in eo.eo_last_error()
    assert eo.lib().eo_sync(None) == eo.EO_ERR_INVALID_ARG
