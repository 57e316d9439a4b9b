"""GPU: the expert kernels' own weight decoders, bit for bit against the oracle.

The grouped GEMM and the decode GEMV decode packed weights with gfx950's scaled
converts, not with the scalar decoders of eo_dequant. eo_dequant_with runs each
family's decoders element by element, followed by the factors that family
applies outside the decode (row scale, NVFP4 global scale) in the same order,
and the result must equal oracle.formats.dequant_expert bit for bit.

Each format's block is written by hand so that every element code meets every
scale byte: every 16-element block holds all 16 e2m1 codes and the scale bytes
run through all 256 values; FP8 data bytes run through all 256 codes; bf16 data
through all 65536 patterns. NaN positions must agree (payloads may differ).
No byte is excluded: e8m0 0x00 (2^-127, a subnormal scale), 0xFF (NaN) and the
scales at which 6 * 2^(e-127) overflows fp32 to infinity decode as the oracle
does.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expert_offload_amd as eo  # noqa: E402
import synth  # noqa: E402
from oracle import formats as OF  # noqa: E402
from synth.workload import make_engine  # noqa: E402

pytestmark = pytest.mark.gpu

H, I = 512, 256


def _codes_fp4(rows, K):
    r = np.arange(rows)[:, None]
    c = np.arange(K)[None, :]
    return ((c + r) % 16).astype(np.uint8)  # all 16 codes in every 16-block


def _pack_nibbles(c):
    c = c.reshape(-1, 2)
    return (c[:, 0] | (c[:, 1] << 4)).astype(np.uint8)


def _scales(rows, nblk, offset):
    return ((np.arange(rows * nblk) + offset) % 256).astype(np.uint8).reshape(rows, nblk)


def _block(fmt):
    rng = np.random.default_rng(7 + fmt)
    if fmt == OF.BF16:
        return (np.arange(3 * H * I) % 65536).astype(np.uint16).view(np.uint8)
    if fmt == OF.FP8:
        d13 = (np.arange(2 * I * H) % 256).astype(np.uint8)
        d2 = ((np.arange(H * I) * 7 + 3) % 256).astype(np.uint8)
        r13 = (rng.standard_normal(2 * I) * 0.01).astype(np.float32)
        r2 = (rng.standard_normal(H) * 0.01).astype(np.float32)
        return np.concatenate([d13, d2, r13.view(np.uint8), r2.view(np.uint8)])
    c13 = _pack_nibbles(_codes_fp4(2 * I, H))
    c2 = _pack_nibbles(_codes_fp4(H, I))
    if fmt == OF.MXFP4:
        return np.concatenate([c13, c2, _scales(2 * I, H // 32, 0).ravel(),
                               _scales(H, I // 32, 77).ravel()])
    g = np.array([1 / 3, 0.1, -2.7], dtype=np.float32)
    return np.concatenate([c13, c2, _scales(2 * I, H // 16, 0).ravel(),
                           _scales(H, I // 16, 131).ravel(), g.view(np.uint8)])


def _write(e, blk):
    ptr, n = eo.eo_pool_expert(e, 0, 0)
    assert n == blk.size
    ctypes.memmove(ptr, blk.ctypes.data, n)


def _scale_index(fmt, n13):
    """Per element, the scale byte it is decoded with (fp4 formats)."""
    bs = 32 if fmt == OF.MXFP4 else 16
    s13 = np.repeat(np.arange(2 * I * H // bs), bs)
    s2 = np.repeat(np.arange(H * I // bs), bs) + 2 * I * H // bs
    return np.concatenate([s13, s2])


FMTS = {"bf16": OF.BF16, "fp8": OF.FP8, "mxfp4": OF.MXFP4, "nvfp4": OF.NVFP4}


@pytest.mark.parametrize("fmt_name", list(FMTS))
def test_kernel_decoders_bit_exact(fmt_name):
    fmt = FMTS[fmt_name]
    shape = synth.LayerShape(f"dec_{fmt_name}", "test", H, 4, 2, I, 1, fmt, 1, 0, shared=0)
    e = make_engine(shape, 0, fill_pool=False)
    try:
        blk = _block(fmt)
        _write(e, blk)
        with np.errstate(over="ignore"):  # MXFP4 scales near 2^127 overflow to inf
            ref = np.concatenate([a.ravel() for a in OF.dequant_expert(blk, H, I, fmt)])
        ref_bits = ref.view(np.uint32)
        ref_nan = np.isnan(ref)
        sbytes = None
        if fmt in (OF.MXFP4, OF.NVFP4):
            n_data = 3 * H * I // 2
            sbytes = blk[n_data:n_data + 3 * H * I // (32 if fmt == OF.MXFP4 else 16)]
            sbytes = sbytes[_scale_index(fmt, 2 * I * H)]
        for dec in (eo.EO_DECODER_SCALAR, eo.EO_DECODER_GEMM, eo.EO_DECODER_GEMV):
            out = np.zeros(3 * H * I, dtype=np.float32)
            eo.eo_dequant_with(e, 0, 0, dec, out)
            nan = np.isnan(out)
            bad = (nan != ref_nan) | (~ref_nan & (out.view(np.uint32) != ref_bits))
            if bad.any():
                where = np.flatnonzero(bad)
                msg = f"{fmt_name} decoder {dec}: {where.size} elements differ"
                if sbytes is not None:
                    msg += f"; scale bytes {sorted(set(int(b) for b in sbytes[where]))[:40]}"
                i0 = where[0]
                msg += f"; first at {i0}: got {out[i0]!r} ({out.view(np.uint32)[i0]:#x}) " \
                       f"want {ref[i0]!r} ({ref_bits[i0]:#x})"
                raise AssertionError(msg)
    finally:
        eo.eo_destroy(e)
