"""Pins for the oracle's expert-block decoding — CPU only.

Code tables are checked exhaustively against the OCP value lists and torch's
float8 conversions; block decoding is checked by exact round trips of
grid-aligned weights through the generator's packer (which pins the layout,
nibble order and gate/up/down order), and on random weights by nearest-grid
brute force.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F


def test_e2m1_table_is_the_ocp_value_set():
    pos = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(F.E2M1[:8]) == pos
    assert list(F.E2M1[8:]) == [-v for v in pos]
    assert np.signbit(F.E2M1[8])


def test_e4m3fn_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(F.E4M3))
    assert np.array_equal(ref[~nan], F.E4M3[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(F.E4M3[~nan]))
    assert F.E4M3[0x7E] == 448.0 and F.E4M3[1] == 2.0 ** -9


def test_e8m0_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ref[255]) and np.isnan(F.E8M0[255])
    assert np.array_equal(ref[:255], F.E8M0[:255])


def test_bf16_decode_matches_torch_rounding():
    rng = np.random.default_rng(0)
    H, I = 64, 32
    w = [rng.standard_normal(s).astype(np.float32) * 0.02 for s in [(I, H), (I, H), (H, I)]]
    blk = synth.pack_expert(*w, synth.FMT_BF16)
    got = F.dequant_expert(blk, H, I, F.BF16)
    for a, b in zip(got, w):
        ref = torch.from_numpy(b).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(a, ref)


def _grid_weights(rng, H, I, fmt):
    """Weights that each format represents exactly."""
    def mx(shape):  # e2m1 grid times 2^j per 32-block, each block holding a 6*2^j
        rows, K = shape
        v = F.E2M1[rng.integers(0, 16, size=shape)]
        j = rng.integers(-12, -2, size=(rows, K // 32))
        v[:, ::32] = 6.0 * np.where(rng.random((rows, K // 32)) < 0.5, 1, -1)
        return (v * np.repeat(2.0 ** j, 32, axis=1)).astype(np.float32)

    def nv(shape, m):  # e2m1 grid times 3.5*2^m, a +-6 in every 16-block
        rows, K = shape
        v = F.E2M1[rng.integers(0, 16, size=shape)]
        v[:, ::16] = 6.0 * np.where(rng.random((rows, K // 16)) < 0.5, 1, -1)
        return (v * 3.5 * 2.0 ** m).astype(np.float32)

    def f8(shape):  # e4m3 grid times 2^j per row, each row holding a 448*2^j
        rows, K = shape
        codes = rng.integers(0, 256, size=shape)
        codes[(codes & 0x7F) == 0x7F] = 0x10  # no NaN
        v = F.E4M3[codes]
        v[:, 0] = 448.0
        j = rng.integers(-14, -6, size=(rows, 1))
        return (v * 2.0 ** j).astype(np.float32)

    shapes = [(I, H), (I, H), (H, I)]
    if fmt == F.MXFP4:
        return [mx(s) for s in shapes]
    if fmt == F.NVFP4:
        return [nv(s, m) for s, m in zip(shapes, (-8, -7, -9))]
    if fmt == F.FP8:
        return [f8(s) for s in shapes]
    return [rng.standard_normal(s).astype(np.float32) for s in shapes]


@pytest.mark.parametrize("fmt", [F.FP32, F.MXFP4, F.NVFP4, F.FP8])
def test_exact_round_trip_on_grid_weights(fmt):
    rng = np.random.default_rng(10 + fmt)
    H, I = 96, 64
    w = _grid_weights(rng, H, I, fmt)
    blk = synth.pack_expert(*w, fmt)
    assert blk.size == F.expert_bytes(H, I, fmt)
    got = F.dequant_expert(blk, H, I, fmt)
    for a, b in zip(got, w):
        assert a.dtype == np.float32 and a.shape == b.shape
        assert np.array_equal(a, b)


def _nearest_ok(v, dq, grid):
    """dq must be a grid point at least as close to v as any other grid point."""
    d_best = np.min(np.abs(v[..., None] - grid), axis=-1)
    return np.all(np.abs(v - dq) <= d_best * (1 + 1e-12) + 1e-30)


def test_mxfp4_random_weights_nearest_grid():
    H, I = 128, 64
    blk, wg, wu, wd = synth.expert_block_with_f32(7, 0, 3, H, I, synth.FMT_MXFP4)
    got = F.dequant_expert(blk, H, I, F.MXFP4)
    for a, b in zip(got, (wg, wu, wd)):
        rows, K = b.shape
        amax = np.abs(b.astype(np.float64)).reshape(rows, K // 32, 32).max(axis=2)
        se = np.floor(np.log2(amax)) - 2
        scale = np.repeat(2.0 ** se, 32, axis=1)
        grid = np.concatenate([F.E2M1[:8], -F.E2M1[1:8]])
        assert _nearest_ok(b / scale, a / scale, grid)


def test_nvfp4_random_weights_error_bound():
    H, I = 128, 64
    blk, wg, wu, wd = synth.expert_block_with_f32(7, 1, 2, H, I, synth.FMT_NVFP4)
    got = F.dequant_expert(blk, H, I, F.NVFP4)
    for a, b in zip(got, (wg, wu, wd)):
        rows, K = b.shape
        blkmax = np.abs(b.astype(np.float64)).reshape(rows, K // 16, 16).max(axis=2)
        # block scale within e4m3 precision of amax/6: error <= half a step (1 at
        # the top of the e2m1 range) of that scale, plus the scale's own rounding
        step = np.repeat(blkmax / 6.0, 16, axis=1)
        assert np.all(np.abs(a - b) <= 1.0 * step * (1 + 2.0 ** -3) + 1e-12)
        rel = np.abs(a - b).max() / np.abs(b).max()
        assert rel < 0.2


def test_fp8_random_weights_error_bound():
    H, I = 64, 32
    blk, wg, wu, wd = synth.expert_block_with_f32(7, 2, 1, H, I, synth.FMT_FP8)
    got = F.dequant_expert(blk, H, I, F.FP8)
    for a, b in zip(got, (wg, wu, wd)):
        s = (np.abs(b.astype(np.float64)).max(axis=1, keepdims=True) / 448.0)
        s = s.astype(np.float32).astype(np.float64)
        # e4m3 normals: half a step is 2^-4 of the value; subnormal step 2^-9
        bound = np.maximum(2.0 ** -4 * np.abs(b), 2.0 ** -10 * s) * (1 + 2.0 ** -20)
        assert np.all(np.abs(a.astype(np.float64) - b) <= bound)
        # the row maximum maps to 448 exactly (up to the fp32 rounding of s)
        rowmax = np.abs(a).max(axis=1).astype(np.float64)
        assert np.allclose(rowmax, np.abs(b).max(axis=1), rtol=2.0 ** -22, atol=0)


# ---- NVFP4 global scale: one rounding after the exact code x block-scale product

def _round_f32(x: "Fraction") -> np.float32:
    """Round a rational to fp32, nearest with ties to even (normal range only)."""
    from fractions import Fraction
    if x == 0:
        return np.float32(0.0)
    sign, a = (-1, -x) if x < 0 else (1, x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert -126 <= e <= 127, "outside the fp32 normal range"
    ulp = Fraction(2) ** (e - 23)
    n, rem = divmod(a, ulp)
    n = int(n)
    if rem > ulp / 2 or (rem == ulp / 2 and n % 2 == 1):
        n += 1
    return np.float32(sign * float(n * ulp))


def _nvfp4_block(c13, c2, s13, s2, g):
    """Pack NVFP4 codes by the documented layout (data | scales | globals),
    even element in the low nibble."""
    def nib(c):
        c = c.reshape(-1, 2).astype(np.uint8)
        return (c[:, 0] | (c[:, 1] << 4)).astype(np.uint8)
    return np.concatenate([nib(c13), nib(c2), s13.ravel().astype(np.uint8),
                           s2.ravel().astype(np.uint8),
                           np.asarray(g, dtype=np.float32).view(np.uint8)])


def test_nvfp4_global_scale_hand_worked():
    # e2m1 code 3 = 1.5, e4m3 code 0x36 = 2^-1 * 1.75 = 0.875: the product is
    # 21/16, exact in fp32. g = fp32(1/3) = 11184811 * 2^-25. Then
    # (21/16) * g = 234881031 * 2^-29 = 0.4375 + 0.4375 ulp (ulp = 2^-25 in
    # [1/4, 1/2)), which rounds down to 0.4375 = 0x3EE00000. The other order,
    # 1.5 * fp32(0.875 * g) = 1.5 * 9786710 * 2^-25 = 14680065 * 2^-25, gives
    # 0x3EE00001: the oracle must produce the first.
    H, I = 16, 16
    c13 = np.zeros((2 * I, H), dtype=np.uint8)
    c2 = np.zeros((H, I), dtype=np.uint8)
    s13 = np.full((2 * I, H // 16), 0x38, dtype=np.uint8)  # 1.0
    s2 = np.full((H, I // 16), 0x38, dtype=np.uint8)
    c13[0, 0] = 3
    s13[0, 0] = 0x36
    c2[5, 7] = 3 | 8     # -1.5
    s2[5, 0] = 0x36
    g = np.array([1 / 3, 1.0, 1 / 3], dtype=np.float32)
    assert g[0].view(np.uint32) == 0x3EAAAAAB
    wg, wu, wd = F.dequant_expert(_nvfp4_block(c13, c2, s13, s2, g), H, I, F.NVFP4)
    assert wg[0, 0].view(np.uint32) == 0x3EE00000
    assert wd[5, 7].view(np.uint32) == 0xBEE00000
    wrong = np.float32(1.5) * (np.float32(0.875) * g[0])
    assert wrong.view(np.uint32) == 0x3EE00001


def test_nvfp4_every_code_and_scale_with_non_power_of_two_globals():
    """Every e2m1 code against every finite e4m3 block scale, under three
    global scales that are not powers of two, against exact rational
    arithmetic rounded once to fp32."""
    from fractions import Fraction
    scales = np.array([s for s in range(256) if (s & 0x7F) != 0x7F], dtype=np.uint8)  # 254
    H = 16 * len(scales)  # one 16-element block per scale code
    I = 16
    codes = np.tile(np.arange(16, dtype=np.uint8), H // 16)  # one of each code per block
    c13 = np.tile(codes, (2 * I, 1))
    s13 = np.tile(scales, (2 * I, 1))
    rng = np.random.default_rng(3)
    c2 = rng.integers(0, 16, size=(H, I)).astype(np.uint8)
    s2 = rng.choice(scales, size=(H, I // 16)).astype(np.uint8)
    g = np.array([1 / 3, 0.1, -2.7], dtype=np.float32)
    wg, wu, wd = F.dequant_expert(_nvfp4_block(c13, c2, s13, s2, g), H, I, F.NVFP4)

    def exact(code, sc, gl):
        s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
        v = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
        se, ee, me = (sc >> 7) & 1, (sc >> 3) & 15, sc & 7
        b = Fraction(me, 8) * Fraction(2) ** -6 if ee == 0 else \
            (1 + Fraction(me, 8)) * Fraction(2) ** (ee - 7)
        sign = (-1) ** (s + se)
        return sign, v * b * Fraction(float(gl))

    differ = 0
    for row, (w, gl) in ((0, (wg, g[0])), (3, (wu, g[1]))):
        for col in range(H):
            sign, x = exact(int(c13[row, col]), int(s13[row, col // 16]), gl)
            ref = _round_f32(sign * x)
            got = w[row, col]
            if x == 0:
                assert got == 0 and np.signbit(got) == (sign * np.sign(float(gl)) < 0)
                continue
            assert got.view(np.uint32) == ref.view(np.uint32), (row, col)
            p = np.float32(F.E2M1[c13[row, col]]) * (np.float32(F.E4M3[s13[row, col // 16]]) * gl)
            differ += int(p.view(np.uint32) != ref.view(np.uint32))
    assert differ > 0  # the multiply order is really exercised
    for r in range(0, H, 97):
        for col in range(I):
            sign, x = exact(int(c2[r, col]), int(s2[r, col // 16]), g[2])
            if x != 0:
                assert wd[r, col].view(np.uint32) == _round_f32(sign * x).view(np.uint32)
