"""ORACLE (test infrastructure only) — expert-block decoding to fp32.

The juejin.cn overview (section 5) lists MXFP4, NVFP4, FP8 and BF16 as the
supported precisions, and the zhichai.net article (section 5) notes that one
model ships natively in MXFP4 and another as an NVFP4 checkpoint. The pages do
not give layouts, so the following readings are used:

* element codes, from their bit fields (OCP MX v1.0 / OCP FP8):
  e2m1: sign, 2 exponent bits (bias 1), 1 mantissa bit; values 0, 0.5, 1, 1.5,
  2, 3, 4, 6 and their negatives. e4m3fn: sign, 4 exponent bits (bias 7),
  3 mantissa bits, subnormals, no infinities, S.1111.111 is NaN. e8m0: 2^(c-127),
  0xFF is NaN.
* MXFP4: v = e2m1 * 2^(e8m0 - 127), one scale per 32 consecutive elements of a
  row (the contraction axis).
* NVFP4: v = (e2m1 * e4m3) * g: the first product is exact in fp32, the multiply
  by the tensor's fp32 global scale g rounds once. One e4m3 scale per 16
  elements; one g each for gate, up and down.
* FP8: v = e4m3fn * s_row, one fp32 scale per output row, one rounding.
* BF16 widens exactly; FP32 is taken as stored.
* Block layout: W13 = [W_gate; W_up] (2I rows of H), then W2 = W_down (H rows of
  I); data sections first, then scales, then (NVFP4) the three global scales.
  The even element of a pair sits in the low nibble.
"""
from __future__ import annotations

import math

import numpy as np

FP32, BF16, MXFP4, NVFP4, FP8 = 0, 1, 2, 3, 4


def _e2m1(code: int) -> float:
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else math.ldexp(1.0 + m / 2.0, e - 1)
    return -mag if s else mag


def _e4m3fn(code: int) -> float:
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    mag = math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7)
    return -mag if s else mag


def _e8m0(code: int) -> float:
    return math.nan if code == 0xFF else math.ldexp(1.0, code - 127)


E2M1 = np.array([_e2m1(c) for c in range(16)], dtype=np.float64)
E4M3 = np.array([_e4m3fn(c) for c in range(256)], dtype=np.float64)
E8M0 = np.array([_e8m0(c) for c in range(256)], dtype=np.float64)


def expert_bytes(H: int, I: int, fmt: int) -> int:
    n = 3 * H * I  # elements of gate + up + down
    if fmt == FP32:
        return 4 * n
    if fmt == BF16:
        return 2 * n
    if fmt == MXFP4:
        return n // 2 + n // 32
    if fmt == NVFP4:
        return n // 2 + n // 16 + 12
    if fmt == FP8:
        return n + 4 * (2 * I + H)
    raise ValueError(fmt)


def _nibbles(b: np.ndarray, rows: int, K: int) -> np.ndarray:
    b = b.reshape(rows, K // 2)
    out = np.empty((rows, K), dtype=np.uint8)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


def dequant_expert(block: np.ndarray, H: int, I: int, fmt: int):
    """(W_gate [I,H], W_up [I,H], W_down [H,I]) as fp32 from one packed block."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    n13, n2 = 2 * I * H, H * I
    if fmt == FP32:
        w = b[:4 * (n13 + n2)].view(np.float32)
        w13, w2 = w[:n13].reshape(2 * I, H), w[n13:].reshape(H, I)
    elif fmt == BF16:
        u = b[:2 * (n13 + n2)].view(np.uint16).astype(np.uint32) << 16
        w = u.view(np.float32)
        w13, w2 = w[:n13].reshape(2 * I, H), w[n13:].reshape(H, I)
    elif fmt == MXFP4:
        d13, d2 = 0, n13 // 2
        s13 = d2 + n2 // 2
        s2 = s13 + n13 // 32
        c13 = _nibbles(b[d13:d2], 2 * I, H)
        c2 = _nibbles(b[d2:s13], H, I)
        sc13 = b[s13:s2].reshape(2 * I, H // 32)
        sc2 = b[s2:s2 + n2 // 32].reshape(H, I // 32)
        w13 = (E2M1[c13] * np.repeat(E8M0[sc13], 32, axis=1)).astype(np.float32)
        w2 = (E2M1[c2] * np.repeat(E8M0[sc2], 32, axis=1)).astype(np.float32)
    elif fmt == NVFP4:
        d13, d2 = 0, n13 // 2
        s13 = d2 + n2 // 2
        s2 = s13 + n13 // 16
        gl = s2 + n2 // 16
        c13 = _nibbles(b[d13:d2], 2 * I, H)
        c2 = _nibbles(b[d2:s13], H, I)
        sc13 = b[s13:s2].reshape(2 * I, H // 16)
        sc2 = b[s2:gl].reshape(H, I // 16)
        g = b[gl:gl + 12].view(np.float32)
        # e2m1 * e4m3 is exact in fp32 (at most 6 significant bits)
        p13 = (E2M1[c13] * np.repeat(E4M3[sc13], 16, axis=1)).astype(np.float32)
        p2 = (E2M1[c2] * np.repeat(E4M3[sc2], 16, axis=1)).astype(np.float32)
        w13 = np.empty_like(p13)
        w13[:I] = p13[:I] * g[0]  # fp32 multiply, one rounding
        w13[I:] = p13[I:] * g[1]
        w2 = p2 * g[2]
    elif fmt == FP8:
        d2 = n13
        s13 = d2 + n2
        s2 = s13 + 4 * 2 * I
        v13 = E4M3[b[:n13].reshape(2 * I, H)].astype(np.float32)
        v2 = E4M3[b[d2:s13].reshape(H, I)].astype(np.float32)
        r13 = b[s13:s2].view(np.float32)
        r2 = b[s2:s2 + 4 * H].view(np.float32)
        w13 = v13 * r13[:, None]
        w2 = v2 * r2[:, None]
    else:
        raise ValueError(fmt)
    return (np.ascontiguousarray(w13[:I]), np.ascontiguousarray(w13[I:]),
            np.ascontiguousarray(w2))
