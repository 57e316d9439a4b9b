"""ORACLE (test infrastructure only) — prefill streaming timing model.

zhichai.net article, section 2, Prefill paragraph: experts are streamed at the
granularity of a whole layer with double buffering — while the GPU computes
layer l, layer l+1's experts cross PCIe — so a prefill chunk takes about the
time to stream the expert pool once, with the expert compute hidden.

Model: copy c_l seconds and compute k_l seconds per layer, two staging buffers.
Copy l+1 may start once copy l is done and buffer (l+1) mod 2 has been released
by compute l-1; compute l starts once copy l and compute l-1 are done. With one
buffer, copy l+1 waits for compute l. Returns the chunk's end time.
"""
from __future__ import annotations


def chunk_time(copy_s, compute_s, buffers: int = 2) -> float:
    L = len(copy_s)
    assert len(compute_s) == L and buffers in (1, 2)
    copy_end = [0.0] * L
    comp_end = [0.0] * L
    copy_start = 0.0
    for l in range(L):
        copy_end[l] = copy_start + copy_s[l]
        comp_start = max(copy_end[l], comp_end[l - 1] if l else 0.0)
        comp_end[l] = comp_start + compute_s[l]
        if buffers == 2:
            copy_start = max(copy_end[l], comp_end[l - 1] if l else 0.0)
        else:
            copy_start = comp_end[l]
    return comp_end[-1] if L else 0.0
