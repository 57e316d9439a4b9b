"""Pins for the prefill streaming timing model — CPU only."""
import json
import os

from oracle.streaming import chunk_time


def test_page_chunk_time(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "prefill_chunk_pages.json")))
    L = 48
    copy = [g["pool_GB"] / g["B_P_GBps"] / L] * L
    comp = [0.002] * L  # compute well below copy: hidden except the last layer
    t = chunk_time(copy, comp)
    lo, hi = g["chunk_seconds_printed"]
    assert abs(t - (sum(copy) + comp[-1])) < 1e-12
    assert lo - 0.01 <= sum(copy) <= hi + 0.01  # 64.4 / 52.7 = 1.222 s


def test_compute_bound_and_single_buffer():
    copy, comp = [1.0] * 5, [3.0] * 5
    assert chunk_time(copy, comp) == 1.0 + 15.0
    # one buffer serialises copy and compute
    assert chunk_time(copy, comp, buffers=1) == 20.0
    assert chunk_time([2.0] * 8, [1.0] * 8, buffers=1) > chunk_time([2.0] * 8, [1.0] * 8)


def test_double_buffer_gain_grows_with_compute_share():
    # the page's ablation: turning double buffering off costs more as the
    # hideable compute share grows (4k < 8k < 16k tokens)
    copy = [1.0] * 16
    losses = []
    for c in (0.2, 0.4, 0.8):
        comp = [c] * 16
        losses.append(1 - chunk_time(copy, comp) / chunk_time(copy, comp, buffers=1))
    assert losses[0] < losses[1] < losses[2]
