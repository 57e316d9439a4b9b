"""bench.py's host-side pieces (CPU only): the per-layer miss-aware bound, the
refusal of more than one GPU, and the sha that ties the committed HBM counters
to the decode GEMV's sources.

The bound of a decode step is the sum over its layer calls of the slowest of
three lanes (zhichai.net article, section 2, Decode paragraph: hits come from
device memory, q* misses over PCIe, the rest from the host cores): HBM reads of
(hits + fills + shared) experts at 8 TB/s, fills at B_P, host experts at B_H.
"""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_miss_aware_bound_hand_worked():
    S = 8_000_000  # bytes per expert: 1 us at 8 TB/s
    bp, bh = 1000, 4000  # MB/s: a fill takes 8 ms, a host expert 2 ms
    log = np.array([[0, 8, 0, 0],    # all hits: 8 us of HBM
                    [1, 6, 1, 1],    # one fill (8 ms) beside one host expert (2 ms)
                    [2, 5, 0, 3]],   # three host experts: 6 ms
                   dtype=np.int32)
    got = bench.miss_aware_bound(log, S, bp, bh, shared=0)
    assert abs(got - (8e-6 + 8e-3 + 6e-3)) < 1e-12
    # a shared expert adds one HBM read per call: only the all-hit call is HBM-bound
    got1 = bench.miss_aware_bound(log, S, bp, bh, shared=1)
    assert abs(got1 - (9e-6 + 8e-3 + 6e-3)) < 1e-12
    assert bench.miss_aware_bound(np.zeros((0, 4), dtype=np.int32), S, bp, bh, 0) is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
    assert r.stdout == ""


def test_gemv_counters_sha_covers_the_gemv_sources():
    # the committed traffic figure applies only to the sources it was taken on
    prof = open(os.path.join(ROOT, "profiles", "hbm_counters_decode_gemv_bf16_48L.md")).read()
    sha = bench.gemv_source_sha256()
    assert len(sha) == 64
    traffic = bench.gemv_traffic()
    if f"source_sha256={sha}" in prof:
        assert traffic[0] is not None and 0.9 < traffic[1] < 1.2
    else:
        assert traffic == (None, None) or traffic[0] is None


def test_prefill_overlap_efficiency_hand_worked():
    # two chunks: 2.0 s of copies and 0.6 s of kernels in all, 1.05 s per chunk:
    # per chunk 1.0 s copy, 0.3 s compute, efficiency 1.0 / 1.05
    st = {"copy_ms": 2000.0, "compute_ms": 600.0, "copy_layers": 96, "compute_layers": 96}
    ov = bench.overlap(st, 1.05, 2)
    assert ov["copy_s"] == 1.0 and ov["compute_s"] == 0.3 and ov["chunk_s"] == 1.05
    assert ov["efficiency"] == round(1.0 / 1.05, 4) and ov["layers_stamped"] == [96, 96]
    # compute the longer of the two: it sets the efficiency
    assert bench.overlap({**st, "compute_ms": 2200.0}, 1.25, 2)["efficiency"] == 0.88
