"""Pins for the oracle's router (logits order, top-k, weights) — CPU only."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import router

U = 2.0 ** -24  # unit roundoff of fp32


def test_logits_exact_on_small_integers():
    # every product and partial sum is an integer below 2^24, so any order is
    # exact and z must equal the integer dot product: pins indexing and terms
    rng = np.random.default_rng(1)
    T, E, H = 5, 7, 512
    x = rng.integers(-8, 9, size=(T, H))
    R = rng.integers(-8, 9, size=(E, H))
    z = router.logits(x.astype(np.float32), R.astype(np.float32))
    assert np.array_equal(z.astype(np.int64), x @ R.T)


def test_logits_order_hand_worked():
    # H = 128: chain i holds terms h = i and h = i + 64.
    # chain 0: 2^24 then +1 -> tie, rounds to even 2^24; chain 1: 1 + 1 = 2.
    # butterfly: p0 stays 2^24 until s = 1, where p0 + p1 = 2^24 + 2 (exact).
    # A left-to-right sum gives 2^24, the correctly rounded sum 2^24 + 4.
    H = 128
    x = np.ones((1, H), dtype=np.float32)
    R = np.zeros((1, H), dtype=np.float32)
    R[0, 0] = 2.0 ** 24
    R[0, 64] = 1.0
    R[0, 1] = 1.0
    R[0, 65] = 1.0
    z = router.logits(x, R)
    assert z[0, 0] == np.float32(2.0 ** 24 + 2)


def test_logits_use_fused_multiply_add():
    # chain 0: acc = 1 * -1 = -1, then fma(1+2^-12, 1+2^-12, -1) = 2^-11 + 2^-24
    # exactly; a separate multiply would round the product to 1 + 2^-11 first.
    H = 128
    x = np.zeros((1, H), dtype=np.float32)
    R = np.zeros((1, H), dtype=np.float32)
    x[0, 0], R[0, 0] = 1.0, -1.0
    a = np.float32(1.0 + 2.0 ** -12)
    x[0, 64], R[0, 64] = a, a
    z = router.logits(x, R)
    assert z[0, 0] == np.float32(2.0 ** -11 + 2.0 ** -24)


@pytest.mark.parametrize("H", [256, 2048])
def test_logits_error_bound(H):
    # recursive-summation bound: depth n = H/64 fused steps + 6 butterfly adds
    rng = np.random.default_rng(H)
    T, E = 8, 16
    x = rng.standard_normal((T, H)).astype(np.float32)
    R = (0.02 * rng.standard_normal((E, H))).astype(np.float32)
    z = router.logits(x, R).astype(np.float64)
    exact = x.astype(np.float64) @ R.astype(np.float64).T
    mag = np.abs(x.astype(np.float64)) @ np.abs(R.astype(np.float64)).T
    n = H // 64 + 6
    gamma = n * U / (1 - n * U)
    assert np.all(np.abs(z - exact) <= gamma * mag)
    assert np.any(z != exact.astype(np.float32))  # rounding does happen


def test_topk_matches_full_sort_with_ties():
    rng = np.random.default_rng(3)
    T, E, k = 40, 16, 4
    z = rng.integers(-3, 4, size=(T, E)).astype(np.float32)  # many ties
    ids = router.topk(z, k)
    for t in range(T):
        order = np.lexsort((np.arange(E), -z[t].astype(np.float64)))
        assert list(ids[t]) == list(order[:k])
    # signed zeros compare equal: the lower id wins
    z0 = np.zeros((1, 4), dtype=np.float32)
    z0[0, 0] = -0.0
    assert list(router.topk(z0, 2)[0]) == [0, 1]


def test_weights_sum_to_one_and_match_full_softmax():
    rng = np.random.default_rng(4)
    T, E, k = 20, 16, 2
    z = rng.standard_normal((T, E)).astype(np.float32)
    ids = router.topk(z, k)
    w = router.weights(z, ids)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)  # ids listed by logit descending
    full = softmax(z.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-14, atol=0)


def test_forced_ids_keep_trace_order():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 128)).astype(np.float32)
    R = rng.standard_normal((8, 128)).astype(np.float32)
    forced = np.array([[5, 1, 7]], dtype=np.int32)
    ids, w, z = router.route(x, R, 3, forced)
    assert list(ids[0]) == [5, 1, 7]
    ref = softmax(z[0, [5, 1, 7]].astype(np.float64))
    assert np.allclose(w[0], ref, rtol=1e-14, atol=0)
