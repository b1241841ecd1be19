"""Pins for the oracle's argmax (the LM head's greedy pick; emit_qwen38_generate,
"Where the speed comes from", item 2; GPU Kernel Lab, "Decode integration"):
the lowest index among IEEE-equal maxima, so -0.0 ties +0.0."""
import itertools

import numpy as np

import oracle


def _textbook(v):
    # stable sort on the negated values (IEEE comparisons, so -0 == +0):
    # the first element is the maximum with the lowest index
    order = np.argsort(-np.asarray(v, dtype=np.float64), kind="stable")
    return int(order[0])


def test_exhaustive_small_vectors():
    vals = [-1.0, -0.0, 0.0, 1.0, 2.0]
    for n in range(1, 6):
        for t in itertools.product(vals, repeat=n):
            v = np.array(t, np.float64)
            assert oracle.argmax_f64(v) == _textbook(v), t
            assert oracle.argmax_f32(v.astype(np.float32)) == _textbook(v), t


def test_ties_and_near_ties():
    n = 151936
    rng = np.random.default_rng(0)
    v = rng.standard_normal(n).astype(np.float32)
    top = np.float32(8.0)
    v[1000] = top
    v[500] = np.nextafter(top, np.float32(0))   # one ulp below: loses
    v[2000] = top                                # exact tie: 1000 wins
    assert oracle.argmax_f32(v) == 1000
    v[3000] = np.nextafter(top, np.float32(np.inf))  # one ulp above: wins despite index
    assert oracle.argmax_f32(v) == 3000
    assert oracle.argmax_f64(v.astype(np.float64)) == 3000


def test_signed_zero_and_edges():
    v = np.array([-1.0, -0.0, 0.0, -2.0], np.float32)
    assert oracle.argmax_f32(v) == 1
    v = np.array([0.0, -0.0], np.float32)
    assert oracle.argmax_f32(v) == 0
    v = np.full(1000, 3.5, np.float32)
    assert oracle.argmax_f32(v) == 0
    v = np.arange(1000, dtype=np.float32)
    assert oracle.argmax_f32(v) == 999
    v = -np.arange(1000, dtype=np.float32)
    assert oracle.argmax_f32(v) == 0
    v = np.full(7, -np.inf, np.float32)
    v[4] = -1e30
    assert oracle.argmax_f32(v) == 4


def test_nan_and_empty_are_rejected():
    assert oracle.argmax_f32(np.array([1.0, np.nan], np.float32)) == -1
    assert oracle.argmax_f32(np.array([], np.float32)) == -1
