"""Pins for oracle.merge: hand-worked example, brute-force delta, finite differences."""
import json
import os

import numpy as np

from oracle import merge

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLD, "merge_tiny.json")))
    e = g["expected"]
    W0, A, B, dW = (np.array(g[k], float) for k in ("W0", "A", "B", "dW"))
    s = g["s"]
    np.testing.assert_array_equal(merge.merge_forward(W0, A, B, s), np.array(e["W"]))
    np.testing.assert_array_equal(merge.merge_forward(None, A, B, s), np.array(e["delta"]))
    b = merge.merge_backward(dW, A, B, s)
    np.testing.assert_array_equal(b["dA"], np.array(e["dA"]))
    np.testing.assert_array_equal(b["dB"], np.array(e["dB"]))


def test_delta_brute_force():
    A, B, s = _rand(1, 3, 5), _rand(2, 4, 3), 0.7
    d = merge.merge_forward(None, A, B, s)
    for n in range(4):
        for k in range(5):
            assert abs(d[n, k] - s * sum(B[n, j] * A[j, k] for j in range(3))) < 1e-12


def test_finite_differences():
    W0, A, B, dW, s = _rand(3, 4, 5), _rand(4, 2, 5), _rand(5, 4, 2), _rand(6, 4, 5), 1.3
    g = merge.merge_backward(dW, A, B, s)

    def loss(A_, B_):
        return float(np.sum(dW * merge.merge_forward(W0, A_, B_, s)))

    h = 1e-6
    for name, arr, pos in (("dA", A, 0), ("dB", B, 1)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = [A.copy(), B.copy()]
            q = [A.copy(), B.copy()]
            p[pos][idx] += h
            q[pos][idx] -= h
            fd[idx] = (loss(*p) - loss(*q)) / (2 * h)
        np.testing.assert_allclose(g[name], fd, rtol=1e-7, atol=1e-8)
