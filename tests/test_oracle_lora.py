"""Pins for oracle.lora against facts that do not come from the oracle itself.

Each test states what fixes the expected value: a hand-worked example, a
brute-force loop over the definition, a special case that reduces to a plain
library product, a finite difference, or an algebraic identity of the layer.
"""
import json
import os

import numpy as np
import pytest

from oracle import lora

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _tiny(seed=0, M=5, N=4, K=6, r=3):
    return _rand(seed, M, K), _rand(seed + 1, N, K), _rand(seed + 2, r, K), _rand(seed + 3, N, r)


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLD, "lora_tiny.json")))
    X, W0, A, B = (np.array(g[k], float) for k in ("X", "W0", "A", "B"))
    bias, dY, s = np.array(g["bias"], float), np.array(g["dY"], float), g["s"]
    e = g["expected"]
    np.testing.assert_array_equal(lora.lora_forward(X, W0, A, B, s, bias), e["Y"])
    gr = lora.lora_backward(dY, X, W0, A, B, s)
    for k in ("dX", "dA", "dB", "db"):
        np.testing.assert_allclose(gr[k], np.array(e[k], float), rtol=0, atol=1e-15)


def test_brute_force_loops():
    X, W0, A, B = _tiny(1, M=3, N=4, K=5, r=2)
    s = 0.7
    Y = lora.lora_forward(X, W0, A, B, s)
    M, K = X.shape
    N, r = B.shape
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                w = W0[n, k]
                for j in range(r):
                    w += s * B[n, j] * A[j, k]
                acc += X[m, k] * w
            assert abs(Y[m, n] - acc) < 1e-12


@pytest.mark.parametrize("which", ["s0", "B0"])
def test_zero_delta_is_base_product(which):
    X, W0, A, B = _tiny(2)
    s = 0.0 if which == "s0" else 1.3
    if which == "B0":
        B = np.zeros_like(B)
    # With no delta the adapted weight is W0 itself, so the result is the plain product bit for bit.
    np.testing.assert_array_equal(lora.lora_forward(X, W0, A, B, s), np.matmul(X, W0.T))
    gr = lora.lora_backward(_rand(9, X.shape[0], W0.shape[0]), X, W0, A, B, s)
    if which == "s0":
        assert not gr["dA"].any() and not gr["dB"].any()
    else:
        assert not gr["dA"].any()  # dA = s.B^T.G vanishes with B = 0


def test_zero_base_is_pure_low_rank():
    X, W0, A, B = _tiny(3)
    s = 1.7
    Y = lora.lora_forward(X, np.zeros_like(W0), A, B, s)
    # Other association order: (X.A^T).B^T, never forming B.A.
    np.testing.assert_allclose(Y, s * ((X @ A.T) @ B.T), rtol=1e-13, atol=1e-13)


def test_affine_in_s():
    X, W0, A, B = _tiny(4)
    y0 = lora.lora_forward(X, W0, A, B, 0.0)
    y1 = lora.lora_forward(X, W0, A, B, 0.8)
    y2 = lora.lora_forward(X, W0, A, B, 1.6)
    np.testing.assert_allclose(y2 - 2 * y1 + y0, 0.0, atol=1e-12)


def test_finite_differences():
    X, W0, A, B = _tiny(5)
    s = 0.9
    bias = _rand(11, W0.shape[0])
    dY = _rand(12, X.shape[0], W0.shape[0])
    gr = lora.lora_backward(dY, X, W0, A, B, s)

    def loss(X_, A_, B_, b_):
        return float(np.sum(dY * lora.lora_forward(X_, W0, A_, B_, s, b_)))

    h = 1e-6
    for name, arr in (("dX", X), ("dA", A), ("dB", B), ("db", bias)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy(); p[idx] += h
            q = arr.copy(); q[idx] -= h
            args = {"dX": (p, A, B, bias), "dA": (X, p, B, bias), "dB": (X, A, p, bias), "db": (X, A, B, p)}[name]
            argsq = {"dX": (q, A, B, bias), "dA": (X, q, B, bias), "dB": (X, A, q, bias), "db": (X, A, B, q)}[name]
            fd[idx] = (loss(*args) - loss(*argsq)) / (2 * h)
        np.testing.assert_allclose(gr[name], fd, rtol=1e-7, atol=1e-7)


def test_gauge_and_euler_identities():
    X, W0, A, B = _tiny(6, M=7, N=5, K=9, r=4)
    s, bias = 1.1, _rand(21, 5)
    dY = _rand(22, 7, 5)
    Y = lora.lora_forward(X, W0, A, B, s, bias)
    gr = lora.lora_backward(dY, X, W0, A, B, s)
    # Y depends on (A, B) only through B.A, so the rescaling A -> (1+t)A, B -> B/(1+t) is a symmetry.
    assert abs(np.sum(gr["dA"] * A) - np.sum(gr["dB"] * B)) < 1e-12
    # <dB, B> = <dY, Y - X.W0^T - b>  (Y - base is linear in B).
    assert abs(np.sum(gr["dB"] * B) - np.sum(dY * (Y - X @ W0.T - bias))) < 1e-12
    # Y - b is linear in X.
    assert abs(np.sum(gr["dX"] * X) - np.sum(dY * (Y - bias))) < 1e-12


def test_sampled_weight_grads_match_full():
    X, W0, A, B = _tiny(7, M=8, N=6, K=10, r=3)
    dY = _rand(31, 8, 6)
    full = lora.lora_backward(dY, X, W0, A, B, 0.6)
    smp = lora.lora_weight_grads_sampled(dY, X, A, B, 0.6, [0, 4, 5], [1, 7])
    np.testing.assert_allclose(smp["dB_rows"], full["dB"][[0, 4, 5]], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(smp["dA_cols"], full["dA"][:, [1, 7]], rtol=1e-13, atol=1e-13)


def test_planted_mistake_is_caught():
    """A transposed factor (the classic slip) must fail the brute-force pin."""
    X, W0, A, B = _tiny(8, M=2, N=3, K=3, r=3)
    wrong = X @ (W0 + 0.5 * (A.T @ B.T)).T     # dW = (B.A)^T instead of B.A
    right = lora.lora_forward(X, W0, A, B, 0.5)
    assert np.max(np.abs(wrong - right)) > 1e-3
