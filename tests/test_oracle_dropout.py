"""Pins for oracle.dropout: reductions to the plain layers, and finite differences through the mask."""
import numpy as np

from oracle import dora, dropout, lora


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _case():
    X, W0, A, B, dY = _rand(1, 4, 7), _rand(2, 5, 7), _rand(3, 2, 7), _rand(4, 5, 2), _rand(5, 4, 5)
    m = np.abs(_rand(6, 5)) + 0.5
    keep = np.array([1, 0, 1, 1, 0, 1, 1])
    return X, W0, A, B, dY, m, keep


def test_reductions():
    X, W0, A, B, dY, m, keep = _case()
    ones, zeros = np.ones(7), np.zeros(7)
    np.testing.assert_array_equal(dropout.lora_forward(X, W0, A, B, 0.7, ones, 0.0), lora.lora_forward(X, W0, A, B, 0.7))
    np.testing.assert_allclose(dropout.lora_forward(X, W0, A, B, 0.7, zeros, 0.3), X @ W0.T, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(dropout.dora_forward(X, W0, A, B, m, 0.7, ones, 0.0)["Y"],
                                  dora.dora_forward(X, W0, A, B, m, 0.7)["Y"])
    base = X @ W0.T * (m / np.sqrt(np.sum(W0 * W0, axis=1)))[None, :]
    np.testing.assert_allclose(dropout.dora_forward(X, W0, A, B, m, 0.7, zeros, 0.3)["Y"], base, rtol=1e-13)
    g = dropout.lora_backward(dY, X, W0, A, B, 0.7, keep, 0.25)
    assert not np.any(g["dA"][:, keep == 0])


def test_finite_differences_through_the_mask():
    X, W0, A, B, dY, m, keep = _case()
    s, p, h = 0.8, 0.25, 1e-6
    for fwd, bwd, extra in ((dropout.lora_forward, dropout.lora_backward, ()),
                            (lambda *a: dropout.dora_forward(*a)["Y"], dropout.dora_backward, (m,))):
        args = lambda A_, B_: (X, W0, A_, B_) + extra + (s, keep, p)  # noqa: E731
        g = bwd(dY, *args(A, B))

        def loss(A_, B_):
            return float(np.sum(dY * fwd(*args(A_, B_))))
        for name, arr, pos in (("dA", A, 0), ("dB", B, 1)):
            fd = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                pa = [A.copy(), B.copy()]
                qa = [A.copy(), B.copy()]
                pa[pos][idx] += h
                qa[pos][idx] -= h
                fd[idx] = (loss(*pa) - loss(*qa)) / (2 * h)
            np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-7)
