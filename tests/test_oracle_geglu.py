"""Pins for oracle.geglu: GELU against the normal distribution function of scipy, its tanh
form, derivatives, the plain-MLP special case and finite differences of every gradient."""
import numpy as np
from scipy.stats import norm

from oracle import geglu


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _proj(seed, n_out, n_in, r, s):
    return (_rand(seed, n_out, n_in), _rand(seed + 1, r, n_in), _rand(seed + 2, n_out, r), s)


def test_gelu_facts():
    e = np.linspace(-8, 8, 161)
    for approx in (False, True):
        assert geglu.gelu(np.array([0.0]), approx)[0] == 0.0
        assert abs(geglu.gelu_grad(np.array([0.0]), approx)[0] - 0.5) < 1e-15
        h = 1e-6
        fd = (geglu.gelu(e + h, approx) - geglu.gelu(e - h, approx)) / (2 * h)
        np.testing.assert_allclose(geglu.gelu_grad(e, approx), fd, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(geglu.gelu(e), e * norm.cdf(e), rtol=1e-13, atol=1e-300)
    assert np.max(np.abs(geglu.gelu(e, True) - geglu.gelu(e))) < 1e-3
    big = np.array([-30.0, 30.0])
    np.testing.assert_allclose(geglu.gelu(big), [0.0, 30.0], atol=1e-12)


def test_zero_adapters_is_plain_mlp():
    X = _rand(1, 5, 6)
    gate, up, down = _proj(10, 7, 6, 2, 0.3), _proj(20, 7, 6, 2, 0.3), _proj(30, 6, 7, 2, 0.3)
    z = lambda p: (p[0], p[1], np.zeros_like(p[2]), p[3])  # noqa: E731
    O = geglu.geglu_mlp_forward(X, z(gate), z(up), z(down))["O"]
    e = X @ gate[0].T
    np.testing.assert_allclose(O, (e * norm.cdf(e) * (X @ up[0].T)) @ down[0].T, rtol=1e-12, atol=1e-12)


def test_finite_differences():
    M, K, H, r = 3, 4, 5, 2
    X = _rand(2, M, K)
    gate, up, down = _proj(40, H, K, r, 0.6), _proj(50, H, K, r, 1.1), _proj(60, K, H, r, 0.4)
    dO = _rand(3, M, K)
    for approx in (False, True):
        gr = geglu.geglu_mlp_backward(dO, X, gate, up, down, approx)

        def loss(X_, g_, u_, d_):
            return float(np.sum(dO * geglu.geglu_mlp_forward(X_, g_, u_, d_, approx)["O"]))

        h = 1e-6
        fd = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            p = X.copy(); p[idx] += h
            q = X.copy(); q[idx] -= h
            fd[idx] = (loss(p, gate, up, down) - loss(q, gate, up, down)) / (2 * h)
        np.testing.assert_allclose(gr["dX"], fd, rtol=1e-6, atol=1e-7)
        projs = {"gate": gate, "up": up, "down": down}
        for name in ("gate", "up", "down"):
            for which, pos in (("dA_", 1), ("dB_", 2)):
                arr = projs[name][pos]
                fd = np.zeros_like(arr)
                for idx in np.ndindex(arr.shape):
                    vals = []
                    for sgn in (1, -1):
                        a2 = arr.copy(); a2[idx] += sgn * h
                        pr = list(projs[name]); pr[pos] = a2
                        pp = dict(projs); pp[name] = tuple(pr)
                        vals.append(loss(X, pp["gate"], pp["up"], pp["down"]))
                    fd[idx] = (vals[0] - vals[1]) / (2 * h)
                np.testing.assert_allclose(gr[which + name], fd, rtol=1e-6, atol=1e-7)
