"""Pins for oracle.swiglu: silu facts, the plain-MLP special case, a hand-worked example, finite differences."""
import json
import math
import os

import numpy as np
from scipy.special import expit

from oracle import swiglu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _proj(seed, n_out, n_in, r, s):
    return (_rand(seed, n_out, n_in), _rand(seed + 1, r, n_in), _rand(seed + 2, n_out, r), s)


def test_silu_facts():
    assert swiglu.silu(np.array([0.0]))[0] == 0.0
    assert swiglu.silu_grad(np.array([0.0]))[0] == 0.5
    e = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(swiglu.silu(e), e * expit(e), rtol=1e-14, atol=1e-300)
    h = 1e-6
    fd = (swiglu.silu(e + h) - swiglu.silu(e - h)) / (2 * h)
    np.testing.assert_allclose(swiglu.silu_grad(e), fd, rtol=1e-6, atol=1e-8)
    assert np.all(np.isfinite(swiglu.silu(np.array([-1e4, 1e4]))))


def test_zero_adapters_is_plain_mlp():
    X = _rand(1, 5, 6)
    gate, up, down = _proj(10, 7, 6, 2, 0.3), _proj(20, 7, 6, 2, 0.3), _proj(30, 6, 7, 2, 0.3)
    z = lambda p: (p[0], p[1], np.zeros_like(p[2]), p[3])  # noqa: E731
    O = swiglu.swiglu_mlp_forward(X, z(gate), z(up), z(down))["O"]
    e = X @ gate[0].T
    plain = ((e * expit(e)) * (X @ up[0].T)) @ down[0].T
    np.testing.assert_allclose(O, plain, rtol=1e-13, atol=1e-13)


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLD, "swiglu_tiny.json")))
    L = math.log(3.0)
    P = {p: (np.array(g[p]["W"], float), np.array(g[p]["A"], float), np.array(g[p]["B"], float), g[p]["s"])
         for p in ("gate", "up", "down")}
    X = np.array(g["X_over_L"], float) * L
    dO = np.array(g["dO"], float)
    e = g["expected"]
    f = swiglu.swiglu_mlp_forward(X, P["gate"], P["up"], P["down"])
    np.testing.assert_allclose(f["O"], np.array(e["O_L2"]) * L * L, rtol=1e-14)
    b = swiglu.swiglu_mlp_backward(dO, X, P["gate"], P["up"], P["down"])
    np.testing.assert_allclose(b["dX"], np.array(e["dX_L"]) * L + np.array(e["dX_L2"]) * L * L, rtol=1e-14)
    for k in ("dA_up", "dB_up", "dA_down", "dB_down"):
        np.testing.assert_allclose(b[k], np.array(e[k + "_L2"]) * L * L, rtol=1e-14, atol=1e-15)
    for k in ("dA_gate", "dB_gate"):
        np.testing.assert_allclose(b[k], np.array(e[k], float), atol=1e-14)


def test_finite_differences():
    M, K, H, r = 3, 4, 5, 2
    X = _rand(2, M, K)
    gate, up, down = _proj(40, H, K, r, 0.6), _proj(50, H, K, r, 1.1), _proj(60, K, H, r, 0.4)
    dO = _rand(3, M, K)
    gr = swiglu.swiglu_mlp_backward(dO, X, gate, up, down)

    def loss(X_, g_, u_, d_):
        return float(np.sum(dO * swiglu.swiglu_mlp_forward(X_, g_, u_, d_)["O"]))

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


def test_sampled_factor_gradients_equal_the_full_backward():
    M, K, H, r = 7, 6, 9, 3
    X = _rand(70, M, K)
    gate, up, down = _proj(71, H, K, r, 0.7), _proj(74, H, K, r, 1.3), _proj(77, K, H, r, 0.45)
    dO = _rand(80, M, K)
    full = swiglu.swiglu_mlp_backward(dO, X, gate, up, down)
    h_idx, k_idx = np.array([0, 4, 8]), np.array([1, 5])
    smp = swiglu.swiglu_mlp_grads_sampled(dO, X, gate, up, down, h_idx, k_idx)
    for p in ("gate", "up"):
        np.testing.assert_allclose(smp["dB_" + p + "_rows"], full["dB_" + p][h_idx], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(smp["dA_" + p + "_cols"], full["dA_" + p][:, k_idx], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(smp["dB_down_rows"], full["dB_down"][k_idx], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(smp["dA_down_cols"], full["dA_down"][:, h_idx], rtol=1e-12, atol=1e-12)
