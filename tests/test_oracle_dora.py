"""Pins for oracle.dora: hand-worked example, closed-form norm, invariances, finite differences."""
import json
import os

import numpy as np

from oracle import dora

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(seed=0, M=5, N=4, K=6, r=3):
    X, W0, A, B = _rand(seed, M, K), _rand(seed + 1, N, K), _rand(seed + 2, r, K), _rand(seed + 3, N, r)
    m = np.abs(_rand(seed + 4, N)) + 0.5
    return X, W0, A, B, m


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLD, "dora_tiny.json")))
    X, W0, A, B = (np.array(g[k], float) for k in ("X", "W0", "A", "B"))
    m, bias, dY = (np.array(g[k], float) for k in ("m", "bias", "dY"))
    s, eps, e = g["s"], g["eps"], g["expected"]
    f = dora.dora_forward(X, W0, A, B, m, s, eps, bias)
    np.testing.assert_allclose(f["nu"], e["nu"], atol=1e-15)
    np.testing.assert_allclose(f["g"], e["g"], atol=1e-15)
    np.testing.assert_allclose(f["Y"], e["Y"], atol=1e-13)
    gr = dora.dora_backward(dY, X, W0, A, B, m, s, eps)
    for k in ("dX", "dA", "dB", "dm"):
        np.testing.assert_allclose(gr[k], np.array(e[k], float), atol=1e-13)


def test_closed_form_norm_equals_explicit():
    """||W0_n + s B_n A||^2 = rowsum(W0^2)_n + 2s <B_n, (W0 A^T)_n> + s^2 B_n (A A^T) B_n^T."""
    _, W0, A, B, _ = _case(1, N=7, K=11, r=3)
    s = 1.3
    P = W0 @ A.T
    Gm = A @ A.T
    closed = np.sqrt(np.sum(W0 ** 2, axis=1) + 2 * s * np.sum(B * P, axis=1)
                     + s * s * np.einsum("nj,jl,nl->n", B, Gm, B))
    np.testing.assert_allclose(dora.row_norm_explicit(W0, A, B, s), closed, rtol=1e-14)
    np.testing.assert_allclose(dora.w0_row_sumsq(W0), np.linalg.norm(W0, axis=1) ** 2, rtol=1e-14)


def test_norm_matches_library_norm():
    _, W0, A, B, _ = _case(2)
    Wp = W0 + 0.4 * (B @ A)
    np.testing.assert_allclose(dora.row_norm_explicit(W0, A, B, 0.4), np.linalg.norm(Wp, axis=1), rtol=1e-14)


def test_direction_invariance():
    X, W0, A, B, m = _case(3)
    y1 = dora.dora_forward(X, W0, A, B, m, 0.8)["Y"]
    y2 = dora.dora_forward(X, 3.5 * W0, A, 3.5 * B, m, 0.8)["Y"]
    np.testing.assert_allclose(y1, y2, rtol=1e-13, atol=1e-13)


def test_unit_scale_reduces_to_base():
    X, W0, A, B, _ = _case(4)
    bias = _rand(40, W0.shape[0])
    m = np.linalg.norm(W0, axis=1)
    f = dora.dora_forward(X, W0, A, np.zeros_like(B), m, 0.9, bias=bias)
    np.testing.assert_allclose(f["g"], 1.0, rtol=1e-15)
    np.testing.assert_allclose(f["Y"], X @ W0.T + bias, rtol=1e-13, atol=1e-13)


def test_finite_differences_through_the_norm():
    X, W0, A, B, m = _case(5, M=4, N=3, K=5, r=2)
    s, bias = 0.7, _rand(50, 3)
    dY = _rand(51, 4, 3)
    gr = dora.dora_backward(dY, X, W0, A, B, m, s)

    def loss(X_, A_, B_, m_):
        return float(np.sum(dY * dora.dora_forward(X_, W0, A_, B_, m_, s, bias=bias)["Y"]))

    h = 1e-6
    for name, pos in (("dX", 0), ("dA", 1), ("dB", 2), ("dm", 3)):
        base = [X, A, B, m]
        arr = base[pos]
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = [a.copy() for a in base]
            q = [a.copy() for a in base]
            p[pos][idx] += h
            q[pos][idx] -= h
            fd[idx] = (loss(*p) - loss(*q)) / (2 * h)
        np.testing.assert_allclose(gr[name], fd, rtol=1e-6, atol=1e-7)


def test_homogeneity_and_gauge_identities():
    X, W0, A, B, m = _case(6, M=6, N=5, K=8, r=3)
    s, bias = 1.2, _rand(60, 5)
    dY = _rand(61, 6, 5)
    Y = dora.dora_forward(X, W0, A, B, m, s, bias=bias)["Y"]
    gr = dora.dora_backward(dY, X, W0, A, B, m, s)
    target = np.sum(dY * (Y - bias))
    assert abs(np.sum(m * gr["dm"]) - target) < 1e-11      # Y - b is 1-homogeneous in m
    assert abs(np.sum(gr["dX"] * X) - target) < 1e-11      # and linear in X
    assert abs(np.sum(gr["dA"] * A) - np.sum(gr["dB"] * B)) < 1e-11   # depends on B.A only


def test_norm_gradient_is_in_the_graph():
    """Dropping the norm term (the DoRA-paper detach) must change dA and dB."""
    X, W0, A, B, m = _case(7)
    dY = _rand(70, X.shape[0], W0.shape[0])
    gr = dora.dora_backward(dY, X, W0, A, B, m, 1.0)
    f = dora.dora_forward(X, W0, A, B, m, 1.0)
    dZ = dY * f["g"][None, :]
    detached_dB = 1.0 * (dZ.T @ X) @ A.T
    assert np.max(np.abs(gr["dB"] - detached_dB)) > 1e-3


def test_eps_clamp_on_a_zero_row():
    X, W0, A, B, m = _case(8)
    W0 = W0.copy(); B = B.copy()
    W0[1] = 0.0
    B[1] = 0.0                            # row 1 of W' is exactly zero, so nu_1 = 0 <= eps
    eps = 1e-12
    f = dora.dora_forward(X, W0, A, B, m, 0.5, eps)
    assert f["nu"][1] == 0.0 and f["g"][1] == m[1] / eps
    assert not f["Y"][:, 1].any()
    dY = _rand(80, X.shape[0], W0.shape[0])
    gr = dora.dora_backward(dY, X, W0, A, B, m, 0.5, eps)
    assert gr["dm"][1] == 0.0                 # dg_1 = <dY_1, Z_1> = 0
    assert np.all(np.isfinite(gr["dA"])) and np.all(np.isfinite(gr["dB"]))
