"""Pins for the column-scaled DoRA ("dora-cols") functions of oracle.dora: hand-worked
example, brute-force column norm, the transposed row form, reductions to the LoRA layer and
the base, finite differences and the eps clamp."""
import json
import os

import numpy as np

from oracle import dora, lora

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(seed, M=4, N=5, K=6, r=2):
    return dict(X=_rand(seed, M, K), W0=_rand(seed + 1, N, K), A=_rand(seed + 2, r, K), B=_rand(seed + 3, N, r),
                m=np.abs(_rand(seed + 4, K)) + 0.5, bias=_rand(seed + 5, N), dY=_rand(seed + 6, M, N), s=0.75)


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLD, "dora_cols_tiny.json")))
    e = g["expected"]
    X, W0, A, B, m, b, dY = (np.array(g[k], float) for k in ("X", "W0", "A", "B", "m", "bias", "dY"))
    f = dora.dora_cols_forward(X, W0, A, B, m, g["s"], g["eps"], b)
    np.testing.assert_allclose(f["nu"], e["nu"], rtol=1e-15)
    np.testing.assert_allclose(f["g"], e["g"], rtol=1e-15)
    np.testing.assert_allclose(f["Y"], e["Y"], rtol=1e-15)
    bw = dora.dora_cols_backward(dY, X, W0, A, B, m, g["s"], g["eps"])
    for k in ("dX", "dA", "dB", "dm"):
        np.testing.assert_allclose(bw[k], np.array(e[k]), rtol=1e-13, atol=1e-14, err_msg=k)


def test_column_norm_brute_force():
    c = _case(1, N=3, K=4, r=2)
    nu = dora.col_norm_explicit(c["W0"], c["A"], c["B"], c["s"])
    for k in range(4):
        col = [c["W0"][n, k] + c["s"] * sum(c["B"][n, j] * c["A"][j, k] for j in range(2)) for n in range(3)]
        assert abs(nu[k] - np.sqrt(sum(v * v for v in col))) < 1e-12
    np.testing.assert_allclose(dora.w0_col_sumsq(c["W0"]), [sum(c["W0"][n, k] ** 2 for n in range(3))
                                                             for k in range(4)], rtol=1e-14)


def test_column_norm_is_row_norm_of_transpose():
    # W'^T = W0^T + s.A^T.B^T: the row form on a layer with weight W0^T, lora_down B^T and
    # lora_up A^T has the same norms
    c = _case(2)
    np.testing.assert_allclose(dora.col_norm_explicit(c["W0"], c["A"], c["B"], c["s"]),
                               dora.row_norm_explicit(c["W0"].T, c["B"].T, c["A"].T, c["s"]), rtol=1e-14)


def test_unit_scale_is_lora():
    c = _case(3)
    m = dora.col_norm_explicit(c["W0"], c["A"], c["B"], c["s"])
    f = dora.dora_cols_forward(c["X"], c["W0"], c["A"], c["B"], m, c["s"], bias=c["bias"])
    np.testing.assert_allclose(f["g"], np.ones_like(m), rtol=1e-14)
    np.testing.assert_allclose(f["Y"], lora.lora_forward(c["X"], c["W0"], c["A"], c["B"], c["s"], c["bias"]),
                               rtol=1e-12, atol=1e-12)
    # the input gradient does not see the norm terms
    bw = dora.dora_cols_backward(c["dY"], c["X"], c["W0"], c["A"], c["B"], m, c["s"])
    np.testing.assert_allclose(bw["dX"], lora.lora_backward(c["dY"], c["X"], c["W0"], c["A"], c["B"], c["s"])["dX"],
                               rtol=1e-12, atol=1e-12)


def test_zero_strength_is_base():
    c = _case(4)
    m = np.sqrt(dora.w0_col_sumsq(c["W0"]))
    f = dora.dora_cols_forward(c["X"], c["W0"], c["A"], c["B"], m, 0.0, bias=c["bias"])
    np.testing.assert_allclose(f["Y"], c["X"] @ c["W0"].T + c["bias"], rtol=1e-12, atol=1e-12)


def test_finite_differences():
    c = _case(5, M=3, N=4, K=5, r=2)
    bw = dora.dora_cols_backward(c["dY"], c["X"], c["W0"], c["A"], c["B"], c["m"], c["s"])

    def loss(X, A, B, m, b):
        return float(np.sum(c["dY"] * dora.dora_cols_forward(X, c["W0"], A, B, m, c["s"], bias=b)["Y"]))

    args = [c["X"], c["A"], c["B"], c["m"], c["bias"]]
    h = 1e-6
    for name, pos in (("dX", 0), ("dA", 1), ("dB", 2), ("dm", 3), ("db", 4)):
        fd = np.zeros_like(args[pos])
        for idx in np.ndindex(args[pos].shape):
            p = [a.copy() for a in args]
            q = [a.copy() for a in args]
            p[pos][idx] += h
            q[pos][idx] -= h
            fd[idx] = (loss(*p) - loss(*q)) / (2 * h)
        np.testing.assert_allclose(bw[name], fd, rtol=2e-7, atol=1e-8, err_msg=name)


def test_eps_clamp_zero_column():
    # a zero column of W' (W0 and A zero there): g_k = m_k / eps, no gradient through nu_k
    c = _case(6, M=3, N=4, K=5, r=2)
    c["W0"][:, 2] = 0.0
    c["A"][:, 2] = 0.0
    eps = 1e-3
    f = dora.dora_cols_forward(c["X"], c["W0"], c["A"], c["B"], c["m"], c["s"], eps)
    assert f["nu"][2] == 0.0 and f["g"][2] == c["m"][2] / eps
    bw = dora.dora_cols_backward(c["dY"], c["X"], c["W0"], c["A"], c["B"], c["m"], c["s"], eps)
    # dm_k = dg_k / eps with dg_k = sum_n G[n,k] W'[n,k] = 0 for the zero column
    assert bw["dm"][2] == 0.0

    def loss(A):
        return float(np.sum(c["dY"] * dora.dora_cols_forward(c["X"], c["W0"], A, c["B"], c["m"], c["s"], eps)["Y"]))

    # finite differences away from the clamped column
    h = 1e-6
    for idx in [(0, 0), (1, 4)]:
        p, q = c["A"].copy(), c["A"].copy()
        p[idx] += h
        q[idx] -= h
        assert abs(bw["dA"][idx] - (loss(p) - loss(q)) / (2 * h)) < 1e-6
