"""Pins for oracle.w8a8: hand-worked codes, exact integer product, round-trip bound, finite differences."""
import json
import os

import numpy as np

from oracle import w8a8

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_worked_codes():
    g = json.load(open(os.path.join(GOLD, "w8a8_quant.json")))
    q, sc = w8a8.quantize_rows_int8(np.array(g["X"], np.float32))
    np.testing.assert_array_equal(q, np.array(g["q"], np.int8))
    # scale * 127 recovers the row absmax to float32 rounding
    np.testing.assert_allclose(sc.astype(np.float64) * 127, g["absmax"], rtol=2e-7)
    assert sc[1] == 0.0


def test_integer_product_is_exact_brute_force():
    rng = np.random.default_rng(3)
    Xq = rng.integers(-127, 128, size=(4, 33)).astype(np.int8)
    Wq = rng.integers(-127, 128, size=(5, 33)).astype(np.int8)
    acc = w8a8.int_product(Xq, Wq)
    for m in range(4):
        for n in range(5):
            assert acc[m, n] == sum(int(Xq[m, k]) * int(Wq[n, k]) for k in range(33))
    # extreme codes at the largest K the layer is quantised at stay far from int32 overflow
    big = np.full((1, 5120), 127, np.int8)
    assert w8a8.int_product(big, big)[0, 0] == 127 * 127 * 5120 < 2 ** 31


def test_round_trip_bound_and_code_range():
    X = (_rand(4, 64, 300) * 3).astype(np.float32)
    q, sc = w8a8.quantize_rows_int8(X)
    assert q.dtype == np.int8 and q.min() >= -127 and q.max() <= 127
    err = np.abs(X.astype(np.float64) - q.astype(np.float64) * sc.astype(np.float64)[:, None])
    assert np.all(err <= sc.astype(np.float64)[:, None] * (0.5 + 1e-6))
    # the row absmax maps to +-127
    assert np.all(np.max(np.abs(q.astype(int)), axis=1) == 127)


def test_forward_special_cases():
    X = _rand(5, 6, 16).astype(np.float32)
    W0 = (_rand(6, 8, 16) / 4).astype(np.float32)
    Wq, sw = w8a8.quantize_rows_int8(W0)
    A, B = _rand(7, 2, 16), _rand(8, 8, 2)
    f0 = w8a8.w8a8_forward(X, Wq, sw, A, B, 0.0)
    Xq, sx = w8a8.quantize_rows_int8(X)
    # With s = 0 the layer is the dequantised integer product
    ref = (Xq.astype(np.int64) @ Wq.astype(np.int64).T) * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    np.testing.assert_array_equal(f0["Y"], ref)
    # the LoRA branch sees the unquantised input: difference to s = 0 is s.(X.A^T).B^T
    f1 = w8a8.w8a8_forward(X, Wq, sw, A, B, 0.5)
    np.testing.assert_allclose(f1["Y"] - f0["Y"], 0.5 * (X.astype(np.float64) @ A.T) @ B.T, rtol=1e-12, atol=1e-12)


def test_finite_differences_of_the_straight_through_backward():
    X = _rand(9, 4, 8)
    W0 = (_rand(10, 5, 8) / 3).astype(np.float32)
    Wq, sw = w8a8.quantize_rows_int8(W0)
    A, B, s = _rand(11, 2, 8), _rand(12, 5, 2), 0.8
    dY = _rand(13, 4, 5)
    gr = w8a8.w8a8_backward(dY, X, Wq, sw, A, B, s)
    Wdq = Wq.astype(np.float64) * sw.astype(np.float64)[:, None]

    def surrogate(X_, A_, B_):   # quantisation of X passed straight through
        return float(np.sum(dY * (X_ @ Wdq.T + s * (X_ @ A_.T) @ B_.T)))

    h = 1e-6
    for name, pos in (("dX", 0), ("dA", 1), ("dB", 2)):
        base = [X, A, B]
        arr = base[pos]
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = [a.copy() for a in base]
            q = [a.copy() for a in base]
            p[pos][idx] += h
            q[pos][idx] -= h
            fd[idx] = (surrogate(*p) - surrogate(*q)) / (2 * h)
        np.testing.assert_allclose(gr[name], fd, rtol=1e-7, atol=1e-7)

    # dA, dB are exact gradients of the real forward too (the quantised base does not depend on A, B)
    def real(A_, B_):
        return float(np.sum(dY * w8a8.w8a8_forward(X, Wq, sw, A_, B_, s)["Y"]))
    fd = np.zeros_like(A)
    for idx in np.ndindex(A.shape):
        p = A.copy(); p[idx] += h
        q = A.copy(); q[idx] -= h
        fd[idx] = (real(p, B) - real(q, B)) / (2 * h)
    np.testing.assert_allclose(gr["dA"], fd, rtol=1e-7, atol=1e-7)


def test_zero_row_gives_zero_scale():
    X = np.zeros((2, 10), np.float32)
    X[1, 3] = -0.5
    q, sc = w8a8.quantize_rows_int8(X)
    assert sc[0] == 0 and not q[0].any()
    assert q[1, 3] == -127


def test_hand_worked_forward_and_backward():
    """The dequantised base plus the low-rank update from the unquantised input, and the
    straight-through backward, on a hand-worked example with power-of-two scales."""
    g = json.load(open(os.path.join(GOLD, "w8a8_forward.json")))
    e = g["expected"]
    X, W0 = np.array(g["X"], np.float64), np.array(g["W0"], np.float64)
    A, B = np.array(g["A"], np.float64), np.array(g["B"], np.float64)
    bias, dY, s = np.array(g["bias"], np.float64), np.array(g["dY"], np.float64), g["s"]
    Wq, sw = w8a8.quantize_rows_int8(W0)
    np.testing.assert_array_equal(Wq, np.array(e["Wq"], np.int8))
    np.testing.assert_array_equal(sw, np.array(e["sw"], np.float32))
    f = w8a8.w8a8_forward(X, Wq, sw, A, B, s, bias)
    np.testing.assert_array_equal(f["Xq"], np.array(e["Xq"], np.int8))
    np.testing.assert_array_equal(f["sx"], np.array(e["sx"], np.float32))
    np.testing.assert_array_equal(f["acc"], np.array(e["acc"], np.int64))
    # dyadic values: the float64 result is exact
    np.testing.assert_array_equal(f["Y"], np.array(e["Y"], np.float64))
    b = w8a8.w8a8_backward(dY, X, Wq, sw, A, B, s)
    for k in ("dX", "dA", "dB"):
        np.testing.assert_array_equal(b[k], np.array(e[k], np.float64), err_msg=k)
