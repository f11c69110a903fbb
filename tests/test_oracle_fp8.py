"""Pins for oracle.fp8: e4m3 rounding against torch's float8_e4m3fn conversion, the
format's fixed points, the quantiser's half-ulp bound and zero rows, a hand-worked forward,
finite differences of the backward."""
import json
import os

import numpy as np
import pytest

from oracle import fp8

GOLD = os.path.join(os.path.dirname(__file__), "golden")
torch = pytest.importorskip("torch")


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_rounding_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 20.0, 120.0)])
    x = np.clip(x, -448, 448).astype(np.float32)
    np.testing.assert_array_equal(fp8.e4m3_round(x), _torch_e4m3(x))


def test_every_value_and_midpoint():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    v = fp8.e4m3_decode(codes)
    # representable values are fixed points, and encode inverts decode (bar the sign of zero)
    np.testing.assert_array_equal(fp8.e4m3_round(v), v)
    np.testing.assert_array_equal(fp8.e4m3_decode(fp8.e4m3_encode(v)), v)
    pos = np.sort(np.unique(v[v >= 0]))
    mids = 0.5 * (pos[:-1] + pos[1:])          # exact in float32 (at most 5 significant bits)
    np.testing.assert_array_equal(fp8.e4m3_round(mids), _torch_e4m3(mids))
    # ties go to the even code
    assert np.all(fp8.e4m3_encode(fp8.e4m3_round(mids)) % 2 == 0)


def test_format_fixed_points():
    np.testing.assert_array_equal(fp8.e4m3_decode([0x38, 0x7E, 0x08, 0x01, 0xB8, 0x00]),
                                  [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, -1.0, 0.0])
    assert fp8.e4m3_round(449.0) == 448.0 and fp8.e4m3_round(-1000.0) == -448.0


def test_quantiser_bound_and_zero_rows():
    rng = np.random.default_rng(1)
    X = (rng.standard_normal((16, 96)) * rng.uniform(0.01, 10, (16, 1))).astype(np.float32)
    X[3] = 0.0
    q, sx = fp8.quantize_rows_fp8(X)
    assert sx[3] == 0 and not np.any(q[3])
    v = fp8.e4m3_decode(q)
    for rrow in range(16):
        if rrow == 3:
            continue
        quot = X[rrow].astype(np.float64) / sx[rrow]
        # half a spacing of the binade (or of the subnormal range) around each code
        _, ex = np.frexp(np.where(np.abs(v[rrow]) > 0, np.abs(v[rrow]), 1.0))
        half = np.ldexp(1.0, np.maximum(ex - 1, -6) - 4)
        assert np.all(np.abs(quot - v[rrow]) <= half * (1 + 1e-6) + 1e-12)
        assert np.max(np.abs(v[rrow])) == 448.0


def test_hand_worked_forward():
    g = json.load(open(os.path.join(GOLD, "fp8_forward.json")))
    e = g["expected"]
    f = fp8.fp8_forward(np.array(g["X"]), np.array(g["Wq"], np.uint8), np.array(g["sw"]), np.array(g["A"], float),
                        np.array(g["B"], float), g["s"], np.array(g["bias"], float))
    np.testing.assert_array_equal(f["Xq"], np.array(e["Xq"], np.uint8))
    np.testing.assert_array_equal(f["sx"], np.array(e["sx"], np.float32))
    np.testing.assert_array_equal(f["acc"], np.array(e["acc"], float))
    np.testing.assert_allclose(f["Y"], np.array(e["Y"]), rtol=1e-12)


def test_backward_finite_differences():
    rng = np.random.default_rng(2)
    M, N, K, r, s = 3, 4, 5, 2, 0.7
    X, A, B, dY = rng.standard_normal((M, K)), rng.standard_normal((r, K)), rng.standard_normal((N, r)), \
        rng.standard_normal((M, N))
    Wq, _ = fp8.quantize_rows_fp8(rng.standard_normal((N, K)))
    sw = rng.uniform(0.01, 0.1, N)
    g = fp8.fp8_backward(dY, X, Wq, sw, A, B, s)
    Wdq = fp8.dequantized_weight(Wq, sw)

    def loss(X_, A_, B_):     # the straight-through layer: dequantised weight, unquantised X
        return float(np.sum(dY * (X_ @ (Wdq + s * B_ @ A_).T)))

    h = 1e-6
    args = [X, A, B]
    for name, pos in (("dX", 0), ("dA", 1), ("dB", 2)):
        fd = np.zeros_like(args[pos])
        for idx in np.ndindex(args[pos].shape):
            p = [a.copy() for a in args]
            q = [a.copy() for a in args]
            p[pos][idx] += h
            q[pos][idx] -= h
            fd[idx] = (loss(*p) - loss(*q)) / (2 * h)
        np.testing.assert_allclose(g[name], fd, rtol=1e-7, atol=1e-8, err_msg=name)
