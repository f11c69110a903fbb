"""Pins for oracle.multi (several adapters over one concatenated base weight): reductions
to oracle.lora, the equivalent single adapter with a block-diagonal up factor, a leaf with
zero scale, brute-force loops and finite differences."""
import numpy as np

from oracle import lora, multi


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(seed, M=5, K=6, n_leaf=(3, 2, 4), r=2):
    L, N = len(n_leaf), sum(n_leaf)
    return dict(X=_rand(seed, M, K), W0=_rand(seed + 1, N, K), A=_rand(seed + 2, L * r, K),
                B=_rand(seed + 3, N, r), bias=_rand(seed + 4, N), dY=_rand(seed + 5, M, N),
                n_leaf=list(n_leaf), s=[0.5, -1.25, 2.0][:L], r=r)


def test_one_leaf_is_lora():
    c = _case(10, n_leaf=(7,))
    c["s"] = [0.75]
    y = multi.multi_forward(c["X"], c["W0"], c["A"], c["B"], c["n_leaf"], c["s"], c["bias"])
    np.testing.assert_allclose(y, lora.lora_forward(c["X"], c["W0"], c["A"], c["B"], 0.75, c["bias"]), rtol=1e-13,
                               atol=1e-13)
    g = multi.multi_backward(c["dY"], c["X"], c["W0"], c["A"], c["B"], c["n_leaf"], c["s"])
    h = lora.lora_backward(c["dY"], c["X"], c["W0"], c["A"], c["B"], 0.75)
    for k in ("dX", "dA", "dB", "db"):
        np.testing.assert_allclose(g[k], h[k], rtol=1e-13, atol=1e-13)


def test_each_leaf_is_its_own_lora():
    c = _case(20)
    r = c["r"]
    y = multi.multi_forward(c["X"], c["W0"], c["A"], c["B"], c["n_leaf"], c["s"], c["bias"])
    g = multi.multi_backward(c["dY"], c["X"], c["W0"], c["A"], c["B"], c["n_leaf"], c["s"])
    dX = np.zeros_like(c["X"])
    a = 0
    for l, n in enumerate(c["n_leaf"]):
        b = a + n
        Al, Bl = c["A"][l * r:(l + 1) * r], c["B"][a:b]
        yl = lora.lora_forward(c["X"], c["W0"][a:b], Al, Bl, c["s"][l], c["bias"][a:b])
        np.testing.assert_allclose(y[:, a:b], yl, rtol=1e-13, atol=1e-13)
        hl = lora.lora_backward(c["dY"][:, a:b], c["X"], c["W0"][a:b], Al, Bl, c["s"][l])
        np.testing.assert_allclose(g["dA"][l * r:(l + 1) * r], hl["dA"], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(g["dB"][a:b], hl["dB"], rtol=1e-13, atol=1e-13)
        dX += hl["dX"]
        a = b
    # the input gradient sums the leaves' contributions
    np.testing.assert_allclose(g["dX"], dX, rtol=1e-12, atol=1e-12)


def test_block_diagonal_single_adapter():
    # one adapter of rank L r with A = A_cat and the up factor block diagonal (leaf l's rows
    # hold s_l.B_l in rank columns l r .. l r + r - 1), scale 1
    c = _case(30)
    r, L, N = c["r"], len(c["n_leaf"]), sum(c["n_leaf"])
    Bbig = np.zeros((N, L * r))
    a = 0
    for l, n in enumerate(c["n_leaf"]):
        Bbig[a:a + n, l * r:(l + 1) * r] = c["s"][l] * c["B"][a:a + n]
        a += n
    y = multi.multi_forward(c["X"], c["W0"], c["A"], c["B"], c["n_leaf"], c["s"])
    np.testing.assert_allclose(y, lora.lora_forward(c["X"], c["W0"], c["A"], Bbig, 1.0), rtol=1e-12, atol=1e-12)
    g = multi.multi_backward(c["dY"], c["X"], c["W0"], c["A"], c["B"], c["n_leaf"], c["s"])
    np.testing.assert_allclose(g["dX"], lora.lora_backward(c["dY"], c["X"], c["W0"], c["A"], Bbig, 1.0)["dX"],
                               rtol=1e-12, atol=1e-12)


def test_zero_scale_leaf_is_base():
    c = _case(40)
    c["s"][1] = 0.0
    y = multi.multi_forward(c["X"], c["W0"], c["A"], c["B"], c["n_leaf"], c["s"])
    a, b = c["n_leaf"][0], c["n_leaf"][0] + c["n_leaf"][1]
    np.testing.assert_allclose(y[:, a:b], c["X"] @ c["W0"][a:b].T, rtol=1e-13, atol=1e-13)
    g = multi.multi_backward(c["dY"], c["X"], c["W0"], c["A"], c["B"], c["n_leaf"], c["s"])
    assert not np.any(g["dA"][c["r"]:2 * c["r"]]) and not np.any(g["dB"][a:b])


def test_brute_force_loops():
    c = _case(50, M=2, K=3, n_leaf=(2, 1), r=1)
    y = multi.multi_forward(c["X"], c["W0"], c["A"], c["B"], c["n_leaf"], c["s"])
    leaf = [0, 0, 1]
    for m in range(2):
        for n in range(3):
            l = leaf[n]
            ref = sum(c["X"][m, k] * (c["W0"][n, k] + c["s"][l] * c["B"][n, 0] * c["A"][l, k]) for k in range(3))
            assert abs(y[m, n] - ref) < 1e-12


def test_finite_differences():
    c = _case(60, M=3, K=4, n_leaf=(2, 3), r=2)
    g = multi.multi_backward(c["dY"], c["X"], c["W0"], c["A"], c["B"], c["n_leaf"], c["s"])

    def loss(X, A, B, bias):
        return float(np.sum(c["dY"] * multi.multi_forward(X, c["W0"], A, B, c["n_leaf"], c["s"], bias)))

    args = [c["X"], c["A"], c["B"], c["bias"]]
    h = 1e-6
    for name, pos in (("dX", 0), ("dA", 1), ("dB", 2), ("db", 3)):
        fd = np.zeros_like(args[pos])
        for idx in np.ndindex(args[pos].shape):
            p = [a.copy() for a in args]
            q = [a.copy() for a in args]
            p[pos][idx] += h
            q[pos][idx] -= h
            fd[idx] = (loss(*p) - loss(*q)) / (2 * h)
        np.testing.assert_allclose(g[name], fd, rtol=1e-7, atol=1e-8)


def test_sampled_grads_match_full():
    c = _case(70, M=6, K=8, n_leaf=(3, 4, 2), r=2)
    g = multi.multi_backward(c["dY"], c["X"], c["W0"], c["A"], c["B"], c["n_leaf"], c["s"])
    rows, cols = [0, 3, 8], [1, 7]
    sm = multi.multi_weight_grads_sampled(c["dY"], c["X"], c["A"], c["B"], c["n_leaf"], c["s"], rows, cols)
    np.testing.assert_allclose(sm["dB_rows"], g["dB"][rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(sm["dA_cols"], g["dA"][:, cols], rtol=1e-13, atol=1e-13)
