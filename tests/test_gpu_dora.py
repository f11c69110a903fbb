"""GPU parity of the row-scaled DoRA linear against the fp64 oracle (explicit norm, materialised W')."""
import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import dora as odora
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu

TOL = 5e-3


def _run(c, eps, with_bias=False, need_dbias=False):
    import lora_dora_linear_amd as L
    X, W0, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
    m = dev(c.t["m"], "f32")
    bias = dev(c.t["bias"], "bf16") if with_bias else None
    c0 = L.dora_prepare(W0)
    Y, U, Z, state = L.dora_linear_fwd(X, W0, A, B, m, c0, c.s, eps, bias=bias)
    g = L.dora_linear_bwd(dY, X, W0, A, B, m, U, Z, state, c.s, eps, need_dbias=need_dbias)
    torch.cuda.synchronize()
    return Y, Z, state, g, c0


def _oracle(c, eps, with_bias=False):
    X, W0, A, B, dY = (c.f64(k) for k in ("X", "W0", "A", "B", "dY"))
    m = c.t["m"].astype(np.float64)
    bias = c.f64("bias") if with_bias else None
    return odora.dora_forward(X, W0, A, B, m, c.s, eps, bias), odora.dora_backward(dY, X, W0, A, B, m, c.s, eps)


@pytest.mark.parametrize("M,N,K,r,s", [(300, 384, 256, 32, 1.0), (200, 512, 384, 16, 0.5), (129, 256, 192, 8, 2.0)])
def test_dora_parity(M, N, K, r, s):
    require_gpu()
    eps = 1e-12
    c = inputs.linear_case(3, M, N, K, r, s, "bf16", with_bias=True, dora=True)
    Y, Z, state, g, c0 = _run(c, eps, with_bias=True, need_dbias=True)
    f, gr = _oracle(c, eps, with_bias=True)
    assert_close(host(Y), f["Y"], TOL, "Y")
    assert_close(host(Z), f["Z"], TOL, "Z")
    nu = host(state[:N])
    gg = host(state[N:2 * N])
    # closed-form norm from the cached row constant vs the explicit norm of W'
    assert_close(nu, f["nu"], 1e-5, "norm")
    assert_close(gg, f["g"], 1e-5, "g")
    assert_close(host(c0), odora.w0_row_sumsq(c.f64("W0")), 1e-6, "rowsum W0^2")
    for k in ("dX", "dA", "dB", "dm"):
        assert_close(host(g[k]), gr[k], TOL, k)
    assert_close(host(g["dbias"]), gr["db"], 1e-5, "dbias")


def test_dora_rank64_norm_terms_and_u_in_one_row_launch():
    """r = 64 with N + r + M = 8256 rows: P = W0.A^T, G = A.A^T and U = X.A^T run as one
    row-projection launch on 32-row blocks (three row segments, each a multiple of 32)."""
    require_gpu()
    eps = 1e-12
    M, N, K, r = 4096, 4096, 256, 64
    c = inputs.linear_case(7, M, N, K, r, 1.0, "bf16", dora=True)
    import lora_dora_linear_amd as L
    X, W0, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
    m = dev(c.t["m"], "f32")
    c0 = L.dora_prepare(W0)
    Y, U, Z, state = L.dora_linear_fwd(X, W0, A, B, m, c0, c.s, eps)
    g = L.dora_linear_bwd(dY, X, W0, A, B, m, U, Z, state, c.s, eps)
    torch.cuda.synchronize()
    f, gr = _oracle(c, eps)
    assert_close(host(U), c.f64("X") @ c.f64("A").T, 1e-5, "U")
    assert_close(host(state[:N]), f["nu"], 1e-5, "norm")
    assert_close(host(Y), f["Y"], TOL, "Y")
    for k in ("dX", "dA", "dB", "dm"):
        assert_close(host(g[k]), gr[k], TOL, k)


@pytest.mark.parametrize("r", [32, 64])
def test_dora_prepacked_factors_match_the_packing_pass(r):
    """V and w.B written packed by the kernels that form them give the same bits as packing
    them in a separate pass (every gradient, equal)."""
    require_gpu()
    from lora_dora_linear_amd import binding
    c = inputs.linear_case(11, 300, 384, 256, r, 1.0, "bf16", with_bias=True, dora=True)
    try:
        binding.set_tuning(3, 1)
        _, _, _, g1, _ = _run(c, 1e-12, with_bias=True, need_dbias=True)
        binding.set_tuning(3, 0)
        _, _, _, g0, _ = _run(c, 1e-12, with_bias=True, need_dbias=True)
    finally:
        binding.set_tuning(3, 1)
    for k in ("dX", "dA", "dB", "dm", "dbias"):
        assert torch.equal(g1[k], g0[k]), k


def test_dora_unit_scale_is_base():
    """B = 0 and m = ||W0_n||: g = 1 and Y = X.W0^T."""
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(3, 300, 384, 256, 16, 1.0, "bf16", zero_B=True, dora=True)
    W0 = c.f64("W0")
    m = np.sqrt(np.sum(W0 * W0, axis=1)).astype(np.float32)
    X, W0d, A, B = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B"))
    md = dev(m, "f32")
    c0 = L.dora_prepare(W0d)
    Y, U, Z, state = L.dora_linear_fwd(X, W0d, A, B, md, c0, c.s, 1e-12)
    torch.cuda.synchronize()
    assert_close(host(state[384:768]), np.ones(384), 1e-5, "g")
    assert_close(host(Y), c.f64("X") @ W0.T, TOL, "Y")


def test_dora_deterministic():
    require_gpu()
    c = inputs.linear_case(3, 300, 384, 256, 32, 1.0, "bf16", dora=True)
    Y1, _, _, g1, _ = _run(c, 1e-12)
    Y2, _, _, g2, _ = _run(c, 1e-12)
    assert torch.equal(Y1, Y2)
    for k in ("dX", "dA", "dB", "dm"):
        assert torch.equal(g1[k], g2[k]), k


def test_dora_full_size_3072():
    """M = 4096, K = N = 3072, r = 32, s = 1, eps = 1e-12: every output against the full oracle."""
    require_gpu()
    eps = 1e-12
    c = inputs.linear_case(3, 4096, 3072, 3072, 32, 1.0, "bf16", dora=True)
    Y, Z, state, g, _ = _run(c, eps)
    f, gr = _oracle(c, eps)
    assert_close(host(Y), f["Y"], TOL, "Y")
    assert_close(host(state[:3072]), f["nu"], 1e-5, "norm")
    for k in ("dX", "dA", "dB", "dm"):
        assert_close(host(g[k]), gr[k], TOL, k)


@pytest.mark.parametrize("M,N,K,r", [(64, 384, 256, 32), (100, 256, 192, 16)])
def test_dora_small_batch_tiles(M, N, K, r):
    """At most 128 tokens: the 128-row tiles of the row-scaled forward and of the input gradient."""
    require_gpu()
    eps = 1e-12
    c = inputs.linear_case(13, M, N, K, r, 0.5, "bf16", with_bias=True, dora=True)
    Y, Z, state, g, _ = _run(c, eps, with_bias=True, need_dbias=True)
    f, gr = _oracle(c, eps, with_bias=True)
    assert_close(host(Y), f["Y"], TOL, "Y")
    assert_close(host(Z), f["Z"], TOL, "Z")
    for k in ("dX", "dA", "dB", "dm"):
        assert_close(host(g[k]), gr[k], TOL, k)
    assert_close(host(g["dbias"]), gr["db"], 1e-5, "dbias")


def test_dora_zero_row_eps_clamp():
    """A row of W' that is exactly zero (W0 and B rows zero): the closed-form norm is 0, the
    clamp max(nu, eps) gives g = m / eps and no gradient flows through the norm there."""
    require_gpu()
    eps = 1e-12
    c = inputs.linear_case(14, 200, 256, 192, 16, 0.75, "bf16", dora=True)
    c.t["W0"][5] = 0
    c.t["B"][5] = 0
    c.t["m"][5] = np.float32(0.75)
    Y, Z, state, g, _ = _run(c, eps)
    f, gr = _oracle(c, eps)
    N = c.N
    nu, gg = host(state[:N]), host(state[N:2 * N])
    assert nu[5] == 0.0
    assert_close(gg, f["g"], 1e-5, "g")
    assert abs(gg[5] - 0.75 / eps) <= 1e-6 * (0.75 / eps)
    assert_close(host(Y), f["Y"], TOL, "Y")
    for k in ("dX", "dA", "dB", "dm"):
        got = host(g[k])
        assert np.all(np.isfinite(got)), k
        assert_close(got, gr[k], TOL, k)


def test_dora_zero_strength():
    """s = 0: the formula with g = m / ||W0_n|| (no short-circuit); the factor gradients vanish."""
    require_gpu()
    eps = 1e-12
    c = inputs.linear_case(15, 300, 384, 256, 32, 0.0, "bf16", dora=True)
    Y, Z, state, g, _ = _run(c, eps)
    f, gr = _oracle(c, eps)
    W0 = c.f64("W0")
    assert_close(host(state[c.N:2 * c.N]), c.t["m"] / np.sqrt(np.sum(W0 * W0, axis=1)), 1e-5, "g")
    assert_close(host(Y), f["Y"], TOL, "Y")
    assert_close(host(g["dX"]), gr["dX"], TOL, "dX")
    assert_close(host(g["dm"]), gr["dm"], TOL, "dm")
    assert not torch.any(g["dA"]) and not torch.any(g["dB"])


@pytest.mark.parametrize("M,N,K,r", [(300, 384, 256, 32), (4096, 3072, 3072, 32)])
def test_dora_without_input_gradient(M, N, K, r):
    """dX not requested: V = (dY.diag(g)).B is projected with g applied to B's rows on load
    (the k-scaled row projection); dA, dB, dm against the oracle and against the dX route."""
    require_gpu()
    import lora_dora_linear_amd as L
    eps = 1e-12
    c = inputs.linear_case(16, M, N, K, r, 1.0, "bf16", dora=True)
    X, W0, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
    m = dev(c.t["m"], "f32")
    c0 = L.dora_prepare(W0)
    Y, U, Z, state = L.dora_linear_fwd(X, W0, A, B, m, c0, c.s, eps)
    g0 = L.dora_linear_bwd(dY, X, W0, A, B, m, U, Z, state, c.s, eps, need_dx=False)
    g1 = L.dora_linear_bwd(dY, X, W0, A, B, m, U, Z, state, c.s, eps, need_dx=True)
    torch.cuda.synchronize()
    assert g0["dX"] is None
    _, gr = _oracle(c, eps)
    for k in ("dA", "dB", "dm"):
        assert_close(host(g0[k]), gr[k], TOL, k)
        assert_close(host(g0[k]), host(g1[k]), TOL, k + " vs dX route")
