"""GPU parity of the column-scaled DoRA linear ("dora-cols") against the fp64 oracle
(explicit column norm of the materialised W').  Tolerances as for the row form: 5e-3 of
max|ref| for bf16 outputs and all gradients, 1e-5 for the norm, g and the column sums of
W0^2 (fp32 sums of exact bf16 products)."""
import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import dora as odora
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu

TOL = 5e-3


def _run(c, eps, with_bias=False, need_dbias=False, need_dx=True, keep_u=True):
    import lora_dora_linear_amd as L
    X, W0, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
    m = dev(c.t["m"], "f32")
    bias = dev(c.t["bias"], "bf16") if with_bias else None
    c0 = L.dora_cols_prepare(W0)
    Y, U, Xs, state = L.dora_cols_linear_fwd(X, W0, A, B, m, c0, c.s, eps, bias=bias)
    g = L.dora_cols_linear_bwd(dY, X, Xs, W0, A, B, m, U if keep_u else None, state, c.s, eps, need_dx=need_dx,
                               need_dbias=need_dbias)
    torch.cuda.synchronize()
    return Y, Xs, state, g, c0


def _oracle(c, eps, with_bias=False):
    X, W0, A, B, dY = (c.f64(k) for k in ("X", "W0", "A", "B", "dY"))
    m = c.t["m"].astype(np.float64)
    bias = c.f64("bias") if with_bias else None
    return (odora.dora_cols_forward(X, W0, A, B, m, c.s, eps, bias),
            odora.dora_cols_backward(dY, X, W0, A, B, m, c.s, eps))


SHAPES = [
    # M, N, K, r, s   (256-column tiles with a ragged row tail; 128-row tiles; 192 columns; r = 64)
    (300, 512, 384, 16, 1.0),
    (100, 256, 256, 8, 0.5),
    (257, 384, 640, 32, 2.0),
    (64, 192, 128, 64, 1.0),
]


@pytest.mark.parametrize("M,N,K,r,s", SHAPES)
def test_dora_cols_parity(M, N, K, r, s):
    require_gpu()
    eps = 1e-12
    c = inputs.linear_case(4, M, N, K, r, s, "bf16", with_bias=True, dora_cols=True)
    Y, Xs, state, g, c0 = _run(c, eps, with_bias=True, need_dbias=True)
    f, gr = _oracle(c, eps, with_bias=True)
    assert_close(host(c0), odora.w0_col_sumsq(c.f64("W0")), 1e-6, "colsum W0^2")
    assert_close(host(state[:K]), f["nu"], 1e-5, "norm")
    assert_close(host(state[K:2 * K]), f["g"], 1e-5, "g")
    assert_close(host(Y), f["Y"], TOL, "Y")
    assert_close(host(Xs), f["Xs"], 2.0 ** -8, "Xs")
    for k in ("dX", "dA", "dB", "dm"):
        assert_close(host(g[k]), gr[k], TOL, k)
    assert_close(host(g["dbias"]), gr["db"], 1e-5, "dbias")


def test_dora_cols_no_dx_recomputed_u():
    require_gpu()
    c = inputs.linear_case(5, 300, 512, 384, 16, 1.0, "bf16", dora_cols=True)
    Y, Xs, state, g, c0 = _run(c, 1e-12, need_dx=False, keep_u=False)
    assert g["dX"] is None
    f, gr = _oracle(c, 1e-12)
    for k in ("dA", "dB", "dm"):
        assert_close(host(g[k]), gr[k], TOL, k)


def test_dora_cols_unit_scale_is_base():
    """B = 0 and m = ||W0[:,k]||: g = 1 and Y = X.W0^T."""
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(6, 300, 384, 256, 16, 1.0, "bf16", zero_B=True, dora_cols=True)
    W0 = c.f64("W0")
    m = np.sqrt(np.sum(W0 * W0, axis=0)).astype(np.float32)
    X, W0d, A, B = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B"))
    c0 = L.dora_cols_prepare(W0d)
    Y, U, Xs, state = L.dora_cols_linear_fwd(X, W0d, A, B, dev(m, "f32"), c0, c.s, 1e-12)
    torch.cuda.synchronize()
    assert_close(host(state[256:512]), np.ones(256), 1e-5, "g")
    assert_close(host(Y), c.f64("X") @ W0.T, TOL, "Y")


def test_dora_cols_zero_column_eps_clamp():
    """A zero column of W' (W0 and A zero there): nu = 0, g = m / eps on that column, and no
    gradient through the clamped norm."""
    require_gpu()
    eps = 1e-3
    c = inputs.linear_case(7, 300, 256, 256, 16, 1.0, "bf16", dora_cols=True)
    for k in ("W0", "A"):
        c.t[k] = c.t[k].copy()
        c.t[k][:, 5] = 0
    c.t["m"] = c.t["m"].copy()
    c.t["m"][5] = 1e-3       # g = 1 on the clamped column keeps Xs in range
    Y, Xs, state, g, c0 = _run(c, eps)
    f, gr = _oracle(c, eps)
    assert host(state[5])[()] == 0.0
    assert_close(host(state[256:512]), f["g"], 1e-5, "g")
    assert_close(host(Y), f["Y"], TOL, "Y")
    for k in ("dX", "dA", "dB", "dm"):
        assert_close(host(g[k]), gr[k], TOL, k)


def test_dora_cols_deterministic():
    require_gpu()
    c = inputs.linear_case(8, 300, 384, 256, 32, 1.0, "bf16", dora_cols=True)
    Y1, _, _, g1, _ = _run(c, 1e-12)
    Y2, _, _, g2, _ = _run(c, 1e-12)
    assert torch.equal(Y1, Y2)
    for k in ("dX", "dA", "dB", "dm"):
        assert torch.equal(g1[k], g2[k]), k


def test_dora_cols_full_size():
    """M = 4096, K = N = 3072, r = 32, s = 1, eps = 1e-12: every output against the full oracle."""
    require_gpu()
    c = inputs.linear_case(9, 4096, 3072, 3072, 32, 1.0, "bf16", with_bias=True, dora_cols=True)
    Y, Xs, state, g, c0 = _run(c, 1e-12, with_bias=True, need_dbias=True)
    f, gr = _oracle(c, 1e-12, with_bias=True)
    assert_close(host(state[:3072]), f["nu"], 1e-5, "norm")
    assert_close(host(Y), f["Y"], TOL, "Y")
    for k in ("dX", "dA", "dB", "dm"):
        assert_close(host(g[k]), gr[k], TOL, k)
    assert_close(host(g["dbias"]), gr["db"], 1e-5, "dbias")
