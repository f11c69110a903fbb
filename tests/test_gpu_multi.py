"""GPU parity of the fused QKV leaves (several adapters over one concatenated base weight)
against the fp64 oracle, through the C interface.

Routes: one rank-(L r) projection plus one four-wave GEMM whose low-rank k-tile takes each
column's own leaf (256- and 192-column tiles, with and without the bf16 hi + lo split of
s.U, leaf boundaries inside a tile), and the per-leaf fallback (128 rows or fewer, L r above
64).  Tolerance max|gpu - ref| / max|ref| per tensor: 5e-3 for bf16 outputs and factor
gradients (as for the single adapter), 1e-5 for U and dbias (fp32 sums of bf16 products).
"""
import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import multi as omulti
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu

BF16_TOL = 5e-3

CASES = [
    # M, K, leaf widths, r, what it exercises
    (300, 256, (320, 192, 256), 16, "four-wave 256-column tiles, boundary at column 320 inside a tile, L r = 48"),
    (300, 384, (128, 384), 16, "four-wave, L r = 32: s.U as a bf16 hi + lo pair"),
    (300, 256, (192, 320, 64), 8, "four-wave 192-column tiles (576 columns), three boundaries"),
    (100, 256, (128, 64, 64), 8, "128 rows or fewer: one product per leaf"),
    (300, 256, (256, 256, 256), 32, "L r = 96 above the k-tile: one product per leaf"),
    (257, 128, (64,) * 8, 8, "eight leaves of 64 columns, L r = 64, ragged rows"),
]


def _run(c, need_dbias=True, save_u=True, need_dx=True):
    import lora_dora_linear_amd as L
    X, W0, A, B, dY, bias = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY", "bias"))
    Y, U = L.lora_multi_linear_fwd(X, W0, A, B, c.n_leaf, c.s_leaf, bias=bias, save_u=save_u)
    g = L.lora_multi_linear_bwd(dY, X, W0, A, B, c.n_leaf, c.s_leaf, U=U, need_dx=need_dx, need_dbias=need_dbias)
    torch.cuda.synchronize()
    return Y, U, g


@pytest.mark.parametrize("M,K,leaves,r,what", CASES)
def test_multi_parity(M, K, leaves, r, what):
    require_gpu()
    s_leaf = [0.5, -1.5, 2.0, 1.0, 0.25, -0.75, 1.25, 3.0][:len(leaves)]
    c = inputs.multi_case(7, M, K, leaves, r, s_leaf, with_bias=True)
    Y, U, g = _run(c)
    X, W0, A, B, dY, bias = (c.f64(k) for k in ("X", "W0", "A", "B", "dY", "bias"))
    Yr = omulti.multi_forward(X, W0, A, B, c.n_leaf, c.s_leaf, bias)
    gr = omulti.multi_backward(dY, X, W0, A, B, c.n_leaf, c.s_leaf)
    assert_close(host(Y), Yr, BF16_TOL, "Y")
    assert_close(host(U), X @ A.T, 1e-5, "U")
    for k in ("dX", "dA", "dB"):
        assert_close(host(g[k]), gr[k], BF16_TOL, k)
    assert_close(host(g["dbias"]), gr["db"], 1e-5, "dbias")
    # every leaf's block on its own: a wrong leaf at a boundary shows here even when the
    # whole-tensor error stays small
    a = 0
    for l, n in enumerate(c.n_leaf):
        assert_close(host(Y[:, a:a + n]), Yr[:, a:a + n], BF16_TOL, f"Y leaf {l}")
        assert_close(host(g["dA"][l * r:(l + 1) * r]), gr["dA"][l * r:(l + 1) * r], BF16_TOL, f"dA leaf {l}")
        assert_close(host(g["dB"][a:a + n]), gr["dB"][a:a + n], BF16_TOL, f"dB leaf {l}")
        a += n


def test_multi_recomputed_u_and_no_dx():
    require_gpu()
    c = inputs.multi_case(8, 300, 256, (320, 192, 256), 16, [0.5, -1.5, 2.0], with_bias=True)
    import lora_dora_linear_amd as L
    X, W0, A, B, dY, bias = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY", "bias"))
    Y, U = L.lora_multi_linear_fwd(X, W0, A, B, c.n_leaf, c.s_leaf, bias=bias, save_u=False)
    assert U is None
    g = L.lora_multi_linear_bwd(dY, X, W0, A, B, c.n_leaf, c.s_leaf, U=None, need_dx=False)
    torch.cuda.synchronize()
    assert g["dX"] is None and g["dbias"] is None
    Xf, W0f, Af, Bf, dYf, bf = (c.f64(k) for k in ("X", "W0", "A", "B", "dY", "bias"))
    assert_close(host(Y), omulti.multi_forward(Xf, W0f, Af, Bf, c.n_leaf, c.s_leaf, bf), BF16_TOL, "Y")
    gr = omulti.multi_backward(dYf, Xf, W0f, Af, Bf, c.n_leaf, c.s_leaf)
    for k in ("dA", "dB"):
        assert_close(host(g[k]), gr[k], BF16_TOL, k)


def test_multi_matches_separate_layers():
    # the fused call against three single-adapter calls on the column blocks: the leaf
    # columns of Y and the factor gradients agree to bf16 rounding of the two routes
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.multi_case(9, 512, 512, (512, 256, 256), 16, [1.0, 0.5, 2.0])
    X, W0, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
    Y, U = L.lora_multi_linear_fwd(X, W0, A, B, c.n_leaf, c.s_leaf)
    a = 0
    for l, n in enumerate(c.n_leaf):
        Yl, _ = L.lora_linear_fwd(X, W0[a:a + n], A[l * 16:(l + 1) * 16].contiguous(), B[a:a + n].contiguous(),
                                  c.s_leaf[l])
        torch.cuda.synchronize()
        assert_close(host(Y[:, a:a + n]), host(Yl), 2 * 2.0 ** -8, f"Y leaf {l}")
        a += n


def test_multi_full_size_sampled():
    # a Llama-style fused QKV at 4096 tokens: hidden 4096, q 4096 and grouped k, v 1024 each,
    # rank 16 per leaf; outputs checked on sampled rows, factor gradients on sampled rows /
    # columns (the oracle's full [N,K] gradient would take minutes on the host)
    require_gpu()
    M, K, leaves, r = 4096, 4096, (4096, 1024, 1024), 16
    c = inputs.multi_case(3, M, K, leaves, r, [2.0, 2.0, 2.0])
    import lora_dora_linear_amd as L
    X, W0, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
    Y, U = L.lora_multi_linear_fwd(X, W0, A, B, c.n_leaf, c.s_leaf)
    g = L.lora_multi_linear_bwd(dY, X, W0, A, B, c.n_leaf, c.s_leaf, U=U)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(M, 48, replace=False))
    Xf, W0f, Af, Bf, dYf = (c.f64(k) for k in ("X", "W0", "A", "B", "dY"))
    Wp = omulti.adapted_weight(W0f, Af, Bf, c.n_leaf, c.s_leaf)
    assert_close(host(Y[rows]), Xf[rows] @ Wp.T, BF16_TOL, "Y rows")
    assert_close(host(g["dX"][rows]), dYf[rows] @ Wp, BF16_TOL, "dX rows")
    n_rows = np.array([0, 1, 4095, 4096, 4097, 5119, 5120, 6143])
    k_cols = np.array([0, 63, 64, 2047, 4095])
    sm = omulti.multi_weight_grads_sampled(dYf, Xf, Af, Bf, c.n_leaf, c.s_leaf, n_rows, k_cols)
    assert_close(host(g["dB"][n_rows]), sm["dB_rows"], BF16_TOL, "dB rows")
    assert_close(host(g["dA"][:, k_cols]), sm["dA_cols"], BF16_TOL, "dA cols")
