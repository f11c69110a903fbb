"""GPU parity of the SwiGLU LoRA MLP against the fp64 oracle."""
import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import swiglu as osw
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu

TOL = 5e-3
# H = silu(E) * Gu is formed from the stored bf16 E and Gu (when the gate and up products
# run as two GEMMs) and rounded once more: three roundings of 2^-9 relative, the one of E
# amplified by e.silu'(e)/silu(e) = 1 + e(1 - sigmoid(e)) <= 1.28 where silu(e) > 0 is not
# small, bound the error at (1.28 + 2) 2^-9 = 6.4e-3 of max|H|.
TOL_H = 7e-3


def _dev_proj(c, tag, s):
    return (dev(c.t["W" + tag], "bf16"), dev(c.t["A" + tag], "bf16"), dev(c.t["B" + tag], "bf16"), s)


def _run(c):
    import lora_dora_linear_amd as L
    X, dO = dev(c.t["X"], "bf16"), dev(c.t["dY"], "bf16")
    gate, up, down = (_dev_proj(c, t, c.s) for t in ("g", "u", "d"))
    Out, saved = L.swiglu_lora_mlp_fwd(X, gate, up, down)
    g = L.swiglu_lora_mlp_bwd(dO, X, gate, up, down, saved)
    torch.cuda.synchronize()
    return Out, saved, g


@pytest.mark.parametrize("M,K,H,r", [(200, 256, 384, 16), (300, 384, 256, 64)])
def test_swiglu_parity(M, K, H, r):
    require_gpu()
    c = inputs.mlp_case(4, M, K, H, r, 0.25)
    Out, saved, g = _run(c)
    X, dO = c.f64("X"), c.f64("dY")
    P = [c.proj(p) for p in ("gate", "up", "down")]
    f = osw.swiglu_mlp_forward(X, *P)
    b = osw.swiglu_mlp_backward(dO, X, *P)
    assert_close(host(Out), f["O"], TOL, "Out")
    assert_close(host(saved["E"]), f["E"], TOL, "E")
    assert_close(host(saved["Gu"]), f["Gu"], TOL, "Gu")
    assert_close(host(saved["H"]), f["H"], TOL_H, "H")
    assert_close(host(g["dX"]), b["dX"], TOL, "dX")
    for p in ("gate", "up", "down"):
        for w in ("dA_", "dB_"):
            assert_close(host(g[w + p]), b[w + p], TOL, w + p)


@pytest.mark.parametrize("M,K,H,r", [(300, 384, 512, 16), (129, 256, 768, 64)])
def test_swiglu_gate_up_routes(M, K, H, r):
    """Hidden widths a multiple of 256: gate and up as two four-wave products plus the
    streaming activation pass, and (four-wave tiles switched off) as one dual tile; both
    against the oracle, the saved E and Gu of the two routes within rounding of each other."""
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.mlp_case(7, M, K, H, r, 0.25)
    Out1, saved1, g1 = _run(c)
    L.set_tuning(1, 0)
    try:
        Out2, saved2, g2 = _run(c)
    finally:
        L.set_tuning(1, 1)
    X, dO = c.f64("X"), c.f64("dY")
    P = [c.proj(p) for p in ("gate", "up", "down")]
    f = osw.swiglu_mlp_forward(X, *P)
    b = osw.swiglu_mlp_backward(dO, X, *P)
    for Out, saved, g in ((Out1, saved1, g1), (Out2, saved2, g2)):
        assert_close(host(Out), f["O"], TOL, "Out")
        for k in ("E", "Gu"):
            assert_close(host(saved[k]), f[k], TOL, k)
        assert_close(host(saved["H"]), f["H"], TOL_H, "H")
        assert_close(host(g["dX"]), b["dX"], TOL, "dX")
        for p in ("gate", "up", "down"):
            for w in ("dA_", "dB_"):
                assert_close(host(g[w + p]), b[w + p], TOL, w + p)
    # H of the split route is silu(E) * Gu of its own stored E and Gu, rounded once
    E, Gu = host(saved1["E"]), host(saved1["Gu"])
    assert_close(host(saved1["H"]), osw.silu(E) * Gu, 2.0 ** -8, "H from stored E, Gu")


@pytest.mark.parametrize("r", [32, 64])
def test_swiglu_row_projection_32_row_blocks(r):
    """The gate/up row projection runs rank 2r over two factor segments [Ag; Au] (64 and
    128 here); forced onto 32-row blocks it gives the same bits as on 16-row blocks."""
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.mlp_case(9, 300, 256, 512, r, 0.25)
    runs = []
    for mode in (2, 0):
        L.set_tuning(2, mode)
        try:
            runs.append(_run(c))
        finally:
            L.set_tuning(2, 1)
    (O2, s2, g2), (O0, s0, g0) = runs
    assert torch.equal(O2, O0)
    for k in s0:
        assert torch.equal(s2[k], s0[k]), k
    for k in g0:
        assert torch.equal(g2[k], g0[k]), k
    X = c.f64("X")
    P = [c.proj(p) for p in ("gate", "up", "down")]
    assert_close(host(O2), osw.swiglu_mlp_forward(X, *P)["O"], TOL, "Out")


def test_swiglu_zero_adapters_is_plain_mlp():
    require_gpu()
    c = inputs.mlp_case(4, 200, 256, 384, 16, 0.25, zero_B=True)
    Out, _, _ = _run(c)
    X = c.f64("X")
    Wg, Wu, Wd = c.f64("Wg"), c.f64("Wu"), c.f64("Wd")
    e = X @ Wg.T
    plain = (osw.silu(e) * (X @ Wu.T)) @ Wd.T
    assert_close(host(Out), plain, TOL, "Out")


def test_swiglu_full_size_sampled():
    """M 8192, K 4096, H 14336, r 64, s 0.25: sampled rows of Out and dX, and the
    per-projection identity <dA, A> = <dB, B> on the full factor gradients."""
    require_gpu()
    c = inputs.mlp_case(4, 8192, 4096, 14336, 64, 0.25)
    Out, saved, g = _run(c)
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(8192, 4, replace=False))
    P = [c.proj(p) for p in ("gate", "up", "down")]
    X, dO = c.f64("X")[rows], c.f64("dY")[rows]
    f = osw.swiglu_mlp_forward(X, *P)
    assert_close(host(Out[rows]), f["O"], TOL, "Out rows")
    dXr = osw.swiglu_mlp_dx_rows(dO, X, *P)
    assert_close(host(g["dX"][rows]), dXr, TOL, "dX rows")
    for p, tag in (("gate", "g"), ("up", "u"), ("down", "d")):
        A, B = c.f64("A" + tag), c.f64("B" + tag)
        lhs = float(np.sum(host(g["dA_" + p]) * A))
        rhs = float(np.sum(host(g["dB_" + p]) * B))
        assert abs(lhs - rhs) <= 5e-3 * max(abs(lhs), abs(rhs), 1e-6), (p, lhs, rhs)
