"""GPU parity of the SwiGLU LoRA MLP against the fp64 oracle."""
import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import swiglu as osw
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu

TOL = 5e-3


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


def test_swiglu_prepacked_factors_match_the_packing_pass():
    """r = 64 (dAg, dAu as two rank-64 column projections): V_g and V_u written packed by their
    row projections give the same bits as packing them in a separate pass."""
    require_gpu()
    from lora_dora_linear_amd import binding
    c = inputs.mlp_case(9, 300, 256, 384, 64, 0.25)
    try:
        binding.set_tuning(3, 1)
        _, _, g1 = _run(c)
        binding.set_tuning(3, 0)
        _, _, g0 = _run(c)
    finally:
        binding.set_tuning(3, 1)
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g0[k]), k


@pytest.mark.parametrize("M,K,H,r", [(200, 256, 384, 16), (300, 384, 256, 64), (64, 256, 512, 32),
                                     (100, 192, 256, 16), (300, 256, 320, 16)])
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
    assert_close(host(saved["H"]), f["H"], TOL, "H")
    assert_close(host(g["dX"]), b["dX"], TOL, "dX")
    for p in ("gate", "up", "down"):
        for w in ("dA_", "dB_"):
            assert_close(host(g[w + p]), b[w + p], TOL, w + p)


@pytest.mark.parametrize("M,K,H,r", [(300, 384, 512, 16), (129, 256, 768, 64), (513, 256, 384, 32)])
def test_swiglu_gate_up_routes(M, K, H, r):
    """Gate and up in one dual tile per 128 hidden units with h = silu(e) u formed from the
    fp32 accumulators: the four-wave tile (hidden width a multiple of 128, more than 128
    tokens; ragged row tails) and, four-wave tiles switched off, the eight-wave dual tile;
    both against the oracle."""
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
        assert_close(host(saved["H"]), f["H"], TOL, "H")
        assert_close(host(g["dX"]), b["dX"], TOL, "dX")
        for p in ("gate", "up", "down"):
            for w in ("dA_", "dB_"):
                assert_close(host(g[w + p]), b[w + p], TOL, w + p)


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
    """M 8192, K 4096, H 14336, r 64, s 0.25: Out and dX on 16 sampled rows; every factor
    gradient on sampled rows / columns of the weight-shaped gradients, element by element."""
    require_gpu()
    c = inputs.mlp_case(4, 8192, 4096, 14336, 64, 0.25)
    Out, saved, g = _run(c)
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(8192, 16, replace=False))
    P = [c.proj(p) for p in ("gate", "up", "down")]
    X, dO = c.f64("X"), c.f64("dY")
    f = osw.swiglu_mlp_forward(X[rows], *P)
    assert_close(host(Out[rows]), f["O"], TOL, "Out rows")
    for k in ("E", "Gu", "H"):
        assert_close(host(saved[k][rows]), f[k], TOL, k + " rows")
    dXr = osw.swiglu_mlp_dx_rows(dO[rows], X[rows], *P)
    assert_close(host(g["dX"][rows]), dXr, TOL, "dX rows")
    h_idx = np.sort(rng.choice(14336, 16, replace=False))
    k_idx = np.sort(rng.choice(4096, 16, replace=False))
    smp = osw.swiglu_mlp_grads_sampled(dO, X, *P, h_idx, k_idx)
    for p in ("gate", "up"):
        assert_close(host(g["dB_" + p][h_idx]), smp["dB_" + p + "_rows"], TOL, "dB_" + p)
        assert_close(host(g["dA_" + p][:, k_idx]), smp["dA_" + p + "_cols"], TOL, "dA_" + p)
    assert_close(host(g["dB_down"][k_idx]), smp["dB_down_rows"], TOL, "dB_down")
    assert_close(host(g["dA_down"][:, h_idx]), smp["dA_down_cols"], TOL, "dA_down")
