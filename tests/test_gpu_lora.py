"""GPU parity of the LoRA linear (forward and backward) against the fp64 oracle.

All calls go through the C interface (ctypes binding) on the same seeded inputs
the oracle receives.  Tolerance: max|gpu - ref| / max|ref| per tensor, 1e-5
(outputs) and 1e-4 (gradients) for fp32, 5e-3 for bf16.
"""
import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import lora as olora
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu

BF16_TOL = 5e-3


def _run(c, with_bias=False, need_dbias=False):
    import lora_dora_linear_amd as L
    kind = c.dtype
    X, W0, A, B, dY = (dev(c.t[k], kind) for k in ("X", "W0", "A", "B", "dY"))
    bias = dev(c.t["bias"], kind) if with_bias else None
    Y, U = L.lora_linear_fwd(X, W0, A, B, c.s, bias=bias)
    g = L.lora_linear_bwd(dY, X, W0, A, B, c.s, U=U, need_dbias=need_dbias)
    torch.cuda.synchronize()
    return Y, U, g


def _oracle(c, with_bias=False):
    X, W0, A, B, dY = (c.f64(k) for k in ("X", "W0", "A", "B", "dY"))
    bias = c.f64("bias") if with_bias else None
    return olora.lora_forward(X, W0, A, B, c.s, bias), olora.lora_backward(dY, X, W0, A, B, c.s), X @ A.T


# ---------------------------------------------------------------- fp32, the tiny configuration
@pytest.mark.parametrize("variant", ["s2", "s0", "B0", "W00"])
def test_fp32_tiny(variant):
    require_gpu()
    s = 0.0 if variant == "s0" else 2.0
    c = inputs.linear_case(1, 64, 256, 256, 8, s, "f32", with_bias=True,
                           zero_B=(variant == "B0"), zero_W0=(variant == "W00"))
    Y, U, g = _run(c, with_bias=True, need_dbias=True)
    Yr, gr, Ur = _oracle(c, with_bias=True)
    assert_close(host(Y), Yr, 1e-5, "Y")
    assert_close(host(U), Ur, 1e-5, "U")
    for k in ("dX", "dA", "dB"):
        if not np.any(gr[k]):
            assert not np.any(host(g[k])), k
        else:
            assert_close(host(g[k]), gr[k], 1e-4, k)
    assert_close(host(g["dbias"]), gr["db"], 1e-4, "dbias")
    if variant in ("s0", "B0"):
        X, W0 = c.f64("X"), c.f64("W0")
        assert_close(host(Y), X @ W0.T + c.f64("bias"), 1e-5, "Y vs base")


# fp32 layers small enough for the one-launch forward / backward (M <= 256, N and K multiples
# of 16 up to 1024, r <= 16), a ragged M tail, r not a multiple of 4, and shapes just outside
# those limits (the multi-launch path): each against the oracle, and the factor gradients the
# same bits with U saved and with U recomputed.
F32_SHAPES = [
    (37, 80, 48, 5),      # ragged M, odd r
    (200, 1024, 64, 16),  # four row blocks per wave in the dA / dB jobs, N at its limit
    (256, 32, 1024, 3),   # K at its limit
    (1, 16, 16, 1),       # one row, one rank
    (64, 250, 256, 8),    # N not a multiple of 16: multi-launch
    (300, 256, 256, 8),   # M above 256: multi-launch
    (64, 256, 256, 17),   # r above 16: multi-launch
]


@pytest.mark.parametrize("M,N,K,r", F32_SHAPES)
def test_fp32_small_shapes(M, N, K, r):
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(5, M, N, K, r, 1.5, "f32", with_bias=True)
    Y, U, g = _run(c, with_bias=True, need_dbias=True)
    Yr, gr, Ur = _oracle(c, with_bias=True)
    assert_close(host(Y), Yr, 1e-5, "Y")
    assert_close(host(U), Ur, 1e-5, "U")
    for k in ("dX", "dA", "dB"):
        assert_close(host(g[k]), gr[k], 1e-4, k)
    assert_close(host(g["dbias"]), gr["db"], 1e-4, "dbias")
    X, W0, A, B, dY = (dev(c.t[k], "f32") for k in ("X", "W0", "A", "B", "dY"))
    g2 = L.lora_linear_bwd(dY, X, W0, A, B, c.s, U=None)
    torch.cuda.synchronize()
    for k in ("dA", "dB"):
        assert torch.equal(g[k], g2[k]), k + " with U recomputed"


# ---------------------------------------------------------------- bf16 at several tile shapes with a ragged M tail
SHAPES = [
    # M, N, K, r     (256x256 tiles, 256x192, 256x128, 128-row tiles; r not a multiple of 16; r = 128)
    (300, 512, 384, 16),
    (300, 576, 256, 32),
    (257, 384, 640, 48),
    (100, 640, 128, 8),
    (64, 192, 128, 128),
]


@pytest.mark.parametrize("M,N,K,r", SHAPES)
def test_bf16_parity(M, N, K, r):
    require_gpu()
    c = inputs.linear_case(2, M, N, K, r, 0.5, "bf16", with_bias=True)
    Y, U, g = _run(c, with_bias=True, need_dbias=True)
    Yr, gr, Ur = _oracle(c, with_bias=True)
    assert_close(host(Y), Yr, BF16_TOL, "Y")
    assert_close(host(U), Ur, 1e-5, "U")
    for k in ("dX", "dA", "dB"):
        assert_close(host(g[k]), gr[k], BF16_TOL, k)
    assert_close(host(g["dbias"]), gr["db"], 1e-5, "dbias")


def test_bf16_pure_low_rank_path():
    """W0 = 0: everything in Y comes from the rank-r epilogue, so it cannot hide under the base term."""
    require_gpu()
    c = inputs.linear_case(2, 300, 512, 384, 16, 0.5, "bf16", zero_W0=True)
    Y, U, g = _run(c)
    Yr, gr, _ = _oracle(c)
    assert_close(host(Y), Yr, BF16_TOL, "Y")
    assert_close(host(g["dX"]), gr["dX"], BF16_TOL, "dX")


def _excess_over_rounding(gpu_bf16, ref):
    """max over elements of (|gpu - ref| - half a bf16 unit in the last place of ref), at least
    0, divided by max|ref|: the error left once the output's own rounding is allowed for."""
    g = host(gpu_bf16)
    ref = np.asarray(ref, np.float64)
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-300))) - 8)
    return float(np.max(np.maximum(np.abs(g - ref) - half_ulp, 0.0)) / np.max(np.abs(ref)))


def test_bf16_low_rank_term_keeps_precision():
    """W0 = 0 on the four-wave tiles (rank 16): the low-rank term enters the MFMAs as the bf16
    pair hi + lo of s.U (resp. s.V), so beyond the output's own rounding Y and dX carry only
    fp32-level error (~1e-6 of max|ref|).  A single bf16 rounding of s.U would leave ~1e-3."""
    require_gpu()
    c = inputs.linear_case(19, 300, 512, 512, 16, 0.5, "bf16", zero_W0=True)
    Y, U, g = _run(c)
    Yr, gr, _ = _oracle(c)
    for name, got, ref in (("Y", Y, Yr), ("dX", g["dX"], gr["dX"])):
        e = _excess_over_rounding(got, ref)
        print(f"{name}: error beyond the bf16 rounding = {e:.2e} of max|ref|")
        assert e < 2e-5, (name, e)


def test_bf16_zero_delta_bitwise():
    """s = 0 and B = 0 give bit-identical outputs, equal to X.W0^T within tolerance."""
    require_gpu()
    c0 = inputs.linear_case(2, 300, 512, 384, 16, 0.0, "bf16")
    cB = inputs.linear_case(2, 300, 512, 384, 16, 0.7, "bf16", zero_B=True)
    Y0, _, g0 = _run(c0)
    YB, _, gB = _run(cB)
    assert torch.equal(Y0, YB)
    assert torch.equal(g0["dX"], gB["dX"])
    X, W0 = c0.f64("X"), c0.f64("W0")
    assert_close(host(Y0), X @ W0.T, BF16_TOL, "Y vs X.W0^T")
    assert not torch.any(g0["dA"]) and not torch.any(g0["dB"])
    assert not torch.any(gB["dA"])


def test_bf16_fused_down_projection():
    """U = X.A^T computed inside the base GEMM's K-loop matches the separate pass."""
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(3, 300, 512, 384, 16, 0.5, "bf16", with_bias=True)
    X, W0, A, B = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B"))
    bias = dev(c.t["bias"], "bf16")
    Y1, U1 = L.lora_linear_fwd(X, W0, A, B, c.s, bias=bias)
    L.set_tuning(0, 1)
    try:
        Y2, U2 = L.lora_linear_fwd(X, W0, A, B, c.s, bias=bias)
    finally:
        L.set_tuning(0, 0)
    torch.cuda.synchronize()
    Yr, _, Ur = _oracle(c, with_bias=True)
    assert_close(host(Y2), Yr, BF16_TOL, "Y fused")
    assert_close(host(U2), Ur, 1e-5, "U fused")
    assert_close(host(Y2), host(Y1), BF16_TOL, "fused vs separate")


@pytest.mark.parametrize("M,N,K,r", [
    # the four-wave 256x256 tiles (forward Y when N % 256 == 0, input gradient dX when
    # K % 256 == 0): odd and single k-tile counts, one and two 32-rank steps of the
    # low-rank term, ragged row counts
    (300, 512, 320, 16),
    (300, 320, 512, 16),
    (129, 256, 64, 48),
    (129, 64, 256, 48),
    (513, 768, 448, 64),
    (513, 448, 768, 64),
    (260, 256, 256, 8),
    # the 192-column four-wave forward tile (N a multiple of 192 whose 256-column tiles
    # underfill the chip; 768 above takes it too): odd k-tile count, N not a multiple of 256
    (300, 384, 320, 16),
    (129, 576, 256, 8),
])
def test_bf16_four_wave_tiles(M, N, K, r):
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(6, M, N, K, r, 0.5, "bf16", with_bias=True)
    X, W0, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
    bias = dev(c.t["bias"], "bf16")

    def run():
        Y, U = L.lora_linear_fwd(X, W0, A, B, c.s, bias=bias)
        g = L.lora_linear_bwd(dY, X, W0, A, B, c.s, U=U)
        return Y, U, g["dX"]

    Y4, U4, dX4 = run()
    L.set_tuning(1, 0)
    try:
        Y8, _, dX8 = run()
    finally:
        L.set_tuning(1, 1)
    Y4b, _, dX4b = run()
    torch.cuda.synchronize()
    Yr, gr, Ur = _oracle(c, with_bias=True)
    assert_close(host(Y4), Yr, BF16_TOL, "Y four-wave")
    assert_close(host(U4), Ur, 1e-5, "U")
    assert_close(host(dX4), gr["dX"], BF16_TOL, "dX four-wave")
    assert_close(host(Y8), Yr, BF16_TOL, "Y eight-wave")
    assert_close(host(dX8), gr["dX"], BF16_TOL, "dX eight-wave")
    assert torch.equal(Y4, Y4b) and torch.equal(dX4, dX4b)


@pytest.mark.parametrize("M,N,K,r", [(300, 512, 640, 64), (129, 384, 256, 48), (200, 256, 192, 128)])
def test_bf16_row_projection_32_row_blocks(M, N, K, r):
    """Rank 33..128 row projections (U = X.A^T, V = dY.B with B read transposed) on 32-row
    blocks, forced at small M: the same bits as on 16-row blocks, and against the oracle
    (ragged last block, ragged last chunk of K)."""
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(8, M, N, K, r, 0.5, "bf16")
    runs = []
    for mode in (2, 0):
        L.set_tuning(2, mode)
        try:
            Y, U, g = _run(c)
        finally:
            L.set_tuning(2, 1)
        runs.append((Y, U, g))
    (Y2, U2, g2), (Y0, U0, g0) = runs
    assert torch.equal(U2, U0) and torch.equal(Y2, Y0)
    for k in ("dX", "dA", "dB"):
        assert torch.equal(g2[k], g0[k]), k
    Yr, gr, Ur = _oracle(c)
    assert_close(host(U2), Ur, 1e-5, "U")
    assert_close(host(Y2), Yr, BF16_TOL, "Y")
    for k in ("dX", "dA", "dB"):
        assert_close(host(g2[k]), gr[k], BF16_TOL, k)


def test_bf16_deterministic():
    require_gpu()
    c = inputs.linear_case(4, 300, 512, 384, 16, 0.5, "bf16")
    Y1, _, g1 = _run(c)
    Y2, _, g2 = _run(c)
    assert torch.equal(Y1, Y2)
    for k in ("dX", "dA", "dB"):
        assert torch.equal(g1[k], g2[k]), k


def test_empty_batch():
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(5, 0, 256, 256, 16, 0.5, "bf16")
    X, W0, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
    Y, U = L.lora_linear_fwd(X, W0, A, B, c.s)
    g = L.lora_linear_bwd(dY, X, W0, A, B, c.s, U=U, need_dbias=True)
    torch.cuda.synchronize()
    assert Y.shape == (0, 256)
    assert not torch.any(g["dA"]) and not torch.any(g["dB"]) and not torch.any(g["dbias"])


def test_full_size_4096_sampled():
    """M = K = N = 4096, r = 16, s = 0.5 (the benchmark launch configuration): sampled rows / entries."""
    require_gpu()
    c = inputs.linear_case(2, 4096, 4096, 4096, 16, 0.5, "bf16")
    Y, U, g = _run(c)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(4096, 24, replace=False))
    X, W0, A, B, dY = (c.f64(k) for k in ("X", "W0", "A", "B", "dY"))
    Yr = olora.lora_forward(X[rows], W0, A, B, c.s)
    assert_close(host(Y[rows]), Yr, BF16_TOL, "Y rows")
    dXr = olora.lora_backward(dY[rows], X[rows], W0, A, B, c.s)["dX"]
    assert_close(host(g["dX"][rows]), dXr, BF16_TOL, "dX rows")
    ncols = np.sort(rng.choice(4096, 16, replace=False))
    kcols = np.sort(rng.choice(4096, 16, replace=False))
    smp = olora.lora_weight_grads_sampled(dY, X, A, B, c.s, ncols, kcols)
    assert_close(host(g["dB"][ncols]), smp["dB_rows"], BF16_TOL, "dB rows")
    assert_close(host(g["dA"][:, kcols]), smp["dA_cols"], BF16_TOL, "dA cols")


@pytest.mark.parametrize("dtype,M,N,K,r", [("bf16", 300, 512, 384, 16), ("f32", 64, 256, 256, 8)])
def test_without_input_gradient(dtype, M, N, K, r):
    """dX not requested: the factor gradients are the same bits as with dX."""
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(17, M, N, K, r, 0.5, dtype)
    X, W0, A, B, dY = (dev(c.t[k], dtype) for k in ("X", "W0", "A", "B", "dY"))
    Y, U = L.lora_linear_fwd(X, W0, A, B, c.s)
    g0 = L.lora_linear_bwd(dY, X, W0, A, B, c.s, U=U, need_dx=False)
    g1 = L.lora_linear_bwd(dY, X, W0, A, B, c.s, U=U, need_dx=True)
    g2 = L.lora_linear_bwd(dY, X, W0, A, B, c.s, U=None, need_dx=False)
    torch.cuda.synchronize()
    assert g0["dX"] is None
    _, gr, _ = _oracle(c)
    tol = BF16_TOL if dtype == "bf16" else 1e-4
    for k in ("dA", "dB"):
        assert_close(host(g0[k]), gr[k], tol, k)
        assert torch.equal(g0[k], g1[k]), k
        assert torch.equal(g0[k], g2[k]), k + " with U recomputed"


def test_fp32_tiny_latency():
    """c1 (fp32, 64 x 256 x 256, r = 8): forward + backward time on the GPU, printed (launch-bound)."""
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(1, 64, 256, 256, 8, 2.0, "f32")
    X, W0, A, B, dY = (dev(c.t[k], "f32") for k in ("X", "W0", "A", "B", "dY"))

    def step():
        Y, U = L.lora_linear_fwd(X, W0, A, B, c.s)
        return L.lora_linear_bwd(dY, X, W0, A, B, c.s, U=U)

    for _ in range(20):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(200):
        g = step()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / 200 * 1e3
    print(f"c1 fp32 tiny LoRA fwd+bwd: {us:.1f} us per step (binding calls included)")
    _, gr, _ = _oracle(c)
    assert_close(host(g["dX"]), gr["dX"], 1e-4, "dX")
