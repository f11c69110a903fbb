"""GPU parity of the 8-bit float (e4m3) base with the LoRA epilogue against the oracle.

The quantiser's codes are compared exactly (both sides divide in float32 and round to the
nearest e4m3 value, ties to even; compared as decoded values, so that a negative quotient
rounding to zero may keep its sign bit); the scales bit for bit; outputs and gradients use
the 5e-3 tolerance of the bf16 layer.
"""
import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import fp8 as of8
from oracle import lora as olora
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu

TOL = 5e-3


def _case(M, N, K, r, s=0.5, seed=11):
    c = inputs.linear_case(seed, M, N, K, r, s, "bf16", with_bias=True)
    W0f = inputs.normal(seed, 1, (N, K), 1.0 / np.sqrt(K), "f32")
    return c, W0f


def _codes(t):
    return of8.e4m3_decode(t.cpu().numpy())


def test_fp8_quantizers_exact():
    require_gpu()
    import lora_dora_linear_amd as L
    c, W0f = _case(300, 512, 640, 32)
    Xq, sx = L.fp8_quantize_rows(dev(c.t["X"], "bf16"))
    Wq, sw = L.fp8_quantize_weight(dev(W0f, "f32"))
    Wqb, swb = L.fp8_quantize_weight(dev(c.t["W0"], "bf16"))
    torch.cuda.synchronize()
    q_ref, s_ref = of8.quantize_rows_fp8(inputs.bf16_bits_to_f32(c.t["X"]))
    np.testing.assert_array_equal(_codes(Xq), of8.e4m3_decode(q_ref))
    np.testing.assert_array_equal(sx.cpu().numpy(), s_ref)
    wq_ref, sw_ref = of8.quantize_rows_fp8(W0f)
    np.testing.assert_array_equal(_codes(Wq), of8.e4m3_decode(wq_ref))
    np.testing.assert_array_equal(sw.cpu().numpy(), sw_ref)
    wqb_ref, swb_ref = of8.quantize_rows_fp8(inputs.bf16_bits_to_f32(c.t["W0"]))
    np.testing.assert_array_equal(_codes(Wqb), of8.e4m3_decode(wqb_ref))
    np.testing.assert_array_equal(swb.cpu().numpy(), swb_ref)
    Z = torch.zeros((3, 128), dtype=torch.bfloat16, device="cuda")
    zq, zs = L.fp8_quantize_rows(Z)
    torch.cuda.synchronize()
    assert not torch.any(zq) and not torch.any(zs)


@pytest.mark.parametrize("K", [512, 5120])
def test_fp8_quantize_rows_one_read(K):
    require_gpu()
    import lora_dora_linear_amd as L
    rng = np.random.default_rng(K + 1)
    x = (rng.standard_normal((130, K)) * rng.uniform(1e-3, 1e3, (130, 1))).astype(np.float32)
    x[9] = 0.0
    bits = inputs.f32_to_bf16_bits(x)
    Xq, sx = L.fp8_quantize_rows(dev(bits, "bf16"))
    torch.cuda.synchronize()
    q_ref, s_ref = of8.quantize_rows_fp8(inputs.bf16_bits_to_f32(bits))
    np.testing.assert_array_equal(_codes(Xq), of8.e4m3_decode(q_ref))
    np.testing.assert_array_equal(sx.cpu().numpy(), s_ref)


def _run(c, W0f, need_dx=True, with_bias=True):
    import lora_dora_linear_amd as L
    X, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "A", "B", "dY"))
    bias = dev(c.t["bias"], "bf16") if with_bias else None
    Wq, sw = L.fp8_quantize_weight(dev(W0f, "f32"))
    Y, Xq, sx, U = L.fp8_lora_linear_fwd(X, Wq, sw, A, B, c.s, bias=bias)
    g = L.fp8_lora_linear_bwd(dY, X, Wq, sw, A, B, c.s, U=U, need_dx=need_dx)
    torch.cuda.synchronize()
    return Y, Xq, sx, g


SHAPES = [
    # M, N, K, r   (256-column tiles, ragged rows; 128-column tiles; odd k-tile count; r = 64; M <= 128)
    (300, 512, 640, 32),
    (129, 256, 256, 16),
    (64, 384, 256, 32),
    (100, 128, 384, 16),
    (300, 256, 512, 64),
    (513, 768, 1024, 8),
    (4097, 4096, 256, 16),     # enough tiles for the 256-column tile, one ragged row
]


@pytest.mark.parametrize("M,N,K,r", SHAPES)
def test_fp8_parity(M, N, K, r):
    require_gpu()
    c, W0f = _case(M, N, K, r)
    Y, Xq, sx, g = _run(c, W0f)
    Wq_ref, sw_ref = of8.quantize_rows_fp8(W0f)
    X, A, B, dY, bias = (c.f64(k) for k in ("X", "A", "B", "dY", "bias"))
    f = of8.fp8_forward(X, Wq_ref, sw_ref, A, B, c.s, bias)
    b = of8.fp8_backward(dY, X, Wq_ref, sw_ref, A, B, c.s)
    np.testing.assert_array_equal(_codes(Xq), of8.e4m3_decode(f["Xq"]))
    assert_close(host(Y), f["Y"], TOL, "Y")
    for k in ("dX", "dA", "dB"):
        assert_close(host(g[k]), b[k], TOL, k)


def test_fp8_base_only_and_no_dx():
    """B = 0: Y is the dequantised e4m3 product alone; need_dx = False leaves dX unset."""
    require_gpu()
    c, W0f = _case(300, 512, 512, 16)
    c.t["B"] = np.zeros_like(c.t["B"])
    Y, Xq, sx, g = _run(c, W0f, need_dx=False, with_bias=False)
    assert g["dX"] is None
    Wq_ref, sw_ref = of8.quantize_rows_fp8(W0f)
    f = of8.fp8_forward(c.f64("X"), Wq_ref, sw_ref, c.f64("A"), c.f64("B"), c.s)
    assert_close(host(Y), f["acc"] * f["sx"][:, None].astype(np.float64) * sw_ref[None, :].astype(np.float64),
                 TOL, "Y base")


@pytest.mark.parametrize("M", [1024, 2048, 4096, 8192, 16384])
def test_fp8_full_size_sampled(M):
    """K = N = 5120, r = 32, s = 0.5, every token count of the sweep (tails split three, four
    and two ways over k at 1024, 4096 and 8192 tokens): sampled rows and gradient entries."""
    require_gpu()
    c, W0f = _case(M, 5120, 5120, 32)
    Y, Xq, sx, g = _run(c, W0f, with_bias=False)
    Wq_ref, sw_ref = of8.quantize_rows_fp8(W0f)
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(M, 16, replace=False))
    X, A, B, dY = (c.f64(k) for k in ("X", "A", "B", "dY"))
    f = of8.fp8_forward(X[rows], Wq_ref, sw_ref, A, B, c.s)
    assert_close(host(Y[rows]), f["Y"], TOL, "Y rows")
    b = of8.fp8_backward(dY[rows], X[rows], Wq_ref, sw_ref, A, B, c.s)
    assert_close(host(g["dX"][rows]), b["dX"], TOL, "dX rows")
    ncols = np.sort(rng.choice(5120, 12, replace=False))
    kcols = np.sort(rng.choice(5120, 12, replace=False))
    smp = olora.lora_weight_grads_sampled(dY, X, A, B, c.s, ncols, kcols)
    assert_close(host(g["dB"][ncols]), smp["dB_rows"], TOL, "dB rows")
    assert_close(host(g["dA"][:, kcols]), smp["dA_cols"], TOL, "dA cols")
