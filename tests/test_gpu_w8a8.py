"""GPU parity of the int8 (W8A8) base with the LoRA epilogue against the oracle.

The quantiser's integer codes are compared bit for bit (both sides divide in
float32 and round half to even); the raw int32 product is compared bit for bit
with an int64 product; outputs and gradients use the 5e-3 tolerance.
"""
import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import lora as olora
from oracle import w8a8 as ow
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu

TOL = 5e-3


def _case(M, N, K, r, s=0.5, seed=5):
    c = inputs.linear_case(seed, M, N, K, r, s, "bf16", with_bias=False)
    W0f = inputs.normal(seed, 1, (N, K), 1.0 / np.sqrt(K), "f32")    # float32 base weight
    return c, W0f


def test_quantizers_bit_exact():
    require_gpu()
    import lora_dora_linear_amd as L
    c, W0f = _case(300, 512, 640, 32)
    Xq, sx = L.w8a8_quantize_rows(dev(c.t["X"], "bf16"))
    Wq, sw = L.w8a8_quantize_weight(dev(W0f, "f32"))
    torch.cuda.synchronize()
    q_ref, s_ref = ow.quantize_rows_int8(inputs.bf16_bits_to_f32(c.t["X"]))
    np.testing.assert_array_equal(Xq.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(sx.cpu().numpy(), s_ref)
    wq_ref, sw_ref = ow.quantize_rows_int8(W0f)
    np.testing.assert_array_equal(Wq.cpu().numpy(), wq_ref)
    np.testing.assert_array_equal(sw.cpu().numpy(), sw_ref)
    # zero rows
    Z = torch.zeros((3, 128), dtype=torch.bfloat16, device="cuda")
    zq, zs = L.w8a8_quantize_rows(Z)
    torch.cuda.synchronize()
    assert not torch.any(zq) and not torch.any(zs)


@pytest.mark.parametrize("K", [512, 5120, 8192])
def test_quantize_rows_bit_exact_one_read(K):
    """Rows of a multiple of 512 up to 8192 elements are quantised from one read of the row
    (kept in registers); codes and scales must equal the oracle's bit for bit."""
    require_gpu()
    import lora_dora_linear_amd as L
    rng = np.random.default_rng(K)
    x = rng.standard_normal((130, K)).astype(np.float32)
    x[7] = 0.0                                       # a zero row: scale 0, codes 0
    bits = inputs.f32_to_bf16_bits(x)
    Xq, sx = L.w8a8_quantize_rows(dev(bits, "bf16"))
    torch.cuda.synchronize()
    q_ref, s_ref = ow.quantize_rows_int8(inputs.bf16_bits_to_f32(bits))
    np.testing.assert_array_equal(Xq.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(sx.cpu().numpy(), s_ref)


@pytest.mark.parametrize("M,N,K", [(300, 512, 640), (100, 192, 256), (1024, 1024, 1024)])
def test_int8_raw_product_exact(M, N, K):
    require_gpu()
    import lora_dora_linear_amd as L
    rng = np.random.default_rng(7)
    a = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    b = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    C = L.int8_gemm_raw(dev(a, "i8"), dev(b, "i8"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(C.cpu().numpy().astype(np.int64), ow.int_product(a, b))


def _run(c, W0f, need_dx=True, bias=None):
    import lora_dora_linear_amd as L
    X, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "A", "B", "dY"))
    Wq, sw = L.w8a8_quantize_weight(dev(W0f, "f32"))
    Y, Xq, sx, U = L.w8a8_lora_linear_fwd(X, Wq, sw, A, B, c.s, bias=None if bias is None else dev(bias, "bf16"))
    g = L.w8a8_lora_linear_bwd(dY, X, Wq, sw, A, B, c.s, U=U, need_dx=need_dx)
    torch.cuda.synchronize()
    return Y, Xq, sx, g


@pytest.mark.parametrize("M,N,K,r", [(300, 512, 640, 32), (129, 256, 256, 16), (64, 384, 256, 32),
                                     (100, 192, 384, 16)])
def test_w8a8_parity(M, N, K, r):
    require_gpu()
    c, W0f = _case(M, N, K, r)
    Y, Xq, sx, g = _run(c, W0f)
    Wq_ref, sw_ref = ow.quantize_rows_int8(W0f)
    X, A, B, dY = (c.f64(k) for k in ("X", "A", "B", "dY"))
    f = ow.w8a8_forward(X, Wq_ref, sw_ref, A, B, c.s)
    b = ow.w8a8_backward(dY, X, Wq_ref, sw_ref, A, B, c.s)
    np.testing.assert_array_equal(Xq.cpu().numpy(), f["Xq"])
    assert_close(host(Y), f["Y"], TOL, "Y")
    for k in ("dX", "dA", "dB"):
        assert_close(host(g[k]), b[k], TOL, k)


@pytest.mark.parametrize("M", [1024, 2048, 4096, 8192, 16384])
def test_w8a8_full_size_sampled(M):
    """K = N = 5120, r = 32, s = 0.5 at every point of the M sweep: sampled rows and entries."""
    require_gpu()
    c, W0f = _case(M, 5120, 5120, 32)
    Y, Xq, sx, g = _run(c, W0f)
    Wq_ref, sw_ref = ow.quantize_rows_int8(W0f)
    rng = np.random.default_rng(2)
    rows = np.sort(rng.choice(M, 16, replace=False))
    X, A, B, dY = (c.f64(k) for k in ("X", "A", "B", "dY"))
    f = ow.w8a8_forward(X[rows], Wq_ref, sw_ref, A, B, c.s)
    assert_close(host(Y[rows]), f["Y"], TOL, "Y rows")
    b = ow.w8a8_backward(dY[rows], X[rows], Wq_ref, sw_ref, A, B, c.s)
    assert_close(host(g["dX"][rows]), b["dX"], TOL, "dX rows")
    ncols = np.sort(rng.choice(5120, 12, replace=False))
    kcols = np.sort(rng.choice(5120, 12, replace=False))
    smp = olora.lora_weight_grads_sampled(dY, X, A, B, c.s, ncols, kcols)
    assert_close(host(g["dB"][ncols]), smp["dB_rows"], TOL, "dB rows")
    assert_close(host(g["dA"][:, kcols]), smp["dA_cols"], TOL, "dA cols")


def test_w8a8_bias_and_no_input_gradient():
    """Bias added after the dequantised base and the low-rank term; with dX not requested
    the factor gradients are the same bits."""
    require_gpu()
    c, W0f = _case(300, 512, 640, 32, seed=18)
    bias = inputs.normal(18, 6, (512,), 0.5, "bf16")
    Y, Xq, sx, g = _run(c, W0f, need_dx=True, bias=bias)
    Y2, _, _, g2 = _run(c, W0f, need_dx=False, bias=bias)
    Wq_ref, sw_ref = ow.quantize_rows_int8(W0f)
    X, A, B, dY = (c.f64(k) for k in ("X", "A", "B", "dY"))
    f = ow.w8a8_forward(X, Wq_ref, sw_ref, A, B, c.s, bias=inputs.bf16_bits_to_f64(bias))
    assert_close(host(Y), f["Y"], TOL, "Y with bias")
    assert torch.equal(Y, Y2)
    assert g2["dX"] is None
    b = ow.w8a8_backward(dY, X, Wq_ref, sw_ref, A, B, c.s)
    for k in ("dA", "dB"):
        assert_close(host(g2[k]), b[k], TOL, k)
        assert torch.equal(g[k], g2[k]), k


@pytest.mark.parametrize("M,N,K,r", [(300, 512, 640, 32), (513, 768, 256, 16), (129, 256, 384, 48)])
def test_w8a8_int8_forward_routes(M, N, K, r):
    """The W8A8 forward on the four-wave int8 tile (exact int32 accumulators dequantised after
    the loop, then the low-rank k-tile; the default when N is a multiple of 256 and 256 x 128
    tiles would not fit the chip in one round, forced here) and, four-wave tiles switched off,
    on the eight-wave tile: both against the oracle; ragged row tails, rank 16 / 32 with the
    hi + lo low-rank term and rank 48 without."""
    require_gpu()
    import lora_dora_linear_amd as L
    c, W0f = _case(M, N, K, r, seed=19)
    X, A, B = (dev(c.t[k], "bf16") for k in ("X", "A", "B"))
    bias = inputs.normal(19, 6, (N,), 0.5, "bf16")
    Wq, sw = L.w8a8_quantize_weight(dev(W0f, "f32"))
    L.set_tuning(1, 2)         # the four-wave int8 tile at these small sizes too
    try:
        Y4, Xq, sx, U = L.w8a8_lora_linear_fwd(X, Wq, sw, A, B, c.s, bias=dev(bias, "bf16"))
    finally:
        L.set_tuning(1, 1)
    L.set_tuning(1, 0)
    try:
        Y8, _, _, _ = L.w8a8_lora_linear_fwd(X, Wq, sw, A, B, c.s, bias=dev(bias, "bf16"))
    finally:
        L.set_tuning(1, 1)
    torch.cuda.synchronize()
    Wq_ref, sw_ref = ow.quantize_rows_int8(W0f)
    f = ow.w8a8_forward(c.f64("X"), Wq_ref, sw_ref, c.f64("A"), c.f64("B"), c.s, bias=inputs.bf16_bits_to_f64(bias))
    assert_close(host(Y4), f["Y"], TOL, "Y four-wave")
    assert_close(host(Y8), f["Y"], TOL, "Y eight-wave")
