"""Strided operands through the C interface: inputs that are row-major views into wider
buffers (leading dimension above the row length) and outputs written into column slices of
wider buffers.  Results must equal those of the dense call bit for bit (same kernels, same
tiles), match the oracle, and leave every column outside the slices untouched."""
import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import dora as odora
from oracle import lora as olora
from oracle import swiglu as osw
from oracle import w8a8 as ow
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _embed(t, pad_left, pad_right):
    """The same values as a column slice of a wider buffer filled with a sentinel."""
    big = torch.full((t.shape[0], pad_left + t.shape[1] + pad_right), SENTINEL, dtype=t.dtype, device=t.device)
    big[:, pad_left:pad_left + t.shape[1]] = t
    return big, big[:, pad_left:pad_left + t.shape[1]]


def _slot(shape, dtype, pad_left=32, pad_right=32):
    big = torch.full((shape[0], pad_left + shape[1] + pad_right), SENTINEL, dtype=dtype, device="cuda")
    return big, big[:, pad_left:pad_left + shape[1]]


def _untouched(big, view_cols, pad_left=32):
    left = big[:, :pad_left].float()
    right = big[:, pad_left + view_cols:].float()
    return bool(torch.all(left == SENTINEL)) and bool(torch.all(right == SENTINEL))


@pytest.mark.parametrize("dtype,M,N,K,r", [
    ("bf16", 300, 512, 512, 16),      # four-wave forward and input-gradient tiles
    ("bf16", 200, 384, 192, 32),      # 192-wide forward tile, eight-wave input gradient
    ("bf16", 100, 256, 320, 8),       # 128-row tiles
    ("f32", 64, 256, 256, 8),         # fp32 path
])
def test_lora_strided(dtype, M, N, K, r):
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(31, M, N, K, r, 0.5, dtype)
    X, W0, A, B, dY = (dev(c.t[k], dtype) for k in ("X", "W0", "A", "B", "dY"))
    Yd, Ud = L.lora_linear_fwd(X, W0, A, B, c.s)
    gd = L.lora_linear_bwd(dY, X, W0, A, B, c.s, U=Ud)
    _, Xs = _embed(X, 16, 48)
    _, W0s = _embed(W0, 64, 8)
    _, dYs = _embed(dY, 8, 24)
    tdt = X.dtype
    Ybig, Ys = _slot((M, N), tdt)
    Ubig, Us = _slot((M, r), torch.float32, 4, 12)
    dXbig, dXs = _slot((M, K), tdt)
    L.lora_linear_fwd(Xs, W0s, A, B, c.s, Y=Ys, U=Us)
    gs = L.lora_linear_bwd(dYs, Xs, W0s, A, B, c.s, U=Us, dX=dXs)
    torch.cuda.synchronize()
    assert torch.equal(Ys, Yd) and torch.equal(Us, Ud)
    assert torch.equal(dXs, gd["dX"])
    for k in ("dA", "dB"):
        assert torch.equal(gs[k], gd[k]), k
    assert _untouched(Ybig, N) and _untouched(dXbig, K) and _untouched(Ubig, r, 4)
    tol_o, tol_g = (5e-3, 5e-3) if dtype == "bf16" else (1e-5, 1e-4)
    Xf, W0f, Af, Bf, dYf = (c.f64(k) for k in ("X", "W0", "A", "B", "dY"))
    assert_close(host(Ys), olora.lora_forward(Xf, W0f, Af, Bf, c.s), tol_o, "Y")
    gr = olora.lora_backward(dYf, Xf, W0f, Af, Bf, c.s)
    for k in ("dX", "dA", "dB"):
        assert_close(host(gs[k]), gr[k], tol_g, k)


def test_lora_fp32_odd_strides():
    """fp32 rows whose strides are not a multiple of four floats (16-byte aligned bases, odd
    leading dimensions): the one-launch small-layer kernels load rows 16 bytes at a time and
    are not taken, the general fp32 products are; results match the oracle, and the columns
    outside the output slices stay untouched."""
    require_gpu()
    import lora_dora_linear_amd as L
    M, N, K, r = 64, 256, 256, 8
    c = inputs.linear_case(32, M, N, K, r, 0.5, "f32", with_bias=True)
    X, W0, A, B, dY, bias = (dev(c.t[k], "f32") for k in ("X", "W0", "A", "B", "dY", "bias"))
    _, Xs = _embed(X, 4, 1)
    _, W0s = _embed(W0, 8, 3)
    _, dYs = _embed(dY, 4, 5)
    Ybig, Ys = _slot((M, N), torch.float32, 4, 1)
    Ubig, Us = _slot((M, r), torch.float32, 4, 1)
    dXbig, dXs = _slot((M, K), torch.float32, 4, 3)
    assert Xs.stride(0) % 4 and W0s.stride(0) % 4 and dYs.stride(0) % 4 and Ys.stride(0) % 4
    L.lora_linear_fwd(Xs, W0s, A, B, c.s, bias=bias, Y=Ys, U=Us)
    gs = L.lora_linear_bwd(dYs, Xs, W0s, A, B, c.s, U=Us, dX=dXs, need_dbias=True)
    torch.cuda.synchronize()
    assert _untouched(Ybig, N, 4) and _untouched(dXbig, K, 4) and _untouched(Ubig, r, 4)
    Xf, W0f, Af, Bf, dYf = (c.f64(k) for k in ("X", "W0", "A", "B", "dY"))
    assert_close(host(Ys), olora.lora_forward(Xf, W0f, Af, Bf, c.s, bias=c.f64("bias")), 1e-5, "Y")
    assert_close(host(Us), Xf @ Af.T, 1e-5, "U")
    gr = olora.lora_backward(dYf, Xf, W0f, Af, Bf, c.s)
    for k in ("dX", "dA", "dB"):
        assert_close(host(gs[k]), gr[k], 1e-4, k)
    assert_close(host(gs["dbias"]), gr["db"], 1e-4, "dbias")


def test_dora_strided():
    require_gpu()
    import lora_dora_linear_amd as L
    eps = 1e-12
    c = inputs.linear_case(32, 300, 384, 256, 32, 1.0, "bf16", dora=True)
    X, W0, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
    m = dev(c.t["m"], "f32")
    c0 = L.dora_prepare(W0)
    Yd, Ud, Zd, std = L.dora_linear_fwd(X, W0, A, B, m, c0, c.s, eps)
    gd = L.dora_linear_bwd(dY, X, W0, A, B, m, Ud, Zd, std, c.s, eps)
    _, Xs = _embed(X, 8, 8)
    _, W0s = _embed(W0, 32, 0)
    _, dYs = _embed(dY, 0, 64)
    c1 = L.dora_prepare(W0s)
    Ybig, Ys = _slot((300, 384), torch.bfloat16)
    dXbig, dXs = _slot((300, 256), torch.bfloat16)
    Y, U, Z, st = L.dora_linear_fwd(Xs, W0s, A, B, m, c1, c.s, eps, Y=Ys)
    g = L.dora_linear_bwd(dYs, Xs, W0s, A, B, m, U, Z, st, c.s, eps, dX=dXs)
    torch.cuda.synchronize()
    assert torch.equal(c1, c0) and torch.equal(Ys, Yd) and torch.equal(Z, Zd)
    for k in ("dX", "dA", "dB", "dm"):
        assert torch.equal(g[k], gd[k]), k
    assert _untouched(Ybig, 384) and _untouched(dXbig, 256)
    f = odora.dora_forward(c.f64("X"), c.f64("W0"), c.f64("A"), c.f64("B"), c.t["m"], c.s, eps)
    assert_close(host(Ys), f["Y"], 5e-3, "Y")


def test_w8a8_strided():
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(33, 300, 512, 640, 32, 0.5, "bf16")
    W0f = inputs.normal(33, 1, (512, 640), 1.0 / np.sqrt(640), "f32")
    X, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "A", "B", "dY"))
    Wq, sw = L.w8a8_quantize_weight(dev(W0f, "f32"))
    Yd, Xqd, sxd, Ud = L.w8a8_lora_linear_fwd(X, Wq, sw, A, B, c.s)
    gd = L.w8a8_lora_linear_bwd(dY, X, Wq, sw, A, B, c.s, U=Ud)
    _, Xs = _embed(X, 24, 8)
    _, Wqs = _embed(Wq, 32, 16)
    _, dYs = _embed(dY, 8, 8)
    Xq2, sx2 = L.w8a8_quantize_rows(Xs)
    Ybig, Ys = _slot((300, 512), torch.bfloat16)
    dXbig, dXs = _slot((300, 640), torch.bfloat16)
    Y, Xq, sx, U = L.w8a8_lora_linear_fwd(Xs, Wqs, sw, A, B, c.s, Y=Ys)
    g = L.w8a8_lora_linear_bwd(dYs, Xs, Wqs, sw, A, B, c.s, U=U, dX=dXs)
    C1 = L.int8_gemm_raw(Xq, Wq)
    C2 = L.int8_gemm_raw(_embed(Xq, 16, 16)[1], Wqs)
    torch.cuda.synchronize()
    assert torch.equal(Xq2, Xqd) and torch.equal(sx2, sxd) and torch.equal(C1, C2)
    assert torch.equal(Ys, Yd) and torch.equal(Xq, Xqd)
    for k in ("dX", "dA", "dB"):
        assert torch.equal(g[k], gd[k]), k
    assert _untouched(Ybig, 512) and _untouched(dXbig, 640)
    Wq_ref, sw_ref = ow.quantize_rows_int8(W0f)
    f = ow.w8a8_forward(c.f64("X"), Wq_ref, sw_ref, c.f64("A"), c.f64("B"), c.s)
    assert_close(host(Ys), f["Y"], 5e-3, "Y")


def test_swiglu_strided():
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.mlp_case(34, 300, 256, 512, 16, 0.25)
    X, dO = dev(c.t["X"], "bf16"), dev(c.t["dY"], "bf16")
    gate, up, down = ((dev(c.t["W" + t], "bf16"), dev(c.t["A" + t], "bf16"), dev(c.t["B" + t], "bf16"), c.s)
                      for t in ("g", "u", "d"))
    Od, sd = L.swiglu_lora_mlp_fwd(X, gate, up, down)
    gd = L.swiglu_lora_mlp_bwd(dO, X, gate, up, down, sd)
    _, Xs = _embed(X, 8, 56)
    _, dOs = _embed(dO, 32, 32)
    Obig, Os = _slot((300, 256), torch.bfloat16)
    dXbig, dXs = _slot((300, 256), torch.bfloat16)
    O, saved = L.swiglu_lora_mlp_fwd(Xs, gate, up, down, Out=Os)
    g = L.swiglu_lora_mlp_bwd(dOs, Xs, gate, up, down, saved, dX=dXs)
    torch.cuda.synchronize()
    assert torch.equal(Os, Od)
    for k in saved:
        assert torch.equal(saved[k], sd[k]), k
    for k in gd:
        assert torch.equal(g[k], gd[k]), k
    assert _untouched(Obig, 256) and _untouched(dXbig, 256)
    P = [c.proj(p) for p in ("gate", "up", "down")]
    assert_close(host(Os), osw.swiglu_mlp_forward(c.f64("X"), *P)["O"], 5e-3, "Out")
