"""Weight-space dropout through the C interface (mask lora_down's dropped input features, run
the layer with s / (1 - p), mask the factor gradient) against the oracle's definition: the
LoRA linear (bf16 and fp32) and the row-scaled DoRA linear, whose norm sees the same mask."""
import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import dropout as od
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu


def _keep(K, seed, p):
    return (np.random.default_rng(seed).random(K) >= p).astype(np.uint8)


@pytest.mark.parametrize("dtype,M,N,K,r", [("bf16", 300, 512, 512, 16), ("bf16", 4096, 4096, 4096, 16),
                                           ("f32", 64, 256, 256, 8)])
def test_lora_dropout(dtype, M, N, K, r):
    require_gpu()
    import lora_dora_linear_amd as L
    p = 0.25
    c = inputs.linear_case(71, M, N, K, r, 0.5, dtype)
    keep = _keep(K, 71, p)
    X, W0, A, B, dY = (dev(c.t[k], dtype) for k in ("X", "W0", "A", "B", "dY"))
    kd = torch.from_numpy(keep).cuda()
    Ad = L.lora_dropout_mask(A, kd)
    Y, U = L.lora_linear_fwd(X, W0, Ad, B, c.s / (1 - p))
    g = L.lora_linear_bwd(dY, X, W0, Ad, B, c.s / (1 - p), U=U)
    L.lora_dropout_grad(g["dA"], kd)
    torch.cuda.synchronize()
    assert torch.equal(Ad[:, torch.from_numpy(keep == 0).cuda()], torch.zeros_like(Ad[:, :int((keep == 0).sum())]))
    tol_o, tol_g = (5e-3, 5e-3) if dtype == "bf16" else (1e-5, 1e-4)
    Xf, W0f, Af, Bf, dYf = (c.f64(k) for k in ("X", "W0", "A", "B", "dY"))
    if M <= 512:
        assert_close(host(Y), od.lora_forward(Xf, W0f, Af, Bf, c.s, keep, p), tol_o, "Y")
        gr = od.lora_backward(dYf, Xf, W0f, Af, Bf, c.s, keep, p)
        for k in ("dX", "dA", "dB"):
            assert_close(host(g[k]), gr[k], tol_g, k)
    else:
        rows = np.sort(np.random.default_rng(5).choice(M, 16, replace=False))
        assert_close(host(Y[rows]), od.lora_forward(Xf[rows], W0f, Af, Bf, c.s, keep, p), tol_o, "Y rows")
        gr = od.lora_backward(dYf[rows], Xf[rows], W0f, Af, Bf, c.s, keep, p)
        assert_close(host(g["dX"][rows]), gr["dX"], tol_g, "dX rows")
    assert not torch.any(g["dA"][:, torch.from_numpy(keep == 0).cuda()])


def test_dora_dropout():
    require_gpu()
    import lora_dora_linear_amd as L
    p, eps = 0.3, 1e-12
    c = inputs.linear_case(72, 300, 384, 256, 32, 1.0, "bf16", dora=True)
    keep = _keep(256, 72, p)
    X, W0, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
    m = dev(c.t["m"], "f32")
    kd = torch.from_numpy(keep).cuda()
    Ad = L.lora_dropout_mask(A, kd)
    c0 = L.dora_prepare(W0)
    sp = c.s / (1 - p)
    Y, U, Z, st = L.dora_linear_fwd(X, W0, Ad, B, m, c0, sp, eps)
    g = L.dora_linear_bwd(dY, X, W0, Ad, B, m, U, Z, st, sp, eps)
    L.lora_dropout_grad(g["dA"], kd)
    torch.cuda.synchronize()
    Xf, W0f, Af, Bf, dYf = (c.f64(k) for k in ("X", "W0", "A", "B", "dY"))
    mf = c.t["m"].astype(np.float64)
    f = od.dora_forward(Xf, W0f, Af, Bf, mf, c.s, keep, p, eps)
    assert_close(host(Y), f["Y"], 5e-3, "Y")
    assert_close(host(st[:384]), f["nu"], 1e-5, "norm with the dropped factor")
    gr = od.dora_backward(dYf, Xf, W0f, Af, Bf, mf, c.s, keep, p, eps)
    for k in ("dX", "dA", "dB", "dm"):
        assert_close(host(g[k]), gr[k], 5e-3, k)
