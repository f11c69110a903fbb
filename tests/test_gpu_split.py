"""The split reduction of the output tiles past the last full round of the 256 compute units.

With a workspace of ldl_workspace_bytes the LoRA, int8 and e4m3 products split those tiles
over k into fp32 partials that a fixup pass sums in order; with one byte less the same calls
run them unsplit.  Both must match the fp64 oracle (sampled rows inside and outside the
split tiles), agree with each other to the bf16 output rounding, and the split results must
repeat bit for bit.  Shapes: 15 tiles (every tile split, four ways), and 272 tiles (one full
round of 256, the last 16 tiles split four ways: rows 4096..4351)."""
import numpy as np
import pytest

from lora_dora_linear_amd import binding, inputs
from oracle import fp8 as of8
from oracle import lora as olora
from oracle import w8a8 as ow
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu

TOL = 5e-3
SHAPES = [(768, 1280, 1024, 16), (4352, 4096, 256, 16)]


def _unsplit_ws(op, M, N, K, r, dtype, device):
    """The workspace minus one byte: everything a call needs except the split partials."""
    n = binding.workspace_bytes(op, M, N, K, r, dtype)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device), n - 1


def _rows(M):
    rng = np.random.default_rng(M)
    lo = rng.choice(min(M, 4096), 12, replace=False)
    hi = rng.choice(np.arange(4096, M), 12, replace=False) if M > 4096 else np.array([], int)
    return np.sort(np.concatenate([lo, hi]).astype(int))


def _lora(c, bias):
    import lora_dora_linear_amd as L
    X, W0, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
    Y, U = L.lora_linear_fwd(X, W0, A, B, c.s, bias=bias)
    g = L.lora_linear_bwd(dY, X, W0, A, B, c.s, U=U)
    torch.cuda.synchronize()
    return Y, g["dX"], g["dA"], g["dB"]


@pytest.mark.parametrize("M,N,K,r", SHAPES)
def test_lora_split_matches_unsplit_and_oracle(M, N, K, r, monkeypatch):
    require_gpu()
    c = inputs.linear_case(41, M, N, K, r, 0.5, "bf16", with_bias=True)
    bias = dev(c.t["bias"], "bf16")
    s1 = _lora(c, bias)
    s2 = _lora(c, bias)
    for a, b in zip(s1, s2):
        assert torch.equal(a, b)                     # the split path repeats bit for bit
    monkeypatch.setattr(binding, "_ws", _unsplit_ws)
    u = _lora(c, bias)
    for name, a, b in zip(("Y", "dX", "dA", "dB"), s1, u):
        assert_close(host(a), host(b), TOL, name + " split vs unsplit")
    rows = _rows(M)
    X, W0, A, B, dY = (c.f64(k) for k in ("X", "W0", "A", "B", "dY"))
    Yr = olora.lora_forward(X[rows], W0, A, B, c.s, bias=c.f64("bias"))
    assert_close(host(s1[0][rows]), Yr, TOL, "Y rows")
    b = olora.lora_backward(dY[rows], X[rows], W0, A, B, c.s)
    assert_close(host(s1[1][rows]), b["dX"], TOL, "dX rows")


def _eight_bit(kind, c, W0f):
    import lora_dora_linear_amd as L
    X, A, B, dY = (dev(c.t[k], "bf16") for k in ("X", "A", "B", "dY"))
    if kind == "int8":
        Wq, sw = L.w8a8_quantize_weight(dev(W0f, "f32"))
        Y, _, _, U = L.w8a8_lora_linear_fwd(X, Wq, sw, A, B, c.s)
        g = L.w8a8_lora_linear_bwd(dY, X, Wq, sw, A, B, c.s, U=U)
    else:
        Wq, sw = L.fp8_quantize_weight(dev(W0f, "f32"))
        Y, _, _, U = L.fp8_lora_linear_fwd(X, Wq, sw, A, B, c.s)
        g = L.fp8_lora_linear_bwd(dY, X, Wq, sw, A, B, c.s, U=U)
    torch.cuda.synchronize()
    return Y, g["dX"]


@pytest.mark.parametrize("kind", ["int8", "e4m3"])
def test_eight_bit_split_matches_unsplit_and_oracle(kind, monkeypatch):
    require_gpu()
    M, N, K, r = 4352, 4096, 256, 16
    c = inputs.linear_case(43, M, N, K, r, 0.5, "bf16")
    W0f = inputs.normal(43, 1, (N, K), 1.0 / np.sqrt(K), "f32")
    s1 = _eight_bit(kind, c, W0f)
    s2 = _eight_bit(kind, c, W0f)
    for a, b in zip(s1, s2):
        assert torch.equal(a, b)
    monkeypatch.setattr(binding, "_ws", _unsplit_ws)
    u = _eight_bit(kind, c, W0f)
    for name, a, b in zip(("Y", "dX"), s1, u):
        assert_close(host(a), host(b), TOL, name + " split vs unsplit")
    rows = _rows(M)
    X, A, B, dY = (c.f64(k) for k in ("X", "A", "B", "dY"))
    if kind == "int8":
        Wq_ref, sw_ref = ow.quantize_rows_int8(W0f)
        f = ow.w8a8_forward(X[rows], Wq_ref, sw_ref, A, B, c.s)
        b = ow.w8a8_backward(dY[rows], X[rows], Wq_ref, sw_ref, A, B, c.s)
    else:
        Wq_ref, sw_ref = of8.quantize_rows_fp8(W0f)
        f = of8.fp8_forward(X[rows], Wq_ref, sw_ref, A, B, c.s)
        b = of8.fp8_backward(dY[rows], X[rows], Wq_ref, sw_ref, A, B, c.s)
    assert_close(host(s1[0][rows]), f["Y"], TOL, "Y rows")
    assert_close(host(s1[1][rows]), b["dX"], TOL, "dX rows")
