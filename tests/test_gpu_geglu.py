"""GPU parity of the GeGLU LoRA MLP (exact and tanh forms of GELU) against the fp64 oracle,
on the four-wave routes (dual gate/up tile with the activation in its epilogue, plain input
gradient plus the streaming gated backward) and the eight-wave routes (fused epilogues)."""
import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import geglu as og
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu

TOL = 5e-3


def _run(c, approximate):
    import lora_dora_linear_amd as L
    X, dO = dev(c.t["X"], "bf16"), dev(c.t["dY"], "bf16")
    gate, up, down = ((dev(c.t["W" + t], "bf16"), dev(c.t["A" + t], "bf16"), dev(c.t["B" + t], "bf16"), c.s)
                      for t in ("g", "u", "d"))
    Out, saved = L.geglu_lora_mlp_fwd(X, gate, up, down, approximate=approximate)
    g = L.geglu_lora_mlp_bwd(dO, X, gate, up, down, saved, approximate=approximate)
    torch.cuda.synchronize()
    return Out, saved, g


@pytest.mark.parametrize("approximate", [False, True])
@pytest.mark.parametrize("M,K,H,r,four", [(300, 256, 512, 16, 1), (300, 384, 256, 64, 1), (100, 192, 320, 16, 1),
                                          (300, 256, 512, 32, 0)])
def test_geglu_parity(M, K, H, r, four, approximate):
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.mlp_case(61, M, K, H, r, 0.25)
    L.set_tuning(1, four)
    try:
        Out, saved, g = _run(c, approximate)
    finally:
        L.set_tuning(1, 1)
    X, dO = c.f64("X"), c.f64("dY")
    P = [c.proj(p) for p in ("gate", "up", "down")]
    f = og.geglu_mlp_forward(X, *P, approximate=approximate)
    b = og.geglu_mlp_backward(dO, X, *P, approximate=approximate)
    assert_close(host(Out), f["O"], TOL, "Out")
    for k in ("E", "Gu", "H"):
        assert_close(host(saved[k]), f[k], TOL, k)
    assert_close(host(g["dX"]), b["dX"], TOL, "dX")
    for p in ("gate", "up", "down"):
        for w in ("dA_", "dB_"):
            assert_close(host(g[w + p]), b[w + p], TOL, w + p)


def test_geglu_forms_differ_and_swiglu_unchanged():
    """The exact and tanh forms give different (close) hidden activations, and the SwiGLU entry
    point is untouched by the activation parameter."""
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.mlp_case(62, 300, 256, 512, 16, 0.25)
    _, s0, _ = _run(c, False)
    _, s1, _ = _run(c, True)
    X = dev(c.t["X"], "bf16")
    gate, up, down = ((dev(c.t["W" + t], "bf16"), dev(c.t["A" + t], "bf16"), dev(c.t["B" + t], "bf16"), c.s)
                      for t in ("g", "u", "d"))
    _, sw = L.swiglu_lora_mlp_fwd(X, gate, up, down)
    torch.cuda.synchronize()
    assert torch.equal(s0["E"], s1["E"]) and torch.equal(s0["E"], sw["E"])
    h0, h1 = host(s0["H"]), host(s1["H"])
    # the two forms differ by less than 1e-3 of |e| before rounding; stored in bf16, an element
    # can move by one unit (2^-7 of its magnitude) more
    assert 0 < np.max(np.abs(h0 - h1)) <= 2.0 ** -6 * np.max(np.abs(h0))
    assert not torch.equal(s0["H"], sw["H"])
