"""GPU parity of the LoRA merge (W0 + s.B.A formed explicitly) and its backward against the
fp64 oracle: bf16 outputs at 5e-3, fp32 at 1e-5; factor gradients at 5e-3 (bf16 inputs) and
1e-4 (fp32)."""
import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import merge as om
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,N,K,r", [("bf16", 4096, 4096, 16), ("bf16", 300, 640, 48), ("bf16", 129, 192, 128),
                                         ("bf16", 64, 256, 8), ("f32", 64, 256, 8), ("f32", 200, 96, 33)])
def test_merge_parity(dtype, N, K, r):
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(51, 1, N, K, r, 0.5, dtype)
    dW = inputs.normal(51, 7, (N, K), 1.0, dtype)
    W0, A, B = (dev(c.t[k], dtype) for k in ("W0", "A", "B"))
    W = L.lora_merge_fwd(W0, A, B, c.s)
    D = L.lora_merge_fwd(None, A, B, c.s)
    g = L.lora_merge_bwd(dev(dW, dtype), A, B, c.s)
    torch.cuda.synchronize()
    W0f, Af, Bf = c.f64("W0"), c.f64("A"), c.f64("B")
    tol_o, tol_g = (5e-3, 5e-3) if dtype == "bf16" else (1e-5, 1e-4)
    assert_close(host(W), om.merge_forward(W0f, Af, Bf, c.s), tol_o, "W")
    assert_close(host(D), om.merge_forward(None, Af, Bf, c.s), tol_o, "delta")
    gr = om.merge_backward(inputs.to_f64(dW, dtype), Af, Bf, c.s)
    assert_close(host(g["dA"]), gr["dA"], tol_g, "dA")
    assert_close(host(g["dB"]), gr["dB"], tol_g, "dB")


def test_merge_in_place_and_strided():
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(52, 1, 256, 384, 16, 0.75, "bf16")
    W0, A, B = (dev(c.t[k], "bf16") for k in ("W0", "A", "B"))
    ref = L.lora_merge_fwd(W0, A, B, c.s)
    big = torch.full((256, 384 + 64), 3.0, dtype=torch.bfloat16, device="cuda")
    L.lora_merge_fwd(W0, A, B, c.s, out=big[:, 32:32 + 384])
    W1 = W0.clone()
    L.lora_merge_fwd(W1, A, B, c.s, out=W1)            # merged into the base weight
    torch.cuda.synchronize()
    assert torch.equal(big[:, 32:32 + 384], ref) and torch.equal(W1, ref)
    assert bool(torch.all(big[:, :32] == 3.0)) and bool(torch.all(big[:, 32 + 384:] == 3.0))
    assert_close(host(ref), om.merge_forward(c.f64("W0"), c.f64("A"), c.f64("B"), c.s), 5e-3, "W")
