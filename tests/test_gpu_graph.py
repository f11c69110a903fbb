"""The LoRA (fp32 and bf16), DoRA and SwiGLU-MLP forward + backward, each captured into one
HIP graph (through torch's graph capture on the C interface's stream argument) and replayed: every replay, with eager work and
synchronisations between replays, must give the eager result bit for bit.  None of the
library's launch sequences records a memset (zeroing runs as a kernel)."""
import ctypes

import pytest

from lora_dora_linear_amd import binding, inputs
from tests.gpu_util import dev, require_gpu, torch

pytestmark = pytest.mark.gpu


def _step_fn(c, dt_code):
    L = binding.lib()
    M, N, K, r, s = c.M, c.N, c.K, c.r, c.s
    kind = c.dtype
    X, W0, A, B, dY = (dev(c.t[k], kind) for k in ("X", "W0", "A", "B", "dY"))
    t = X.dtype
    out = {"Y": torch.empty((M, N), dtype=t, device="cuda"), "U": torch.empty((M, r), dtype=torch.float32, device="cuda"),
           "dX": torch.empty((M, K), dtype=t, device="cuda"),
           "dA": torch.empty((r, K), dtype=torch.float32, device="cuda"),
           "dB": torch.empty((N, r), dtype=torch.float32, device="cuda")}
    nb = binding.workspace_bytes("lora_bwd", M, N, K, r, dt_code)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    P = lambda x: ctypes.c_void_p(x.data_ptr())  # noqa: E731

    def step():
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert L.lora_linear_fwd(M, N, K, r, s, dt_code, P(X), K, P(W0), K, P(A), P(B), None, P(out["Y"]), N,
                                 P(out["U"]), r, P(ws), 0, st) == 0
        assert L.lora_linear_bwd(M, N, K, r, s, dt_code, P(dY), N, P(X), K, P(W0), K, P(A), P(B), P(out["U"]), r,
                                 P(out["dX"]), K, P(out["dA"]), P(out["dB"]), None, P(ws), nb, st) == 0
    return step, out


@pytest.mark.parametrize("dtype,M,N,K,r", [("f32", 64, 256, 256, 8), ("bf16", 300, 512, 512, 16)])
def test_graph_replays_equal_eager(dtype, M, N, K, r):
    require_gpu()
    c = inputs.linear_case(41, M, N, K, r, 0.5, dtype)
    step, out = _step_fn(c, 0 if dtype == "f32" else 1)
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()
        torch.cuda.current_stream().synchronize()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(4):
        for v in out.values():
            v.fill_(float("nan") if v.is_floating_point() else 0)     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k], ref[k]), (i, k)
        step()                                                          # and an eager step
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k], ref[k]), (i, k, "eager")


def _capture_and_replay(fn):
    """fn() -> dict of output tensors.  Eager result, then fn captured into one graph and
    replayed four times with eager work in between: every replay equal to the eager result."""
    ref = {k: v.clone() for k, v in fn().items() if v is not None}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        fn()
        torch.cuda.current_stream().synchronize()
        with torch.cuda.graph(g, stream=side):
            out = fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(4):
        for k in ref:
            out[k].fill_(float("nan") if out[k].is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(out[k], ref[k]), (i, k)
        fn()                                                            # eager work between replays
        torch.cuda.synchronize()


def test_graph_dora_replays_equal_eager():
    """DoRA rows (r = 32): one row-projection launch for P, G and U, factors packed by the
    kernels that form them, split reductions."""
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.linear_case(43, 300, 384, 256, 32, 1.0, "bf16", with_bias=True, dora=True)
    X, W0, A, B, dY, bias = (dev(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY", "bias"))
    m = dev(c.t["m"], "f32")
    c0 = L.dora_prepare(W0)
    torch.cuda.synchronize()

    def fn():
        Y, U, Z, state = L.dora_linear_fwd(X, W0, A, B, m, c0, c.s, 1e-12, bias=bias)
        g = L.dora_linear_bwd(dY, X, W0, A, B, m, U, Z, state, c.s, 1e-12, need_dbias=True)
        return {"Y": Y, "U": U, "Z": Z, "state": state, **g}
    _capture_and_replay(fn)


def test_graph_swiglu_replays_equal_eager():
    """SwiGLU MLP (r = 64): dual gate/up tile, four-wave NN over the two stacked weights,
    activation pass, pre-packed rank factors."""
    require_gpu()
    import lora_dora_linear_amd as L
    c = inputs.mlp_case(44, 300, 256, 384, 64, 0.25)
    X, dO = dev(c.t["X"], "bf16"), dev(c.t["dY"], "bf16")
    gate, up, down = ((dev(c.t["W" + t], "bf16"), dev(c.t["A" + t], "bf16"), dev(c.t["B" + t], "bf16"), c.s)
                      for t in ("g", "u", "d"))

    def fn():
        Out, saved = L.swiglu_lora_mlp_fwd(X, gate, up, down)
        g = L.swiglu_lora_mlp_bwd(dO, X, gate, up, down, saved)
        return {"Out": Out, **{k: v for k, v in saved.items()}, **g}
    _capture_and_replay(fn)
