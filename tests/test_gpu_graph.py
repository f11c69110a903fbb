"""The LoRA forward + backward captured into one HIP graph (through torch's graph capture
on the C interface's stream argument) and replayed: every replay, with eager work and
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
