"""The LoRA backward entry point that allocates nothing (lora_linear_bwd_noalloc): its
workspace is the library's fixed per-device scratch array.  Called through the C
interface, its outputs must equal those of lora_linear_bwd (same kernels, caller-owned
workspace) bit for bit, on consecutive calls whose sizes shrink (the scratch keeps the
previous call's contents), and match the fp64 oracle."""
import ctypes

import numpy as np
import pytest

from lora_dora_linear_amd import inputs
from oracle import lora as olora
from tests.gpu_util import assert_close, dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu

LDL_E_WORKSPACE = -3


def _tensors(c):
    return tuple(dev(c.t[k], c.dtype) for k in ("X", "W0", "A", "B", "dY"))


def test_noalloc_matches_workspace_entry_point_on_shrinking_calls():
    require_gpu()
    import lora_dora_linear_amd as L
    cases = [(4096, 4096, 4096, 16, "bf16"), (300, 512, 384, 32, "bf16"), (64, 256, 256, 8, "f32")]
    for i, (M, N, K, r, dt) in enumerate(cases):
        c = inputs.linear_case(21 + i, M, N, K, r, 0.5, dt)
        X, W0, A, B, dY = _tensors(c)
        Y, U = L.lora_linear_fwd(X, W0, A, B, c.s)
        g0 = L.lora_linear_bwd_noalloc(dY, X, W0, A, B, c.s, U=U, need_dbias=True)
        g1 = L.lora_linear_bwd(dY, X, W0, A, B, c.s, U=U, need_dbias=True)
        torch.cuda.synchronize()
        for k in ("dX", "dA", "dB", "dbias"):
            assert torch.equal(g0[k], g1[k]), (M, N, K, r, k)
        tol = 5e-3 if dt == "bf16" else 1e-4
        Xf, W0f, Af, Bf, dYf = (c.f64(k) for k in ("X", "W0", "A", "B", "dY"))
        if M <= 512:
            gr = olora.lora_backward(dYf, Xf, W0f, Af, Bf, c.s)
            for k in ("dX", "dA", "dB"):
                assert_close(host(g0[k]), gr[k], tol, k)
        else:
            rows = np.sort(np.random.default_rng(3).choice(M, 16, replace=False))
            dXr = olora.lora_backward(dYf[rows], Xf[rows], W0f, Af, Bf, c.s)["dX"]
            assert_close(host(g0["dX"][rows]), dXr, tol, "dX rows")
            nc = np.sort(np.random.default_rng(4).choice(N, 12, replace=False))
            kc = np.sort(np.random.default_rng(5).choice(K, 12, replace=False))
            smp = olora.lora_weight_grads_sampled(dYf, Xf, Af, Bf, c.s, nc, kc)
            assert_close(host(g0["dB"][nc]), smp["dB_rows"], tol, "dB rows")
            assert_close(host(g0["dA"][:, kc]), smp["dA_cols"], tol, "dA cols")


def test_noalloc_takes_no_device_memory_and_rejects_oversize():
    require_gpu()
    import lora_dora_linear_amd as L
    lib = L.lib()
    c = inputs.linear_case(25, 1024, 1024, 1024, 16, 0.5, "bf16")
    X, W0, A, B, dY = _tensors(c)
    Y, U = L.lora_linear_fwd(X, W0, A, B, c.s)
    dX = torch.empty((1024, 1024), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((16, 1024), dtype=torch.float32, device="cuda")
    dB = torch.empty((1024, 16), dtype=torch.float32, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = (1024, 1024, 1024, 16, 0.5, 1, P(dY), 1024, P(X), 1024, P(W0), 1024, P(A), P(B), P(U), 16, P(dX), 1024,
            P(dA), P(dB), None, stream)
    assert lib.lora_linear_bwd_noalloc(*args) == 0
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        assert lib.lora_linear_bwd_noalloc(*args) == 0
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    # a size whose workspace exceeds the scratch is refused before anything is enqueued
    cap = int(lib.ldl_noalloc_scratch_bytes())
    assert cap == 32 << 20
    big = (16384, 8192, 8192, 128)
    assert lib.ldl_workspace_bytes(1, *big, 1) > cap
    bad = (*big, 0.5, 1, P(dY), 0, P(X), 0, P(W0), 0, P(A), P(B), None, 0, P(dX), 0, P(dA), P(dB), None, stream)
    assert lib.lora_linear_bwd_noalloc(*bad) == LDL_E_WORKSPACE
