#!/usr/bin/env python3
"""Throughput of the fused LoRA linear, forward + backward, on one MI355X.

Default workload: bf16 LoRA linear, M = 4096 tokens, K = N = 4096, r = 16,
s = 0.5 (X ~ N(0,1), W0, A ~ N(0, 1/K), B ~ N(0, 0.02 variance), dY ~ N(0,1)).
One step = lora_linear_fwd + lora_linear_bwd (Y, U, dX, dA, dB) with every
input already resident in HBM.  Algorithmic work per step:
4MNK + 6Mr(K+N) FLOP (no B.A product, no weight gradient of the frozen W0).

Prints ONE JSON line.  Extra workloads (--workload dora|swiglu|w8a8) print their
own line in the same format for the other layer variants.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2516.6    # TFLOP/s dense bf16 MFMA, MI355X (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_INT8 = 5033.2    # TOP/s dense int8 MFMA (and TFLOP/s dense fp8)
PEAK_HBM = 8000.0     # GB/s

METRIC = "fused LoRA/DoRA linear fwd+bwd TFLOP/s and % of bf16 MFMA peak (1 GPU)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the engine clock ramps up over the first ~100 steps (~30 ms) of back-to-back work;
    # 200 untimed steps reach the sustained clock, 1000 timed steps take about 0.3 s
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="lora", choices=["lora", "dora", "dora_cols", "qkv", "swiglu", "geglu", "w8a8", "fp8", "tiny",
                                                           "merge"])
    ap.add_argument("--M", type=int, default=None, help="token count override (w8a8 / fp8 sweep point)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fused-downproj", type=int, default=None, choices=[0, 1])
    ap.add_argument("--gemm-4wave", type=int, default=None, choices=[0, 1],
                    help="four-wave 256x256 tile for the plain NT products (library default 1)")
    ap.add_argument("--step-times", action="store_true",
                    help="also report every timed step's duration (fence-free events between steps)")
    ap.add_argument("--copy-calibrate", type=int, default=None, metavar="MIB",
                    help="only run device-to-device copies of MIB MiB (reference kernel for the HBM byte counters)")
    return ap.parse_args()


# HBM traffic of the dominant kernel, taken with rocprofv3 counter runs and kept
# with its kernel trace under profiles/; it is reported only while the GEMM
# sources still hash to the value recorded with the counters.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lora_bf16_4096_r16_gemm_traffic.md")
GEMM_SOURCES = ("lora_dora_linear_amd/csrc/gemm_tile.hpp", "lora_dora_linear_amd/csrc/gemm16.hpp",
                "lora_dora_linear_amd/csrc/gemm.hip", "lora_dora_linear_amd/csrc/common.hpp")


def gemm_source_hash():
    import hashlib
    h = hashlib.sha1()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel_key):
    """Bytes per launch (fetch + write, copy-calibrated) recorded for kernel_key, or None if stale/absent."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    for ln in lines:
        if ln.startswith("traffic-record: "):
            rec = json.loads(ln[len("traffic-record: "):])
            if rec.get("kernel") == kernel_key and rec.get("source_sha1") == gemm_source_hash():
                return rec["fetch_bytes"] * rec["fetch_scale"] + rec["write_bytes"] * rec["write_scale"]
    return None


def copy_calibrate(mib):
    import torch
    torch.cuda.set_device(0)
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}))


class TimingEvents:
    """n HIP timing events created with hipEventDisableSystemFence: recording one then costs no
    system-scope fence (cache write-back and invalidate), which with default events left ~5 us
    gaps around every timed launch and slowed the step itself.  They are read only after a
    device-wide synchronisation, so the missing host-visibility fence changes no result."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")    # the runtime torch has loaded
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.arr[i] = ev

    def record(self, i, stream):
        if self.hip.hipEventRecord(self.arr[i], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def between_ms(self, i, j):
        """Milliseconds from this set's event i to its event j."""
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[i], self.arr[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def elapsed_ms(self, stop, i):
        """Milliseconds from this set's event i to stop's event i."""
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[i], stop.arr[i]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_lora(M_sample, N, K, r, s, min_seconds=10.0, min_repeats=3):
    """The fp64 oracle (as it stands) on the first M_sample rows of the same workload, repeated
    until about min_seconds of CPU work (median of the repeats)."""
    from threadpoolctl import threadpool_info

    from lora_dora_linear_amd import inputs
    from oracle import lora as olora
    c = inputs.linear_case(2, M_sample, N, K, r, s, "bf16")
    X, W0, A, B, dY = (c.f64(k) for k in ("X", "W0", "A", "B", "dY"))
    times = []
    while len(times) < min_repeats or sum(times) < min_seconds:
        t0 = time.perf_counter()
        olora.lora_forward(X, W0, A, B, s)
        olora.lora_backward(dY, X, W0, A, B, s)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    flops = 4.0 * M_sample * N * K + 6.0 * M_sample * r * (K + N)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{M_sample} of the 4096 token rows (same N, K, r), fp64 forward + backward materialising "
                      f"B.A and dY^T.X, median of {len(times)} runs ({sum(times):.1f} s of CPU work): {dt:.2f} s each",
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(), "blas_threads": int(threads), "seconds": dt}


def tiny(args, torch, np, binding, inputs, L, up, P, st, check):
    """The fp32 workload of 64 tokens, K = N = 256, r = 8, s = 2: launch-bound, so the line
    reports the step time, eagerly and as one replayed HIP graph of the same launches."""
    M, N, K, r, s = 64, 256, 256, 8, 2.0
    dev = torch.device("cuda", 0)
    c = inputs.linear_case(1, M, N, K, r, s, "f32")
    X, W0, A, B, dY = (up(c.t[k], "f32") for k in ("X", "W0", "A", "B", "dY"))
    f32 = torch.float32
    Y = torch.empty((M, N), dtype=f32, device=dev)
    U = torch.empty((M, r), dtype=f32, device=dev)
    dX = torch.empty((M, K), dtype=f32, device=dev)
    dA = torch.empty((r, K), dtype=f32, device=dev)
    dB = torch.empty((N, r), dtype=f32, device=dev)
    nb = binding.workspace_bytes("lora_bwd", M, N, K, r, 0)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)

    def step():
        check(L.lora_linear_fwd(M, N, K, r, s, 0, P(X), K, P(W0), K, P(A), P(B), None, P(Y), N, P(U), r, P(ws), 0,
                                st()), "lora_linear_fwd")
        check(L.lora_linear_bwd(M, N, K, r, s, 0, P(dY), N, P(X), K, P(W0), K, P(A), P(B), P(U), r, P(dX), K, P(dA),
                                P(dB), None, P(ws), nb, st()), "lora_linear_bwd")

    K_steps = args.steps
    for _ in range(args.warmup):
        step()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(K_steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K_steps
    # the same step captured once and replayed (launch overhead of the nine kernels gone)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()
        torch.cuda.current_stream().synchronize()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(K_steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_graph = t0.elapsed_time(t1) / K_steps
    flops = 4.0 * M * N * K + 6.0 * M * r * (K + N)
    print(json.dumps({"metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 4), "unit": "TFLOP/s", "n_gpus": 1,
                      "steps": K_steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
                      "us_per_step": round(ms * 1e3, 2), "us_per_step_graph_replay": round(ms_graph * 1e3, 2),
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
                      "data": "synthetic",
                      "config": {"workload": f"fp32 LoRA linear fwd+bwd, M={M}, K=N={K}, r={r}, s={s} "
                                             "(launch-bound: report the step time)",
                                 "M": M, "N": N, "K": K, "r": r, "s": s}}))


def merge(args, torch, np, binding, inputs, L, up, P, st, check):
    """LoRA merge of a 4096 x 4096 bf16 weight with a rank-16 adapter: W = W0 + s.B.A (one
    HBM-bound kernel: read W0, write W) and the merge backward (dA, dB from a weight
    gradient).  The roofline is the forward kernel's HBM rate."""
    N, K, r, s = 4096, 4096, 16, 0.5
    dev = torch.device("cuda", 0)
    c = inputs.linear_case(2, 1, N, K, r, s, "bf16")
    W0, A, B = (up(c.t[k], "bf16") for k in ("W0", "A", "B"))
    dW = up(inputs.normal(2, 7, (N, K), 1.0, "bf16"), "bf16")
    W = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    nb = binding.workspace_bytes("merge_bwd", 0, N, K, r)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    K_steps = args.steps
    e0, e1 = TimingEvents(K_steps), TimingEvents(K_steps)

    def step(i=None):
        if i is not None:
            e0.record(i, st())
        check(L.lora_merge_fwd(N, K, r, s, 1, P(W0), K, P(A), P(B), P(W), K, st()), "lora_merge_fwd")
        if i is not None:
            e1.record(i, st())
        check(L.lora_merge_bwd(N, K, r, s, 1, P(dW), K, P(A), P(B), P(dA), P(dB), P(ws), nb, st()), "lora_merge_bwd")

    for _ in range(args.warmup):
        step()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(K_steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K_steps
    fwd_us = 1e3 * sum(e0.elapsed_ms(e1, i) for i in range(K_steps)) / K_steps
    fwd_bytes = 2.0 * N * K * 2 + (N + K) * r * 2          # read W0, write W, read the factors
    gbs = fwd_bytes / (fwd_us * 1e-6) / 1e9
    flops = 2.0 * N * K * r + 4.0 * N * K * r
    print(json.dumps({"metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
                      "n_gpus": 1, "steps": K_steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                      "data": "synthetic",
                      "config": {"workload": f"bf16 LoRA merge fwd+bwd, N=K={K}, r={r}, s={s}", "N": N, "K": K,
                                 "r": r, "s": s},
                      "roofline": {"bound": "hbm", "kernel": "merge forward (merge_kernel)",
                                   "achieved": round(gbs, 1), "peak": PEAK_HBM, "unit": "GB/s",
                                   "frac": round(gbs / PEAK_HBM, 4), "traffic": None},
                      "kernels": {"merge forward (merge_kernel)": {"avg_us": round(fwd_us, 2)}}}))


def main():
    args = parse()
    if args.copy_calibrate:
        copy_calibrate(args.copy_calibrate)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the layer's data-parallel "
                                   "sharding over several GPUs (rows of X per GPU, one all-reduce of "
                                   "the factor gradients) is not implemented",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from lora_dora_linear_amd import binding, inputs
    L = binding.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.fused_downproj is not None:
        binding.set_tuning(0, args.fused_downproj)
    if args.gemm_4wave is not None:
        binding.set_tuning(1, args.gemm_4wave)

    def up(arr, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)

    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)  # noqa: E731

    def check(code, name):
        if code != 0:
            raise RuntimeError(f"{name}: {binding.status_string(code)}")

    bf = torch.bfloat16
    f32 = torch.float32
    wl = args.workload
    if wl == "tiny":
        tiny(args, torch, np, binding, inputs, L, up, P, st, check)
        return
    if wl == "merge":
        merge(args, torch, np, binding, inputs, L, up, P, st, check)
        return
    gemm_kinds = (0, 1)
    gemm_flops = {}
    prep = None          # (call, kernel, bytes): a one-time preparation timed apart from the step
    if wl == "lora":
        M, N, K, r, s = 4096, 4096, 4096, 16, 0.5
        c = inputs.linear_case(2, M, N, K, r, s, "bf16")
        X, W0, A, B, dY = (up(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
        Y = torch.empty((M, N), dtype=bf, device=dev)
        U = torch.empty((M, r), dtype=f32, device=dev)
        dX = torch.empty((M, K), dtype=bf, device=dev)
        dA = torch.empty((r, K), dtype=f32, device=dev)
        dB = torch.empty((N, r), dtype=f32, device=dev)
        nf = binding.workspace_bytes("lora_fwd", M, N, K, r)
        nb = binding.workspace_bytes("lora_bwd", M, N, K, r)
        ws = torch.empty(max(nf, nb, 256), dtype=torch.uint8, device=dev)

        def step():
            check(L.lora_linear_fwd(M, N, K, r, s, 1, P(X), K, P(W0), K, P(A), P(B), None, P(Y), N, P(U), r, P(ws),
                                    nf, st()), "lora_linear_fwd")
            check(L.lora_linear_bwd(M, N, K, r, s, 1, P(dY), N, P(X), K, P(W0), K, P(A), P(B), P(U), r, P(dX), K,
                                    P(dA), P(dB), None, P(ws), nb, st()), "lora_linear_bwd")
        flops = 4.0 * M * N * K + 6.0 * M * r * (K + N)
        gemm_flops = {0: 2.0 * M * N * K + 2.0 * M * N * r, 1: 2.0 * M * N * K + 2.0 * M * K * r}
        config = {"workload": f"bf16 LoRA linear fwd+bwd, M={M} tokens (4x1024), K=N={K}, r={r}, s={s}",
                  "M": M, "N": N, "K": K, "r": r, "s": s, "B_init": "N(0, 0.02) read as variance"}
    elif wl == "dora":
        M, N, K, r, s, eps = 4096, 3072, 3072, 32, 1.0, 1e-12
        c = inputs.linear_case(3, M, N, K, r, s, "bf16", dora=True)
        X, W0, A, B, dY = (up(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
        m = up(c.t["m"], "f32")
        w0sq = torch.empty((N,), dtype=f32, device=dev)
        prep = (lambda: check(L.dora_prepare(N, K, 1, P(W0), K, P(w0sq), st()), "dora_prepare"),  # noqa: E731
                "rowsumsq_kernel (cached rowsum(W0^2), once per frozen weight)", 2.0 * N * K + 4.0 * N)
        prep[0]()
        Y = torch.empty((M, N), dtype=bf, device=dev)
        Z = torch.empty((M, N), dtype=bf, device=dev)
        U = torch.empty((M, r), dtype=f32, device=dev)
        state = torch.empty((binding.dora_state_floats(N, r),), dtype=f32, device=dev)
        dX = torch.empty((M, K), dtype=bf, device=dev)
        dA = torch.empty((r, K), dtype=f32, device=dev)
        dB = torch.empty((N, r), dtype=f32, device=dev)
        dm = torch.empty((N,), dtype=f32, device=dev)
        nb = binding.workspace_bytes("dora_bwd", M, N, K, r)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)

        def step():
            check(L.dora_linear_fwd(M, N, K, r, s, eps, 1, P(X), K, P(W0), K, P(A), P(B), P(m), P(w0sq), None, P(Y),
                                    N, P(U), r, P(Z), N, P(state), P(ws), 0, st()), "dora_linear_fwd")
            check(L.dora_linear_bwd(M, N, K, r, s, eps, 1, P(dY), N, P(X), K, P(W0), K, P(A), P(B), P(m), P(U), r,
                                    P(Z), N, P(state), P(dX), K, P(dA), P(dB), P(dm), None, P(ws), nb, st()),
                  "dora_linear_bwd")
        lora_flops = 4.0 * M * N * K + 6.0 * M * r * (K + N)
        dora_flops = 2.0 * N * K * r * 2 + 2.0 * r * r * K       # P = W0.A^T and (w.B)^T.W0, plus G = A.A^T
        flops = lora_flops + dora_flops
        gemm_flops = {0: 2.0 * M * N * K + 2.0 * M * N * r, 1: 2.0 * M * N * K + 2.0 * M * K * r}
        config = {"workload": f"bf16 DoRA (row-scaled) linear fwd+bwd, M={M}, K=N={K}, r={r}, s={s}, eps={eps}",
                  "M": M, "N": N, "K": K, "r": r, "s": s}
    elif wl == "dora_cols":
        M, N, K, r, s, eps = 4096, 3072, 3072, 32, 1.0, 1e-12
        c = inputs.linear_case(3, M, N, K, r, s, "bf16", dora_cols=True)
        X, W0, A, B, dY = (up(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
        m = up(c.t["m"], "f32")
        w0sq = torch.empty((K,), dtype=f32, device=dev)
        prep = (lambda: check(L.dora_cols_prepare(N, K, 1, P(W0), K, P(w0sq), st()), "dora_cols_prepare"),  # noqa
                "col_sumsq_kernel (cached column sums of W0^2, once per frozen weight)", 2.0 * N * K + 4.0 * K)
        prep[0]()
        Y = torch.empty((M, N), dtype=bf, device=dev)
        Xs = torch.empty((M, K), dtype=bf, device=dev)
        U = torch.empty((M, r), dtype=f32, device=dev)
        state = torch.empty((binding.dora_state_floats(K, r),), dtype=f32, device=dev)
        dX = torch.empty((M, K), dtype=bf, device=dev)
        dA = torch.empty((r, K), dtype=f32, device=dev)
        dB = torch.empty((N, r), dtype=f32, device=dev)
        dm = torch.empty((K,), dtype=f32, device=dev)
        nf = binding.workspace_bytes("dora_cols_fwd", M, N, K, r)
        nb = binding.workspace_bytes("dora_cols_bwd", M, N, K, r)
        ws = torch.empty(max(nf, nb, 256), dtype=torch.uint8, device=dev)

        def step():
            check(L.dora_cols_linear_fwd(M, N, K, r, s, eps, 1, P(X), K, P(W0), K, P(A), P(B), P(m), P(w0sq), None,
                                         P(Y), N, P(U), r, P(Xs), K, P(state), P(ws), nf, st()), "dora_cols_linear_fwd")
            check(L.dora_cols_linear_bwd(M, N, K, r, s, eps, 1, P(dY), N, P(X), K, P(Xs), K, P(W0), K, P(A), P(B),
                                         P(m), P(U), r, P(state), P(dX), K, P(dA), P(dB), P(dm), None, P(ws), nb, st()),
                  "dora_cols_linear_bwd")
        lora_flops = 4.0 * M * N * K + 6.0 * M * r * (K + N)
        dora_flops = 2.0 * N * K * r * 2 + 2.0 * N * r * r        # Pc = B^T.W0 and W0.(A.diag(w))^T, plus Gc
        flops = lora_flops + dora_flops
        gemm_flops = {0: 2.0 * M * N * K + 2.0 * M * N * r, 1: 2.0 * M * N * K + 2.0 * M * K * r}
        config = {"workload": f"bf16 DoRA (column-scaled) linear fwd+bwd, M={M}, K=N={K}, r={r}, s={s}, eps={eps}",
                  "M": M, "N": N, "K": K, "r": r, "s": s}
    elif wl == "qkv":
        M, K, r = 4096, 4096, 16
        leaves, s_leaf = (4096, 1024, 1024), (2.0, 2.0, 2.0)
        N, nl = sum(leaves), len(leaves)
        c = inputs.multi_case(6, M, K, leaves, r, s_leaf)
        X, W0, A, B, dY = (up(c.t[k], "bf16") for k in ("X", "W0", "A", "B", "dY"))
        nleaf = (ctypes.c_int * nl)(*leaves)
        sleaf = (ctypes.c_float * nl)(*s_leaf)
        Y = torch.empty((M, N), dtype=bf, device=dev)
        U = torch.empty((M, nl * r), dtype=f32, device=dev)
        dX = torch.empty((M, K), dtype=bf, device=dev)
        dA = torch.empty((nl * r, K), dtype=f32, device=dev)
        dB = torch.empty((N, r), dtype=f32, device=dev)
        nb = binding.multi_workspace_bytes("lora_bwd", M, K, leaves, r)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        cp = lambda a: ctypes.cast(a, ctypes.c_void_p)  # noqa: E731

        def step():
            check(L.lora_multi_linear_fwd(M, K, nl, cp(nleaf), r, cp(sleaf), 1, P(X), K, P(W0), K, P(A), P(B), None,
                                          P(Y), N, P(U), nl * r, P(ws), 0, st()), "lora_multi_linear_fwd")
            check(L.lora_multi_linear_bwd(M, K, nl, cp(nleaf), r, cp(sleaf), 1, P(dY), N, P(X), K, P(W0), K, P(A),
                                          P(B), P(U), nl * r, P(dX), K, P(dA), P(dB), None, P(ws), nb, st()),
                  "lora_multi_linear_bwd")
        flops = 4.0 * M * N * K + 6.0 * M * r * (nl * K + N)
        gemm_flops = {0: 2.0 * M * N * K + 2.0 * M * N * nl * r, 1: 2.0 * M * N * K + 2.0 * M * K * nl * r}
        config = {"workload": f"bf16 fused QKV leaves fwd+bwd, M={M}, K={K}, leaves q/k/v={leaves}, r={r} each, "
                              f"s={s_leaf[0]}", "M": M, "N": N, "K": K, "r": r, "leaves": list(leaves)}
    elif wl in ("swiglu", "geglu"):
        M, K, H, r, s = 8192, 4096, 14336, 64, 0.25
        c = inputs.mlp_case(4, M, K, H, r, s)
        Xd, dO = up(c.t["X"], "bf16"), up(c.t["dY"], "bf16")
        Wt = {k: up(c.t[k], "bf16") for k in ("Wg", "Ag", "Bg", "Wu", "Au", "Bu", "Wd", "Ad", "Bd")}
        Out = torch.empty((M, K), dtype=bf, device=dev)
        E = torch.empty((M, H), dtype=bf, device=dev)
        Gu = torch.empty((M, H), dtype=bf, device=dev)
        Hs = torch.empty((M, H), dtype=bf, device=dev)
        U = torch.empty((M, 3 * r), dtype=f32, device=dev)
        dX = torch.empty((M, K), dtype=bf, device=dev)
        gr = {k: torch.empty(sh, dtype=f32, device=dev) for k, sh in
              (("dAg", (r, K)), ("dBg", (H, r)), ("dAu", (r, K)), ("dBu", (H, r)), ("dAd", (r, H)), ("dBd", (K, r)))}
        nb = binding.workspace_bytes("swiglu_bwd", M, H, K, r)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        w = [P(Wt[k]) for k in ("Wg", "Ag", "Bg", "Wu", "Au", "Bu", "Wd", "Ad", "Bd")]

        if wl == "swiglu":
            fwd, bwd, act = L.swiglu_lora_mlp_fwd, L.swiglu_lora_mlp_bwd, ()
        else:
            fwd, bwd, act = L.geglu_lora_mlp_fwd, L.geglu_lora_mlp_bwd, (0,)   # exact gelu

        def step():
            check(fwd(M, K, H, r, s, s, s, *act, P(Xd), K, *w, P(Out), K, P(E), P(Gu), P(Hs), P(U), P(ws), 0, st()),
                  wl + "_lora_mlp_fwd")
            check(bwd(M, K, H, r, s, s, s, *act, P(dO), K, P(Xd), K, *w, P(E), P(Gu), P(Hs), P(U), P(dX), K,
                      P(gr["dAg"]), P(gr["dBg"]), P(gr["dAu"]), P(gr["dBu"]), P(gr["dAd"]), P(gr["dBd"]), P(ws), nb,
                      st()), wl + "_lora_mlp_bwd")
        base = 2.0 * M * K * H * 3 * 2           # three projections, forward + input gradient
        lora = 3 * (6.0 * M * r * (K + H))
        flops = base + lora
        # timed: the down projection (NT, four-wave) and dX over the 2H reduction (NN, eight-wave)
        gemm_flops = {0: 2.0 * M * K * H + 2.0 * M * K * r, 1: 2.0 * M * K * 2 * H + 2.0 * M * K * 2 * r}
        actname = "SwiGLU" if wl == "swiglu" else "GeGLU (exact gelu)"
        config = {"workload": f"bf16 LoRA MLP with fused {actname} fwd+bwd, M={M}, K={K}, H={H}, r={r}, s={s}",
                  "M": M, "K": K, "H": H, "r": r, "s": s}
    else:
        M = args.M or 4096
        N, K, r, s = 5120, 5120, 32, 0.5
        c = inputs.linear_case(5, M, N, K, r, s, "bf16")
        X, A, B, dY = (up(c.t[k], "bf16") for k in ("X", "A", "B", "dY"))
        W0f = up(inputs.normal(5, 1, (N, K), 1.0 / np.sqrt(K), "f32"), "f32")
        f8 = wl == "fp8"
        pre = "fp8" if f8 else "w8a8"
        code_t = torch.uint8 if f8 else torch.int8
        Wq = torch.empty((N, K), dtype=code_t, device=dev)
        sw = torch.empty((N,), dtype=f32, device=dev)
        prep = (lambda: check(getattr(L, pre + "_quantize_weight")(N, K, 0, P(W0f), K, P(Wq), P(sw), st()),  # noqa
                              pre + "_quantize_weight"),
                ("e4m3" if f8 else "int8") + " per-channel codes of the frozen fp32 weight (once per weight)",
                4.0 * N * K + 1.0 * N * K + 4.0 * N)
        prep[0]()
        fwd, bwd = getattr(L, pre + "_lora_linear_fwd"), getattr(L, pre + "_lora_linear_bwd")
        Y = torch.empty((M, N), dtype=bf, device=dev)
        Xq = torch.empty((M, K), dtype=code_t, device=dev)
        sx = torch.empty((M,), dtype=f32, device=dev)
        U = torch.empty((M, r), dtype=f32, device=dev)
        dX = torch.empty((M, K), dtype=bf, device=dev)
        dA = torch.empty((r, K), dtype=f32, device=dev)
        dB = torch.empty((N, r), dtype=f32, device=dev)
        nf = binding.workspace_bytes("w8a8_fwd", M, N, K, r)
        nb = binding.workspace_bytes("w8a8_bwd", M, N, K, r)
        ws = torch.empty(max(nf, nb, 256), dtype=torch.uint8, device=dev)

        def step():
            check(fwd(M, N, K, r, s, P(X), K, P(Wq), K, P(sw), P(A), P(B), None, P(Y), N, P(Xq), P(sx), P(U), r,
                      P(ws), nf, st()), pre + "_lora_linear_fwd")
            check(bwd(M, N, K, r, s, P(dY), N, P(X), K, P(Wq), K, P(sw), P(A), P(B), P(U), r, P(dX), K, P(dA), P(dB),
                      P(ws), nb, st()), pre + "_lora_linear_bwd")
        flops = 4.0 * M * N * K + 6.0 * M * r * (K + N)   # 8-bit ops of the base counted with the bf16 ones
        gemm_flops = {0: 2.0 * M * N * K + 2.0 * M * N * r, 1: 2.0 * M * N * K + 2.0 * M * K * r}
        base = "e4m3 (fp8)" if f8 else "W8A8 int8"
        config = {"workload": f"{base} base + bf16 LoRA fwd+bwd, M={M}, K=N={K}, r={r}, s={s}",
                  "M": M, "N": N, "K": K, "r": r, "s": s}

    # ------------------------------------------------------------------ warmup, then the timed region
    # (the per-kernel timing events are created first, so that nothing idles the GPU between
    # the warm-up and the timed steps)
    K_steps = args.steps
    # hook 2: the gated MLP backward's activation pass (dE, dGu from dH, E, Gu in place)
    hook_kinds = tuple(gemm_kinds) + ((2,) if wl in ("swiglu", "geglu") else ())
    evs = {k: (TimingEvents(K_steps), TimingEvents(K_steps)) for k in hook_kinds}
    for _ in range(args.warmup):
        step()
    keep = []
    for k in hook_kinds:
        a, b = evs[k][0].arr, evs[k][1].arr
        keep.append((a, b))
        check(L.ldl_set_kernel_events(k, a, b, K_steps), "ldl_set_kernel_events")
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = TimingEvents(K_steps + 1) if args.step_times else None
    torch.cuda.synchronize()
    t_start.record()
    if marks is not None:
        marks.record(0, st())
    for i in range(K_steps):
        step()
        if marks is not None:
            marks.record(i + 1, st())
    t_stop.record()
    torch.cuda.synchronize()
    for k in hook_kinds:
        L.ldl_set_kernel_events(k, None, None, 0)
    ms = t_start.elapsed_time(t_stop) / K_steps
    value = flops / (ms * 1e-3) / 1e12

    kern = {}
    for k in gemm_kinds:
        times = [evs[k][0].elapsed_ms(evs[k][1], i) for i in range(K_steps)]
        avg = sum(times) / len(times)
        kern[k] = {"avg_us": avg * 1e3, "tflops": gemm_flops[k] / (avg * 1e-3) / 1e12}
    act_pass = None
    if 2 in hook_kinds:
        # reads dH, E, Gu and writes dE, dGu: 10 bytes per hidden unit and token (bf16)
        times = [evs[2][0].elapsed_ms(evs[2][1], i) for i in range(K_steps)]
        avg = sum(times) / len(times)
        nbytes = 10 * M * H
        act_pass = {"kernel": "swiglu_bwd_kernel (dE, dGu in place over dH)", "avg_us": round(avg * 1e3, 2),
                    "bytes": nbytes, "GB/s": round(nbytes / (avg * 1e-3) / 1e9, 1),
                    "frac_hbm": round(nbytes / (avg * 1e-3) / 1e9 / 8000.0, 4)}

    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K_steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": {"w8a8": "int8+bf16", "fp8": "e4m3+bf16"}.get(wl, "bf16"), "data": "synthetic",
           "config": config, "pct_bf16_peak": round(100.0 * value / PEAK_BF16, 2)}
    if kern:
        dom = max(kern, key=lambda k: kern[k]["avg_us"])
        # the LoRA and DoRA products (N a multiple of 256) run on the four-wave tile unless
        # it is switched off
        four = wl in ("lora", "dora", "dora_cols", "qkv") and args.gemm_4wave != 0
        names = {0: "forward base GEMM (" + ("gemm16_kernel NT" if four else "gemm_kernel NT") + ")",
                 1: "input-gradient GEMM (" + ("gemm16_kernel NN" if four else "gemm_kernel NN") + ")"}
        if wl in ("swiglu", "geglu"):
            names = {0: "down-projection GEMM (" + ("gemm16_kernel NT" if args.gemm_4wave != 0 else "gemm_kernel NT")
                        + ")",
                     1: "input-gradient GEMM over gate and up (" +
                        ("gemm16_kernel NN over the two stacked weights" if args.gemm_4wave != 0 else "gemm_kernel NN")
                        + ")"}
        if wl == "fp8":
            names[0] = "forward base GEMM (gemm_f8_kernel NT, e4m3 block-scaled MFMA)"
        if wl in ("w8a8", "fp8"):
            if wl == "w8a8":
                names[0] = "forward base GEMM (int8 NT tile: gemm16_kernel, or gemm_kernel 256x128 at few tiles)"
            names[1] = ("input-gradient GEMM (gemm16_kernel NN on the weight dequantised to bf16 once per step)"
                        if M >= 512 else "input-gradient GEMM (gemm_kernel NN, 8-bit weight widened to bf16 in LDS)")
        peak = PEAK_INT8 if (wl in ("w8a8", "fp8") and dom == 0) else PEAK_BF16
        traffic = recorded_traffic(f"{wl}:{names[dom]}")
        out["roofline"] = {"bound": "mfma", "kernel": names[dom], "achieved": round(kern[dom]["tflops"], 1),
                           "peak": peak, "unit": "TFLOP/s", "frac": round(kern[dom]["tflops"] / peak, 4),
                           "traffic": None if traffic is None else int(traffic)}
        out["kernels"] = {names[k]: {"avg_us": round(v["avg_us"], 2), "TFLOP/s": round(v["tflops"], 1)}
                          for k, v in kern.items()}
    if marks is not None:
        out["step_us"] = [round(1e3 * marks.between_ms(i, i + 1), 1) for i in range(K_steps)]
    if act_pass is not None:
        out["activation_pass"] = act_pass
    if prep is not None:
        # not part of the step: once per frozen weight; timed here over 20 calls
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        prep[0]()
        p0.record()
        for _ in range(20):
            prep[0]()
        p1.record()
        torch.cuda.synchronize()
        us = p0.elapsed_time(p1) / 20 * 1e3
        out["prepare"] = {"kernel": prep[1], "us": round(us, 2), "bytes": int(prep[2]),
                          "GB/s": round(prep[2] / (us * 1e-6) / 1e9, 1)}
    if wl == "lora" and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_lora(4096, 4096, 4096, 16, 0.5)
        out["cpu_baseline"].pop("seconds", None)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
