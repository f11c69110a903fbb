"""Thin Python binding of liblora_dora_linear.so (ctypes).

Argument marshalling only: each wrapper checks dtypes / devices / contiguity,
allocates the outputs and the workspace with torch (PyTorch serves as the
device-memory and stream provider), and calls the C entry point of the same
name on torch's current stream.  Every step of the computation runs in the HIP
kernels; there is no fallback: if the library is missing the call raises.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblora_dora_linear.so")

LDL_F32, LDL_BF16 = 0, 1
OPS = {"lora_fwd": 0, "lora_bwd": 1, "dora_fwd": 2, "dora_bwd": 3,
       "swiglu_fwd": 4, "swiglu_bwd": 5, "w8a8_fwd": 6, "w8a8_bwd": 7}

_lib = None

_i, _f, _p, _z = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

# C signatures (argument types, return type) of every exported entry point.
SIGNATURES = {
    "ldl_status_string": ([_i], ctypes.c_char_p),
    "ldl_version": ([], _i),
    "ldl_set_tuning": ([_i, _i], _i),
    "ldl_set_kernel_events": ([_i, ctypes.POINTER(_p), ctypes.POINTER(_p), _i], _i),
    "ldl_workspace_bytes": ([_i, _i, _i, _i, _i, _i], _z),
    "dora_state_floats": ([_i, _i], _z),
    "lora_linear_fwd": ([_i, _i, _i, _i, _f, _i, _p, _p, _p, _p, _p, _p, _p, _p, _z, _p], _i),
    "lora_linear_bwd": ([_i, _i, _i, _i, _f, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _z, _p], _i),
    "lora_linear_bwd_noalloc": ([_i, _i, _i, _i, _f, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p], _i),
    "ldl_noalloc_scratch_bytes": ([], _z),
    "dora_prepare": ([_i, _i, _i, _p, _p, _p], _i),
    "dora_linear_fwd": ([_i, _i, _i, _i, _f, _f, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _z, _p], _i),
    "dora_linear_bwd": ([_i, _i, _i, _i, _f, _f, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                         _p, _z, _p], _i),
    "swiglu_lora_mlp_fwd": ([_i, _i, _i, _i, _f, _f, _f] + [_p] * 16 + [_z, _p], _i),
    "swiglu_lora_mlp_bwd": ([_i, _i, _i, _i, _f, _f, _f] + [_p] * 23 + [_z, _p], _i),
    "w8a8_quantize_weight": ([_i, _i, _i, _p, _p, _p, _p], _i),
    "w8a8_quantize_rows": ([_i, _i, _p, _p, _p, _p], _i),
    "int8_gemm_raw": ([_i, _i, _i, _p, _p, _p, _p], _i),
    "w8a8_lora_linear_fwd": ([_i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _z, _p], _i),
    "w8a8_lora_linear_bwd": ([_i, _i, _i, _i, _f] + [_p] * 11 + [_z, _p], _i),
}


class LdlError(RuntimeError):
    pass


def lib():
    """The loaded library with every signature declared (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library missing: {LIB_PATH}; build it with "
                               "`python -m lora_dora_linear_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


# ------------------------------------------------------------------ helpers
def status_string(code):
    return lib().ldl_status_string(int(code)).decode()


def _check(code, name):
    if code != 0:
        raise LdlError(f"{name} failed: {status_string(code)} (status {code})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t):
    if t.dtype == torch.bfloat16:
        return LDL_BF16
    if t.dtype == torch.float32:
        return LDL_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, dtype=None, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def workspace_bytes(op, M, N, K, r, dtype=LDL_BF16):
    return int(lib().ldl_workspace_bytes(OPS[op] if isinstance(op, str) else op, M, N, K, r, dtype))


def _ws(op, M, N, K, r, dtype, device):
    n = workspace_bytes(op, M, N, K, r, dtype)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device), n


def set_tuning(key, value):
    _check(lib().ldl_set_tuning(int(key), int(value)), "ldl_set_tuning")


def dora_state_floats(N, r):
    return int(lib().dora_state_floats(N, r))


# ------------------------------------------------------------------ LoRA
def lora_linear_fwd(X, W0, A, B, s, bias=None, save_u=True):
    """Y = X.W0^T + s.(X.A^T).B^T (+ bias).  Returns (Y, U or None)."""
    M, K = X.shape
    N, r = B.shape
    dt = X.dtype
    for t, n, sh in ((X, "X", (M, K)), (W0, "W0", (N, K)), (A, "A", (r, K)), (B, "B", (N, r))):
        _need(t, n, dt, sh)
    if bias is not None:
        _need(bias, "bias", dt, (N,))
    Y = torch.empty((M, N), dtype=dt, device=X.device)
    U = torch.empty((M, r), dtype=torch.float32, device=X.device) if save_u else None
    ws, n = _ws("lora_fwd", M, N, K, r, _dt(X), X.device)
    _check(lib().lora_linear_fwd(M, N, K, r, float(s), _dt(X), _ptr(X), _ptr(W0), _ptr(A), _ptr(B), _ptr(bias),
                                 _ptr(Y), _ptr(U), _ptr(ws), n, _stream()), "lora_linear_fwd")
    return Y, U


def lora_linear_bwd(dY, X, W0, A, B, s, U=None, need_dx=True, need_dbias=False):
    """Returns dict(dX, dA, dB, dbias) of the LoRA linear."""
    M, K = X.shape
    N, r = B.shape
    dt = X.dtype
    for t, n, sh in ((dY, "dY", (M, N)), (X, "X", (M, K)), (W0, "W0", (N, K)), (A, "A", (r, K)), (B, "B", (N, r))):
        _need(t, n, dt, sh)
    if U is not None:
        _need(U, "U", torch.float32, (M, r))
    dev = X.device
    dX = torch.empty((M, K), dtype=dt, device=dev) if need_dx else None
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    db = torch.empty((N,), dtype=torch.float32, device=dev) if need_dbias else None
    ws, n = _ws("lora_bwd", M, N, K, r, _dt(X), dev)
    _check(lib().lora_linear_bwd(M, N, K, r, float(s), _dt(X), _ptr(dY), _ptr(X), _ptr(W0), _ptr(A), _ptr(B), _ptr(U),
                                 _ptr(dX), _ptr(dA), _ptr(dB), _ptr(db), _ptr(ws), n, _stream()), "lora_linear_bwd")
    return {"dX": dX, "dA": dA, "dB": dB, "dbias": db}


def lora_linear_bwd_noalloc(dY, X, W0, A, B, s, U=None, need_dx=True, need_dbias=False):
    """lora_linear_bwd on the library's fixed per-device scratch (no workspace is allocated)."""
    M, K = X.shape
    N, r = B.shape
    dt = X.dtype
    for t, n, sh in ((dY, "dY", (M, N)), (X, "X", (M, K)), (W0, "W0", (N, K)), (A, "A", (r, K)), (B, "B", (N, r))):
        _need(t, n, dt, sh)
    if U is not None:
        _need(U, "U", torch.float32, (M, r))
    dev = X.device
    dX = torch.empty((M, K), dtype=dt, device=dev) if need_dx else None
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    db = torch.empty((N,), dtype=torch.float32, device=dev) if need_dbias else None
    _check(lib().lora_linear_bwd_noalloc(M, N, K, r, float(s), _dt(X), _ptr(dY), _ptr(X), _ptr(W0), _ptr(A), _ptr(B),
                                         _ptr(U), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(db), _stream()),
           "lora_linear_bwd_noalloc")
    return {"dX": dX, "dA": dA, "dB": dB, "dbias": db}


# ------------------------------------------------------------------ DoRA
def dora_prepare(W0):
    N, K = W0.shape
    _need(W0, "W0")
    out = torch.empty((N,), dtype=torch.float32, device=W0.device)
    _check(lib().dora_prepare(N, K, _dt(W0), _ptr(W0), _ptr(out), _stream()), "dora_prepare")
    return out


def dora_linear_fwd(X, W0, A, B, m, w0_sumsq, s, eps=1e-12, bias=None):
    """Returns (Y, U, Z, state) where state = [norm | g | P | G] (fp32)."""
    M, K = X.shape
    N, r = B.shape
    dt = X.dtype
    for t, n, sh in ((X, "X", (M, K)), (W0, "W0", (N, K)), (A, "A", (r, K)), (B, "B", (N, r))):
        _need(t, n, dt, sh)
    _need(m, "m", torch.float32, (N,))
    _need(w0_sumsq, "w0_sumsq", torch.float32, (N,))
    if bias is not None:
        _need(bias, "bias", dt, (N,))
    dev = X.device
    Y = torch.empty((M, N), dtype=dt, device=dev)
    Z = torch.empty((M, N), dtype=dt, device=dev)
    U = torch.empty((M, r), dtype=torch.float32, device=dev)
    state = torch.empty((dora_state_floats(N, r),), dtype=torch.float32, device=dev)
    ws, n = _ws("dora_fwd", M, N, K, r, _dt(X), dev)
    _check(lib().dora_linear_fwd(M, N, K, r, float(s), float(eps), _dt(X), _ptr(X), _ptr(W0), _ptr(A), _ptr(B),
                                 _ptr(m), _ptr(w0_sumsq), _ptr(bias), _ptr(Y), _ptr(U), _ptr(Z), _ptr(state),
                                 _ptr(ws), n, _stream()), "dora_linear_fwd")
    return Y, U, Z, state


def dora_linear_bwd(dY, X, W0, A, B, m, U, Z, state, s, eps=1e-12, need_dx=True, need_dbias=False):
    """Returns dict(dX, dA, dB, dm, dbias)."""
    M, K = X.shape
    N, r = B.shape
    dt = X.dtype
    for t, n, sh in ((dY, "dY", (M, N)), (X, "X", (M, K)), (W0, "W0", (N, K)), (A, "A", (r, K)),
                     (B, "B", (N, r)), (Z, "Z", (M, N))):
        _need(t, n, dt, sh)
    _need(m, "m", torch.float32, (N,))
    _need(U, "U", torch.float32, (M, r))
    _need(state, "state", torch.float32, (dora_state_floats(N, r),))
    dev = X.device
    dX = torch.empty((M, K), dtype=dt, device=dev) if need_dx else None
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    dm = torch.empty((N,), dtype=torch.float32, device=dev)
    db = torch.empty((N,), dtype=torch.float32, device=dev) if need_dbias else None
    ws, n = _ws("dora_bwd", M, N, K, r, _dt(X), dev)
    _check(lib().dora_linear_bwd(M, N, K, r, float(s), float(eps), _dt(X), _ptr(dY), _ptr(X), _ptr(W0), _ptr(A),
                                 _ptr(B), _ptr(m), _ptr(U), _ptr(Z), _ptr(state), _ptr(dX), _ptr(dA), _ptr(dB),
                                 _ptr(dm), _ptr(db), _ptr(ws), n, _stream()), "dora_linear_bwd")
    return {"dX": dX, "dA": dA, "dB": dB, "dm": dm, "dbias": db}


# ------------------------------------------------------------------ SwiGLU MLP
def swiglu_lora_mlp_fwd(X, gate, up, down):
    """gate/up/down = (W, A, B, s).  Returns (Out, saved) with saved = dict(E, Gu, H, U)."""
    M, K = X.shape
    (Wg, Ag, Bg, sg), (Wu, Au, Bu, su), (Wd, Ad, Bd, sd) = gate, up, down
    H, r = Bg.shape
    bf = torch.bfloat16
    _need(X, "X", bf, (M, K))
    for t, n, sh in ((Wg, "Wg", (H, K)), (Ag, "Ag", (r, K)), (Bg, "Bg", (H, r)), (Wu, "Wu", (H, K)),
                     (Au, "Au", (r, K)), (Bu, "Bu", (H, r)), (Wd, "Wd", (K, H)), (Ad, "Ad", (r, H)),
                     (Bd, "Bd", (K, r))):
        _need(t, n, bf, sh)
    dev = X.device
    Out = torch.empty((M, K), dtype=bf, device=dev)
    E = torch.empty((M, H), dtype=bf, device=dev)
    Gu = torch.empty((M, H), dtype=bf, device=dev)
    Hs = torch.empty((M, H), dtype=bf, device=dev)
    U = torch.empty((M, 3 * r), dtype=torch.float32, device=dev)
    ws, n = _ws("swiglu_fwd", M, H, K, r, LDL_BF16, dev)
    _check(lib().swiglu_lora_mlp_fwd(M, K, H, r, float(sg), float(su), float(sd), _ptr(X), _ptr(Wg), _ptr(Ag),
                                     _ptr(Bg), _ptr(Wu), _ptr(Au), _ptr(Bu), _ptr(Wd), _ptr(Ad), _ptr(Bd), _ptr(Out),
                                     _ptr(E), _ptr(Gu), _ptr(Hs), _ptr(U), _ptr(ws), n, _stream()),
           "swiglu_lora_mlp_fwd")
    return Out, {"E": E, "Gu": Gu, "H": Hs, "U": U}


def swiglu_lora_mlp_bwd(dOut, X, gate, up, down, saved, need_dx=True):
    M, K = X.shape
    (Wg, Ag, Bg, sg), (Wu, Au, Bu, su), (Wd, Ad, Bd, sd) = gate, up, down
    H, r = Bg.shape
    bf = torch.bfloat16
    _need(dOut, "dOut", bf, (M, K))
    dev = X.device
    f32 = torch.float32
    dX = torch.empty((M, K), dtype=bf, device=dev) if need_dx else None
    out = {"dX": dX,
           "dA_gate": torch.empty((r, K), dtype=f32, device=dev), "dB_gate": torch.empty((H, r), dtype=f32, device=dev),
           "dA_up": torch.empty((r, K), dtype=f32, device=dev), "dB_up": torch.empty((H, r), dtype=f32, device=dev),
           "dA_down": torch.empty((r, H), dtype=f32, device=dev), "dB_down": torch.empty((K, r), dtype=f32, device=dev)}
    ws, n = _ws("swiglu_bwd", M, H, K, r, LDL_BF16, dev)
    _check(lib().swiglu_lora_mlp_bwd(M, K, H, r, float(sg), float(su), float(sd), _ptr(dOut), _ptr(X), _ptr(Wg),
                                     _ptr(Ag), _ptr(Bg), _ptr(Wu), _ptr(Au), _ptr(Bu), _ptr(Wd), _ptr(Ad), _ptr(Bd),
                                     _ptr(saved["E"]), _ptr(saved["Gu"]), _ptr(saved["H"]), _ptr(saved["U"]),
                                     _ptr(dX), _ptr(out["dA_gate"]), _ptr(out["dB_gate"]), _ptr(out["dA_up"]),
                                     _ptr(out["dB_up"]), _ptr(out["dA_down"]), _ptr(out["dB_down"]), _ptr(ws), n,
                                     _stream()), "swiglu_lora_mlp_bwd")
    return out


# ------------------------------------------------------------------ W8A8
def w8a8_quantize_weight(W0):
    N, K = W0.shape
    _need(W0, "W0")
    Wq = torch.empty((N, K), dtype=torch.int8, device=W0.device)
    sw = torch.empty((N,), dtype=torch.float32, device=W0.device)
    _check(lib().w8a8_quantize_weight(N, K, _dt(W0), _ptr(W0), _ptr(Wq), _ptr(sw), _stream()), "w8a8_quantize_weight")
    return Wq, sw


def w8a8_quantize_rows(X):
    M, K = X.shape
    _need(X, "X", torch.bfloat16)
    Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    sx = torch.empty((M,), dtype=torch.float32, device=X.device)
    _check(lib().w8a8_quantize_rows(M, K, _ptr(X), _ptr(Xq), _ptr(sx), _stream()), "w8a8_quantize_rows")
    return Xq, sx


def int8_gemm_raw(Xq, Wq):
    M, K = Xq.shape
    N = Wq.shape[0]
    _need(Xq, "Xq", torch.int8, (M, K))
    _need(Wq, "Wq", torch.int8, (N, K))
    C = torch.empty((M, N), dtype=torch.int32, device=Xq.device)
    _check(lib().int8_gemm_raw(M, N, K, _ptr(Xq), _ptr(Wq), _ptr(C), _stream()), "int8_gemm_raw")
    return C


def w8a8_lora_linear_fwd(X, Wq, sw, A, B, s, bias=None, save=True):
    """Returns (Y, Xq, sx, U)."""
    M, K = X.shape
    N, r = B.shape
    bf = torch.bfloat16
    _need(X, "X", bf, (M, K))
    _need(Wq, "Wq", torch.int8, (N, K))
    _need(sw, "sw", torch.float32, (N,))
    _need(A, "A", bf, (r, K))
    _need(B, "B", bf, (N, r))
    if bias is not None:
        _need(bias, "bias", bf, (N,))
    dev = X.device
    Y = torch.empty((M, N), dtype=bf, device=dev)
    Xq = torch.empty((M, K), dtype=torch.int8, device=dev) if save else None
    sx = torch.empty((M,), dtype=torch.float32, device=dev) if save else None
    U = torch.empty((M, r), dtype=torch.float32, device=dev) if save else None
    ws, n = _ws("w8a8_fwd", M, N, K, r, LDL_BF16, dev)
    _check(lib().w8a8_lora_linear_fwd(M, N, K, r, float(s), _ptr(X), _ptr(Wq), _ptr(sw), _ptr(A), _ptr(B), _ptr(bias),
                                      _ptr(Y), _ptr(Xq), _ptr(sx), _ptr(U), _ptr(ws), n, _stream()),
           "w8a8_lora_linear_fwd")
    return Y, Xq, sx, U


def w8a8_lora_linear_bwd(dY, X, Wq, sw, A, B, s, U=None, need_dx=True):
    M, K = X.shape
    N, r = B.shape
    bf = torch.bfloat16
    _need(dY, "dY", bf, (M, N))
    dev = X.device
    dX = torch.empty((M, K), dtype=bf, device=dev) if need_dx else None
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    ws, n = _ws("w8a8_bwd", M, N, K, r, LDL_BF16, dev)
    _check(lib().w8a8_lora_linear_bwd(M, N, K, r, float(s), _ptr(dY), _ptr(X), _ptr(Wq), _ptr(sw), _ptr(A), _ptr(B),
                                      _ptr(U), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), n, _stream()),
           "w8a8_lora_linear_bwd")
    return {"dX": dX, "dA": dA, "dB": dB}
