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
       "swiglu_fwd": 4, "swiglu_bwd": 5, "w8a8_fwd": 6, "w8a8_bwd": 7, "merge_bwd": 8,
       "dora_cols_fwd": 9, "dora_cols_bwd": 10}

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
    "lora_linear_fwd": ([_i, _i, _i, _i, _f, _i, _p, _i, _p, _i, _p, _p, _p, _p, _i, _p, _i, _p, _z, _p], _i),
    "lora_linear_bwd": ([_i, _i, _i, _i, _f, _i, _p, _i, _p, _i, _p, _i, _p, _p, _p, _i, _p, _i, _p, _p, _p,
                         _p, _z, _p], _i),
    "lora_linear_bwd_noalloc": ([_i, _i, _i, _i, _f, _i, _p, _i, _p, _i, _p, _i, _p, _p, _p, _i, _p, _i, _p, _p,
                                 _p, _p], _i),
    "ldl_noalloc_scratch_bytes": ([], _z),
    "ldl_multi_workspace_bytes": ([_i, _i, _i, _i, _p, _i], _z),
    "lora_multi_linear_fwd": ([_i, _i, _i, _p, _i, _p, _i, _p, _i, _p, _i, _p, _p, _p, _p, _i, _p, _i, _p, _z, _p],
                              _i),
    "lora_multi_linear_bwd": ([_i, _i, _i, _p, _i, _p, _i, _p, _i, _p, _i, _p, _i, _p, _p, _p, _i, _p, _i, _p, _p,
                               _p, _p, _z, _p], _i),
    "lora_dropout_mask": ([_i, _i, _i, _p, _p, _p, _p], _i),
    "lora_dropout_grad": ([_i, _i, _p, _p, _p], _i),
    "lora_merge_fwd": ([_i, _i, _i, _f, _i, _p, _i, _p, _p, _p, _i, _p], _i),
    "lora_merge_bwd": ([_i, _i, _i, _f, _i, _p, _i, _p, _p, _p, _p, _p, _z, _p], _i),
    "dora_prepare": ([_i, _i, _i, _p, _i, _p, _p], _i),
    "dora_linear_fwd": ([_i, _i, _i, _i, _f, _f, _i, _p, _i, _p, _i, _p, _p, _p, _p, _p, _p, _i, _p, _i, _p, _i,
                         _p, _p, _z, _p], _i),
    "dora_linear_bwd": ([_i, _i, _i, _i, _f, _f, _i, _p, _i, _p, _i, _p, _i, _p, _p, _p, _p, _i, _p, _i, _p,
                         _p, _i, _p, _p, _p, _p, _p, _z, _p], _i),
    "swiglu_lora_mlp_fwd": ([_i, _i, _i, _i, _f, _f, _f, _p, _i] + [_p] * 9 + [_p, _i] + [_p] * 5 + [_z, _p], _i),
    "swiglu_lora_mlp_bwd": ([_i, _i, _i, _i, _f, _f, _f, _p, _i, _p, _i] + [_p] * 13 + [_p, _i] + [_p] * 7
                            + [_z, _p], _i),
    "geglu_lora_mlp_fwd": ([_i, _i, _i, _i, _f, _f, _f, _i, _p, _i] + [_p] * 9 + [_p, _i] + [_p] * 5 + [_z, _p],
                           _i),
    "geglu_lora_mlp_bwd": ([_i, _i, _i, _i, _f, _f, _f, _i, _p, _i, _p, _i] + [_p] * 13 + [_p, _i] + [_p] * 7
                           + [_z, _p], _i),
    "dora_cols_prepare": ([_i, _i, _i, _p, _i, _p, _p], _i),
    "dora_cols_linear_fwd": ([_i, _i, _i, _i, _f, _f, _i, _p, _i, _p, _i, _p, _p, _p, _p, _p, _p, _i, _p, _i, _p,
                              _i, _p, _p, _z, _p], _i),
    "dora_cols_linear_bwd": ([_i, _i, _i, _i, _f, _f, _i, _p, _i, _p, _i, _p, _i, _p, _i, _p, _p, _p, _p, _i, _p,
                              _p, _i, _p, _p, _p, _p, _p, _z, _p], _i),
    "w8a8_quantize_weight": ([_i, _i, _i, _p, _i, _p, _p, _p], _i),
    "w8a8_quantize_rows": ([_i, _i, _p, _i, _p, _p, _p], _i),
    "int8_gemm_raw": ([_i, _i, _i, _p, _i, _p, _i, _p, _i, _p], _i),
    "fp8_quantize_weight": ([_i, _i, _i, _p, _i, _p, _p, _p], _i),
    "fp8_quantize_rows": ([_i, _i, _p, _i, _p, _p, _p], _i),
    "fp8_lora_linear_fwd": ([_i, _i, _i, _i, _f, _p, _i, _p, _i, _p, _p, _p, _p, _p, _i, _p, _p, _p, _i, _p, _z,
                             _p], _i),
    "fp8_lora_linear_bwd": ([_i, _i, _i, _i, _f, _p, _i, _p, _i, _p, _i, _p, _p, _p, _p, _i, _p, _i, _p, _p, _p,
                             _z, _p], _i),
    "w8a8_lora_linear_fwd": ([_i, _i, _i, _i, _f, _p, _i, _p, _i, _p, _p, _p, _p, _p, _i, _p, _p, _p, _i, _p, _z,
                              _p], _i),
    "w8a8_lora_linear_bwd": ([_i, _i, _i, _i, _f, _p, _i, _p, _i, _p, _i, _p, _p, _p, _p, _i, _p, _i, _p, _p, _p,
                              _z, _p], _i),
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


def _mat(t, name, dtype, shape):
    """A 2-D row-major operand that may be a strided view (unit column stride); returns its
    leading dimension (row stride in elements) for the C call."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.shape[0] > 1 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must be row-major with unit column stride")
    return int(t.stride(0)) if t.shape[0] > 1 else int(t.shape[1])


def _out(t, name, dtype, shape, device):
    """A caller-provided output (possibly a strided view) or a new dense tensor, and its ld."""
    if t is None:
        t = torch.empty(shape, dtype=dtype, device=device)
    return t, _mat(t, name, dtype, shape)


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
def lora_linear_fwd(X, W0, A, B, s, bias=None, save_u=True, Y=None, U=None):
    """Y = X.W0^T + s.(X.A^T).B^T (+ bias).  Returns (Y, U or None).  X, W0 (and given
    outputs Y, U) may be row-major strided views."""
    M, K = X.shape
    N, r = B.shape
    dt = X.dtype
    ldx = _mat(X, "X", dt, (M, K))
    ldw = _mat(W0, "W0", dt, (N, K))
    _need(A, "A", dt, (r, K))
    _need(B, "B", dt, (N, r))
    if bias is not None:
        _need(bias, "bias", dt, (N,))
    Y, ldy = _out(Y, "Y", dt, (M, N), X.device)
    ldu = 0
    if save_u or U is not None:
        U, ldu = _out(U, "U", torch.float32, (M, r), X.device)
    ws, n = _ws("lora_fwd", M, N, K, r, _dt(X), X.device)
    _check(lib().lora_linear_fwd(M, N, K, r, float(s), _dt(X), _ptr(X), ldx, _ptr(W0), ldw, _ptr(A), _ptr(B),
                                 _ptr(bias), _ptr(Y), ldy, _ptr(U), ldu, _ptr(ws), n, _stream()), "lora_linear_fwd")
    return Y, U


def _lora_bwd_args(dY, X, W0, A, B, U, need_dx, need_dbias, dX):
    M, K = X.shape
    N, r = B.shape
    dt = X.dtype
    lddy = _mat(dY, "dY", dt, (M, N))
    ldx = _mat(X, "X", dt, (M, K))
    ldw = _mat(W0, "W0", dt, (N, K))
    _need(A, "A", dt, (r, K))
    _need(B, "B", dt, (N, r))
    ldu = _mat(U, "U", torch.float32, (M, r)) if U is not None else 0
    dev = X.device
    lddx = 0
    if need_dx:
        dX, lddx = _out(dX, "dX", dt, (M, K), dev)
    else:
        dX = None
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    db = torch.empty((N,), dtype=torch.float32, device=dev) if need_dbias else None
    args = (M, N, K, r, None, _dt(X), _ptr(dY), lddy, _ptr(X), ldx, _ptr(W0), ldw, _ptr(A), _ptr(B), _ptr(U), ldu,
            _ptr(dX), lddx, _ptr(dA), _ptr(dB), _ptr(db))
    return args, {"dX": dX, "dA": dA, "dB": dB, "dbias": db}


def lora_linear_bwd(dY, X, W0, A, B, s, U=None, need_dx=True, need_dbias=False, dX=None):
    """Returns dict(dX, dA, dB, dbias) of the LoRA linear.  dY, X, W0, U (and a given dX)
    may be row-major strided views."""
    args, out = _lora_bwd_args(dY, X, W0, A, B, U, need_dx, need_dbias, dX)
    M, N, K, r = args[:4]
    args = args[:4] + (float(s),) + args[5:]
    ws, n = _ws("lora_bwd", M, N, K, r, _dt(X), X.device)
    _check(lib().lora_linear_bwd(*args, _ptr(ws), n, _stream()), "lora_linear_bwd")
    return out


def lora_linear_bwd_noalloc(dY, X, W0, A, B, s, U=None, need_dx=True, need_dbias=False, dX=None):
    """lora_linear_bwd on the library's fixed per-device scratch (no workspace is allocated)."""
    args, out = _lora_bwd_args(dY, X, W0, A, B, U, need_dx, need_dbias, dX)
    args = args[:4] + (float(s),) + args[5:]
    _check(lib().lora_linear_bwd_noalloc(*args, _stream()), "lora_linear_bwd_noalloc")
    return out


# ------------------------------------------------------------------ fused QKV leaves
def _leaf_arrays(n_leaf, s_leaf):
    L = len(n_leaf)
    if len(s_leaf) != L:
        raise ValueError("n_leaf and s_leaf must have the same length")
    return L, (ctypes.c_int * L)(*[int(n) for n in n_leaf]), (ctypes.c_float * L)(*[float(v) for v in s_leaf])


def multi_workspace_bytes(op, M, K, n_leaf, r):
    L = len(n_leaf)
    arr = (ctypes.c_int * L)(*[int(n) for n in n_leaf])
    return int(lib().ldl_multi_workspace_bytes(OPS[op] if isinstance(op, str) else op, M, K, L,
                                               ctypes.cast(arr, _p), r))


def lora_multi_linear_fwd(X, W0, A, B, n_leaf, s_leaf, bias=None, save_u=True, Y=None, U=None):
    """Several adapters over one concatenated base weight: Y[:, leaf l] = X.W0_l^T +
    s_l.(X.A_l^T).B_l^T (+ bias).  A = [A_1; ..; A_L] [L r, K], B = [B_1; ..; B_L] [N, r].
    Returns (Y, U [M, L r] or None)."""
    M, K = X.shape
    N, r = B.shape
    L, nl, sl = _leaf_arrays(n_leaf, s_leaf)
    if sum(int(n) for n in n_leaf) != N:
        raise ValueError("the leaf widths must add up to the rows of B")
    dt = X.dtype
    ldx = _mat(X, "X", dt, (M, K))
    ldw = _mat(W0, "W0", dt, (N, K))
    _need(A, "A", dt, (L * r, K))
    _need(B, "B", dt, (N, r))
    if bias is not None:
        _need(bias, "bias", dt, (N,))
    Y, ldy = _out(Y, "Y", dt, (M, N), X.device)
    ldu = 0
    if save_u or U is not None:
        U, ldu = _out(U, "U", torch.float32, (M, L * r), X.device)
    n = multi_workspace_bytes("lora_fwd", M, K, n_leaf, r)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=X.device)
    _check(lib().lora_multi_linear_fwd(M, K, L, ctypes.cast(nl, _p), r, ctypes.cast(sl, _p), _dt(X), _ptr(X), ldx,
                                       _ptr(W0), ldw, _ptr(A), _ptr(B), _ptr(bias), _ptr(Y), ldy, _ptr(U), ldu,
                                       _ptr(ws), n, _stream()), "lora_multi_linear_fwd")
    return Y, U


def lora_multi_linear_bwd(dY, X, W0, A, B, n_leaf, s_leaf, U=None, need_dx=True, need_dbias=False, dX=None):
    """Gradients of the fused leaves: dict(dX, dA [L r, K], dB [N, r], dbias)."""
    M, K = X.shape
    N, r = B.shape
    L, nl, sl = _leaf_arrays(n_leaf, s_leaf)
    dt = X.dtype
    lddy = _mat(dY, "dY", dt, (M, N))
    ldx = _mat(X, "X", dt, (M, K))
    ldw = _mat(W0, "W0", dt, (N, K))
    _need(A, "A", dt, (L * r, K))
    _need(B, "B", dt, (N, r))
    ldu = _mat(U, "U", torch.float32, (M, L * r)) if U is not None else 0
    dev = X.device
    lddx = 0
    if need_dx:
        dX, lddx = _out(dX, "dX", dt, (M, K), dev)
    else:
        dX = None
    dA = torch.empty((L * r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    db = torch.empty((N,), dtype=torch.float32, device=dev) if need_dbias else None
    n = multi_workspace_bytes("lora_bwd", M, K, n_leaf, r)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    _check(lib().lora_multi_linear_bwd(M, K, L, ctypes.cast(nl, _p), r, ctypes.cast(sl, _p), _dt(X), _ptr(dY), lddy,
                                       _ptr(X), ldx, _ptr(W0), ldw, _ptr(A), _ptr(B), _ptr(U), ldu, _ptr(dX), lddx,
                                       _ptr(dA), _ptr(dB), _ptr(db), _ptr(ws), n, _stream()), "lora_multi_linear_bwd")
    return {"dX": dX, "dA": dA, "dB": dB, "dbias": db}


# ------------------------------------------------------------------ weight-space dropout
def lora_dropout_mask(A, keep):
    """A . diag(keep): lora_down with the dropped input features zeroed (keep: uint8 [K])."""
    r, K = A.shape
    _need(A, "A", A.dtype, (r, K))
    _need(keep, "keep", torch.uint8, (K,))
    out = torch.empty_like(A)
    _check(lib().lora_dropout_mask(r, K, _dt(A), _ptr(A), _ptr(keep), _ptr(out), _stream()), "lora_dropout_mask")
    return out


def lora_dropout_grad(dA, keep):
    """Zeroes the dropped columns of a factor gradient dA [r, K] (fp32) in place; returns dA."""
    r, K = dA.shape
    _need(dA, "dA", torch.float32, (r, K))
    _need(keep, "keep", torch.uint8, (K,))
    _check(lib().lora_dropout_grad(r, K, _ptr(keep), _ptr(dA), _stream()), "lora_dropout_grad")
    return dA


# ------------------------------------------------------------------ LoRA merge
def lora_merge_fwd(W0, A, B, s, out=None):
    """W = W0 + s.B.A (W0 None: the delta s.B.A).  out may be W0 itself (merge in place) or a
    strided view."""
    r, K = A.shape
    N = B.shape[0]
    dt = A.dtype
    _need(A, "A", dt, (r, K))
    _need(B, "B", dt, (N, r))
    ldw = _mat(W0, "W0", dt, (N, K)) if W0 is not None else 0
    out, ldo = _out(out, "out", dt, (N, K), A.device)
    _check(lib().lora_merge_fwd(N, K, r, float(s), _dt(A), _ptr(W0), ldw, _ptr(A), _ptr(B), _ptr(out), ldo,
                                _stream()), "lora_merge_fwd")
    return out


def lora_merge_bwd(dW, A, B, s):
    """dA = s.B^T.dW, dB = s.dW.A^T for a gradient dW of the merged weight."""
    r, K = A.shape
    N = B.shape[0]
    dt = A.dtype
    lddw = _mat(dW, "dW", dt, (N, K))
    _need(A, "A", dt, (r, K))
    _need(B, "B", dt, (N, r))
    dA = torch.empty((r, K), dtype=torch.float32, device=A.device)
    dB = torch.empty((N, r), dtype=torch.float32, device=A.device)
    n = workspace_bytes("merge_bwd", 0, N, K, r, _dt(A))
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=A.device)
    _check(lib().lora_merge_bwd(N, K, r, float(s), _dt(A), _ptr(dW), lddw, _ptr(A), _ptr(B), _ptr(dA), _ptr(dB),
                                _ptr(ws), n, _stream()), "lora_merge_bwd")
    return {"dA": dA, "dB": dB}


# ------------------------------------------------------------------ DoRA
def dora_prepare(W0):
    N, K = W0.shape
    ldw = _mat(W0, "W0", W0.dtype, (N, K))
    out = torch.empty((N,), dtype=torch.float32, device=W0.device)
    _check(lib().dora_prepare(N, K, _dt(W0), _ptr(W0), ldw, _ptr(out), _stream()), "dora_prepare")
    return out


def dora_linear_fwd(X, W0, A, B, m, w0_sumsq, s, eps=1e-12, bias=None, Y=None):
    """Returns (Y, U, Z, state) where state = [norm | g | P | G] (fp32)."""
    M, K = X.shape
    N, r = B.shape
    dt = X.dtype
    ldx = _mat(X, "X", dt, (M, K))
    ldw = _mat(W0, "W0", dt, (N, K))
    _need(A, "A", dt, (r, K))
    _need(B, "B", dt, (N, r))
    _need(m, "m", torch.float32, (N,))
    _need(w0_sumsq, "w0_sumsq", torch.float32, (N,))
    if bias is not None:
        _need(bias, "bias", dt, (N,))
    dev = X.device
    Y, ldy = _out(Y, "Y", dt, (M, N), dev)
    Z = torch.empty((M, N), dtype=dt, device=dev)
    U = torch.empty((M, r), dtype=torch.float32, device=dev)
    state = torch.empty((dora_state_floats(N, r),), dtype=torch.float32, device=dev)
    ws, n = _ws("dora_fwd", M, N, K, r, _dt(X), dev)
    _check(lib().dora_linear_fwd(M, N, K, r, float(s), float(eps), _dt(X), _ptr(X), ldx, _ptr(W0), ldw, _ptr(A),
                                 _ptr(B), _ptr(m), _ptr(w0_sumsq), _ptr(bias), _ptr(Y), ldy, _ptr(U), r, _ptr(Z), N,
                                 _ptr(state), _ptr(ws), n, _stream()), "dora_linear_fwd")
    return Y, U, Z, state


def dora_linear_bwd(dY, X, W0, A, B, m, U, Z, state, s, eps=1e-12, need_dx=True, need_dbias=False, dX=None):
    """Returns dict(dX, dA, dB, dm, dbias)."""
    M, K = X.shape
    N, r = B.shape
    dt = X.dtype
    lddy = _mat(dY, "dY", dt, (M, N))
    ldx = _mat(X, "X", dt, (M, K))
    ldw = _mat(W0, "W0", dt, (N, K))
    _need(A, "A", dt, (r, K))
    _need(B, "B", dt, (N, r))
    ldz = _mat(Z, "Z", dt, (M, N))
    _need(m, "m", torch.float32, (N,))
    ldu = _mat(U, "U", torch.float32, (M, r))
    _need(state, "state", torch.float32, (dora_state_floats(N, r),))
    dev = X.device
    lddx = 0
    if need_dx:
        dX, lddx = _out(dX, "dX", dt, (M, K), dev)
    else:
        dX = None
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    dm = torch.empty((N,), dtype=torch.float32, device=dev)
    db = torch.empty((N,), dtype=torch.float32, device=dev) if need_dbias else None
    ws, n = _ws("dora_bwd", M, N, K, r, _dt(X), dev)
    _check(lib().dora_linear_bwd(M, N, K, r, float(s), float(eps), _dt(X), _ptr(dY), lddy, _ptr(X), ldx, _ptr(W0),
                                 ldw, _ptr(A), _ptr(B), _ptr(m), _ptr(U), ldu, _ptr(Z), ldz, _ptr(state), _ptr(dX),
                                 lddx, _ptr(dA), _ptr(dB), _ptr(dm), _ptr(db), _ptr(ws), n, _stream()),
           "dora_linear_bwd")
    return {"dX": dX, "dA": dA, "dB": dB, "dm": dm, "dbias": db}


# ------------------------------------------------------------------ DoRA, column form
def dora_cols_prepare(W0):
    """Column sums of W0^2 ([K] fp32), once per frozen W0."""
    N, K = W0.shape
    ldw = _mat(W0, "W0", W0.dtype, (N, K))
    out = torch.empty((K,), dtype=torch.float32, device=W0.device)
    _check(lib().dora_cols_prepare(N, K, _dt(W0), _ptr(W0), ldw, _ptr(out), _stream()), "dora_cols_prepare")
    return out


def dora_cols_linear_fwd(X, W0, A, B, m, w0_colsq, s, eps=1e-12, bias=None, Y=None):
    """Column-scaled DoRA forward.  Returns (Y, U, Xs, state) with Xs = X.diag(g) (bf16)
    and state = [norm | g | Pc | Gc] (fp32, dora_state_floats(K, r))."""
    M, K = X.shape
    N, r = B.shape
    dt = X.dtype
    ldx = _mat(X, "X", dt, (M, K))
    ldw = _mat(W0, "W0", dt, (N, K))
    _need(A, "A", dt, (r, K))
    _need(B, "B", dt, (N, r))
    _need(m, "m", torch.float32, (K,))
    _need(w0_colsq, "w0_colsq", torch.float32, (K,))
    if bias is not None:
        _need(bias, "bias", dt, (N,))
    dev = X.device
    Y, ldy = _out(Y, "Y", dt, (M, N), dev)
    Xs = torch.empty((M, K), dtype=dt, device=dev)
    U = torch.empty((M, r), dtype=torch.float32, device=dev)
    state = torch.empty((dora_state_floats(K, r),), dtype=torch.float32, device=dev)
    ws, n = _ws("dora_cols_fwd", M, N, K, r, _dt(X), dev)
    _check(lib().dora_cols_linear_fwd(M, N, K, r, float(s), float(eps), _dt(X), _ptr(X), ldx, _ptr(W0), ldw,
                                      _ptr(A), _ptr(B), _ptr(m), _ptr(w0_colsq), _ptr(bias), _ptr(Y), ldy, _ptr(U), r,
                                      _ptr(Xs), K, _ptr(state), _ptr(ws), n, _stream()), "dora_cols_linear_fwd")
    return Y, U, Xs, state


def dora_cols_linear_bwd(dY, X, Xs, W0, A, B, m, U, state, s, eps=1e-12, need_dx=True, need_dbias=False, dX=None):
    """Returns dict(dX, dA, dB, dm [K], dbias) of the column-scaled layer (U may be None)."""
    M, K = X.shape
    N, r = B.shape
    dt = X.dtype
    lddy = _mat(dY, "dY", dt, (M, N))
    ldx = _mat(X, "X", dt, (M, K))
    ldxs = _mat(Xs, "Xs", dt, (M, K))
    ldw = _mat(W0, "W0", dt, (N, K))
    _need(A, "A", dt, (r, K))
    _need(B, "B", dt, (N, r))
    _need(m, "m", torch.float32, (K,))
    ldu = _mat(U, "U", torch.float32, (M, r)) if U is not None else 0
    _need(state, "state", torch.float32, (dora_state_floats(K, r),))
    dev = X.device
    lddx = 0
    if need_dx:
        dX, lddx = _out(dX, "dX", dt, (M, K), dev)
    else:
        dX = None
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    dm = torch.empty((K,), dtype=torch.float32, device=dev)
    db = torch.empty((N,), dtype=torch.float32, device=dev) if need_dbias else None
    ws, n = _ws("dora_cols_bwd", M, N, K, r, _dt(X), dev)
    _check(lib().dora_cols_linear_bwd(M, N, K, r, float(s), float(eps), _dt(X), _ptr(dY), lddy, _ptr(X), ldx,
                                      _ptr(Xs), ldxs, _ptr(W0), ldw, _ptr(A), _ptr(B), _ptr(m), _ptr(U), ldu,
                                      _ptr(state), _ptr(dX), lddx, _ptr(dA), _ptr(dB), _ptr(dm), _ptr(db), _ptr(ws), n,
                                      _stream()), "dora_cols_linear_bwd")
    return {"dX": dX, "dA": dA, "dB": dB, "dm": dm, "dbias": db}


# ------------------------------------------------------------------ SwiGLU MLP
def swiglu_lora_mlp_fwd(X, gate, up, down, Out=None):
    """gate/up/down = (W, A, B, s).  Returns (Out, saved) with saved = dict(E, Gu, H, U)."""
    return _glu_fwd("swiglu_lora_mlp_fwd", (), X, gate, up, down, Out)


def geglu_lora_mlp_fwd(X, gate, up, down, approximate=False, Out=None):
    """The GeGLU MLP (gelu exact, or its tanh form when approximate); as swiglu_lora_mlp_fwd."""
    return _glu_fwd("geglu_lora_mlp_fwd", (int(bool(approximate)),), X, gate, up, down, Out)


def _glu_fwd(name, extra, X, gate, up, down, Out):
    M, K = X.shape
    (Wg, Ag, Bg, sg), (Wu, Au, Bu, su), (Wd, Ad, Bd, sd) = gate, up, down
    H, r = Bg.shape
    bf = torch.bfloat16
    ldx = _mat(X, "X", bf, (M, K))
    for t, n, sh in ((Wg, "Wg", (H, K)), (Ag, "Ag", (r, K)), (Bg, "Bg", (H, r)), (Wu, "Wu", (H, K)),
                     (Au, "Au", (r, K)), (Bu, "Bu", (H, r)), (Wd, "Wd", (K, H)), (Ad, "Ad", (r, H)),
                     (Bd, "Bd", (K, r))):
        _need(t, n, bf, sh)
    dev = X.device
    Out, ldo = _out(Out, "Out", bf, (M, K), dev)
    E = torch.empty((M, H), dtype=bf, device=dev)
    Gu = torch.empty((M, H), dtype=bf, device=dev)
    Hs = torch.empty((M, H), dtype=bf, device=dev)
    U = torch.empty((M, 3 * r), dtype=torch.float32, device=dev)
    ws, n = _ws("swiglu_fwd", M, H, K, r, LDL_BF16, dev)
    _check(getattr(lib(), name)(M, K, H, r, float(sg), float(su), float(sd), *extra, _ptr(X), ldx, _ptr(Wg),
                                _ptr(Ag), _ptr(Bg), _ptr(Wu), _ptr(Au), _ptr(Bu), _ptr(Wd), _ptr(Ad), _ptr(Bd),
                                _ptr(Out), ldo, _ptr(E), _ptr(Gu), _ptr(Hs), _ptr(U), _ptr(ws), n, _stream()), name)
    return Out, {"E": E, "Gu": Gu, "H": Hs, "U": U}


def swiglu_lora_mlp_bwd(dOut, X, gate, up, down, saved, need_dx=True, dX=None):
    return _glu_bwd("swiglu_lora_mlp_bwd", (), dOut, X, gate, up, down, saved, need_dx, dX)


def geglu_lora_mlp_bwd(dOut, X, gate, up, down, saved, approximate=False, need_dx=True, dX=None):
    return _glu_bwd("geglu_lora_mlp_bwd", (int(bool(approximate)),), dOut, X, gate, up, down, saved, need_dx, dX)


def _glu_bwd(name, extra, dOut, X, gate, up, down, saved, need_dx, dX):
    M, K = X.shape
    (Wg, Ag, Bg, sg), (Wu, Au, Bu, su), (Wd, Ad, Bd, sd) = gate, up, down
    H, r = Bg.shape
    bf = torch.bfloat16
    lddo = _mat(dOut, "dOut", bf, (M, K))
    ldx = _mat(X, "X", bf, (M, K))
    dev = X.device
    f32 = torch.float32
    lddx = 0
    if need_dx:
        dX, lddx = _out(dX, "dX", bf, (M, K), dev)
    else:
        dX = None
    out = {"dX": dX,
           "dA_gate": torch.empty((r, K), dtype=f32, device=dev), "dB_gate": torch.empty((H, r), dtype=f32, device=dev),
           "dA_up": torch.empty((r, K), dtype=f32, device=dev), "dB_up": torch.empty((H, r), dtype=f32, device=dev),
           "dA_down": torch.empty((r, H), dtype=f32, device=dev), "dB_down": torch.empty((K, r), dtype=f32, device=dev)}
    ws, n = _ws("swiglu_bwd", M, H, K, r, LDL_BF16, dev)
    _check(getattr(lib(), name)(M, K, H, r, float(sg), float(su), float(sd), *extra, _ptr(dOut), lddo, _ptr(X), ldx,
                                _ptr(Wg), _ptr(Ag), _ptr(Bg), _ptr(Wu), _ptr(Au), _ptr(Bu), _ptr(Wd), _ptr(Ad),
                                _ptr(Bd), _ptr(saved["E"]), _ptr(saved["Gu"]), _ptr(saved["H"]), _ptr(saved["U"]),
                                _ptr(dX), lddx, _ptr(out["dA_gate"]), _ptr(out["dB_gate"]), _ptr(out["dA_up"]),
                                _ptr(out["dB_up"]), _ptr(out["dA_down"]), _ptr(out["dB_down"]), _ptr(ws), n,
                                _stream()), name)
    return out


# ------------------------------------------------------------------ W8A8
def _quantize_weight8(W0, fn, code_dtype):
    N, K = W0.shape
    ldw = _mat(W0, "W0", W0.dtype, (N, K))
    Wq = torch.empty((N, K), dtype=code_dtype, device=W0.device)
    sw = torch.empty((N,), dtype=torch.float32, device=W0.device)
    _check(getattr(lib(), fn)(N, K, _dt(W0), _ptr(W0), ldw, _ptr(Wq), _ptr(sw), _stream()), fn)
    return Wq, sw


def _quantize_rows8(X, fn, code_dtype):
    M, K = X.shape
    ldx = _mat(X, "X", torch.bfloat16, (M, K))
    Xq = torch.empty((M, K), dtype=code_dtype, device=X.device)
    sx = torch.empty((M,), dtype=torch.float32, device=X.device)
    _check(getattr(lib(), fn)(M, K, _ptr(X), ldx, _ptr(Xq), _ptr(sx), _stream()), fn)
    return Xq, sx


def w8a8_quantize_weight(W0):
    """Per-output-channel int8 codes (int8 [N,K]) and scales (fp32 [N])."""
    return _quantize_weight8(W0, "w8a8_quantize_weight", torch.int8)


def w8a8_quantize_rows(X):
    return _quantize_rows8(X, "w8a8_quantize_rows", torch.int8)


def fp8_quantize_weight(W0):
    """Per-output-channel e4m3 codes (as uint8 [N,K]: the byte of each code) and scales."""
    return _quantize_weight8(W0, "fp8_quantize_weight", torch.uint8)


def fp8_quantize_rows(X):
    return _quantize_rows8(X, "fp8_quantize_rows", torch.uint8)


def int8_gemm_raw(Xq, Wq):
    M, K = Xq.shape
    N = Wq.shape[0]
    ldxq = _mat(Xq, "Xq", torch.int8, (M, K))
    ldwq = _mat(Wq, "Wq", torch.int8, (N, K))
    C = torch.empty((M, N), dtype=torch.int32, device=Xq.device)
    _check(lib().int8_gemm_raw(M, N, K, _ptr(Xq), ldxq, _ptr(Wq), ldwq, _ptr(C), N, _stream()), "int8_gemm_raw")
    return C


def _lora8_fwd(fn, code_dtype, X, Wq, sw, A, B, s, bias, save, Y):
    M, K = X.shape
    N, r = B.shape
    bf = torch.bfloat16
    ldx = _mat(X, "X", bf, (M, K))
    ldw = _mat(Wq, "Wq", code_dtype, (N, K))
    _need(sw, "sw", torch.float32, (N,))
    _need(A, "A", bf, (r, K))
    _need(B, "B", bf, (N, r))
    if bias is not None:
        _need(bias, "bias", bf, (N,))
    dev = X.device
    Y, ldy = _out(Y, "Y", bf, (M, N), dev)
    Xq = torch.empty((M, K), dtype=code_dtype, device=dev) if save else None
    sx = torch.empty((M,), dtype=torch.float32, device=dev) if save else None
    U = torch.empty((M, r), dtype=torch.float32, device=dev) if save else None
    ws, n = _ws("w8a8_fwd", M, N, K, r, LDL_BF16, dev)
    _check(getattr(lib(), fn)(M, N, K, r, float(s), _ptr(X), ldx, _ptr(Wq), ldw, _ptr(sw), _ptr(A), _ptr(B),
                              _ptr(bias), _ptr(Y), ldy, _ptr(Xq), _ptr(sx), _ptr(U), r, _ptr(ws), n, _stream()), fn)
    return Y, Xq, sx, U


def _lora8_bwd(fn, code_dtype, dY, X, Wq, sw, A, B, s, U, need_dx, dX):
    M, K = X.shape
    N, r = B.shape
    bf = torch.bfloat16
    lddy = _mat(dY, "dY", bf, (M, N))
    ldx = _mat(X, "X", bf, (M, K))
    ldw = _mat(Wq, "Wq", code_dtype, (N, K))
    ldu = _mat(U, "U", torch.float32, (M, r)) if U is not None else 0
    dev = X.device
    lddx = 0
    if need_dx:
        dX, lddx = _out(dX, "dX", bf, (M, K), dev)
    else:
        dX = None
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    ws, n = _ws("w8a8_bwd", M, N, K, r, LDL_BF16, dev)
    _check(getattr(lib(), fn)(M, N, K, r, float(s), _ptr(dY), lddy, _ptr(X), ldx, _ptr(Wq), ldw, _ptr(sw), _ptr(A),
                              _ptr(B), _ptr(U), ldu, _ptr(dX), lddx, _ptr(dA), _ptr(dB), _ptr(ws), n, _stream()), fn)
    return {"dX": dX, "dA": dA, "dB": dB}


def w8a8_lora_linear_fwd(X, Wq, sw, A, B, s, bias=None, save=True, Y=None):
    """int8 base + LoRA.  Returns (Y, Xq, sx, U)."""
    return _lora8_fwd("w8a8_lora_linear_fwd", torch.int8, X, Wq, sw, A, B, s, bias, save, Y)


def w8a8_lora_linear_bwd(dY, X, Wq, sw, A, B, s, U=None, need_dx=True, dX=None):
    return _lora8_bwd("w8a8_lora_linear_bwd", torch.int8, dY, X, Wq, sw, A, B, s, U, need_dx, dX)


def fp8_lora_linear_fwd(X, Wq, sw, A, B, s, bias=None, save=True, Y=None):
    """e4m3 base + LoRA (Wq: uint8 bytes of the e4m3 codes).  Returns (Y, Xq, sx, U)."""
    return _lora8_fwd("fp8_lora_linear_fwd", torch.uint8, X, Wq, sw, A, B, s, bias, save, Y)


def fp8_lora_linear_bwd(dY, X, Wq, sw, A, B, s, U=None, need_dx=True, dX=None):
    return _lora8_bwd("fp8_lora_linear_bwd", torch.uint8, dY, X, Wq, sw, A, B, s, U, need_dx, dX)
