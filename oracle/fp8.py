"""8-bit float (e4m3) base with a LoRA epilogue, plain definition (oracle; test use only).

Source passages ("nunchaku-style kernel fusion - 20-30% faster training", OneTrainer PR
#1680):
  * LoRA-epilogue commit: the 8-bit matmul core serves both 8-bit dtypes (the per-axis
    quantiser dispatches on them) with the per-row dequant scale plus the rank-tiled
    low-rank update as its epilogue; the low-rank branch sees the layer's unquantised input.
  * MXFP8 commit: the block-scaled 8-bit float instruction with every block scale equal to
    1.0 computes the same product as the plain 8-bit float product, at the full 8-bit rate.

Readings where the pages are silent (also listed in the design notes):
  * the 8-bit float format is e4m3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormals, no infinities, largest finite value 448);
  * symmetric per-row quantisation: scale = absmax / 448 in float32, code = e4m3 rounding
    (nearest, ties to even) of the float32 quotient x / scale, clamped to +-448; an all-zero
    row gets scale 0 and codes 0;
  * the base product is the exact product of the decoded codes (float64 here, where it is
    exact), dequantised as acc . sx[m] . sw[n];
  * backward as for the int8 base: the quantisation of X is passed straight through and the
    base weight in the backward is the dequantised diag(sw).Wq.

Pins (tests/test_oracle_fp8.py): the rounding against torch's float8_e4m3fn conversion
(values in range and every midpoint), the format's fixed points (1.0, 448, the smallest
normal and subnormal), the half-ulp bound of the quantiser, zero rows, a hand-worked forward
(tests/golden/fp8_forward.json), finite differences of dA, dB and of the straight-through dX.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_round(x):
    """Nearest e4m3 value (ties to even) of each element, as float64; |x| <= 448 expected
    (larger magnitudes are clamped to 448)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # binade exponent e with 2^e <= a < 2^(e+1); values below the smallest normal 2^-6 use
    # the subnormal spacing 2^-9
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex - 1, -6)
    quantum = np.ldexp(1.0, e - 3)
    v = np.rint(a / quantum) * quantum          # a / quantum is exact; rint rounds half to even
    v = np.minimum(v, E4M3_MAX)
    return np.where(x < 0, -v, v)


def e4m3_decode(codes):
    """Value of e4m3 byte codes (float64); 0x7f / 0xff (NaN) are not produced here."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    v = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    return sign * v


def e4m3_encode(values):
    """Byte codes of values that are exactly e4m3 (as returned by e4m3_round); zero -> 0x00."""
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    normal = a >= 2.0 ** -6
    e = np.where(normal, ex - 1 + 7, 0)
    m = np.where(normal, np.rint((a / np.ldexp(1.0, ex - 1) - 1.0) * 8), np.rint(a / 2.0 ** -9))
    code = (e.astype(np.int64) << 3) | m.astype(np.int64)
    code = np.where(a > 0, code | np.where(v < 0, 0x80, 0), 0)
    return code.astype(np.uint8)


def quantize_rows_fp8(X):
    """Per-row symmetric e4m3 codes.  Returns (codes uint8 [R,C], scale float32 [R]).

    scale_r = float32(absmax_r) / 448 in float32; code = e4m3(clamp(float32(x) / scale_r))
    with the quotient in float32; scale 0 gives code 0.
    """
    Xf = np.asarray(X, dtype=np.float32)
    absmax = np.max(np.abs(Xf), axis=1) if Xf.shape[1] else np.zeros(Xf.shape[0], np.float32)
    scale = (absmax.astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    quot = (Xf / safe[:, None]).astype(np.float32)
    q = e4m3_round(np.clip(quot.astype(np.float64), -E4M3_MAX, E4M3_MAX))
    q = np.where(scale[:, None] > 0, q, 0.0)
    return e4m3_encode(q), scale


def fp8_product(Xq, Wq):
    """Exact product of the decoded codes, Xq . Wq^T (float64 holds it exactly here)."""
    return e4m3_decode(Xq) @ e4m3_decode(Wq).T


def fp8_forward(X, Wq, sw, A, B, s, bias=None):
    """Y = (Xq.Wq^T) . sx[m] . sw[n] + s.X.(B.A)^T (+ b); Xq, sx from quantize_rows_fp8(X).

    Returns dict(Y, Xq, sx, acc)."""
    X = np.asarray(X, dtype=np.float64)
    Xq, sx = quantize_rows_fp8(X)
    acc = fp8_product(Xq, Wq)
    delta = np.asarray(B, np.float64) @ np.asarray(A, np.float64)
    Y = acc * sx.astype(np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    Y = Y + float(s) * (X @ delta.T)
    if bias is not None:
        Y = Y + np.asarray(bias, np.float64)[None, :]
    return {"Y": Y, "Xq": Xq, "sx": sx, "acc": acc}


def dequantized_weight(Wq, sw):
    return e4m3_decode(Wq) * np.asarray(sw, np.float64)[:, None]


def fp8_backward(dY, X, Wq, sw, A, B, s):
    """Straight-through backward.  Returns dict(dX, dA, dB)."""
    dY, X = np.asarray(dY, np.float64), np.asarray(X, np.float64)
    A, B = np.asarray(A, np.float64), np.asarray(B, np.float64)
    G = dY.T @ X
    return {
        "dX": dY @ (dequantized_weight(Wq, sw) + float(s) * (B @ A)),
        "dA": float(s) * (B.T @ G),
        "dB": float(s) * (G @ A.T),
    }
