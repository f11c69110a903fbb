"""int8 base (W8A8) with a LoRA epilogue, plain definition (oracle; test use only).

Source passages ("nunchaku-style kernel fusion - 20-30% faster training",
OneTrainer PR #1680):
  * LoRA-epilogue commit: a shared 8-bit matmul core whose epilogues are the
    raw product, a per-row dequant scale, or that scale plus a rank-tiled
    low-rank update; the autograd Function owns the down-projection, so the
    low-rank branch is fed the layer's (unquantised) input; the LoRA dgrad is
    folded into the backward epilogue; quantize_axiswise quantises per axis.
  * the comment on activations: the int32 product is never materialised, the
    kernel goes straight to bf16.
  * unification commit: one mm_8bit(a, b, out_dtype, scale_m, scale_n,
    lora_xd, lora_up) with optional epilogue operands.

Readings where the pages are silent (also listed in the design notes):
  * symmetric per-row quantisation with divisor 127 and codes clamped to
    [-127, 127]; scale = absmax / 127; an all-zero row gets scale 0 and codes 0;
  * the code is round-half-to-even of x / scale, with the scale and the quotient
    computed in float32 (the precision in which both implementations take this
    integer decision);
  * the base product is exact integer arithmetic (int64 here), dequantised as
    acc . sx[m] . sw[n];
  * the LoRA branch sees the bf16 input X, not its quantised copy;
  * backward: the quantisation of X is passed straight through, and the base
    weight in the backward is the dequantised weight diag(sw).Wq, so
    dX = dY.(diag(sw).Wq + s.B.A); dA = s.B^T.(dY^T.X); dB = s.(dY^T.X).A^T.

Pins (tests/test_oracle_w8a8.py): hand-worked quantiser codes
(tests/golden/w8a8_quant.json), brute-force Python-int product, round-trip
bound |x - sx.q| <= sx/2, zero rows, finite differences of dA, dB and of the
straight-through dX.
"""

import numpy as np


def quantize_rows_int8(X):
    """Per-row symmetric int8 codes.  Returns (q int8 [R,C], scale float32 [R]).

    scale_r = float32(absmax_r) / 127 in float32; q = clamp(rint(float32(x) / scale_r), -127, 127)
    with the quotient in float32 and rint = round half to even; scale 0 gives q = 0.
    """
    Xf = np.asarray(X, dtype=np.float32)
    absmax = np.max(np.abs(Xf), axis=1) if Xf.shape[1] else np.zeros(Xf.shape[0], np.float32)
    scale = (absmax.astype(np.float32) / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    quot = (Xf / safe[:, None]).astype(np.float32)
    q = np.clip(np.rint(quot), -127, 127)
    q = np.where(scale[:, None] > 0, q, 0).astype(np.int8)
    return q, scale


def int_product(Xq, Wq):
    """Exact integer product Xq . Wq^T in int64 (no rounding possible at these sizes)."""
    return np.asarray(Xq, dtype=np.int64) @ np.asarray(Wq, dtype=np.int64).T


def w8a8_forward(X, Wq, sw, A, B, s, bias=None):
    """Y = (Xq.Wq^T) . sx[m] . sw[n] + s.X.(B.A)^T (+ b); Xq, sx from quantize_rows_int8(X).

    Returns dict(Y, Xq, sx, acc).
    """
    X = np.asarray(X, dtype=np.float64)
    Xq, sx = quantize_rows_int8(X)
    acc = int_product(Xq, Wq)
    delta = np.asarray(B, np.float64) @ np.asarray(A, np.float64)
    Y = acc.astype(np.float64) * sx.astype(np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    Y = Y + float(s) * (X @ delta.T)
    if bias is not None:
        Y = Y + np.asarray(bias, np.float64)[None, :]
    return {"Y": Y, "Xq": Xq, "sx": sx, "acc": acc}


def dequantized_weight(Wq, sw):
    return np.asarray(Wq, np.float64) * np.asarray(sw, np.float64)[:, None]


def w8a8_backward(dY, X, Wq, sw, A, B, s):
    """Straight-through backward.  Returns dict(dX, dA, dB)."""
    dY = np.asarray(dY, np.float64)
    X = np.asarray(X, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    Wdq = dequantized_weight(Wq, sw)
    G = dY.T @ X
    return {
        "dX": dY @ (Wdq + float(s) * (B @ A)),
        "dA": float(s) * (B.T @ G),
        "dB": float(s) * (G @ A.T),
    }
