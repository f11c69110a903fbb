"""LoRA bypass layer, materialised definition in float64 (oracle; test use only).

Source passages:
  * "How Unsloth's FastLoRA Kernel Differs from Standard LoRA Implementations",
    section "Fused Forward Pass Architecture": the layer output is the input
    times the adapted weight W + dW with dW the product of the two low-rank
    factors; the fused form must give the same result.
  * Same page, section "Custom Backward Pass Implementation": the gradients of
    the two factors are pre-scaled by the LoRA scaling factor.
  * "nunchaku-style kernel fusion - 20-30% faster training" (OneTrainer PR),
    the LoRA-epilogue and autotune-key commit messages: lora_down is [r,K]
    (row-major) and lora_up is [N,r]; the update is lora_xd . up^T.

Orientation (the reading used throughout): W0 [N,K], A [r,K], B [N,r],
dW = B.A [N,K], W' = W0 + s.dW, Y = X.W'^T + b.

Pins (tests/test_oracle_lora.py): hand-worked integer example
(tests/golden/lora_tiny.json), brute-force triple loop, s = 0 / B = 0 reduce to
X.W0^T, W0 = 0 reduces to s.(X.A^T).B^T, central finite differences of every
gradient, the gauge identity <dA,A> = <dB,B>, the Euler identity
<dX,X> = <dY,Y-b>.
"""

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def adapted_weight(W0, A, B, s):
    """W' = W0 + s.(B.A), built explicitly ([N,K]); the thing the fused path never forms."""
    W0, A, B = _f64(W0), _f64(A), _f64(B)
    delta = B @ A
    return W0 + float(s) * delta


def lora_forward(X, W0, A, B, s, bias=None):
    """Y = X.W'^T (+ b).  Returns Y [M,N] float64."""
    X = _f64(X)
    Wp = adapted_weight(W0, A, B, s)
    Y = X @ Wp.T
    if bias is not None:
        Y = Y + _f64(bias)[None, :]
    return Y


def lora_backward(dY, X, W0, A, B, s):
    """Gradients of <dY, Y> for Y = X.W'^T + b with W0 frozen.

    G = dY^T.X is the (materialised) gradient of W'; the chain rule through
    W' = W0 + s.B.A gives dA = s.B^T.G and dB = s.G.A^T; dX = dY.W';
    db = column sums of dY.  Returns a dict with dX, dA, dB, db.
    """
    dY, X = _f64(dY), _f64(X)
    A, B = _f64(A), _f64(B)
    Wp = adapted_weight(W0, A, B, s)
    G = dY.T @ X
    return {
        "dX": dY @ Wp,
        "dA": float(s) * (B.T @ G),
        "dB": float(s) * (G @ A.T),
        "db": dY.sum(axis=0),
    }


def lora_weight_grads_sampled(dY, X, A, B, s, n_rows, k_cols):
    """The same dA / dB definitions restricted to chosen entries.

    dB[n_rows, :] = s.(dY[:, n_rows]^T.X).A^T and dA[:, k_cols] = s.B^T.(dY^T.X[:, k_cols]),
    i.e. G is built only for the requested rows / columns.  Used to check very
    large shapes where the full [N,K] product would take too long on the host.
    """
    dY, X, A, B = _f64(dY), _f64(X), _f64(A), _f64(B)
    n_rows = np.asarray(n_rows)
    k_cols = np.asarray(k_cols)
    G_rows = dY[:, n_rows].T @ X            # [len(n_rows), K]
    G_cols = dY.T @ X[:, k_cols]            # [N, len(k_cols)]
    return {
        "dB_rows": float(s) * (G_rows @ A.T),
        "dA_cols": float(s) * (B.T @ G_cols),
    }
