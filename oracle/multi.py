"""Several LoRA adapters over one concatenated base weight (fused QKV), plain definition in
float64 (oracle; test use only).

Source passages:
  * "How Unsloth's FastLoRA Kernel Differs from Standard LoRA Implementations", section
    "Fused Forward Pass Architecture": a dedicated autograd Function serves the attention
    query / key / value projections.
  * "nunchaku-style kernel fusion - 20-30% faster training" (OneTrainer PR), the commit
    that adds the LoRA epilogue: fused-qkv adapters take the same fused path, each leaf
    using only its own rows of lora_up.

Reading: the base weight is the row concatenation W0 = [W0_1; ..; W0_L] ([N,K], N the sum
of the leaf widths N_l); leaf l has its own adapter A_l [r,K], B_l [N_l,r] and scale s_l.
The adapted weight keeps the row blocks, W'_l = W0_l + s_l.B_l.A_l, and the layer is
Y = X.W'^T (+ b): the columns of leaf l see only that leaf's adapter.  Factors are passed
concatenated, A_cat = [A_1; ..; A_L] ([L r, K]) and B_cat = [B_1; ..; B_L] ([N, r]).

Backward with W0 frozen: G = dY^T.X is the gradient of W'; per leaf the chain rule gives
dA_l = s_l.B_l^T.G_l and dB_l = s_l.G_l.A_l^T with G_l the leaf's rows of G; dX = dY.W';
db = column sums of dY.

Pins (tests/test_oracle_multi.py): one leaf reduces to oracle.lora; each leaf's column
block equals oracle.lora on that leaf alone; the whole layer equals a single LoRA of rank
L r whose up factor is block diagonal; a leaf with s_l = 0 gives X.W0_l^T; brute-force
loops on a tiny case; central finite differences of every gradient.
"""

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _bounds(n_leaf):
    ends = np.cumsum(np.asarray(n_leaf, dtype=np.int64))
    return [(int(e - n), int(e)) for n, e in zip(n_leaf, ends)]


def adapted_weight(W0, A_cat, B_cat, n_leaf, s_leaf):
    """W' [N,K] with row block l equal to W0_l + s_l.B_l.A_l (built explicitly)."""
    W0, A_cat, B_cat = _f64(W0), _f64(A_cat), _f64(B_cat)
    r = A_cat.shape[0] // len(n_leaf)
    Wp = W0.copy()
    for l, (a, b) in enumerate(_bounds(n_leaf)):
        Wp[a:b] += float(s_leaf[l]) * (B_cat[a:b] @ A_cat[l * r:(l + 1) * r])
    return Wp


def multi_forward(X, W0, A_cat, B_cat, n_leaf, s_leaf, bias=None):
    """Y = X.W'^T (+ b), [M,N] float64."""
    Y = _f64(X) @ adapted_weight(W0, A_cat, B_cat, n_leaf, s_leaf).T
    if bias is not None:
        Y = Y + _f64(bias)[None, :]
    return Y


def multi_backward(dY, X, W0, A_cat, B_cat, n_leaf, s_leaf):
    """Gradients of <dY, Y>: dict with dX [M,K], dA [L r, K], dB [N, r], db [N]."""
    dY, X, A_cat, B_cat = _f64(dY), _f64(X), _f64(A_cat), _f64(B_cat)
    r = A_cat.shape[0] // len(n_leaf)
    Wp = adapted_weight(W0, A_cat, B_cat, n_leaf, s_leaf)
    G = dY.T @ X
    dA = np.zeros_like(A_cat)
    dB = np.zeros_like(B_cat)
    for l, (a, b) in enumerate(_bounds(n_leaf)):
        s = float(s_leaf[l])
        dA[l * r:(l + 1) * r] = s * (B_cat[a:b].T @ G[a:b])
        dB[a:b] = s * (G[a:b] @ A_cat[l * r:(l + 1) * r].T)
    return {"dX": dY @ Wp, "dA": dA, "dB": dB, "db": dY.sum(axis=0)}


def multi_weight_grads_sampled(dY, X, A_cat, B_cat, n_leaf, s_leaf, n_rows, k_cols):
    """dB at chosen rows and dA at chosen columns, from the same definitions with G built
    only where needed (for shapes too large for the full [N,K] product on the host)."""
    dY, X, A_cat, B_cat = _f64(dY), _f64(X), _f64(A_cat), _f64(B_cat)
    r = A_cat.shape[0] // len(n_leaf)
    bounds = _bounds(n_leaf)
    leaf_of = np.concatenate([np.full(b - a, l) for l, (a, b) in enumerate(bounds)])
    n_rows, k_cols = np.asarray(n_rows), np.asarray(k_cols)
    G_rows = dY[:, n_rows].T @ X
    dB_rows = np.stack([float(s_leaf[leaf_of[n]]) * (G_rows[i] @ A_cat[leaf_of[n] * r:(leaf_of[n] + 1) * r].T)
                        for i, n in enumerate(n_rows)])
    G_cols = dY.T @ X[:, k_cols]
    dA_cols = np.concatenate([float(s_leaf[l]) * (B_cat[a:b].T @ G_cols[a:b]) for l, (a, b) in enumerate(bounds)])
    return {"dB_rows": dB_rows, "dA_cols": dA_cols}
