"""LoRA MLP with the SwiGLU activation, materialised definition in float64 (oracle; test use only).

Source passages ("How Unsloth's FastLoRA Kernel Differs from Standard LoRA
Implementations"):
  * section "Fused Forward Pass Architecture": the LoRA MLP applies a LoRA
    matmul to the gate and the up projection, then h = silu(e) * g, then the
    down projection (also LoRA).
  * section "Activation Function Fusion": the activation is fused with the
    LoRA projections; the arithmetic is unchanged by that fusion.
  * section "Custom Backward Pass Implementation": hand-written backward
    for the MLP, factor gradients pre-scaled by each adapter's scale.

Readings: silu(e) = e.sigmoid(e); no bias; no dropout; each projection has its
own (A, B, s).  Every projection uses the LoRA convention of oracle.lora.

Forward:  E = X.Wg'^T,  Gu = X.Wu'^T,  H = silu(E) * Gu,  O = H.Wd'^T.
Backward (chain rule, materialised):
  dH = dO.Wd',  Gd = dO^T.H
  dE = dH * Gu * silu'(E),  silu'(e) = sig(e).(1 + e.(1 - sig(e)))
  dGu = dH * silu(E)
  dX = dE.Wg' + dGu.Wu',  Gg = dE^T.X,  Gu_w = dGu^T.X
  dA_p = s_p.B_p^T.G_p,  dB_p = s_p.G_p.A_p^T   for p in gate, up, down.

Pins (tests/test_oracle_swiglu.py): silu(0) = 0 and silu'(0) = 1/2, silu'
against a central difference of silu, all B = 0 reduces to the plain MLP
written with scipy.special.expit, hand-worked example
(tests/golden/swiglu_tiny.json), finite differences of every gradient.
"""

import numpy as np

from .lora import adapted_weight


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sigmoid(e):
    """Logistic function, evaluated without overflow for large |e|."""
    e = _f64(e)
    out = np.empty_like(e)
    pos = e >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-e[pos]))
    ex = np.exp(e[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def silu(e):
    e = _f64(e)
    return e * sigmoid(e)


def silu_grad(e):
    """d silu / d e = sig(e).(1 + e.(1 - sig(e)))."""
    e = _f64(e)
    sg = sigmoid(e)
    return sg * (1.0 + e * (1.0 - sg))


def swiglu_mlp_forward(X, gate, up, down):
    """gate/up/down are tuples (W, A, B, s) in the LoRA convention.

    Returns dict(O, E, Gu, H).
    """
    X = _f64(X)
    Wg = adapted_weight(*gate)
    Wu = adapted_weight(*up)
    Wd = adapted_weight(*down)
    E = X @ Wg.T
    Gu = X @ Wu.T
    H = silu(E) * Gu
    O = H @ Wd.T
    return {"O": O, "E": E, "Gu": Gu, "H": H}


def swiglu_mlp_backward(dO, X, gate, up, down):
    """Gradients of <dO, O>.  Returns dict(dX, dA_gate, dB_gate, dA_up, dB_up, dA_down, dB_down)."""
    dO, X = _f64(dO), _f64(X)
    Wg = adapted_weight(*gate)
    Wu = adapted_weight(*up)
    Wd = adapted_weight(*down)
    E = X @ Wg.T
    Gu = X @ Wu.T
    H = silu(E) * Gu
    dH = dO @ Wd
    Gd = dO.T @ H
    dE = dH * Gu * silu_grad(E)
    dGu = dH * silu(E)
    Gg = dE.T @ X
    Gup = dGu.T @ X
    out = {"dX": dE @ Wg + dGu @ Wu}
    for name, (W, A, B, s), G in (("gate", gate, Gg), ("up", up, Gup), ("down", down, Gd)):
        A, B = _f64(A), _f64(B)
        out["dA_" + name] = float(s) * (B.T @ G)
        out["dB_" + name] = float(s) * (G @ A.T)
    return out


def swiglu_mlp_dx_rows(dO_rows, X_rows, gate, up, down):
    """dX for a subset of rows only: each row of dX depends on its own row of X and dO."""
    return swiglu_mlp_backward(dO_rows, X_rows, gate, up, down)["dX"]


def swiglu_mlp_grads_sampled(dO, X, gate, up, down, h_idx, k_idx):
    """The factor-gradient definitions of swiglu_mlp_backward restricted to chosen entries.

    The activations E, Gu, H and the hidden-side gradient dH = dO.Wd' are built in full
    (every entry below is a reduction over all tokens); the weight-shaped gradients
    G_p are formed only for the requested rows / columns:
      G_gate = dE^T.X, G_up = dGu^T.X ([H,K]):  rows h_idx -> dB_gate[h_idx], dB_up[h_idx];
                                                columns k_idx -> dA_gate[:, k_idx], dA_up[:, k_idx]
      G_down = dO^T.H ([K,H]):                  rows k_idx -> dB_down[k_idx];
                                                columns h_idx -> dA_down[:, h_idx]
    with dA_p = s_p.B_p^T.G_p and dB_p = s_p.G_p.A_p^T.  Used at sizes where the full
    [H,K] products would take too long on the host.
    """
    dO, X = _f64(dO), _f64(X)
    h_idx, k_idx = np.asarray(h_idx), np.asarray(k_idx)
    Wg = adapted_weight(*gate)
    Wu = adapted_weight(*up)
    Wd = adapted_weight(*down)
    E = X @ Wg.T
    Gu = X @ Wu.T
    H = silu(E) * Gu
    dH = dO @ Wd
    dE = dH * Gu * silu_grad(E)
    dGu = dH * silu(E)
    out = {}
    for name, (W, A, B, s), dZ in (("gate", gate, dE), ("up", up, dGu)):
        A, B = _f64(A), _f64(B)
        G_rows = dZ[:, h_idx].T @ X           # [len(h_idx), K]
        G_cols = dZ.T @ X[:, k_idx]           # [H, len(k_idx)]
        out["dB_" + name + "_rows"] = float(s) * (G_rows @ A.T)
        out["dA_" + name + "_cols"] = float(s) * (B.T @ G_cols)
    W, A, B, s = down
    A, B = _f64(A), _f64(B)
    Gd_rows = dO[:, k_idx].T @ H              # [len(k_idx), H]
    Gd_cols = dO.T @ H[:, h_idx]              # [K, len(h_idx)]
    out["dB_down_rows"] = float(s) * (Gd_rows @ A.T)
    out["dA_down_cols"] = float(s) * (B.T @ Gd_cols)
    return out
