"""DoRA, row-scaled form ("dora-rows"), materialised definition in float64 (oracle; test use only).

Source passages ("LoRA/DoRA fast forward: no weight materialization", Stable
Audio 3 PR):
  * section "What": dora-rows is a row scale of the base-plus-low-rank output;
    the naive parametrisation rebuilds the adapted weight and takes an
    [out,in] norm on every step.
  * section "Fidelity": the norm stays in the autograd graph (no detach as in
    the DoRA paper), eps is 1e-12, strength multiplies inside the delta, and
    the bias is added without the row scale.
  * the commit message: the fast path must compute the same y as the
    materialised weight.

Readings where the pages leave a step open (also listed in the design notes):
  * the norm is taken per output row n over the input axis K (row scale);
  * eps placement: g_n = m_n / max(nu_n, eps), and no gradient flows through
    nu_n where the clamp is active (nu_n <= eps);
  * bias optional, added after the row scale.

Definition:  W' = W0 + s.B.A;  nu_n = ||W'_n||_2  (explicit, from W');
             g_n = m_n / max(nu_n, eps);  Z = X.W'^T;  Y = Z.diag(g) + b.

Column-scaled form ("dora-cols", same page, section "What": the other of the two DoRA
forms the fast path reproduces).  Reading: the norm is taken per input column k over the
output axis N, with a magnitude m [K]; the scale then multiplies the layer input,
  nu_k = ||W'[:,k]||_2;  g_k = m_k / max(nu_k, eps);  W'' = W'.diag(g);
  Y = X.W''^T + b = (X.diag(g)).W'^T + b,
with the same eps clamp, in-graph norm and un-scaled bias as dora-rows.

Pins (tests/test_oracle_dora.py): hand-worked example (tests/golden/dora_tiny.json),
closed-form norm equals the explicit norm, direction invariance under
(W0, B) -> (c.W0, c.B), B = 0 with m = ||W0_n|| reduces to X.W0^T + b,
central finite differences of dX, dA, dB, dm (through the norm), the
identities <m,dm> = <dY,Y-b>, <dA,A> = <dB,B>, <dX,X> = <dY,Y-b>, and the
eps-clamped zero-row case.  dora-cols (tests/test_oracle_dora_cols.py): hand-worked
example (tests/golden/dora_cols_tiny.json), brute-force column norm, the column norm of W'
equal to the row norm of W'^T (oracle.dora's row form on the transposed layer), m = nu
reducing to the LoRA layer, s = 0 with m = ||W0[:,k]|| reducing to X.W0^T + b, central
finite differences of dX, dA, dB, dm, db, and the eps-clamped zero-column case.
"""

import numpy as np

from .lora import adapted_weight


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def row_norm_explicit(W0, A, B, s):
    """nu_n = sqrt(sum_k W'[n,k]^2) from the materialised W' (the naive [out,in] norm)."""
    Wp = adapted_weight(W0, A, B, s)
    return np.sqrt(np.sum(Wp * Wp, axis=1))


def w0_row_sumsq(W0):
    """sum_k W0[n,k]^2: the constant the fast path caches for a frozen W0."""
    W0 = _f64(W0)
    return np.sum(W0 * W0, axis=1)


def dora_forward(X, W0, A, B, m, s, eps=1e-12, bias=None):
    """Returns dict(Y, Z, nu, g).  Z = X.W'^T is the unscaled product."""
    X, m = _f64(X), _f64(m)
    Wp = adapted_weight(W0, A, B, s)
    nu = np.sqrt(np.sum(Wp * Wp, axis=1))
    g = m / np.maximum(nu, eps)
    Z = X @ Wp.T
    Y = Z * g[None, :]
    if bias is not None:
        Y = Y + _f64(bias)[None, :]
    return {"Y": Y, "Z": Z, "nu": nu, "g": g}


def dora_backward(dY, X, W0, A, B, m, s, eps=1e-12):
    """Chain rule through the materialised W' and the explicit norm.

    With dZ = dY.diag(g):
      dg_n   = sum_m dY[m,n] Z[m,n]
      dm_n   = dg_n / max(nu_n, eps)
      dnu_n  = -dg_n m_n / nu_n^2      (0 where nu_n <= eps)
      dW'    = dZ^T.X + diag(dnu/nu).W'          (norm kept in the graph)
      dA = s.B^T.dW',  dB = s.dW'.A^T,  dX = dZ.W',  db = column sums of dY.
    Returns dict(dX, dA, dB, dm, db).
    """
    dY, X, A, B, m = _f64(dY), _f64(X), _f64(A), _f64(B), _f64(m)
    Wp = adapted_weight(W0, A, B, s)
    nu = np.sqrt(np.sum(Wp * Wp, axis=1))
    den = np.maximum(nu, eps)
    g = m / den
    Z = X @ Wp.T
    dg = np.sum(dY * Z, axis=0)
    dm = dg / den
    active = nu > eps
    dnu = np.where(active, -dg * m / np.where(active, nu * nu, 1.0), 0.0)
    dZ = dY * g[None, :]
    coef = np.where(active, dnu / np.where(active, nu, 1.0), 0.0)
    dWp = dZ.T @ X + coef[:, None] * Wp
    return {
        "dX": dZ @ Wp,
        "dA": float(s) * (B.T @ dWp),
        "dB": float(s) * (dWp @ A.T),
        "dm": dm,
        "db": dY.sum(axis=0),
    }


# ----------------------------------------------------------------------------- dora-cols
def col_norm_explicit(W0, A, B, s):
    """nu_k = sqrt(sum_n W'[n,k]^2) from the materialised W' (the naive [out,in] norm)."""
    Wp = adapted_weight(W0, A, B, s)
    return np.sqrt(np.sum(Wp * Wp, axis=0))


def w0_col_sumsq(W0):
    """sum_n W0[n,k]^2: the constant the fast path caches for a frozen W0 (column form)."""
    W0 = _f64(W0)
    return np.sum(W0 * W0, axis=0)


def dora_cols_forward(X, W0, A, B, m, s, eps=1e-12, bias=None):
    """Returns dict(Y, Xs, nu, g) with Xs = X.diag(g), the scaled layer input."""
    X, m = _f64(X), _f64(m)
    Wp = adapted_weight(W0, A, B, s)
    nu = np.sqrt(np.sum(Wp * Wp, axis=0))
    g = m / np.maximum(nu, eps)
    Wpp = Wp * g[None, :]
    Y = X @ Wpp.T
    if bias is not None:
        Y = Y + _f64(bias)[None, :]
    return {"Y": Y, "Xs": X * g[None, :], "nu": nu, "g": g}


def dora_cols_backward(dY, X, W0, A, B, m, s, eps=1e-12):
    """Chain rule through W'' = W'.diag(g) with the explicit column norm kept in the graph.

      G      = dY^T.X                     (gradient of W'')
      dg_k   = sum_n G[n,k] W'[n,k]
      dm_k   = dg_k / max(nu_k, eps)
      dnu_k  = -dg_k m_k / nu_k^2        (0 where nu_k <= eps)
      dW'    = G.diag(g) + W'.diag(dnu/nu)
      dA = s.B^T.dW',  dB = s.dW'.A^T,  dX = dY.W'',  db = column sums of dY.
    Returns dict(dX, dA, dB, dm, db).
    """
    dY, X, A, B, m = _f64(dY), _f64(X), _f64(A), _f64(B), _f64(m)
    Wp = adapted_weight(W0, A, B, s)
    nu = np.sqrt(np.sum(Wp * Wp, axis=0))
    den = np.maximum(nu, eps)
    g = m / den
    G = dY.T @ X
    dg = np.sum(G * Wp, axis=0)
    dm = dg / den
    active = nu > eps
    dnu = np.where(active, -dg * m / np.where(active, nu * nu, 1.0), 0.0)
    coef = np.where(active, dnu / np.where(active, nu, 1.0), 0.0)
    dWp = G * g[None, :] + Wp * coef[None, :]
    return {
        "dX": dY @ (Wp * g[None, :]),
        "dA": float(s) * (B.T @ dWp),
        "dB": float(s) * (dWp @ A.T),
        "dm": dm,
        "db": dY.sum(axis=0),
    }
