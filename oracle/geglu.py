"""LoRA MLP with the GeGLU activation, materialised definition in float64 (oracle; test use only).

Source passages ("How Unsloth's FastLoRA Kernel Differs from Standard LoRA Implementations"):
  * section "Activation Function Fusion": the LoRA update is injected while the SwiGLU and
    GeGLU activations are computed (apply_lora_mlp_geglu_* beside apply_lora_mlp_swiglu);
  * section "Fused Forward Pass Architecture": gate and up projections with LoRA, the gated
    activation, then the down projection with LoRA.

Readings: h = gelu(e) * g with gelu(e) = e.Phi(e), Phi the standard normal distribution
function (exact form), or the tanh form 0.5 e (1 + tanh(sqrt(2/pi) (e + 0.044715 e^3)))
(the "approximate" variant); no bias; no dropout; each projection has its own (A, B, s) in
the LoRA convention of oracle.lora.

Forward:  E = X.Wg'^T,  Gu = X.Wu'^T,  H = gelu(E) * Gu,  O = H.Wd'^T.
Backward: dH = dO.Wd',  Gd = dO^T.H,  dE = dH * Gu * gelu'(E),  dGu = dH * gelu(E),
          dX = dE.Wg' + dGu.Wu',  G_gate = dE^T.X,  G_up = dGu^T.X,
          dA_p = s_p.B_p^T.G_p,  dB_p = s_p.G_p.A_p^T.

Pins (tests/test_oracle_geglu.py): gelu(0) = 0 and gelu'(0) = 1/2 for both forms, the exact
form against scipy.stats.norm.cdf, the tanh form within 1e-3 of the exact one, both
derivatives against central differences, all B = 0 equals the plain MLP written with
scipy.stats.norm.cdf, finite differences of every gradient.
"""

import math

import numpy as np

from .lora import adapted_weight

_SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _Phi(x):
    """Standard normal distribution function, as 0.5 erfc(-x / sqrt 2) (no cancellation for x < 0)."""
    return 0.5 * np.vectorize(math.erfc, otypes=[np.float64])(-_f64(x) / math.sqrt(2.0))


def gelu(e, approximate=False):
    e = _f64(e)
    if approximate:
        return 0.5 * e * (1.0 + np.tanh(_SQRT_2_OVER_PI * (e + 0.044715 * e ** 3)))
    return e * _Phi(e)


def gelu_grad(e, approximate=False):
    """d gelu / d e: Phi(e) + e.phi(e) (exact form); the derivative of the tanh form."""
    e = _f64(e)
    if approximate:
        t = np.tanh(_SQRT_2_OVER_PI * (e + 0.044715 * e ** 3))
        return 0.5 * (1.0 + t) + 0.5 * e * (1.0 - t * t) * _SQRT_2_OVER_PI * (1.0 + 3 * 0.044715 * e * e)
    return _Phi(e) + e * np.exp(-0.5 * e * e) / math.sqrt(2.0 * math.pi)


def geglu_mlp_forward(X, gate, up, down, approximate=False):
    """gate/up/down are tuples (W, A, B, s).  Returns dict(O, E, Gu, H)."""
    X = _f64(X)
    Wg, Wu, Wd = adapted_weight(*gate), adapted_weight(*up), adapted_weight(*down)
    E = X @ Wg.T
    Gu = X @ Wu.T
    H = gelu(E, approximate) * Gu
    return {"O": H @ Wd.T, "E": E, "Gu": Gu, "H": H}


def geglu_mlp_backward(dO, X, gate, up, down, approximate=False):
    """Gradients of <dO, O>.  Returns dict(dX, dA_gate, dB_gate, dA_up, dB_up, dA_down, dB_down)."""
    dO, X = _f64(dO), _f64(X)
    Wg, Wu, Wd = adapted_weight(*gate), adapted_weight(*up), adapted_weight(*down)
    E = X @ Wg.T
    Gu = X @ Wu.T
    H = gelu(E, approximate) * Gu
    dH = dO @ Wd
    dE = dH * Gu * gelu_grad(E, approximate)
    dGu = dH * gelu(E, approximate)
    out = {"dX": dE @ Wg + dGu @ Wu}
    for name, (W, A, B, s), G in (("gate", gate, dE.T @ X), ("up", up, dGu.T @ X), ("down", down, dO.T @ H)):
        A, B = _f64(A), _f64(B)
        out["dA_" + name] = float(s) * (B.T @ G)
        out["dB_" + name] = float(s) * (G @ A.T)
    return out
