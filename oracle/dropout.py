"""Weight-space dropout of the adapters, plain definition in float64 (oracle; test use only).

Source passage: "LoRA/DoRA fast forward: no weight materialization" (Stable Audio PR),
section "Fidelity": weight-space dropout is drawn once per forward and shared with the norm
terms.  Reading (the pages give no formula): a keep mask over the input features of the
lora_down factor, the same for every rank, drawn once per forward (here passed in), with
the usual inverted-dropout scale, d_k = keep_k / (1 - p); the adapter then uses A.diag(d)
everywhere A appears: in the low-rank product and, for DoRA, in the norm of the adapted
weight.  With keep all ones and p = 0 the layer is the plain one.

  LoRA:  W' = W0 + s.B.(A.diag(d)),  Y = X.W'^T (+ b)
  DoRA:  the row-scaled layer of oracle.dora with A.diag(d) in place of A
  gradients: those of the layer with A.diag(d), then dA = dA_d.diag(d) (chain rule)

Pins (tests/test_oracle_dropout.py): keep all ones with p = 0 equals the plain layer; keep
all zeros leaves the base (LoRA) / the magnitude-scaled base (DoRA); central finite
differences of dA and dB through the mask.
"""

import numpy as np

from . import dora, lora


def drop_scale(keep, p):
    """d_k = keep_k / (1 - p)."""
    return np.asarray(keep, np.float64) / (1.0 - float(p))


def lora_forward(X, W0, A, B, s, keep, p, bias=None):
    Ad = np.asarray(A, np.float64) * drop_scale(keep, p)[None, :]
    return lora.lora_forward(X, W0, Ad, B, s, bias)


def lora_backward(dY, X, W0, A, B, s, keep, p):
    d = drop_scale(keep, p)
    g = lora.lora_backward(dY, X, W0, np.asarray(A, np.float64) * d[None, :], B, s)
    g["dA"] = g["dA"] * d[None, :]
    return g


def dora_forward(X, W0, A, B, m, s, keep, p, eps=1e-12, bias=None):
    Ad = np.asarray(A, np.float64) * drop_scale(keep, p)[None, :]
    return dora.dora_forward(X, W0, Ad, B, m, s, eps, bias)


def dora_backward(dY, X, W0, A, B, m, s, keep, p, eps=1e-12):
    d = drop_scale(keep, p)
    g = dora.dora_backward(dY, X, W0, np.asarray(A, np.float64) * d[None, :], B, m, s, eps)
    g["dA"] = g["dA"] * d[None, :]
    return g
