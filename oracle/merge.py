"""LoRA merge, plain definition in float64 (oracle; test use only).

Source passage: "Fused Kernels (experimental)" (LyCORIS kernel docs), section "What is
fused": each algorithm has a merge forward (the weight delta) and a merge backward besides
its bypass kernels; the lora family has both fused.  Orientation as in oracle.lora:
W0 [N,K], A = lora_down [r,K], B = lora_up [N,r].

  merge forward:  W' = W0 + s.B.A   (the delta s.B.A alone when no W0 is given)
  merge backward: for a gradient dW of the merged weight,
                  dA = s.B^T.dW,  dB = s.dW.A^T   (chain rule through s.B.A)

Pins (tests/test_oracle_merge.py): hand-worked example (tests/golden/merge_tiny.json),
brute-force triple loop of the delta, central finite differences of <dW, W'> in A and B.
"""

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def merge_forward(W0, A, B, s):
    """W0 + s.B.A, or s.B.A when W0 is None ([N,K] float64)."""
    delta = float(s) * (_f64(B) @ _f64(A))
    return delta if W0 is None else _f64(W0) + delta


def merge_backward(dW, A, B, s):
    """Gradients of <dW, W0 + s.B.A> in A and B.  Returns dict(dA, dB)."""
    dW, A, B = _f64(dW), _f64(A), _f64(B)
    return {"dA": float(s) * (B.T @ dW), "dB": float(s) * (dW @ A.T)}
