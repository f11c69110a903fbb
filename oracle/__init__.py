"""Plain fp64 CPU oracle for the fused LoRA / DoRA adapted linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, headers,
tables or helpers with the HIP library in ``lora_dora_linear_amd/``.

What it computes and why it is written the slow way
---------------------------------------------------
The pages say the fused path reaches exactly the result of the materialised
adapted weight, only without building it ("LoRA/DoRA fast forward: no weight
materialization", section "What"; "How Unsloth's FastLoRA Kernel Differs from
Standard LoRA Implementations", FAQ on memory use).  So every function here is
the plain definition written out in float64: it deliberately builds
dW = B.A, W' = W0 + s.dW, the explicit row norm of W', and the weight-shaped
gradient G = dY^T.X, and then applies the textbook chain rule.  numpy's
``matmul`` serves as the only library primitive; there is no blocking, fusion
or reordering.

Conventions (shared with the library's C interface, restated here):
  X [M,K], W0 [N,K], A = lora_down [r,K], B = lora_up [N,r], Y [M,N], dY [M,N].
  s is the single scalar that multiplies the low-rank delta (strength
  multiplies inside the delta: "LoRA/DoRA fast forward", section "Fidelity").

Modules
  lora   - LoRA bypass forward/backward.
  dora   - DoRA (row-scaled, "dora-rows") forward/backward with the explicit norm.
  swiglu - LoRA MLP with the SwiGLU activation (gate, up, down adapters).
  w8a8   - per-row / per-channel int8 quantiser and the int8 base + LoRA layer.
  merge  - the LoRA merge (adapted weight formed explicitly) and its backward.
  geglu  - LoRA MLP with the GeGLU activation (exact and tanh forms of GELU).
  dropout - weight-space dropout of the adapters (a keep mask over lora_down's inputs).
  multi  - several adapters over one concatenated base weight (fused QKV).
  fp8    - per-row e4m3 quantiser and the 8-bit float base + LoRA layer.

Parity status of every function is listed in its own docstring; functions
with no independent pin say "parity unpinned".
"""

from . import lora, dora, swiglu, w8a8, merge, geglu, dropout, multi, fp8  # noqa: F401
