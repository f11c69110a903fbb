"""Fused LoRA / DoRA adapted linear layer for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C interface in
include/lora_dora_linear.h (library: liblora_dora_linear.so in this package).
`binding` is the thin ctypes layer with the same entry-point names; `inputs`
draws the seeded synthetic tensors used by the tests and the benchmark.
"""

_EXPORTS = (
    "lora_linear_fwd", "lora_linear_bwd", "lora_linear_bwd_noalloc", "lora_dropout_mask", "lora_dropout_grad", "lora_merge_fwd", "lora_merge_bwd", "lora_multi_linear_fwd", "lora_multi_linear_bwd", "multi_workspace_bytes", "dora_prepare", "dora_linear_fwd", "dora_linear_bwd",
    "dora_cols_prepare", "dora_cols_linear_fwd", "dora_cols_linear_bwd",
    "swiglu_lora_mlp_fwd", "swiglu_lora_mlp_bwd", "geglu_lora_mlp_fwd", "geglu_lora_mlp_bwd", "w8a8_quantize_weight", "w8a8_quantize_rows",
    "int8_gemm_raw", "w8a8_lora_linear_fwd", "w8a8_lora_linear_bwd",
    "fp8_quantize_weight", "fp8_quantize_rows", "fp8_lora_linear_fwd", "fp8_lora_linear_bwd", "workspace_bytes",
    "dora_state_floats", "set_tuning", "status_string", "lib", "LdlError",
)


def __getattr__(name):
    # load the binding (and with it torch and the HIP library) only when used
    if name in _EXPORTS:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
