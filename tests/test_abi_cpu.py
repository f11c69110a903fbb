"""CPU checks of the C boundary: the library loads, exports every declared entry
point, and rejects bad arguments on the host before any HIP call is made."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_dora_linear.h")
LIB = os.path.join(ROOT, "lora_dora_linear_amd", "liblora_dora_linear.so")

OK, INVAL, UNSUP, WS = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|void)\s*\**\s*(\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.skip("library not built (run __graft_entry__.build())")
    from lora_dora_linear_amd import binding
    return binding.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("lora_linear_fwd", "lora_linear_bwd", "dora_linear_fwd", "dora_linear_bwd", "dora_prepare",
              "swiglu_lora_mlp_fwd", "swiglu_lora_mlp_bwd", "w8a8_lora_linear_fwd", "w8a8_lora_linear_bwd",
              "w8a8_quantize_weight", "w8a8_quantize_rows", "int8_gemm_raw", "ldl_workspace_bytes",
              "ldl_status_string", "dora_state_floats", "ldl_set_tuning", "ldl_version"):
        assert n in names, n


def test_library_exports_every_declared_symbol(L):
    raw = ctypes.CDLL(LIB)
    for n in declared_functions():
        assert hasattr(raw, n), f"missing export {n}"
    from lora_dora_linear_amd import binding
    assert set(binding.SIGNATURES) == set(declared_functions())


def test_status_strings_and_version(L):
    assert L.ldl_status_string(0) == b"ok"
    for c in (INVAL, UNSUP, WS, -4):
        assert len(L.ldl_status_string(c)) > 5
    assert L.ldl_status_string(12345) == b"unknown status"
    assert L.ldl_version() >= 100


def test_workspace_sizes(L):
    for op in range(8):
        n1 = L.ldl_workspace_bytes(op, 4096, 4096, 4096, 16, 1)
        n2 = L.ldl_workspace_bytes(op, 8192, 4096, 4096, 16, 1)
        assert n1 % 256 == 0 and n2 >= n1
    assert L.ldl_workspace_bytes(1, -1, 64, 64, 16, 1) == 0
    assert L.ldl_workspace_bytes(99, 64, 64, 64, 16, 1) == 0
    assert L.dora_state_floats(3072, 32) == 2 * 3072 + 3072 * 32 + 32 * 32
    # the backward needs at least V (M x r fp32) and B^T
    assert L.ldl_workspace_bytes(1, 4096, 4096, 4096, 16, 1) >= 4096 * 16 * 4


def test_tuning_switch(L):
    assert L.ldl_set_tuning(0, 1) == OK
    assert L.ldl_set_tuning(0, 0) == OK
    assert L.ldl_set_tuning(0, 7) == INVAL
    assert L.ldl_set_tuning(42, 0) == INVAL
    for v in (0, 2, 1):
        assert L.ldl_set_tuning(2, v) == OK
    assert L.ldl_set_tuning(2, 3) == INVAL


# fake, 256-aligned, never dereferenced: every call below fails validation first
P = ctypes.c_void_p(0x100000)
P2 = ctypes.c_void_p(0x200000)
MIS = ctypes.c_void_p(0x100008)   # not 16-byte aligned
NUL = None


def test_lora_fwd_validation(L):
    f = L.lora_linear_fwd
    # null weight
    assert f(64, 64, 64, 16, 0.5, 1, P, NUL, P, P, NUL, P, P, P, 1 << 20, NUL) == INVAL
    # bad dtype, negative sizes
    assert f(64, 64, 64, 16, 0.5, 7, P, P, P, P, NUL, P, P, P, 1 << 20, NUL) == INVAL
    assert f(-1, 64, 64, 16, 0.5, 1, P, P, P, P, NUL, P, P, P, 1 << 20, NUL) == INVAL
    assert f(64, 64, 64, 0, 0.5, 1, P, P, P, P, NUL, P, P, P, 1 << 20, NUL) == INVAL
    # shapes the bf16 kernels do not take
    assert f(64, 100, 64, 16, 0.5, 1, P, P, P, P, NUL, P, P, P, 1 << 20, NUL) == UNSUP
    assert f(64, 64, 96, 16, 0.5, 1, P, P, P, P, NUL, P, P, P, 1 << 20, NUL) == UNSUP
    assert f(64, 64, 64, 129, 0.5, 1, P, P, P, P, NUL, P, P, P, 1 << 20, NUL) == UNSUP
    # misaligned pointer
    assert f(64, 64, 64, 16, 0.5, 1, MIS, P, P, P, NUL, P, P, P, 1 << 20, NUL) == UNSUP
    # no U_save and no workspace
    assert f(64, 64, 64, 16, 0.5, 1, P, P, P, P, NUL, P, NUL, NUL, 0, NUL) == WS


def test_lora_bwd_validation(L):
    f = L.lora_linear_bwd
    need = L.ldl_workspace_bytes(1, 64, 64, 64, 16, 1)
    assert f(64, 64, 64, 16, 0.5, 1, P, P, P, P, P, NUL, P, NUL, P, NUL, P, need, NUL) == INVAL  # dA null
    assert f(64, 64, 64, 16, 0.5, 1, P, P, P, P, P, NUL, P, P, P, NUL, P, need - 256, NUL) == WS
    assert f(64, 64, 72, 16, 0.5, 1, P, P, P, P, P, NUL, P, P, P, NUL, P, need, NUL) == UNSUP


def test_dora_validation(L):
    assert L.dora_prepare(64, 64, 1, NUL, P, NUL) == INVAL
    assert L.dora_prepare(0, 64, 1, P, P, NUL) == INVAL
    f = L.dora_linear_fwd
    # fp32 DoRA is not offered; r must be a multiple of 8; state required
    assert f(64, 64, 64, 16, 1.0, 1e-12, 0, P, P, P, P, P, P, NUL, P, P, P, P, NUL, 0, NUL) == UNSUP
    assert f(64, 64, 64, 12, 1.0, 1e-12, 1, P, P, P, P, P, P, NUL, P, P, P, P, NUL, 0, NUL) == UNSUP
    assert f(64, 64, 64, 16, 1.0, 1e-12, 1, P, P, P, P, P, P, NUL, P, P, P, NUL, NUL, 0, NUL) == INVAL
    assert f(64, 64, 64, 16, 1.0, -1.0, 1, P, P, P, P, P, P, NUL, P, P, P, P, NUL, 0, NUL) == INVAL
    b = L.dora_linear_bwd
    need = L.ldl_workspace_bytes(3, 64, 64, 64, 16, 1)
    args = [64, 64, 64, 16, 1.0, 1e-12, 1, P, P, P, P, P, P, P, P, P, P, P, P, P, NUL, P, need, NUL]
    a2 = list(args); a2[-2] = need - 256
    assert b(*a2) == WS
    a3 = list(args); a3[18] = NUL   # dm
    assert b(*a3) == INVAL


def test_swiglu_and_w8a8_validation(L):
    f = L.swiglu_lora_mlp_fwd
    ps = [P] * 15 + [NUL]        # 15 tensors, then the (absent) workspace
    assert f(64, 64, 64, 65, 0.25, 0.25, 0.25, *ps, 0, NUL) == UNSUP      # r > 64
    assert f(64, 96, 64, 16, 0.25, 0.25, 0.25, *ps, 0, NUL) == UNSUP      # K not a multiple of 64
    ps2 = list(ps); ps2[1] = NUL
    assert f(64, 64, 64, 16, 0.25, 0.25, 0.25, *ps2, 0, NUL) == INVAL
    w = L.w8a8_lora_linear_fwd
    need = L.ldl_workspace_bytes(6, 64, 128, 128, 16, 1)
    assert w(64, 128, 192, 16, 0.5, P, P, P, P, P, NUL, P, NUL, NUL, NUL, P, 1 << 22, NUL) == UNSUP  # K % 128
    assert w(64, 128, 128, 16, 0.5, P, P, P, P, P, NUL, P, P, NUL, NUL, P, need, NUL) == INVAL       # Xq w/o sx
    assert w(64, 128, 128, 16, 0.5, P, P, P, P, P, NUL, P, NUL, NUL, NUL, P, need - 256, NUL) == WS
    assert L.int8_gemm_raw(64, 128, 96, P, P, P, NUL) == UNSUP
    assert L.w8a8_quantize_weight(64, 64, 3, P, P, P, NUL) == INVAL
    assert L.w8a8_quantize_rows(64, 12, P, P, P, NUL) == UNSUP


def test_workspace_query_with_empty_batch(L):
    # M == 0 is valid everywhere; the size queries must not divide by zero
    for op in range(8):
        assert L.ldl_workspace_bytes(op, 0, 256, 256, 16, 1) % 256 == 0


def test_binding_argument_counts_match_the_header():
    from lora_dora_linear_amd import binding
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    decl = {}
    for m in re.finditer(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|void)\s*\**\s*(\w+)\s*\(([^;]*?)\);", src,
                         re.M | re.S):
        decl[m.group(1)] = len([a for a in m.group(2).split(",") if a.strip() and a.strip() != "void"])
    assert set(decl) == set(binding.SIGNATURES)
    for name, n in decl.items():
        assert len(binding.SIGNATURES[name][0]) == n, name
