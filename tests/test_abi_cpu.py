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
              "ldl_status_string", "dora_state_floats", "ldl_set_tuning", "ldl_version", "lora_linear_bwd_noalloc",
              "ldl_noalloc_scratch_bytes", "lora_merge_fwd", "lora_merge_bwd", "geglu_lora_mlp_fwd",
              "lora_dropout_mask", "lora_dropout_grad",
              "geglu_lora_mlp_bwd"):
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
    for op in range(9):
        n1 = L.ldl_workspace_bytes(op, 4096, 4096, 4096, 16, 1)
        n2 = L.ldl_workspace_bytes(op, 8192, 4096, 4096, 16, 1)
        assert n1 % 256 == 0 and n2 >= n1
    assert L.ldl_workspace_bytes(1, -1, 64, 64, 16, 1) == 0
    assert L.ldl_workspace_bytes(99, 64, 64, 64, 16, 1) == 0
    assert L.dora_state_floats(3072, 32) == 2 * 3072 + 3072 * 32 + 32 * 32
    # the backward needs at least V (M x r fp32)
    assert L.ldl_workspace_bytes(1, 4096, 4096, 4096, 16, 1) >= 4096 * 16 * 4


def test_workspace_counts_split_partials(L):
    """The LoRA forward's workspace holds fp32 partials for the tiles past the last full round
    of the 256 compute units: 4096 x 5120 outputs are 320 tiles of 256 x 256, the 64 past the
    first round split four ways (256 x 256 fp32 = 256 KiB per block); 4096 x 4096 (256 tiles)
    has no tail, the forward's other workspace does not depend on N, and fp32 calls never split."""
    fwd = 0
    a = L.ldl_workspace_bytes(fwd, 4096, 5120, 4096, 16, 1)
    b = L.ldl_workspace_bytes(fwd, 4096, 4096, 4096, 16, 1)
    assert a - b == 64 * 4 * 256 * 256 * 4
    # 1024 tokens: 80 tiles each split three ways, against 64 tiles split four ways at 4096 columns
    a = L.ldl_workspace_bytes(fwd, 1024, 5120, 4096, 16, 1)
    b = L.ldl_workspace_bytes(fwd, 1024, 4096, 4096, 16, 1)
    assert a - b == 80 * 3 * 256 * 256 * 4 - 64 * 4 * 256 * 256 * 4
    assert L.ldl_workspace_bytes(fwd, 4096, 5120, 4096, 16, 0) == L.ldl_workspace_bytes(fwd, 4096, 4096, 4096, 16, 0)


def test_tuning_switch(L):
    assert L.ldl_set_tuning(0, 1) == OK
    assert L.ldl_set_tuning(0, 0) == OK
    assert L.ldl_set_tuning(0, 7) == INVAL
    for v in (0, 2, 1):
        assert L.ldl_set_tuning(1, v) == OK
    assert L.ldl_set_tuning(1, 3) == INVAL
    assert L.ldl_set_tuning(42, 0) == INVAL
    for v in (0, 2, 1):
        assert L.ldl_set_tuning(2, v) == OK
    assert L.ldl_set_tuning(2, 3) == INVAL
    for v in (0, 1):
        assert L.ldl_set_tuning(3, v) == OK
    assert L.ldl_set_tuning(3, 2) == INVAL


def test_kernel_event_hook_arguments(L):
    """Kinds 0 (forward GEMM), 1 (input-gradient GEMM) and 2 (gated-MLP activation pass) take
    a hook; turning one off (count 0, no arrays) records nothing and needs no GPU."""
    for kind in (0, 1, 2):
        assert L.ldl_set_kernel_events(kind, None, None, 0) == OK
    assert L.ldl_set_kernel_events(3, None, None, 0) == INVAL
    assert L.ldl_set_kernel_events(-1, None, None, 0) == INVAL
    assert L.ldl_set_kernel_events(0, None, None, -1) == INVAL
    assert L.ldl_set_kernel_events(2, None, None, 4) == INVAL      # events missing


# fake, 256-aligned, never dereferenced: every call below fails validation first
P = ctypes.c_void_p(0x100000)
P2 = ctypes.c_void_p(0x200000)
MIS = ctypes.c_void_p(0x100008)   # not 16-byte aligned
NUL = None


def lora_fwd_args(M=64, N=64, K=64, r=16, dtype=1, **kw):
    a = dict(X=P, ldx=0, W0=P, ldw=0, A=P, B=P, bias=NUL, Y=P, ldy=0, U=P, ldu=0, ws=P, nws=1 << 20)
    a.update(kw)
    return (M, N, K, r, 0.5, dtype, a["X"], a["ldx"], a["W0"], a["ldw"], a["A"], a["B"], a["bias"], a["Y"],
            a["ldy"], a["U"], a["ldu"], a["ws"], a["nws"], NUL)


def lora_bwd_args(L, M=64, N=64, K=64, r=16, dtype=1, **kw):
    need = L.ldl_workspace_bytes(1, M, N, K, r, dtype) if M >= 0 else 0
    a = dict(dY=P, lddy=0, X=P, ldx=0, W0=P, ldw=0, A=P, B=P, U=NUL, ldu=0, dX=P, lddx=0, dA=P, dB=P, db=NUL,
             ws=P, nws=need)
    a.update(kw)
    return (M, N, K, r, 0.5, dtype, a["dY"], a["lddy"], a["X"], a["ldx"], a["W0"], a["ldw"], a["A"], a["B"],
            a["U"], a["ldu"], a["dX"], a["lddx"], a["dA"], a["dB"], a["db"], a["ws"], a["nws"], NUL)


def test_lora_fwd_validation(L):
    f = L.lora_linear_fwd
    assert f(*lora_fwd_args(W0=NUL)) == INVAL                          # null weight
    assert f(*lora_fwd_args(dtype=7)) == INVAL                         # bad dtype
    assert f(*lora_fwd_args(M=-1)) == INVAL
    assert f(*lora_fwd_args(r=0)) == INVAL
    assert f(*lora_fwd_args(N=100)) == UNSUP                           # shapes the bf16 kernels do not take
    assert f(*lora_fwd_args(K=96)) == UNSUP
    assert f(*lora_fwd_args(r=129)) == UNSUP
    assert f(*lora_fwd_args(X=MIS)) == UNSUP                           # misaligned pointer
    assert f(*lora_fwd_args(U=NUL, ws=NUL, nws=0)) == WS               # no U_save and no workspace


def test_leading_dimension_validation(L):
    f = L.lora_linear_fwd
    # below the row length: invalid; not a whole number of 16-byte groups: unsupported
    assert f(*lora_fwd_args(ldx=32)) == INVAL
    assert f(*lora_fwd_args(ldw=-8)) == INVAL
    assert f(*lora_fwd_args(ldy=63)) == INVAL
    assert f(*lora_fwd_args(ldu=8)) == INVAL
    assert f(*lora_fwd_args(ldx=68)) == UNSUP
    assert f(*lora_fwd_args(ldy=100)) == UNSUP
    assert f(*lora_fwd_args(ldu=18)) == UNSUP
    # the fp32 path takes any leading dimension at least the row length (the call then stops
    # at the missing workspace, before anything is enqueued)
    assert f(*lora_fwd_args(dtype=0, ldx=97, ldy=101, ldw=96, N=100, K=96, U=NUL, ldu=0, ws=NUL, nws=0)) == WS
    assert f(*lora_fwd_args(ldx=72, ldy=80, ldw=128, U=NUL, ws=NUL, nws=0)) == WS
    # a leading dimension whose rows reach past 2 GiB
    assert f(*lora_fwd_args(M=70000, ldx=1 << 15, K=64)) == UNSUP
    b = L.lora_linear_bwd
    assert b(*lora_bwd_args(L, lddy=56)) == INVAL
    assert b(*lora_bwd_args(L, lddx=60)) == INVAL
    assert b(*lora_bwd_args(L, lddx=72, ws=NUL)) == INVAL               # valid ld, then the null workspace
    assert b(*lora_bwd_args(L, lddy=66)) == UNSUP
    d = L.dora_prepare
    assert d(64, 64, 1, P, 32, P, NUL) == INVAL
    assert d(64, 64, 1, P, 68, P, NUL) == UNSUP
    q = L.w8a8_quantize_rows
    assert q(64, 128, P, 120, P, P, NUL) == INVAL
    assert q(64, 128, P, 132, P, P, NUL) == UNSUP
    r = L.int8_gemm_raw
    assert r(64, 128, 128, P, 136, P, 0, P, 0, NUL) == UNSUP           # int8 rows: multiples of 16 bytes
    assert r(64, 128, 128, P, 0, P, 0, P, 100, NUL) == INVAL


def test_lora_bwd_validation(L):
    f = L.lora_linear_bwd
    assert f(*lora_bwd_args(L, dA=NUL)) == INVAL
    need = L.ldl_workspace_bytes(1, 64, 64, 64, 16, 1)
    assert f(*lora_bwd_args(L, nws=need - 256)) == WS
    assert f(*lora_bwd_args(L, K=72)) == UNSUP
    n = L.lora_linear_bwd_noalloc
    cap = L.ldl_noalloc_scratch_bytes()
    assert cap == 32 << 20
    big = lora_bwd_args(L, M=16384, N=8192, K=8192, r=128)
    assert L.ldl_workspace_bytes(1, 16384, 8192, 8192, 128, 1) > cap
    assert n(*(big[:21] + (NUL,))) == WS                                # refused before any HIP call


def dora_fwd_args(**kw):
    a = dict(M=64, N=64, K=64, r=16, eps=1e-12, dtype=1, X=P, ldx=0, W0=P, ldw=0, A=P, B=P, m=P, c=P, bias=NUL,
             Y=P, ldy=0, U=P, ldu=0, Z=P, ldz=0, state=P)
    a.update(kw)
    return (a["M"], a["N"], a["K"], a["r"], 1.0, a["eps"], a["dtype"], a["X"], a["ldx"], a["W0"], a["ldw"], a["A"],
            a["B"], a["m"], a["c"], a["bias"], a["Y"], a["ldy"], a["U"], a["ldu"], a["Z"], a["ldz"], a["state"], NUL,
            0, NUL)


def test_dora_validation(L):
    assert L.dora_prepare(64, 64, 1, NUL, 0, P, NUL) == INVAL
    assert L.dora_prepare(0, 64, 1, P, 0, P, NUL) == INVAL
    f = L.dora_linear_fwd
    # fp32 DoRA is not offered; r must be a multiple of 8; state required
    assert f(*dora_fwd_args(dtype=0)) == UNSUP
    assert f(*dora_fwd_args(r=12)) == UNSUP
    assert f(*dora_fwd_args(state=NUL)) == INVAL
    assert f(*dora_fwd_args(eps=-1.0)) == INVAL
    assert f(*dora_fwd_args(ldz=40)) == INVAL
    b = L.dora_linear_bwd
    need = L.ldl_workspace_bytes(3, 64, 64, 64, 16, 1)
    args = [64, 64, 64, 16, 1.0, 1e-12, 1, P, 0, P, 0, P, 0, P, P, P, P, 0, P, 0, P, P, 0, P, P, P, NUL, P, need, NUL]
    a2 = list(args); a2[-2] = need - 256
    assert b(*a2) == WS
    a3 = list(args); a3[25] = NUL   # dm
    assert b(*a3) == INVAL


def test_swiglu_and_w8a8_validation(L):
    f = L.swiglu_lora_mlp_fwd

    def sw(M=64, K=64, H=64, r=16, **kw):
        a = dict(X=P, ldx=0, Wg=P, Out=P, ldo=0)
        a.update(kw)
        return (M, K, H, r, 0.25, 0.25, 0.25, a["X"], a["ldx"], a["Wg"], P, P, P, P, P, P, P, P, a["Out"], a["ldo"],
                P, P, P, P, NUL, 0, NUL)
    assert f(*sw(r=65)) == UNSUP              # r > 64
    assert f(*sw(K=96)) == UNSUP              # K not a multiple of 64
    assert f(*sw(Wg=NUL)) == INVAL
    assert f(*sw(ldo=32)) == INVAL
    g = L.geglu_lora_mlp_fwd
    a = list(sw(r=65)); a.insert(7, 0)
    assert g(*a) == UNSUP
    a = list(sw()); a.insert(7, 2)
    assert g(*a) == INVAL                      # approximate must be 0 or 1
    w = L.w8a8_lora_linear_fwd
    need = L.ldl_workspace_bytes(6, 64, 128, 128, 16, 1)

    def wa(M=64, N=128, K=128, **kw):
        a = dict(ldx=0, ldw=0, Xq=NUL, sx=NUL, ws=P, nws=need, ldy=0)
        a.update(kw)
        return (M, N, K, 16, 0.5, P, a["ldx"], P, a["ldw"], P, P, P, NUL, P, a["ldy"], a["Xq"], a["sx"], NUL, 0,
                a["ws"], a["nws"], NUL)
    assert w(*wa(K=192, nws=1 << 22)) == UNSUP                                   # K % 128
    assert w(*wa(Xq=P)) == INVAL                                                 # Xq without sx
    assert w(*wa(nws=need - 256)) == WS
    assert w(*wa(ldw=136)) == UNSUP                                              # int8 rows of 16 bytes
    assert L.int8_gemm_raw(64, 128, 96, P, 0, P, 0, P, 0, NUL) == UNSUP
    assert L.w8a8_quantize_weight(64, 64, 3, P, 0, P, P, NUL) == INVAL
    assert L.w8a8_quantize_rows(64, 12, P, 0, P, P, NUL) == UNSUP


def test_merge_validation(L):
    f = L.lora_merge_fwd
    assert f(64, 72, 16, 0.5, 1, P, 0, P, P, P, 0, NUL) == UNSUP            # bf16: K % 64
    assert f(64, 60, 16, 0.5, 0, P, 0, P, P, P, 0, NUL) == UNSUP            # fp32: K % 8
    assert f(64, 64, 129, 0.5, 1, P, 0, P, P, P, 0, NUL) == UNSUP           # r > 128
    assert f(64, 64, 16, 0.5, 1, P, 0, NUL, P, P, 0, NUL) == INVAL          # A null
    assert f(64, 64, 16, 0.5, 1, P, 72, P, P, P, 0, NUL) == INVAL           # in place with different strides
    assert f(64, 64, 16, 0.5, 1, P, 0, P, P, P2, 60, NUL) == INVAL          # ldo below the row length
    assert f(64, 64, 16, 0.5, 2, P, 0, P, P, P2, 0, NUL) == INVAL           # dtype
    b = L.lora_merge_bwd
    need = L.ldl_workspace_bytes(8, 0, 64, 64, 16, 1)
    assert need > 0
    assert b(64, 64, 16, 0.5, 1, P, 0, P, P, P, P, P, need - 256, NUL) == WS
    assert b(64, 64, 16, 0.5, 1, P, 0, P, P, NUL, P, P, need, NUL) == INVAL


def _ints(*v):
    return ctypes.cast((ctypes.c_int * len(v))(*v), ctypes.c_void_p)


def _floats(*v):
    return ctypes.cast((ctypes.c_float * len(v))(*v), ctypes.c_void_p)


def test_multi_leaf_validation(L):
    n3, s3 = _ints(128, 64, 64), _floats(0.5, 1.0, 2.0)
    q = L.ldl_multi_workspace_bytes

    def fwd(M=64, K=64, nl=3, n=n3, r=16, sl=s3, dtype=1, ldy=0, U=P, nws=0):
        return L.lora_multi_linear_fwd(M, K, nl, n, r, sl, dtype, P, 0, P, 0, P, P, NUL, P, ldy, U, 0, P, nws, NUL)

    assert fwd(nl=0) == INVAL
    assert fwd(n=NUL) == INVAL
    assert fwd(sl=NUL) == INVAL
    assert fwd(nl=9, n=_ints(*[64] * 9), sl=_floats(*[1.0] * 9)) == UNSUP       # more than eight leaves
    assert fwd(n=_ints(128, 100, 64)) == UNSUP                                   # leaf width % 64
    assert fwd(n=_ints(128, 0, 64)) == INVAL                                     # empty leaf
    assert fwd(r=12) == UNSUP                                                    # r % 8
    assert fwd(r=48) == UNSUP                                                    # L r = 144 > 128
    assert fwd(dtype=0) == UNSUP                                                 # fp32 not taken
    assert fwd(dtype=2) == INVAL
    assert fwd(ldy=200) == INVAL                                                 # ldy below N = 256
    assert fwd(U=NUL, nws=q(0, 64, 64, 3, n3, 16) - 256) == WS
    assert q(0, 64, 64, 3, n3, 16) == 64 * 48 * 4
    assert q(0, 64, 64, 0, n3, 16) == 0 and q(5, 64, 64, 3, n3, 16) == 0
    need = q(1, 64, 64, 3, n3, 16)
    assert need > 0

    def bwd(dA=P, nws=need, dtype=1):
        return L.lora_multi_linear_bwd(64, 64, 3, n3, 16, s3, dtype, P, 0, P, 0, P, 0, P, P, NUL, 0, P, 0, dA, P,
                                       NUL, P, nws, NUL)

    assert bwd(nws=need - 256) == WS
    assert bwd(dA=NUL) == INVAL
    assert bwd(dtype=0) == UNSUP


def test_dora_cols_validation(L):
    f = L.dora_cols_linear_fwd
    need = L.ldl_workspace_bytes(9, 64, 64, 64, 16, 1)
    assert need > 0 and L.ldl_workspace_bytes(10, 64, 64, 64, 16, 1) > 0

    def fwd(M=64, N=64, K=64, r=16, dtype=1, Xs=P, st=P, nws=need, eps=1e-12):
        return f(M, N, K, r, 0.5, eps, dtype, P, 0, P, 0, P, P, P, P, NUL, P, 0, NUL, 0, Xs, 0, st, P, nws, NUL)

    assert fwd(r=72) == UNSUP              # r above 64
    assert fwd(r=12) == UNSUP              # r % 8
    assert fwd(dtype=0) == UNSUP
    assert fwd(Xs=NUL) == INVAL            # the scaled input is required
    assert fwd(st=NUL) == INVAL
    assert fwd(eps=-1.0) == INVAL
    assert fwd(nws=need - 256) == WS
    b = L.dora_cols_linear_bwd
    needb = L.ldl_workspace_bytes(10, 64, 64, 64, 16, 1)

    def bwd(dm=P, nws=needb):
        return b(64, 64, 64, 16, 0.5, 1e-12, 1, P, 0, P, 0, P, 0, P, 0, P, P, P, NUL, 0, P, P, 0, P, P, dm, NUL, P,
                 nws, NUL)

    assert bwd(dm=NUL) == INVAL
    assert bwd(nws=needb - 256) == WS
    assert L.dora_cols_prepare(64, 64, 2, P, 0, P, NUL) == INVAL


def test_workspace_query_with_empty_batch(L):
    # M == 0 is valid everywhere; the size queries must not divide by zero
    for op in range(11):
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
