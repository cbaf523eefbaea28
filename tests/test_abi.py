"""The C-ABI library loads, exports every declared symbol and rejects bad
arguments on the host with the documented codes (no GPU needed: every call
here fails validation before anything is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmv.h")

EINVAL, EALIGN, EUNSUPPORTED = 1, 2, 3
A = 0x10000          # a fake, aligned, never dereferenced device address


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qmv_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def qmv():
    import bandwidth_bound_block_amd as q
    return q


def test_every_declared_symbol_is_exported(qmv):
    names = declared_functions()
    assert {"qmv_q8_0", "qmv_q4_0", "qmv_q4_1", "qmv_q4_k", "qmv_q6_k", "qmv_matvec_path", "qmv_matvec_xt", "qmv_i8_requant",
            "qmv_i8_requant_lut", "qmv_moe", "qmv_moe_xt", "qmv_moe_swiglu", "qmv_moe_swiglu_xt", "qmv_moe_combine",
            "qmv_dequant",
            "qmv_chain", "qmv_last_error", "qmv_abi_version"} <= set(names)
    raw = ctypes.CDLL(qmv.library_path())
    for n in names:
        assert hasattr(raw, n), n


def test_header_constants_match_binding(qmv):
    src = open(HEADER).read()
    m = re.search(r"#define\s+QMV_CHAIN_WORKSPACE_BYTES\s+(\d+)", src)
    assert m and int(m.group(1)) == qmv.CHAIN_WORKSPACE_BYTES


def test_abi_version(qmv):
    assert qmv.abi_version() == 1


@pytest.mark.parametrize("name", ["qmv_q8_0", "qmv_q4_0", "qmv_q4_1"])
def test_float_matvec_argument_errors(qmv, name):
    f = getattr(qmv.lib(), name)
    cases = [
        ((0, 8, 64, A, 64, 1, A, 8, None), EINVAL, "null"),
        ((A, 0, 64, A, 64, 1, A, 8, None), EINVAL, "n_rows"),
        ((A, 8, 48, A, 48, 1, A, 8, None), EINVAL, "multiple of 32"),
        ((A, 8, 0, A, 64, 1, A, 8, None), EINVAL, "multiple of 32"),
        ((A, 8, 64, A, 64, 0, A, 8, None), EINVAL, "batch"),
        ((A, 8, 64, A, 64, 9, A, 8, None), EINVAL, "batch"),
        ((A, 8, 64, A, 63, 1, A, 8, None), EINVAL, "ldx"),
        ((A, 8, 64, A, 64, 1, A, 7, None), EINVAL, "ldy"),
        ((A + 2, 8, 64, A, 64, 1, A, 8, None), EALIGN, "aligned"),
        ((A, 8, 64, A + 1, 64, 1, A, 8, None), EALIGN, "aligned"),
        ((A, 8, 64, A, 64, 1, A + 2, 8, None), EALIGN, "aligned"),
        ((A, 8, 64 * 1024 * 1024, A, 64 * 1024 * 1024, 1, A, 8, None), EINVAL, "LDS"),
    ]
    for args, code, word in cases:
        assert f(*args) == code, (args, qmv.last_error())
        assert word in qmv.last_error(), qmv.last_error()


def test_q4_k_argument_errors(qmv):
    """Q4_K: columns in multiples of 256, W 16-byte aligned; the MFMA path
    needs batch >= 2; MoE argument checks; the fused SwiGLU, combine and
    chain entry points refuse the format."""
    f = qmv.lib().qmv_q4_k
    cases = [
        ((0, 8, 256, A, 256, 1, A, 8, None), EINVAL, "null"),
        ((A, 0, 256, A, 256, 1, A, 8, None), EINVAL, "n_rows"),
        ((A, 8, 224, A, 224, 1, A, 8, None), EINVAL, "multiple of 256"),
        ((A, 8, 288, A, 288, 1, A, 8, None), EINVAL, "multiple of 256"),
        ((A, 8, 0, A, 256, 1, A, 8, None), EINVAL, "multiple of 256"),
        ((A, 8, 256, A, 256, 0, A, 8, None), EINVAL, "batch"),
        ((A, 8, 256, A, 256, 9, A, 8, None), EINVAL, "batch"),
        ((A, 8, 256, A, 255, 1, A, 8, None), EINVAL, "ldx"),
        ((A, 8, 256, A, 256, 1, A, 7, None), EINVAL, "ldy"),
        ((A + 4, 8, 256, A, 256, 1, A, 8, None), EALIGN, "16-byte"),
        ((A + 8, 8, 256, A, 256, 1, A, 8, None), EALIGN, "16-byte"),
        ((A, 8, 256, A + 1, 256, 1, A, 8, None), EALIGN, "aligned"),
        ((A, 8, 256, A, 256, 1, A + 2, 8, None), EALIGN, "aligned"),
        ((A, 8, 64 * 1024 * 1024, A, 64 * 1024 * 1024, 1, A, 8, None), EINVAL, "LDS"),
        ((A, 8, 38656, A, 38656, 1, A, 8, None), EINVAL, "LDS"),
    ]
    for args, code, word in cases:
        assert f(*args) == code, (args, qmv.last_error())
        assert word in qmv.last_error(), qmv.last_error()
    L = qmv.lib()
    assert L.qmv_matvec_path(qmv.Q4_K, A, 8, 256, A, 256, 1, A, 8, qmv.PATH_MFMA, None) == EUNSUPPORTED
    assert "matrix-core" in qmv.last_error()
    assert L.qmv_matvec_xt(qmv.Q4_K, A, 8, 256, A, 7, 256, 1, A, 8, 0, None) == EINVAL
    assert "x_type" in qmv.last_error()
    assert L.qmv_dequant(qmv.Q4_K, A, 8, 288, A, None) == EINVAL and "256" in qmv.last_error()
    assert L.qmv_dequant(qmv.Q4_K, A + 4, 8, 256, A, None) == EALIGN
    # MoE experts: routed per pair; argument errors only (nothing launches here)
    assert L.qmv_moe(qmv.Q4_K, A, 144, 2, 8, 256, A, 1, 1, A, 256, 256, A, None) == EINVAL
    assert "expert_stride" in qmv.last_error()
    assert L.qmv_moe(qmv.Q4_K, A, 1152, 2, 8, 288, A, 1, 1, A, 288, 288, A, None) == EINVAL
    assert "multiple of 256" in qmv.last_error()
    assert L.qmv_moe(qmv.Q4_K, A, 1160, 2, 8, 256, A, 1, 1, A, 256, 256, A, None) == EINVAL
    assert L.qmv_moe(qmv.Q4_K, A + 4, 1152, 2, 8, 256, A, 1, 1, A, 256, 256, A, None) == EALIGN
    assert "16-byte" in qmv.last_error()
    assert L.qmv_moe(qmv.Q4_K, A, 1152, 2, 8, 256, A, 9, 1, A, 256, 256, A, None) == EINVAL
    # the fused SwiGLU form: experts of 2 n_ff rows
    assert L.qmv_moe_swiglu(qmv.Q4_K, A, 2288, 2, 8, 256, A, 1, 1, A, 256, 256, A, None) == EINVAL
    assert "expert_stride" in qmv.last_error() and "2304" in qmv.last_error()
    assert L.qmv_moe_swiglu(qmv.Q4_K, A + 4, 2304, 2, 8, 256, A, 1, 1, A, 256, 256, A, None) == EALIGN
    assert L.qmv_moe_swiglu(qmv.Q4_K, A, 2304, 2, 8, 256, A, 9, 1, A, 256, 256, A, None) == EINVAL
    assert L.qmv_moe_swiglu(qmv.Q4_K, A, 2304, 2, 8, 288, A, 1, 1, A, 288, 288, A, None) == EINVAL
    # the fused combine: argument errors only (nothing launches here)
    assert L.qmv_moe_combine(qmv.Q4_K, A, 1136, 2, 8, 256, A, A, 1, 1, A, 256, 256, A, None) == EINVAL
    assert "expert_stride" in qmv.last_error()
    assert L.qmv_moe_combine(qmv.Q4_K, A, 1152, 2, 8, 256, A, A + 2, 1, 1, A, 256, 256, A, None) == EALIGN
    assert L.qmv_moe_combine(qmv.Q4_K, A, 1152, 2, 8, 256, A, None, 1, 1, A, 256, 256, A, None) == EINVAL
    assert L.qmv_moe_combine(qmv.Q4_K, A, 1152, 2, 8, 256, A, A, 1, 17, A, 256, 256, A, None) == EINVAL
    # chains: stage checks before any launch (stages live in host memory)
    for fmt, wal in ((qmv.Q4_K, 16), (qmv.Q6_K, 4)):
        arr = (qmv.ChainStage * 2)()
        arr[0] = qmv.ChainStage(A, A, A, 8, 256, 0, 0)
        arr[1] = qmv.ChainStage(A, A, A, 8, 288, 0, 0)
        ap = ctypes.cast(arr, ctypes.c_void_p)
        assert L.qmv_chain(fmt, ap, 2, A, 1 << 20, None) == EINVAL and "multiple of 256" in qmv.last_error()
        assert L.qmv_chain_noalloc(fmt, ap, 2, None) == EINVAL
        arr[1] = qmv.ChainStage(A + wal // 2, A, A, 8, 256, 0, 0)
        assert L.qmv_chain(fmt, ap, 2, A, 1 << 20, None) == EALIGN
        arr[1] = qmv.ChainStage(A, A, A, 0, 256, 0, 0)
        assert L.qmv_chain_noalloc(fmt, ap, 2, None) == EINVAL and "n_rows" in qmv.last_error()
        assert L.qmv_chain(fmt, ap, 0, A, 1 << 20, None) == EINVAL
        assert L.qmv_chain(fmt, ap, 2, A, 1024, None) == EINVAL and "workspace" in qmv.last_error()
        assert L.qmv_chain_noalloc(fmt, None, 1, None) == EINVAL


def test_q6_k_argument_errors(qmv):
    """Q6_K: columns in multiples of 256, W 4-byte aligned; the MFMA path
    needs batch >= 2; MoE argument checks; the fused SwiGLU, combine and
    chain entry points refuse the format."""
    f = qmv.lib().qmv_q6_k
    cases = [
        ((0, 8, 256, A, 256, 1, A, 8, None), EINVAL, "null"),
        ((A, 0, 256, A, 256, 1, A, 8, None), EINVAL, "n_rows"),
        ((A, 8, 224, A, 224, 1, A, 8, None), EINVAL, "multiple of 256"),
        ((A, 8, 0, A, 256, 1, A, 8, None), EINVAL, "multiple of 256"),
        ((A, 8, 256, A, 256, 9, A, 8, None), EINVAL, "batch"),
        ((A, 8, 256, A, 255, 1, A, 8, None), EINVAL, "ldx"),
        ((A, 8, 256, A, 256, 1, A, 7, None), EINVAL, "ldy"),
        ((A + 2, 8, 256, A, 256, 1, A, 8, None), EALIGN, "4-byte"),
        ((A, 8, 256, A + 1, 256, 1, A, 8, None), EALIGN, "aligned"),
        ((A, 8, 256, A, 256, 1, A + 2, 8, None), EALIGN, "aligned"),
        ((A, 8, 38656, A, 38656, 1, A, 8, None), EINVAL, "LDS"),
    ]
    for args, code, word in cases:
        assert f(*args) == code, (args, qmv.last_error())
        assert word in qmv.last_error(), qmv.last_error()
    L = qmv.lib()
    assert L.qmv_matvec_path(qmv.Q6_K, A, 8, 256, A, 256, 1, A, 8, qmv.PATH_MFMA, None) == EUNSUPPORTED
    assert L.qmv_dequant(qmv.Q6_K, A, 8, 288, A, None) == EINVAL and "256" in qmv.last_error()
    assert L.qmv_moe(qmv.Q6_K, A, 210, 2, 8, 256, A, 1, 1, A, 256, 256, A, None) == EINVAL
    assert "expert_stride" in qmv.last_error()
    assert L.qmv_moe(qmv.Q6_K, A + 2, 1680, 2, 8, 256, A, 1, 1, A, 256, 256, A, None) == EALIGN
    assert L.qmv_moe(qmv.Q6_K, A, 1680, 2, 8, 256, A, 1, 17, A, 256, 256, A, None) == EINVAL
    assert "top_k" in qmv.last_error()
    # the fused forms: argument errors only (nothing launches here)
    assert L.qmv_moe_swiglu(qmv.Q6_K, A, 3356, 2, 8, 256, A, 1, 1, A, 256, 256, A, None) == EINVAL
    assert "expert_stride" in qmv.last_error() and "3360" in qmv.last_error()
    assert L.qmv_moe_swiglu(qmv.Q6_K, A + 2, 3360, 2, 8, 256, A, 1, 1, A, 256, 256, A, None) == EALIGN
    assert L.qmv_moe_combine(qmv.Q6_K, A, 1676, 2, 8, 256, A, A, 1, 1, A, 256, 256, A, None) == EINVAL
    assert L.qmv_moe_combine(qmv.Q6_K, A, 1680, 2, 8, 256, A, A + 2, 1, 1, A, 256, 256, A, None) == EALIGN
    assert L.qmv_dequant(5, A, 8, 256, A, None) == EUNSUPPORTED


def test_matvec_path_argument_errors(qmv):
    f = qmv.lib().qmv_matvec_path
    ok = (A, 8, 256, A, 256, 2, A, 8)
    assert f(qmv.Q4_0, *ok, 7, None) == EINVAL and "unknown path" in qmv.last_error()
    assert f(9, *ok, qmv.PATH_AUTO, None) == EUNSUPPORTED
    # the common checks come first, whatever the path
    assert f(qmv.Q4_0, A, 8, 256, A, 256, 9, A, 8, qmv.PATH_MFMA, None) == EINVAL and "batch" in qmv.last_error()
    assert f(qmv.Q8_0, A + 2, 8, 256, A, 256, 2, A, 8, qmv.PATH_FMA, None) == EALIGN
    # shapes the matrix-core kernel does not take (no launch happens)
    for args in [(A, 8, 256, A, 256, 1, A, 8),          # batch 1
                 (A, 8, 224, A, 224, 2, A, 8),          # 7 blocks per row
                 (A + 4, 8, 256, A, 256, 2, A, 8),      # W not 16-byte aligned
                 (A, 8, 256, A + 4, 256, 2, A, 8),      # x not 16-byte aligned
                 (A, 8, 256, A, 258, 2, A, 8)]:         # ldx not a multiple of 4
        assert f(qmv.Q4_1, *args, qmv.PATH_MFMA, None) == EUNSUPPORTED, args
        assert "matrix-core" in qmv.last_error()


def test_matvec_xt_argument_errors(qmv):
    f = qmv.lib().qmv_matvec_xt
    ok = (A, 8, 256)
    tail = (256, 2, A, 8)
    assert f(qmv.Q4_0, *ok, A, 7, *tail, qmv.PATH_AUTO, None) == EINVAL and "activation type" in qmv.last_error()
    assert f(qmv.Q4_0, *ok, A, qmv.X_F16, *tail, 5, None) == EINVAL and "unknown path" in qmv.last_error()
    assert f(11, *ok, A, qmv.X_BF16, *tail, qmv.PATH_AUTO, None) == EUNSUPPORTED
    # x aligned to its element size: 2 bytes for 16-bit activations, 4 for fp32
    assert f(qmv.Q8_0, *ok, A + 1, qmv.X_F16, *tail, qmv.PATH_AUTO, None) == EALIGN
    assert "2-byte" in qmv.last_error()
    assert f(qmv.Q8_0, *ok, A + 2, qmv.X_F32, *tail, qmv.PATH_AUTO, None) == EALIGN
    # 8-byte vector alignment is only needed by the matrix-core path
    assert f(qmv.Q4_0, *ok, A + 2, qmv.X_BF16, *tail, qmv.PATH_MFMA, None) == EUNSUPPORTED
    assert f(qmv.Q4_0, A, 8, 256, A, qmv.X_F16, 255, 2, A, 8, qmv.PATH_FMA, None) == EINVAL   # ldx < n_cols


def test_int8_argument_errors(qmv):
    f = qmv.lib().qmv_i8_requant
    ok = dict(W=A, N=8, K=64, x=A, ldx=64, B=1, mult=A, shift=A, y=A, ldy=8)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["W"], a["N"], a["K"], a["x"], a["ldx"], a["B"], a["mult"], a["shift"], a["y"], a["ldy"], None)

    assert call(mult=0) == EINVAL
    assert call(K=40) == EINVAL and "multiple of 16" in qmv.last_error()
    assert call(K=131072, ldx=131072) == EINVAL
    assert call(B=9) == EINVAL
    assert call(ldy=7) == EINVAL
    assert call(W=A + 4) == EALIGN
    assert call(x=A + 8) == EALIGN
    assert call(ldx=72) == EALIGN
    assert call(shift=A + 2) == EALIGN


def test_int8_lut_argument_errors(qmv):
    f = qmv.lib().qmv_i8_requant_lut
    assert f(A, 8, 64, A, 64, 1, A, A, 0, A, 8, None) == EINVAL and "table" in qmv.last_error()
    assert f(A, 8, 40, A, 64, 1, A, A, A, A, 8, None) == EINVAL and "multiple of 16" in qmv.last_error()
    assert f(A, 8, 64, A + 8, 64, 1, A, A, A, A, 8, None) == EALIGN


def test_moe_swiglu_and_combine_argument_errors(qmv):
    sw = qmv.lib().qmv_moe_swiglu
    per = 2 * 16 * 2 * 18   # 2 x 16 rows of a 64-column Q4_0 expert
    assert sw(7, A, per, 4, 16, 64, A, 2, 2, A, 64, 0, A, None) == EUNSUPPORTED
    assert sw(1, A, per - 4, 4, 16, 64, A, 2, 2, A, 64, 0, A, None) == EINVAL and "expert_stride" in qmv.last_error()
    assert sw(1, A, per, 4, 16, 64, A, 9, 2, A, 64, 0, A, None) == EINVAL
    assert sw(1, A, per, 4, 16, 64, A, 2, 2, A, 64, 0, A + 2, None) == EALIGN
    cb = qmv.lib().qmv_moe_combine
    per = 16 * 2 * 18
    assert cb(7, A, per, 4, 16, 64, A, A, 2, 2, A, 128, 64, A, None) == EUNSUPPORTED
    assert cb(1, A, per, 4, 16, 64, A, 0, 2, 2, A, 128, 64, A, None) == EINVAL and "null" in qmv.last_error()
    assert cb(1, A, per, 4, 16, 64, A, A + 2, 2, 2, A, 128, 64, A, None) == EALIGN
    assert cb(1, A, per, 4, 16, 64, A, A, 2, 17, A, 128, 64, A, None) == EINVAL and "top_k" in qmv.last_error()
    assert cb(1, A, per, 4, 16, 64, A, A, 2, 2, A, 128, 32, A, None) == EINVAL


def test_moe_xt_argument_errors(qmv):
    per = 16 * 2 * 18
    for name in ("qmv_moe_xt", "qmv_moe_swiglu_xt"):
        f = getattr(qmv.lib(), name)
        p = per * (2 if "swiglu" in name else 1)
        assert f(1, A, p, 4, 16, 64, A, 2, 2, A, 7, 64, 0, A, None) == EINVAL and "activation type" in qmv.last_error()
        assert f(1, A, p, 4, 16, 64, A, 2, 2, A + 1, qmv.X_F16, 64, 0, A, None) == EALIGN
        assert "2-byte" in qmv.last_error()
        assert f(1, A, p, 4, 16, 64, A, 2, 2, A + 2, qmv.X_F32, 64, 0, A, None) == EALIGN
        assert f(9, A, p, 4, 16, 64, A, 2, 2, A, qmv.X_BF16, 64, 0, A, None) == EUNSUPPORTED


def test_moe_argument_errors(qmv):
    f = qmv.lib().qmv_moe
    per = 16 * 2 * 18   # 16 x 64 Q4_0 expert
    ok = dict(fmt=1, W=A, stride=per, E=4, N=16, K=64, ids=A, B=2, T=2, x=A, st_tok=64, st_slot=0, y=A)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["fmt"], a["W"], a["stride"], a["E"], a["N"], a["K"], a["ids"], a["B"], a["T"], a["x"],
                 a["st_tok"], a["st_slot"], a["y"], None)

    assert call(fmt=7) == EUNSUPPORTED
    assert call(ids=0) == EINVAL
    assert call(E=0) == EINVAL
    assert call(T=0) == EINVAL and call(T=17) == EINVAL
    assert call(B=9) == EINVAL
    assert call(stride=per - 4) == EINVAL
    assert call(stride=per + 2) == EINVAL
    assert call(st_tok=32) == EINVAL
    assert call(st_slot=32) == EINVAL
    assert call(y=A + 2) == EALIGN


def test_dequant_argument_errors(qmv):
    f = qmv.lib().qmv_dequant
    assert f(5, A, 4, 64, A, None) == EUNSUPPORTED
    assert f(0, 0, 4, 64, A, None) == EINVAL
    assert f(0, A, 4, 65, A, None) == EINVAL


def test_error_message_is_per_call(qmv):
    f = qmv.lib().qmv_q8_0
    assert f(A, 0, 64, A, 64, 1, A, 8, None) == EINVAL
    assert "n_rows" in qmv.last_error()
    assert f(A, 8, 64, A, 64, 12, A, 8, None) == EINVAL
    assert "batch" in qmv.last_error()


def test_python_binding_rejects_cpu_tensors(qmv):
    import torch
    W = torch.zeros(34 * 2, dtype=torch.uint8)
    x = torch.zeros(64, dtype=torch.float32)
    with pytest.raises(ValueError):
        qmv.qmv_q8_0(W, 1, 64, x)


def test_chain_argument_errors(qmv):
    import ctypes
    f = qmv.lib().qmv_chain

    def call(stages, ws=A, ws_bytes=qmv.CHAIN_WORKSPACE_BYTES, fmt=0):
        arr = (qmv.ChainStage * len(stages))(*stages)
        return f(fmt, ctypes.cast(arr, ctypes.c_void_p), len(stages), ws, ws_bytes, None)

    good = qmv.ChainStage(A, A, A, 16, 4096, 0, 0)
    assert call([good], fmt=9) == EUNSUPPORTED
    assert call([good], ws=0) == EINVAL
    assert call([good], ws_bytes=qmv.CHAIN_WORKSPACE_BYTES - 4) == EINVAL and "workspace" in qmv.last_error()
    assert call([good], ws=A + 2) == EALIGN
    assert call([qmv.ChainStage(A, A, A, 0, 4096, 0, 0)]) == EINVAL
    assert call([good, qmv.ChainStage(A, A, A, 16, 4100, 1, 0)]) == EINVAL and "stage 1" in qmv.last_error()
    assert call([qmv.ChainStage(A, A, A, 16, 65536, 0, 0)]) == EINVAL
    assert call([qmv.ChainStage(A, A + 2, A, 16, 4096, 0, 0)]) == EALIGN
    assert f(0, None, 1, A, qmv.CHAIN_WORKSPACE_BYTES, None) == EINVAL
    arr = (qmv.ChainStage * 1)(good)
    assert f(0, ctypes.cast(arr, ctypes.c_void_p), 0, A, qmv.CHAIN_WORKSPACE_BYTES, None) == EINVAL


def test_chain_noalloc_argument_errors(qmv):
    """Checked before the library looks up its barrier words (no GPU here)."""
    import ctypes
    f = qmv.lib().qmv_chain_noalloc
    arr = (qmv.ChainStage * 1)(qmv.ChainStage(A, A, A, 16, 4096, 0, 0))
    assert f(9, ctypes.cast(arr, ctypes.c_void_p), 1, None) == EUNSUPPORTED
    assert f(0, None, 1, None) == EINVAL and "null" in qmv.last_error()
    assert f(0, ctypes.cast(arr, ctypes.c_void_p), 0, None) == EINVAL and "n_stages" in qmv.last_error()


def test_stream_read_argument_errors(qmv):
    f = qmv.lib().qmv_stream_read
    cases = [
        ((0, 4096, A, 256, None), EINVAL, "null"),
        ((A, 4096, 0, 256, None), EINVAL, "null"),
        ((A, 0, A, 256, None), EINVAL, "multiple of 16"),
        ((A, 4100, A, 256, None), EINVAL, "multiple of 16"),
        ((A, 4096, A, 255, None), EINVAL, "out_words"),
        ((A + 8, 4096, A, 256, None), EALIGN, "aligned"),
        ((A, 4096, A + 2, 256, None), EALIGN, "aligned"),
    ]
    for args, code, msg in cases:
        assert f(*args) == code, args
        assert msg in qmv.last_error(), (args, qmv.last_error())
