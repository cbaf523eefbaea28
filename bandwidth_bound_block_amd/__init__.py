"""Block-quantized matrix x vector products for AMD MI355X (gfx950).

Python binding of ``libqmv.so`` (hand-written HIP, C ABI in
``include/qmv.h``).  This module only marshals arguments: it checks tensor
devices, dtypes and shapes, passes raw device pointers and the current HIP
stream to the library, and turns a non-OK return code into ``QmvError``.
Every step of the computation runs in the library's kernels; there is no
fallback of any kind, and importing this package fails loudly when the
library has not been built.

Entry points (same names as the C ABI):
  qmv_q8_0 / qmv_q4_0 / qmv_q4_1   float block-quantized matvec, batch 1..8
  qmv_q4_k                         the same for Q4_K super-blocks (256 weights, 144 bytes)
  qmv_q6_k                         the same for Q6_K super-blocks (256 weights, 210 bytes)
  qmv_matvec_path                  the same with the kernel family chosen
                                   (PATH_AUTO / PATH_FMA / PATH_MFMA)
  qmv_matvec_xt                    the same with fp32, fp16 or bf16 activations
  qmv_i8_requant                   int8 matvec + per-channel gemmlowp requant
  qmv_i8_requant_lut               the same through a frozen int8 lookup table
  qmv_moe                          grouped MoE expert matvec
  qmv_moe_xt                       the same with fp32, fp16 or bf16 activations
  qmv_moe_swiglu                   MoE gate||up with the SwiGLU step fused
  qmv_moe_swiglu_xt                the same with fp32, fp16 or bf16 activations
  qmv_moe_combine                  MoE down with the router-weighted combine
  qmv_dequant                      stored blocks -> fp32 (test/inspection aid)
  qmv_stream_read                  stream-read ceiling of the device (measurement aid)
  qmv_chain                        batch-1 matvec stages in one persistent launch
  qmv_chain_noalloc                the same with library-held barrier words (no workspace)
"""
import ctypes
import os

__all__ = ["QmvError", "qmv_q8_0", "qmv_q4_0", "qmv_q4_1", "qmv_q4_k", "qmv_q6_k", "qmv_matvec_path", "qmv_matvec_xt", "PATH_AUTO",
           "PATH_FMA", "PATH_MFMA", "X_F32", "X_F16", "X_BF16", "qmv_i8_requant", "qmv_i8_requant_lut",
           "qmv_moe", "qmv_moe_xt", "qmv_moe_swiglu", "qmv_moe_swiglu_xt", "qmv_moe_combine",
           "qmv_dequant", "qmv_stream_read", "qmv_chain", "qmv_chain_noalloc", "ChainStage", "CHAIN_WORKSPACE_BYTES", "abi_version", "last_error",
           "library_path", "lib", "Q8_0", "Q4_0", "Q4_1", "Q4_K", "Q6_K", "FORMATS", "BLOCK_BYTES", "row_bytes"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqmv.so")

Q8_0, Q4_0, Q4_1, Q4_K, Q6_K = 0, 1, 2, 3, 4
FORMATS = {"q8_0": Q8_0, "q4_0": Q4_0, "q4_1": Q4_1, "q4_k": Q4_K, "q6_k": Q6_K}
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q4_1: 20}      # per 32 weights
SUPER_BLOCK = {Q4_K: (256, 144), Q6_K: (256, 210)}   # (weights, bytes) per super-block


def row_bytes(fmt, n_cols):
    """Stored bytes of one row of n_cols weights (0 for an unknown format)."""
    f = FORMATS.get(fmt, fmt)
    if f in SUPER_BLOCK:
        w, b = SUPER_BLOCK[f]
        return n_cols // w * b
    return n_cols // 32 * BLOCK_BYTES.get(f, 0)


PATH_AUTO, PATH_FMA, PATH_MFMA = 0, 1, 2
X_F32, X_F16, X_BF16 = 0, 1, 2
_ERRORS = {1: "QMV_EINVAL", 2: "QMV_EALIGN", 3: "QMV_EUNSUPPORTED", 4: "QMV_EHIP"}
CHAIN_WORKSPACE_BYTES = 40960


class ChainStage(ctypes.Structure):
    """qmv_chain_stage of include/qmv.h."""
    _fields_ = [("W", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("n_rows", ctypes.c_int64), ("n_cols", ctypes.c_int64),
                ("wait", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class QmvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_ERRORS.get(code, code)}: {msg}")
        self.code = code


def library_path():
    return _LIB_PATH


def _open():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built: run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950) first")
    L = ctypes.CDLL(_LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    for name in ("qmv_q8_0", "qmv_q4_0", "qmv_q4_1", "qmv_q4_k", "qmv_q6_k"):
        f = getattr(L, name)
        f.argtypes = [P, i64, i64, P, i64, i32, P, i64, P]
        f.restype = i32
    L.qmv_matvec_path.argtypes = [ctypes.c_int, P, i64, i64, P, i64, i32, P, i64, i32, P]
    L.qmv_matvec_path.restype = i32
    L.qmv_matvec_xt.argtypes = [ctypes.c_int, P, i64, i64, P, i32, i64, i32, P, i64, i32, P]
    L.qmv_matvec_xt.restype = i32
    L.qmv_i8_requant.argtypes = [P, i64, i64, P, i64, i32, P, P, P, i64, P]
    L.qmv_i8_requant.restype = i32
    L.qmv_i8_requant_lut.argtypes = [P, i64, i64, P, i64, i32, P, P, P, P, i64, P]
    L.qmv_i8_requant_lut.restype = i32
    L.qmv_moe.argtypes = [ctypes.c_int, P, i64, i32, i64, i64, P, i32, i32, P, i64, i64, P, P]
    L.qmv_moe.restype = i32
    L.qmv_moe_swiglu.argtypes = [ctypes.c_int, P, i64, i32, i64, i64, P, i32, i32, P, i64, i64, P, P]
    L.qmv_moe_swiglu.restype = i32
    for name in ("qmv_moe_xt", "qmv_moe_swiglu_xt"):
        f = getattr(L, name)
        f.argtypes = [ctypes.c_int, P, i64, i32, i64, i64, P, i32, i32, P, i32, i64, i64, P, P]
        f.restype = i32
    L.qmv_moe_combine.argtypes = [ctypes.c_int, P, i64, i32, i64, i64, P, P, i32, i32, P, i64, i64, P, P]
    L.qmv_moe_combine.restype = i32
    L.qmv_dequant.argtypes = [ctypes.c_int, P, i64, i64, P, P]
    L.qmv_dequant.restype = i32
    L.qmv_stream_read.argtypes = [P, ctypes.c_size_t, P, ctypes.c_size_t, P]
    L.qmv_stream_read.restype = i32
    L.qmv_chain.argtypes = [ctypes.c_int, P, i32, P, ctypes.c_size_t, P]
    L.qmv_chain.restype = i32
    L.qmv_chain_noalloc.argtypes = [ctypes.c_int, P, i32, P]
    L.qmv_chain_noalloc.restype = i32
    L.qmv_last_error.argtypes = []
    L.qmv_last_error.restype = ctypes.c_char_p
    L.qmv_abi_version.argtypes = []
    L.qmv_abi_version.restype = i32
    return L


_lib = _open()


def lib():
    """The raw ctypes handle (C signatures as in include/qmv.h)."""
    return _lib


def last_error():
    return _lib.qmv_last_error().decode()


def abi_version():
    return int(_lib.qmv_abi_version())


def _check(rc):
    if rc != 0:
        raise QmvError(rc, last_error())


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _rows2d(t, name, K):
    """[K] or [B, K] with unit inner stride -> (tensor2d, B, ld)."""
    t2 = t.unsqueeze(0) if t.dim() == 1 else t
    if t2.dim() != 2 or t2.shape[1] != K or t2.stride(1) != 1:
        raise ValueError(f"{name} must be [K] or [B, K] with K={K} and unit inner stride")
    return t2, t2.shape[0], t2.stride(0) if t2.shape[0] > 1 else K


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _matvec(cfn, fmt, W, n_rows, n_cols, x, y, stream):
    torch = _torch()
    _dev(W, "W", torch.uint8)
    _dev(x, "x", torch.float32)
    need = n_rows * row_bytes(fmt, n_cols)
    if W.numel() * W.element_size() < need or not W.is_contiguous():
        raise ValueError(f"W must be contiguous and hold {need} bytes")
    x2, B, ldx = _rows2d(x, "x", n_cols)
    if y is None:
        y = torch.empty((B, n_rows), dtype=torch.float32, device=x.device)
    _dev(y, "y", torch.float32)
    y2, By, ldy = _rows2d(y, "y", n_rows)
    if By != B:
        raise ValueError("y must have as many rows as x")
    _check(cfn(W.data_ptr(), n_rows, n_cols, x2.data_ptr(), ldx, B, y2.data_ptr(), ldy, _stream(stream)))
    return y


def qmv_q8_0(W, n_rows, n_cols, x, y=None, stream=None):
    """y[b] = DEQ_Q8_0(W) @ x[b]; x float32 [K] or [B, K] (B <= 8)."""
    return _matvec(_lib.qmv_q8_0, Q8_0, W, n_rows, n_cols, x, y, stream)


def qmv_q4_0(W, n_rows, n_cols, x, y=None, stream=None):
    """y[b] = DEQ_Q4_0(W) @ x[b]; x float32 [K] or [B, K] (B <= 8)."""
    return _matvec(_lib.qmv_q4_0, Q4_0, W, n_rows, n_cols, x, y, stream)


def qmv_q4_1(W, n_rows, n_cols, x, y=None, stream=None):
    """y[b] = DEQ_Q4_1(W) @ x[b]; x float32 [K] or [B, K] (B <= 8)."""
    return _matvec(_lib.qmv_q4_1, Q4_1, W, n_rows, n_cols, x, y, stream)


def qmv_q4_k(W, n_rows, n_cols, x, y=None, stream=None):
    """y[b] = DEQ_Q4_K(W) @ x[b]; x float32 [K] or [B, K] (B <= 8), K a
    multiple of 256."""
    return _matvec(_lib.qmv_q4_k, Q4_K, W, n_rows, n_cols, x, y, stream)


def qmv_q6_k(W, n_rows, n_cols, x, y=None, stream=None):
    """y[b] = DEQ_Q6_K(W) @ x[b]; x float32 [K] or [B, K] (B <= 8), K a
    multiple of 256."""
    return _matvec(_lib.qmv_q6_k, Q6_K, W, n_rows, n_cols, x, y, stream)


def qmv_matvec_path(fmt, W, n_rows, n_cols, x, path, y=None, stream=None):
    """As qmv_q8_0/q4_0/q4_1/q4_k/q6_k for format fmt (Q8_0, Q4_0, Q4_1,
    Q4_K, Q6_K or its name) with the kernel family `path` (PATH_AUTO,
    PATH_FMA or PATH_MFMA)."""
    f = FORMATS.get(fmt, fmt)
    if f not in FORMATS.values():
        raise ValueError(f"unknown format {fmt!r}")

    def cfn(*a):
        return _lib.qmv_matvec_path(f, *a[:-1], path, a[-1])
    return _matvec(cfn, f, W, n_rows, n_cols, x, y, stream)


def qmv_matvec_xt(fmt, W, n_rows, n_cols, x, path=PATH_AUTO, y=None, stream=None):
    """As qmv_matvec_path with x float32, float16 or bfloat16 [K] or [B, K]
    (widened to fp32 exactly); y is float32."""
    torch = _torch()
    f = FORMATS.get(fmt, fmt)
    if f not in FORMATS.values():
        raise ValueError(f"unknown format {fmt!r}")
    xt = {torch.float32: X_F32, torch.float16: X_F16, torch.bfloat16: X_BF16}.get(x.dtype)
    if xt is None:
        raise ValueError(f"x must be float32, float16 or bfloat16 (got {x.dtype})")
    _dev(W, "W", torch.uint8)
    _dev(x, "x", x.dtype)
    need = n_rows * row_bytes(f, n_cols)
    if W.numel() * W.element_size() < need or not W.is_contiguous():
        raise ValueError(f"W must be contiguous and hold {need} bytes")
    x2, B, ldx = _rows2d(x, "x", n_cols)
    if y is None:
        y = torch.empty((B, n_rows), dtype=torch.float32, device=x.device)
    _dev(y, "y", torch.float32)
    y2, By, ldy = _rows2d(y, "y", n_rows)
    if By != B:
        raise ValueError("y must have as many rows as x")
    _check(_lib.qmv_matvec_xt(f, W.data_ptr(), n_rows, n_cols, x2.data_ptr(), xt, ldx, B, y2.data_ptr(), ldy, path,
                              _stream(stream)))
    return y


def qmv_i8_requant(W, x, mult, shift, y=None, stream=None):
    """int8 [N, K] weights x int8 [K] or [B, K] activations, per-row requant
    (mult, shift int32 [N]) -> int8 [B, N]."""
    return _i8(W, x, mult, shift, None, y, stream)


def qmv_i8_requant_lut(W, x, mult, shift, lut, y=None, stream=None):
    """qmv_i8_requant with the outputs mapped through a frozen table:
    y = lut[y_requant + 128]; lut int8 [256] on the GPU."""
    return _i8(W, x, mult, shift, lut, y, stream)


def _i8(W, x, mult, shift, lut, y, stream):
    torch = _torch()
    _dev(W, "W", torch.int8)
    _dev(x, "x", torch.int8)
    _dev(mult, "mult", torch.int32)
    _dev(shift, "shift", torch.int32)
    if W.dim() != 2 or not W.is_contiguous():
        raise ValueError("W must be a contiguous [N, K] tensor")
    N, K = W.shape
    if mult.numel() != N or shift.numel() != N or not mult.is_contiguous() or not shift.is_contiguous():
        raise ValueError("mult and shift must be contiguous [N]")
    x2, B, ldx = _rows2d(x, "x", K)
    if y is None:
        y = torch.empty((B, N), dtype=torch.int8, device=x.device)
    _dev(y, "y", torch.int8)
    y2, By, ldy = _rows2d(y, "y", N)
    if By != B:
        raise ValueError("y must have as many rows as x")
    if lut is None:
        _check(_lib.qmv_i8_requant(W.data_ptr(), N, K, x2.data_ptr(), ldx, B, mult.data_ptr(), shift.data_ptr(),
                                   y2.data_ptr(), ldy, _stream(stream)))
    else:
        _dev(lut, "lut", torch.int8)
        if lut.numel() != 256 or not lut.is_contiguous():
            raise ValueError("lut must be a contiguous int8 [256] tensor")
        _check(_lib.qmv_i8_requant_lut(W.data_ptr(), N, K, x2.data_ptr(), ldx, B, mult.data_ptr(), shift.data_ptr(),
                                       lut.data_ptr(), y2.data_ptr(), ldy, _stream(stream)))
    return y


def _moe_args(fmt, W_experts, expert_stride_bytes, n_experts, rows, n_cols, expert_ids, x, x_types=None):
    torch = _torch()
    fmt = _fmt(fmt)
    _dev(W_experts, "W_experts", torch.uint8)
    _dev(expert_ids, "expert_ids", torch.int32)
    if x_types is None:
        _dev(x, "x", torch.float32)
    else:
        _dev(x, "x", x.dtype)
        if x.dtype not in x_types:
            raise ValueError("x must be float32, float16 or bfloat16")
    if not W_experts.is_contiguous() or not expert_ids.is_contiguous() or not x.is_contiguous():
        raise ValueError("W_experts, expert_ids and x must be contiguous")
    if expert_ids.dim() != 2:
        raise ValueError("expert_ids must be [B, top_k]")
    B, T = expert_ids.shape
    if x.dim() == 2 and x.shape == (B, n_cols):
        st_tok, st_slot = n_cols, 0
    elif x.dim() == 3 and x.shape == (B, T, n_cols):
        st_tok, st_slot = T * n_cols, n_cols
    else:
        raise ValueError("x must be [B, K] or [B, top_k, K]")
    if W_experts.numel() < (n_experts - 1) * expert_stride_bytes + rows * row_bytes(fmt, n_cols):
        raise ValueError("W_experts is smaller than n_experts expert matrices")
    return torch, fmt, B, T, st_tok, st_slot


def _x_types(torch):
    return {torch.float32: X_F32, torch.float16: X_F16, torch.bfloat16: X_BF16}


def qmv_moe_xt(fmt, W_experts, expert_stride_bytes, n_experts, n_rows, n_cols, expert_ids, x, y=None, stream=None):
    """qmv_moe with x float32, float16 or bfloat16 ([B, K] or [B, top_k, K])."""
    torch = _torch()
    xt = _x_types(torch)
    torch, fmt, B, T, st_tok, st_slot = _moe_args(fmt, W_experts, expert_stride_bytes, n_experts, n_rows, n_cols,
                                                  expert_ids, x, xt)
    if y is None:
        y = torch.empty((B, T, n_rows), dtype=torch.float32, device=x.device)
    _dev(y, "y", torch.float32)
    if y.shape != (B, T, n_rows) or not y.is_contiguous():
        raise ValueError("y must be a contiguous [B, top_k, n_rows] tensor")
    _check(_lib.qmv_moe_xt(fmt, W_experts.data_ptr(), expert_stride_bytes, n_experts, n_rows, n_cols,
                           expert_ids.data_ptr(), B, T, x.data_ptr(), xt[x.dtype], st_tok, st_slot, y.data_ptr(),
                           _stream(stream)))
    return y


def qmv_moe_swiglu_xt(fmt, W_experts, expert_stride_bytes, n_experts, n_ff, n_cols, expert_ids, x, h=None,
                      stream=None):
    """qmv_moe_swiglu with x float32, float16 or bfloat16."""
    torch = _torch()
    xt = _x_types(torch)
    torch, fmt, B, T, st_tok, st_slot = _moe_args(fmt, W_experts, expert_stride_bytes, n_experts, 2 * n_ff, n_cols,
                                                  expert_ids, x, xt)
    if h is None:
        h = torch.empty((B, T, n_ff), dtype=torch.float32, device=x.device)
    _dev(h, "h", torch.float32)
    if h.shape != (B, T, n_ff) or not h.is_contiguous():
        raise ValueError("h must be a contiguous [B, top_k, n_ff] tensor")
    _check(_lib.qmv_moe_swiglu_xt(fmt, W_experts.data_ptr(), expert_stride_bytes, n_experts, n_ff, n_cols,
                                  expert_ids.data_ptr(), B, T, x.data_ptr(), xt[x.dtype], st_tok, st_slot,
                                  h.data_ptr(), _stream(stream)))
    return h


def qmv_moe_swiglu(fmt, W_experts, expert_stride_bytes, n_experts, n_ff, n_cols, expert_ids, x, h=None,
                   stream=None):
    """MoE gate||up with SwiGLU: every expert holds 2*n_ff rows (gate rows,
    then up rows); returns h float32 [B, top_k, n_ff] = SiLU(gate x) * (up x).
    x as qmv_moe."""
    torch, fmt, B, T, st_tok, st_slot = _moe_args(fmt, W_experts, expert_stride_bytes, n_experts, 2 * n_ff, n_cols,
                                                  expert_ids, x)
    if h is None:
        h = torch.empty((B, T, n_ff), dtype=torch.float32, device=x.device)
    _dev(h, "h", torch.float32)
    if h.shape != (B, T, n_ff) or not h.is_contiguous():
        raise ValueError("h must be a contiguous [B, top_k, n_ff] tensor")
    _check(_lib.qmv_moe_swiglu(fmt, W_experts.data_ptr(), expert_stride_bytes, n_experts, n_ff, n_cols,
                               expert_ids.data_ptr(), B, T, x.data_ptr(), st_tok, st_slot, h.data_ptr(),
                               _stream(stream)))
    return h


def qmv_moe_combine(fmt, W_experts, expert_stride_bytes, n_experts, n_rows, n_cols, expert_ids, weights, x,
                    out=None, stream=None):
    """MoE down with the router-weighted combine: out float32 [B, n_rows] =
    sum_s weights[b, s] * DEQ(W_{ids[b,s]}) x_{b,s}.  weights float32
    [B, top_k] on the GPU; x as qmv_moe."""
    torch, fmt, B, T, st_tok, st_slot = _moe_args(fmt, W_experts, expert_stride_bytes, n_experts, n_rows, n_cols,
                                                  expert_ids, x)
    _dev(weights, "weights", torch.float32)
    if weights.shape != (B, T) or not weights.is_contiguous():
        raise ValueError("weights must be a contiguous [B, top_k] tensor")
    if out is None:
        out = torch.empty((B, n_rows), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if out.shape != (B, n_rows) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, n_rows] tensor")
    _check(_lib.qmv_moe_combine(fmt, W_experts.data_ptr(), expert_stride_bytes, n_experts, n_rows, n_cols,
                                expert_ids.data_ptr(), weights.data_ptr(), B, T, x.data_ptr(), st_tok, st_slot,
                                out.data_ptr(), _stream(stream)))
    return out


def qmv_moe(fmt, W_experts, expert_stride_bytes, n_experts, n_rows, n_cols, expert_ids, x, y=None,
            stream=None):
    """Grouped MoE expert matvec.

    expert_ids: int32 [B, top_k] on the GPU.  x: float32 [B, K] (one input per
    token, gate/up) or [B, top_k, K] (one input per token and slot, down).
    Returns y float32 [B, top_k, n_rows]."""
    torch, fmt, B, T, st_tok, st_slot = _moe_args(fmt, W_experts, expert_stride_bytes, n_experts, n_rows, n_cols,
                                                  expert_ids, x)
    if y is None:
        y = torch.empty((B, T, n_rows), dtype=torch.float32, device=x.device)
    _dev(y, "y", torch.float32)
    if y.shape != (B, T, n_rows) or not y.is_contiguous():
        raise ValueError("y must be a contiguous [B, top_k, n_rows] tensor")
    _check(_lib.qmv_moe(fmt, W_experts.data_ptr(), expert_stride_bytes, n_experts, n_rows, n_cols,
                        expert_ids.data_ptr(), B, T, x.data_ptr(), st_tok, st_slot, y.data_ptr(),
                        _stream(stream)))
    return y


def qmv_dequant(fmt, W, n_rows, n_cols, out=None, stream=None):
    """fp32 [n_rows, n_cols] values of the stored blocks."""
    torch = _torch()
    fmt = _fmt(fmt)
    _dev(W, "W", torch.uint8)
    if out is None:
        out = torch.empty((n_rows, n_cols), dtype=torch.float32, device=W.device)
    _dev(out, "out", torch.float32)
    if out.shape != (n_rows, n_cols) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [n_rows, n_cols] tensor")
    _check(_lib.qmv_dequant(fmt, W.data_ptr(), n_rows, n_cols, out.data_ptr(), _stream(stream)))
    return out


def qmv_stream_read(buf, out, stream=None):
    """Reads the uint8 GPU tensor buf once (16-byte non-temporal loads); each
    launched thread writes the XOR of the words it read into out (uint32,
    >= 256 words).  A measurement aid: the device's stream-read ceiling."""
    torch = _torch()
    _dev(buf, "buf", torch.uint8)
    _dev(out, "out", torch.int32)
    if not buf.is_contiguous() or not out.is_contiguous():
        raise ValueError("buf and out must be contiguous")
    _check(_lib.qmv_stream_read(buf.data_ptr(), buf.numel(), out.data_ptr(), out.numel(), _stream(stream)))
    return out


def chain_stages(stages, fmt=None):
    """[(W, n_rows, n_cols, x, y, wait), ...] of GPU tensors -> ctypes array.
    With fmt, each W is checked to hold its n_rows x n_cols blocks."""
    torch = _torch()
    arr = (ChainStage * len(stages))()
    for i, (W, n_rows, n_cols, x, y, wait) in enumerate(stages):
        _dev(W, "W", torch.uint8)
        rb = row_bytes(_fmt(fmt), n_cols) if fmt is not None else 0   # unknown fmt: the library rejects it
        if rb:
            need = n_rows * rb
            if W.numel() < need or not W.is_contiguous():
                raise ValueError(f"stage {i}: W must be contiguous and hold {need} bytes")
        _dev(x, "x", torch.float32)
        _dev(y, "y", torch.float32)
        if x.numel() < n_cols or y.numel() < n_rows or not x.is_contiguous() or not y.is_contiguous():
            raise ValueError(f"stage {i}: x must hold n_cols and y n_rows contiguous floats")
        arr[i] = ChainStage(W.data_ptr(), x.data_ptr(), y.data_ptr(), n_rows, n_cols, 1 if wait else 0, 0)
    return arr


def qmv_chain(fmt, stages, workspace, stream=None):
    """Runs batch-1 matvec stages in one call (see qmv.h): one persistent
    launch for the 32-weight formats, stage groups as launches of their own
    for Q4_K and Q6_K.

    stages: list of (W, n_rows, n_cols, x, y, wait) with GPU tensors, or a
    ctypes array from chain_stages().  workspace: uint8 GPU tensor of at
    least CHAIN_WORKSPACE_BYTES, zero-filled before its first use."""
    torch = _torch()
    _dev(workspace, "workspace", torch.uint8)
    arr = stages if isinstance(stages, ctypes.Array) else chain_stages(stages, fmt)
    _check(_lib.qmv_chain(_fmt(fmt), ctypes.cast(arr, ctypes.c_void_p), len(arr), workspace.data_ptr(),
                          workspace.numel(), _stream(stream)))


def qmv_chain_noalloc(fmt, stages, stream=None):
    """qmv_chain with the barrier words held by the library (no workspace
    argument, nothing allocated; see qmv.h).  stages as for qmv_chain."""
    arr = stages if isinstance(stages, ctypes.Array) else chain_stages(stages, fmt)
    _check(_lib.qmv_chain_noalloc(_fmt(fmt), ctypes.cast(arr, ctypes.c_void_p), len(arr), _stream(stream)))
