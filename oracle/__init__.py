"""The oracle: plain CPU fp64 reference for the block-quantized matvec path.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``bandwidth_bound_block_amd``) never imports it, and the two share no
code: this package wraps ``qmv_oracle.c`` (plain C99, double precision,
compiled with gcc) and ``py_int.py`` (an independent big-integer mirror of
the integer semantics).

Sources (the pages collected on the subject):
  * "One Native Stack for Private, Continuously-Learning AI", Sec. "The
    Unified Quant Core" (formats Q8_0 34 B/32, Q4_0 18 B/32, Q4_K 144 B/256
    and Q6_K 210 B/256, the last two without their layouts; one decoder per
    format) and the QLoRA Lemma (y_i = sum_j DEQ(W)_ij x_j).
  * "Economical Serving and the hanzo.ai Platform", Sec. 2.1 (one stream of
    the weights per token) and Sec. 2.2 (block decoder + traits record).
  * "Blue -- porting zen-nano (Qwen3-0.6B) to deterministic on-chain
    inference", "Quantization recipe" (int8 matvec, per-output-channel
    SaturatingRoundingDoublingHighMul then RoundingDivideByPOT to int8).

Parity status: every function is pinned by the ``-m "not gpu"`` tests.  The
Q4_K and Q6_K layouts are readings (ggml's); agreement with ggml itself is
parity unpinned.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC_PATH = os.path.join(_HERE, "qmv_oracle.c")

Q8_0, Q4_0, Q4_1, Q4_K, Q6_K = 0, 1, 2, 3, 4
FORMATS = {"q8_0": Q8_0, "q4_0": Q4_0, "q4_1": Q4_1, "q4_k": Q4_K, "q6_k": Q6_K}
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q4_1: 20}      # per 32 weights
SUPER_BLOCK = {Q4_K: (256, 144), Q6_K: (256, 210)}   # (weights, bytes) per super-block


def row_bytes(fmt, K):
    """Stored bytes of one row of K weights."""
    fmt = _fmt(fmt)
    if fmt in SUPER_BLOCK:
        w, b = SUPER_BLOCK[fmt]
        assert K % w == 0
        return K // w * b
    assert K % 32 == 0
    return K // 32 * BLOCK_BYTES[fmt]

_lib = None


def build(force=False):
    """Compile qmv_oracle.c with gcc (no fast-math, no FMA contraction)."""
    import subprocess
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-Wextra",
                               "-ffp-contract=off", "-fno-fast-math", "-shared",
                               "-fPIC", "-o", tmp, _SRC_PATH, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        lib.qo_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.qo_f16_to_f64.restype = ctypes.c_double
        lib.qo_dequant.argtypes = [ctypes.c_int, P, i64, i64, P]
        lib.qo_matvec.argtypes = [ctypes.c_int, P, i64, i64, P, i64, i32, P, i64, P, P, i64]
        lib.qo_srdhm.argtypes = [i32, i32]
        lib.qo_srdhm.restype = i32
        lib.qo_rdbpot.argtypes = [i32, i32]
        lib.qo_rdbpot.restype = i32
        lib.qo_requant.argtypes = [i32, i32, i32]
        lib.qo_requant.restype = i32
        lib.qo_matvec_i8.argtypes = [P, i64, i64, P, i64, i32, P, P, P, i64, P, P, i64]
        lib.qo_moe.argtypes = [ctypes.c_int, P, i64, i32, i64, i64, P, i32, i32, P,
                               i64, i64, P, i64, P, P, i64]
        lib.qo_matvec_i8_lut.argtypes = [P, i64, i64, P, i64, i32, P, P, P, P, i64, P, P, i64]
        lib.qo_silu.argtypes = [ctypes.c_double]
        lib.qo_silu.restype = ctypes.c_double
        lib.qo_moe_swiglu.argtypes = [ctypes.c_int, P, i64, i32, i64, i64, P, i32, i32, P,
                                      i64, i64, P, i64, P, P, P, P, P, i64]
        lib.qo_moe_combine.argtypes = [ctypes.c_int, P, i64, i32, i64, i64, P, P, i32, i32, P,
                                       i64, i64, P, i64, P, P, i64]
        for f in ("qo_dequant", "qo_matvec", "qo_matvec_i8", "qo_moe", "qo_matvec_i8_lut",
                  "qo_moe_swiglu", "qo_moe_combine"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def f16_to_f64(h):
    """IEEE binary16 bit pattern(s) -> float64, decoded from the definition."""
    lib = _load()
    h = np.asarray(h, dtype=np.uint16)
    flat = h.reshape(-1)
    out = np.empty(flat.shape, dtype=np.float64)
    for i, v in enumerate(flat):
        out[i] = lib.qo_f16_to_f64(int(v))
    return out.reshape(h.shape)


def dequant(fmt, W, N, K):
    """DEQ(W) as an exact float64 [N, K] array (W: packed block bytes)."""
    lib = _load()
    W = np.ascontiguousarray(W, dtype=np.uint8)
    fmt = _fmt(fmt)
    assert W.size == N * row_bytes(fmt, K)
    out = np.empty((N, K), dtype=np.float64)
    _check(lib.qo_dequant(fmt, _ptr(W), N, K, _ptr(out)), "dequant")
    return out


def matvec(fmt, W, N, K, x, rows=None):
    """Float matvec y = DEQ(W) x, per batch column, in fp64.

    x: float32 [B, K].  rows: optional int64 row indices (sampled parity).
    Returns (y, S), each float64 [B, n_rows], S = sum_j |DEQ(W)_ij x_j|.
    """
    lib = _load()
    fmt = _fmt(fmt)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    B = x.shape[0]
    assert x.shape[1] == K and W.size == N * row_bytes(fmt, K)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
    else:
        n = N
    y = np.empty((B, n), dtype=np.float64)
    S = np.empty((B, n), dtype=np.float64)
    _check(lib.qo_matvec(fmt, _ptr(W), N, K, _ptr(x), K, B, _ptr(rows), n,
                         _ptr(y), _ptr(S), n), "matvec")
    return y, S


def srdhm(a, b):
    """SaturatingRoundingDoublingHighMul on int32 scalars (C oracle)."""
    return int(_load().qo_srdhm(int(a), int(b)))


def rdbpot(x, e):
    """RoundingDivideByPOT on an int32 scalar (C oracle)."""
    return int(_load().qo_rdbpot(int(x), int(e)))


def requant(acc, mult, shift):
    return int(_load().qo_requant(int(acc), int(mult), int(shift)))


def matvec_i8(W, x, mult, shift, rows=None):
    """int8 matvec + per-row requant.  W int8 [N, K]; x int8 [B, K].

    Returns (acc int64 [B, n], y int8 [B, n]).  Raises OverflowError when an
    accumulator leaves int32.
    """
    lib = _load()
    W = np.ascontiguousarray(W, dtype=np.int8)
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.int8)
    mult = np.ascontiguousarray(mult, dtype=np.int32)
    shift = np.ascontiguousarray(shift, dtype=np.int32)
    N, K = W.shape
    B = x.shape[0]
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
    else:
        n = N
    acc = np.empty((B, n), dtype=np.int64)
    y = np.empty((B, n), dtype=np.int8)
    rc = lib.qo_matvec_i8(_ptr(W), N, K, _ptr(x), K, B, _ptr(mult), _ptr(shift),
                          _ptr(rows), n, _ptr(acc), _ptr(y), n)
    if rc == 3:
        raise OverflowError("int8 accumulator does not fit int32")
    _check(rc, "matvec_i8")
    return acc, y


def moe(fmt, W_experts, expert_stride, n_experts, N, K, ids, x_tokens, x_slots=None,
        rows=None):
    """Naive MoE expert matvec: y[b, s] = DEQ(W_{ids[b,s]}) x_{b,s}.

    W_experts: uint8 bytes, expert e at byte offset e*expert_stride.
    ids: int32 [batch, top_k].  x_tokens: float32 [batch, K] used by every
    slot (gate/up) unless x_slots (float32 [batch, top_k, K], down) is given.
    Returns (y, S), float64 [batch, top_k, n_rows].
    """
    lib = _load()
    fmt = _fmt(fmt)
    W_experts = np.ascontiguousarray(W_experts, dtype=np.uint8)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    batch, top_k = ids.shape
    if x_slots is not None:
        xs = np.ascontiguousarray(x_slots, dtype=np.float32)
        assert xs.shape == (batch, top_k, K)
        st_tok, st_slot = top_k * K, K
    else:
        xs = np.ascontiguousarray(x_tokens, dtype=np.float32)
        assert xs.shape == (batch, K)
        st_tok, st_slot = K, 0
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
    else:
        n = N
    y = np.empty((batch, top_k, n), dtype=np.float64)
    S = np.empty((batch, top_k, n), dtype=np.float64)
    _check(lib.qo_moe(fmt, _ptr(W_experts), expert_stride, n_experts, N, K, _ptr(ids),
                      batch, top_k, _ptr(xs), st_tok, st_slot, _ptr(rows), n,
                      _ptr(y), _ptr(S), n), "moe")
    return y, S


def matvec_i8_lut(W, x, mult, shift, lut, rows=None):
    """matvec_i8 with the requantized outputs mapped through a frozen table:
    y = lut[y_requant + 128].  lut: int8 [256].  Returns (acc, y) like
    matvec_i8."""
    lib = _load()
    W = np.ascontiguousarray(W, dtype=np.int8)
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.int8)
    mult = np.ascontiguousarray(mult, dtype=np.int32)
    shift = np.ascontiguousarray(shift, dtype=np.int32)
    lut = np.ascontiguousarray(lut, dtype=np.int8)
    assert lut.shape == (256,)
    N, K = W.shape
    B = x.shape[0]
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
    else:
        n = N
    acc = np.empty((B, n), dtype=np.int64)
    y = np.empty((B, n), dtype=np.int8)
    rc = lib.qo_matvec_i8_lut(_ptr(W), N, K, _ptr(x), K, B, _ptr(mult), _ptr(shift), _ptr(lut),
                              _ptr(rows), n, _ptr(acc), _ptr(y), n)
    if rc == 3:
        raise OverflowError("int8 accumulator does not fit int32")
    _check(rc, "matvec_i8_lut")
    return acc, y


def silu(z):
    """SiLU(z) = z / (1 + e^-z), fp64 (C oracle)."""
    return float(_load().qo_silu(float(z)))


def _moe_x(x_tokens, x_slots, batch, top_k, K):
    if x_slots is not None:
        xs = np.ascontiguousarray(x_slots, dtype=np.float32)
        assert xs.shape == (batch, top_k, K)
        return xs, top_k * K, K
    xs = np.ascontiguousarray(x_tokens, dtype=np.float32)
    assert xs.shape == (batch, K)
    return xs, K, 0


def moe_swiglu(fmt, W_experts, expert_stride, n_experts, F, K, ids, x_tokens, x_slots=None, rows=None):
    """MoE gate/up with SwiGLU: every expert holds 2F rows (gate rows, then up
    rows); h[b, s, i] = SiLU(g) * u with g, u the gate and up rows' matvecs.

    Returns (h, g, u, Sg, Su), float64 [batch, top_k, n_rows]."""
    lib = _load()
    fmt = _fmt(fmt)
    W_experts = np.ascontiguousarray(W_experts, dtype=np.uint8)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    batch, top_k = ids.shape
    xs, st_tok, st_slot = _moe_x(x_tokens, x_slots, batch, top_k, K)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
    else:
        n = F
    out = [np.empty((batch, top_k, n), dtype=np.float64) for _ in range(5)]
    _check(lib.qo_moe_swiglu(fmt, _ptr(W_experts), expert_stride, n_experts, F, K, _ptr(ids), batch, top_k,
                             _ptr(xs), st_tok, st_slot, _ptr(rows), n, *[_ptr(a) for a in out], n), "moe_swiglu")
    return tuple(out)


def moe_combine(fmt, W_experts, expert_stride, n_experts, N, K, ids, weights, x_tokens=None, x_slots=None,
                rows=None):
    """MoE down projection with the router-weighted combine:
    out[b, i] = sum_s w[b, s] * (DEQ(W_{ids[b,s]}) x_{b,s})_i.

    weights: float32 [batch, top_k].  Returns (out, S), float64 [batch, n_rows],
    S[b, i] = sum_s |w[b, s]| * sum_j |DEQ(W)_ij x_j|."""
    lib = _load()
    fmt = _fmt(fmt)
    W_experts = np.ascontiguousarray(W_experts, dtype=np.uint8)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    batch, top_k = ids.shape
    w = np.ascontiguousarray(weights, dtype=np.float32)
    assert w.shape == (batch, top_k)
    xs, st_tok, st_slot = _moe_x(x_tokens, x_slots, batch, top_k, K)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
    else:
        n = N
    out = np.empty((batch, n), dtype=np.float64)
    S = np.empty((batch, n), dtype=np.float64)
    _check(lib.qo_moe_combine(fmt, _ptr(W_experts), expert_stride, n_experts, N, K, _ptr(ids), _ptr(w), batch,
                              top_k, _ptr(xs), st_tok, st_slot, _ptr(rows), n, _ptr(out), _ptr(S), n),
           "moe_combine")
    return out, S
