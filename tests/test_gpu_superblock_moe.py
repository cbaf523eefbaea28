"""MoE experts stored as Q4_K or Q6_K super-blocks (qmv_moe, qmv_moe_xt,
and the fused qmv_moe_swiglu / _xt and qmv_moe_combine) through the C ABI
on an MI355X, against the oracle's per-(token, slot) loop.

Each (token, slot) pair is one grid row of the super-block kernel.  Shapes
are the 30B-A3B-style experts (gate||up 1536 x 2048 with one input per
token, down 2048 x 768 with one input per token and slot: 3 super-blocks
per row), with fewer experts than the workload's 128 so the encoding stays
quick; top-8 distinct ids per token, batch 1, 2 and 8.  Also: expert
strides larger than a matrix, shared and duplicate ids, invalid ids (quiet
NaN rows, the others exact), 16-bit activations (bitwise the fp32 call on
the widened values), zero-heavy experts, and bitwise repeatability.
|y_gpu - y| <= 1e-4 * S + 1e-6 per output.
"""
import functools
import sys

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

FMTS = ["q4_k", "q6_k"]
E, T = 32, 8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    import bandwidth_bound_block_amd as qmv
    assert torch.cuda.is_available()
    return torch, qmv


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def assert_tol(y, yr, S, what=""):
    err = np.abs(np.asarray(y, dtype=np.float64) - yr)
    tol = 1e-4 * S + 1e-6
    bad = err > tol
    assert not np.any(bad), (what, int(bad.sum()), float((err / tol).max()))


@functools.lru_cache(maxsize=None)
def experts(fmt, kind, N, K):
    """E experts of N x K, contiguous (stride = one matrix)."""
    return wl.quant_weights(fmt, f"t/sbmoe/{fmt}/{kind}", E * N, K).reshape(-1)


def run(env, fmt, Wall, stride, N, K, ids, x, x_type=None):
    torch, qmv = env
    Wd, idd, xd = dev(torch, Wall), dev(torch, ids), dev(torch, x)
    if x_type is not None:
        xd = xd.to(x_type)
        y = qmv.qmv_moe_xt(fmt, Wd, stride, E, N, K, idd, xd)
    else:
        y = qmv.qmv_moe(fmt, Wd, stride, E, N, K, idd, xd)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [1, 2, 8])
def test_superblock_moe_30b_shapes(env, fmt, B):
    H, F = wl.MOE_HIDDEN, wl.MOE_FFN
    ids = wl.moe_ids(f"t/sbmoe/ids/{B}", B, T, E)
    for kind, N, K in [("gate_up", 2 * F, H), ("down", H, F)]:
        say(f"{fmt} moe {kind} B={B}")
        Wall = experts(fmt, kind, N, K)
        stride = wl.block_bytes(fmt, N, K)
        if kind == "gate_up":
            x = wl.activations(f"t/sbmoe/x/{kind}/{B}", B, K)
            yr, S = oracle.moe(fmt, Wall, stride, E, N, K, ids, x)
        else:
            x = wl.activations(f"t/sbmoe/x/{kind}/{B}", B * T, K).reshape(B, T, K)
            yr, S = oracle.moe(fmt, Wall, stride, E, N, K, ids, None, x_slots=x)
        y = run(env, fmt, Wall, stride, N, K, ids, x)
        assert_tol(y, yr, S, (fmt, kind, B))


@pytest.mark.parametrize("fmt", FMTS)
def test_superblock_moe_routing_edges(env, fmt):
    """Padded expert strides, every token on the same experts, duplicate ids
    within a token, and invalid ids (-1, n_experts): quiet NaN rows for the
    invalid pairs, every other pair within the bound; two calls bitwise
    equal."""
    torch, qmv = env
    N, K = 300, 1024
    per = wl.block_bytes(fmt, N, K)
    stride = per + 256                       # a multiple of 16 (and of 4)
    Wm = wl.quant_weights(fmt, f"t/sbmoe/edge/{fmt}", E * N, K).reshape(E, per)
    Wall = np.zeros((E, stride), dtype=np.uint8)
    Wall[:, :per] = Wm
    Wall = Wall.reshape(-1)
    B = 3
    ids = np.array([[0, 1, 2, 3, 4, 5, 6, 7], [0, 1, 2, 3, 4, 5, 6, 7], [31, 31, 5, 5, 0, 9, 9, 30]], dtype=np.int32)
    x = wl.activations(f"t/sbmoe/edge/x/{fmt}", B, K)
    yr, S = oracle.moe(fmt, Wall, stride, E, N, K, ids, x)
    y = run(env, fmt, Wall, stride, N, K, ids, x)
    assert_tol(y, yr, S, (fmt, "edges"))
    y2 = run(env, fmt, Wall, stride, N, K, ids, x)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    bad = ids.copy()
    bad[0, 3] = -1
    bad[2, 7] = E
    yb = run(env, fmt, Wall, stride, N, K, bad, x)
    assert np.all(np.isnan(yb[0, 3])) and np.all(np.isnan(yb[2, 7]))
    ok = np.ones((B, T), dtype=bool)
    ok[0, 3] = ok[2, 7] = False
    assert np.array_equal(yb[ok].view(np.uint32), y[ok].view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
def test_superblock_moe_x16_and_zero_heavy(env, fmt):
    """fp16 / bf16 activations give bitwise the fp32 call on the widened
    values; zero-heavy experts stay within the bound."""
    torch, qmv = env
    N, K, B = 256, 2048, 2
    Wall = experts(fmt, "x16", N, K)
    stride = wl.block_bytes(fmt, N, K)
    ids = wl.moe_ids(f"t/sbmoe/x16/{fmt}", B, T, E)
    x = wl.activations(f"t/sbmoe/x16/x/{fmt}", B, K)
    for kind, tt in [("f16", torch.float16), ("bf16", torch.bfloat16)]:
        y16 = run(env, fmt, Wall, stride, N, K, ids, x, x_type=tt)
        xw = torch.from_numpy(x).to(tt).float().numpy()
        y32 = run(env, fmt, Wall, stride, N, K, ids, xw)
        assert np.array_equal(y16.view(np.uint32), y32.view(np.uint32)), kind
    Wz, xz = wl.zero_heavy(fmt, f"t/sbmoe/zh/{fmt}", E * N, K, B=B)
    Wz = Wz.reshape(-1)
    yr, S = oracle.moe(fmt, Wz, stride, E, N, K, ids, xz)
    y = run(env, fmt, Wz, stride, N, K, ids, xz)
    assert_tol(y, yr, S, (fmt, "zero-heavy"))


# ------------------------------------------------------------------ fused SwiGLU
def swiglu_bound(h, g, u, Sg, Su):
    """|h_gpu - h| for h = SiLU(g) u from fp32 g, u within the matvec bound
    (tg, tu): |SiLU'| <= 1.1, so |dh| <= 1.1 tg (|u| + tu) + (|SiLU(g)| +
    1.1 tg) tu, plus the fp32 epilogue (a few ulps of h)."""
    tg, tu = 1e-4 * Sg + 1e-6, 1e-4 * Su + 1e-6
    sg = np.abs(g / (1.0 + np.exp(-g)))
    return 1.1 * tg * (np.abs(u) + tu) + (sg + 1.1 * tg) * tu + 2.0 ** -20 * np.abs(h) + 1e-30


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [1, 2, 8])
def test_superblock_moe_swiglu_30b_shapes(env, fmt, B):
    """Super-block experts of gate||up 1536 x 2048 (gate rows, then up rows), top-8
    per token: h against the oracle within the propagated bound on sampled
    rows, and the gate and up sums those of qmv_moe on the same experts (h
    == SiLU(g) u up to the epilogue's rounding)."""
    torch, qmv = env
    H, F = wl.MOE_HIDDEN, wl.MOE_FFN
    Wall = experts(fmt, "gate_up", 2 * F, H)
    stride = wl.block_bytes(fmt, 2 * F, H)
    ids = wl.moe_ids(f"t/sbmoe/sw/ids/{B}", B, T, E)
    x = wl.activations(f"t/sbmoe/sw/x/{B}", B, H)
    say(f"{fmt} moe swiglu B={B}")
    Wd, idd, xd = dev(torch, Wall), dev(torch, ids), dev(torch, x)
    h = qmv.qmv_moe_swiglu(fmt, Wd, stride, E, F, H, idd, xd)
    y = qmv.qmv_moe(fmt, Wd, stride, E, 2 * F, H, idd, xd)
    torch.cuda.synchronize()
    h, y = h.cpu().numpy(), y.cpu().numpy().astype(np.float64)
    rows = np.sort(np.random.default_rng(B).choice(F, size=96, replace=False))
    hr, g, u, Sg, Su = oracle.moe_swiglu(fmt, Wall, stride, E, F, H, ids, x, rows=rows)
    err = np.abs(h[:, :, rows].astype(np.float64) - hr)
    bound = swiglu_bound(hr, g, u, Sg, Su)
    assert np.all(err <= bound), float((err / bound).max())
    g32, u32 = y[:, :, :F], y[:, :, F:]
    href = g32 / (1.0 + np.exp(-g32)) * u32
    assert np.all(np.abs(h - href) <= 2.0 ** -21 * np.abs(href) + 1e-37)


@pytest.mark.parametrize("fmt", FMTS)
def test_superblock_moe_swiglu_edges(env, fmt):
    """Padded strides, duplicate and invalid ids (quiet NaN rows, the others
    within the bound), per-slot inputs, 16-bit activations (bitwise the fp32
    call on the widened values), a ragged row count."""
    torch, qmv = env
    F, K = 300, 1024
    per = wl.block_bytes(fmt, 2 * F, K)
    stride = per + 512
    Wm = wl.quant_weights(fmt, "t/sbmoe/swedge", E * 2 * F, K).reshape(E, per)
    Wall = np.zeros((E, stride), dtype=np.uint8)
    Wall[:, :per] = Wm
    Wall = Wall.reshape(-1)
    ids = np.array([[0, 1, 2, 3, 4, 5, 6, 7], [31, 31, 5, 5, 0, 9, -1, 30], [3, 1, 4, 1, 5, 9, 2, E]],
                   dtype=np.int32)
    B = ids.shape[0]
    x = wl.activations("t/sbmoe/swedge/x", B, K)
    Wd, idd = dev(torch, Wall), dev(torch, ids)
    say(f"{fmt} moe swiglu edges")
    h = qmv.qmv_moe_swiglu(fmt, Wd, stride, E, F, K, idd, dev(torch, x))
    torch.cuda.synchronize()
    h = h.cpu().numpy()
    valid = (ids >= 0) & (ids < E)
    assert np.all(np.isnan(h[~valid])) and not np.any(np.isnan(h[valid]))
    hr, g, u, Sg, Su = oracle.moe_swiglu(fmt, Wall, stride, E, F, K, np.where(valid, ids, 0).astype(np.int32), x)
    err = np.abs(h[valid].astype(np.float64) - hr[valid])
    assert np.all(err <= swiglu_bound(hr[valid], g[valid], u[valid], Sg[valid], Su[valid]))
    for kind, tt in [("f16", torch.float16), ("bf16", torch.bfloat16)]:
        xh = dev(torch, x).to(tt)
        h16 = qmv.qmv_moe_swiglu_xt(fmt, Wd, stride, E, F, K, idd, xh)
        h32 = qmv.qmv_moe_swiglu(fmt, Wd, stride, E, F, K, idd, xh.float())
        torch.cuda.synchronize()
        assert torch.equal(h16.view(torch.int32), h32.view(torch.int32)), kind
    # one input per token and slot
    xs = wl.activations("t/sbmoe/swedge/xs", B * T, K).reshape(B, T, K)
    hs = qmv.qmv_moe_swiglu(fmt, Wd, stride, E, F, K, idd, dev(torch, xs))
    torch.cuda.synchronize()
    hs = hs.cpu().numpy()
    hr, g, u, Sg, Su = oracle.moe_swiglu(fmt, Wall, stride, E, F, K, np.where(valid, ids, 0).astype(np.int32),
                                         None, x_slots=xs)
    err = np.abs(hs[valid].astype(np.float64) - hr[valid])
    assert np.all(err <= swiglu_bound(hr[valid], g[valid], u[valid], Sg[valid], Su[valid]))


# ------------------------------------------------------------------ fused combine
def combine_bound(S, w):
    """The combine's bound: the weighted matvec bounds plus the fp32
    multiply-add chain over at most 16 slots."""
    return (1e-4 + 16 * 2.0 ** -24) * S + 1e-6 * np.abs(w).sum(axis=1, keepdims=True) + 1e-30


def combine(env, fmt, Wall, stride, N, K, ids, w, x, n_experts=E):
    torch, qmv = env
    out = qmv.qmv_moe_combine(fmt, dev(torch, Wall), stride, n_experts, N, K, dev(torch, ids), dev(torch, w),
                              dev(torch, x))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [1, 2, 8])
def test_superblock_moe_combine_30b_shapes(env, fmt, B):
    """Super-block down experts 2048 x 768 (3 super-blocks per row), one input per
    (token, slot), router weights summing to 1: against the oracle, and
    against the weighted sum of qmv_moe's per-slot outputs."""
    H, F = wl.MOE_HIDDEN, wl.MOE_FFN
    Wall = experts(fmt, "down", H, F)
    stride = wl.block_bytes(fmt, H, F)
    ids = wl.moe_ids(f"t/sbmoe/cb/ids/{B}", B, T, E)
    w = wl.router_weights(f"t/sbmoe/cb/w/{B}", B, T)
    x = wl.activations(f"t/sbmoe/cb/x/{B}", B * T, F).reshape(B, T, F)
    say(f"{fmt} moe combine B={B}")
    out = combine(env, fmt, Wall, stride, H, F, ids, w, x)
    ref, S = oracle.moe_combine(fmt, Wall, stride, E, H, F, ids, w, x_slots=x)
    err = np.abs(out.astype(np.float64) - ref)
    assert np.all(err <= combine_bound(S, w)), float((err / combine_bound(S, w)).max())
    y = run(env, fmt, Wall, stride, H, F, ids, x).astype(np.float64)
    mix = np.einsum("bs,bsn->bn", w.astype(np.float64), y)
    assert np.all(np.abs(out - mix) <= T * 2.0 ** -24 * np.einsum("bs,bsn->bn", np.abs(w), np.abs(y)) + 1e-37)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", ["one_hot_dup", "invalid", "chunked_slots", "token_inputs"])
def test_superblock_moe_combine_edges(env, fmt, case):
    """Six experts.  One-hot weights (out equals one slot's qmv_moe output
    bitwise) with duplicated ids and a padded stride, an invalid id (the
    token's row becomes NaN), top_k 16 on rows of 16384 columns (one slot
    vector staged at a time), one input per token; Q6_K refuses the fused
    form."""
    torch, qmv = env
    E6 = 6
    if case == "one_hot_dup":
        N, K, ids = 300, 1024, np.array([[2, 5, 2], [0, 0, 1]], dtype=np.int32)
    elif case == "invalid":
        N, K, ids = 96, 512, np.array([[1, 3], [7, 2], [4, 4]], dtype=np.int32)
    elif case == "chunked_slots":
        N, K, ids = 300, 16384, np.array([[i % E6 for i in range(16)]], dtype=np.int32)
    else:
        N, K, ids = 128, 2048, np.array([[5, 1, 0, 3], [2, 2, 4, 1]], dtype=np.int32)
    B, Tk = ids.shape
    per = wl.block_bytes(fmt, N, K)
    stride = per + (256 if case == "one_hot_dup" else 0)
    Wm = wl.quant_weights(fmt, f"t/sbmoe/cb/{case}", E6 * N, K).reshape(E6, per)
    Wall = np.zeros((E6, stride), dtype=np.uint8)
    Wall[:, :per] = Wm
    Wall = Wall.reshape(-1)
    w = wl.router_weights(f"t/sbmoe/cb/w/{case}", B, Tk)
    say(f"{fmt} moe combine edge {case}")
    if case == "token_inputs":
        x = wl.activations(f"t/sbmoe/cb/x/{case}", B, K)
        out = combine(env, fmt, Wall, stride, N, K, ids, w, x, E6)
        ref, S = oracle.moe_combine(fmt, Wall, stride, E6, N, K, ids, w, x_tokens=x)
    else:
        x = wl.activations(f"t/sbmoe/cb/x/{case}", B * Tk, K).reshape(B, Tk, K)
        if case == "one_hot_dup":
            w = np.zeros((B, Tk), dtype=np.float32)
            w[0, 2] = 1.0
            w[1, 1] = 1.0
        out = combine(env, fmt, Wall, stride, N, K, ids, w, x, E6)
        if case == "invalid":
            valid = np.all((ids >= 0) & (ids < E6), axis=1)
            assert np.all(np.isnan(out[~valid])) and not np.any(np.isnan(out[valid]))
            ids_ok = np.where((ids >= 0) & (ids < E6), ids, 0).astype(np.int32)
            ref, S = oracle.moe_combine(fmt, Wall, stride, E6, N, K, ids_ok, w, x_slots=x)
            out, ref, S, w = out[valid], ref[valid], S[valid], w[valid]
        elif case == "chunked_slots":
            ref, S = oracle.moe_combine(fmt, Wall, stride, E6, N, K, ids, w, x_slots=x)
        else:
            ref, S = oracle.moe_combine(fmt, Wall, stride, E6, N, K, ids, w, x_slots=x)
            y = qmv.qmv_moe(fmt, dev(torch, Wall), stride, E6, N, K, dev(torch, ids), dev(torch, x))
            torch.cuda.synchronize()
            y = y.cpu().numpy()
            assert np.array_equal(out[0].view(np.uint32), y[0, 2].view(np.uint32))
            assert np.array_equal(out[1].view(np.uint32), y[1, 1].view(np.uint32))
    err = np.abs(out.astype(np.float64) - ref)
    assert np.all(err <= combine_bound(S, w)), (case, float((err / combine_bound(S, w)).max()))
