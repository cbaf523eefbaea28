"""MoE experts stored as Q4_K or Q6_K super-blocks (qmv_moe, qmv_moe_xt)
through the C ABI on an MI355X, against the oracle's per-(token, slot)
loop.

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
