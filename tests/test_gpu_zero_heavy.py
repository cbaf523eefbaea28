"""The accuracy bound on rows made mostly of zero weights, on every kernel
family, against the oracle.

The bound |y_gpu - y| <= 1e-4 * sum_j |w_j x_j| + 1e-6 is relative to the
row's own sum of |w x|.  A block term that folds an offset as a separate sum
(d * (sum c x - 8 sum x) for Q4_0, d * sum c x + m * sum x for Q4_1) rounds
two numbers of size ~sum |x| and subtracts them; on rows whose weights are
zero where the activations are large it misses the bound by orders of
magnitude.  The inputs here (workloads.zero_heavy) are exactly that: Q8_0
code 0, Q4_0 code 8 and Q4_1 codes k with d*k + m = 0 on 15 of every 16
columns, which carry activations ~1e3, and arbitrary codes on the rest,
which carry activations ~1e-3.  Every launch choice is reached: the
per-block and whole-line batch-1 kernels, the persistent chain, the FMA
kernels at batch 3 and 8, the matrix-core kernel at batch 2..8, the MoE
per-pair, grouping, SwiGLU and combine kernels, and 16-bit activations.
"""
import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

FMTS = ["q8_0", "q4_0", "q4_1"]


@pytest.fixture(scope="module")
def env():
    import torch
    import bandwidth_bound_block_amd as qmv
    assert torch.cuda.is_available()
    return torch, qmv


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def check(y, yr, S, what):
    err = np.abs(np.asarray(y, dtype=np.float64) - yr)
    tol = 1e-4 * S + 1e-6
    assert np.all(err <= tol), (what, int((err > tol).sum()), float((err / tol).max()))


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_heavy_batch1_kernels(env, fmt):
    """Batch 1: the per-block kernel (64 blocks per row, and a 4-byte
    offset W) and the whole-line kernel (256 blocks per row)."""
    torch, qmv = env
    f = {"q8_0": qmv.qmv_q8_0, "q4_0": qmv.qmv_q4_0, "q4_1": qmv.qmv_q4_1}[fmt]
    for N, K in [(130, 2048), (40, 8192), (3, 14336), (7, 96)]:
        say(f"zero-heavy b1 {fmt} {N}x{K}")
        W, x = wl.zero_heavy(fmt, f"t/zh/b1/{fmt}/{N}x{K}", N, K)
        yr, S = oracle.matvec(fmt, W, N, K, x)
        Wd, xd = dev(torch, W), dev(torch, x)
        y = f(Wd, N, K, xd)
        buf = torch.zeros(W.size + 16, dtype=torch.uint8, device="cuda:0")
        Wo = buf[4:4 + W.size]
        Wo.copy_(Wd.reshape(-1))
        y_off = f(Wo, N, K, xd)
        torch.cuda.synchronize()
        check(y.cpu().numpy(), yr, S, (fmt, N, K))
        check(y_off.cpu().numpy(), yr, S, (fmt, N, K, "offset W"))


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_heavy_chain(env, fmt):
    """qmv_chain: a shared-input group run as one whole-line launch (q||k||v
    shape at 2048 columns, and > 8192 rows, two rows per wave step for Q4),
    and six stages through the persistent chain kernel, the last waiting at
    a stage barrier."""
    torch, qmv = env
    ws = torch.zeros(qmv.CHAIN_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    groups = {"qkv": [2048, 512, 512], "big": [5001, 4000], "six": [300, 77, 1, 513, 64, 129]}
    K = 2048
    for gname, rows in groups.items():
        say(f"zero-heavy chain {fmt} {gname}")
        Ws, xs = [], None
        for i, N in enumerate(rows):
            W, x = wl.zero_heavy(fmt, f"t/zh/chain/{fmt}/{gname}/{i}", N, K)
            Ws.append(W)
            if xs is None:
                xs = wl.zero_heavy(fmt, f"t/zh/chain/{fmt}/{gname}/x", 1, K)[1]
        xd = dev(torch, xs)[0]
        stages = []
        for i, (N, W) in enumerate(zip(rows, Ws)):
            y = torch.full((N,), float("nan"), device="cuda:0")
            stages.append((dev(torch, W), N, K, xd, y, 1 if (gname == "six" and i == len(rows) - 1) else 0))
        qmv.qmv_chain(fmt, stages, ws)
        torch.cuda.synchronize()
        assert int(ws.view(torch.int32)[2].item()) == 0
        for (W, (_, N, _, _, y, _)) in zip(Ws, stages):
            yr, S = oracle.matvec(fmt, W, N, K, xs)
            check(y.cpu().numpy()[None], yr, S, (fmt, gname, N))


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_heavy_batches(env, fmt):
    """Batch 3 and 8 on the FMA kernels, batch 2, 5 and 8 on the matrix
    cores, and the entry point's own choice at batch 4."""
    torch, qmv = env
    N, K = 70, 2048
    for B, path in [(3, qmv.PATH_FMA), (8, qmv.PATH_FMA), (2, qmv.PATH_MFMA), (5, qmv.PATH_MFMA),
                    (8, qmv.PATH_MFMA), (4, qmv.PATH_AUTO)]:
        say(f"zero-heavy {fmt} B={B} path={path}")
        W, x = wl.zero_heavy(fmt, f"t/zh/batch/{fmt}/{B}", N, K, B=B)
        y = qmv.qmv_matvec_path(fmt, dev(torch, W), N, K, dev(torch, x), path)
        torch.cuda.synchronize()
        yr, S = oracle.matvec(fmt, W, N, K, x)
        check(y.cpu().numpy(), yr, S, (fmt, B, path))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_zero_heavy_x16(env, fmt, kind):
    """16-bit activations (widened exactly): batch 1 and batch 4 on the FMA
    and matrix-core kernels, against the oracle on the widened values."""
    torch, qmv = env
    N, K = 70, 4096
    W, x = wl.zero_heavy(fmt, f"t/zh/x16/{fmt}/{kind}", N, K, B=4)
    tt = torch.float16 if kind == "f16" else torch.bfloat16
    x16 = torch.from_numpy(x).to(tt)
    xw = x16.float().numpy()
    yr, S = oracle.matvec(fmt, W, N, K, xw)
    Wd, xd = dev(torch, W), x16.to("cuda:0")
    for B, path in [(1, qmv.PATH_AUTO), (4, qmv.PATH_FMA), (4, qmv.PATH_MFMA)]:
        y = qmv.qmv_matvec_xt(fmt, Wd, N, K, xd[:B], path=path)
        torch.cuda.synchronize()
        check(y.cpu().numpy(), yr[:B], S[:B], (fmt, kind, B, path))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [1, 2, 8])
def test_zero_heavy_moe(env, fmt, B):
    """qmv_moe: gate/up shape (768 x 2048, one input per token) and down
    shape (2048 x 768, one input per token and slot); batch 1 takes the
    per-pair route, 2 and 8 the grouping kernel."""
    torch, qmv = env
    E, T = 16, 8
    for kind, N, K in [("gate", 768, 2048), ("down", 2048, 768)]:
        say(f"zero-heavy moe {fmt} {kind} B={B}")
        Wall, _ = wl.zero_heavy(fmt, f"t/zh/moe/{fmt}/{kind}", E * N, K)
        Wall = Wall.reshape(-1)
        stride = wl.block_bytes(fmt, N, K)
        ids = wl.moe_ids(f"t/zh/moe/ids/{B}", B, T, E)
        if kind == "gate":
            x = wl.zero_heavy(fmt, f"t/zh/moe/{fmt}/{kind}/x/{B}", 1, K, B=B)[1]
            yr, S = oracle.moe(fmt, Wall, stride, E, N, K, ids, x)
        else:
            x = wl.zero_heavy(fmt, f"t/zh/moe/{fmt}/{kind}/x/{B}", 1, K, B=B * T)[1].reshape(B, T, K)
            yr, S = oracle.moe(fmt, Wall, stride, E, N, K, ids, None, x_slots=x)
        y = qmv.qmv_moe(fmt, dev(torch, Wall), stride, E, N, K, dev(torch, ids), dev(torch, x))
        torch.cuda.synchronize()
        check(y.cpu().numpy(), yr, S, (fmt, kind, B))


def swiglu_bound(h, g, u, Sg, Su):
    """|h_gpu - h| for h = SiLU(g) u from fp32 g, u within the matvec bound
    (tg, tu): |SiLU'| <= 1.1, so |dh| <= 1.1 tg (|u| + tu) + (|SiLU(g)| +
    1.1 tg) tu, plus the fp32 epilogue (a few ulps of h)."""
    tg, tu = 1e-4 * Sg + 1e-6, 1e-4 * Su + 1e-6
    sg = np.abs(g / (1.0 + np.exp(-g)))
    return 1.1 * tg * (np.abs(u) + tu) + (sg + 1.1 * tg) * tu + 2.0 ** -20 * np.abs(h) + 1e-30


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [1, 4])
def test_zero_heavy_moe_swiglu(env, fmt, B):
    """qmv_moe_swiglu on gate||up experts of 2 x 768 rows (batch 1: the
    per-pair route with paired rows; batch 4: the grouping kernel)."""
    torch, qmv = env
    E, T, F, K = 16, 8, 768, 2048
    Wall, _ = wl.zero_heavy(fmt, f"t/zh/swiglu/{fmt}", E * 2 * F, K)
    Wall = Wall.reshape(-1)
    stride = 2 * wl.block_bytes(fmt, F, K)
    ids = wl.moe_ids(f"t/zh/swiglu/ids/{B}", B, T, E)
    x = wl.zero_heavy(fmt, f"t/zh/swiglu/{fmt}/x/{B}", 1, K, B=B)[1]
    h = qmv.qmv_moe_swiglu(fmt, dev(torch, Wall), stride, E, F, K, dev(torch, ids), dev(torch, x))
    torch.cuda.synchronize()
    hr, g, u, Sg, Su = oracle.moe_swiglu(fmt, Wall, stride, E, F, K, ids, x)
    bound = swiglu_bound(hr, g, u, Sg, Su)
    err = np.abs(h.cpu().numpy().astype(np.float64) - hr)
    assert np.all(err <= bound), (fmt, B, float((err / bound).max()))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [1, 8])
def test_zero_heavy_moe_combine(env, fmt, B):
    """qmv_moe_combine on down experts of 2048 x 768, one input per (token,
    slot), router weights summing to 1."""
    torch, qmv = env
    E, T, N, K = 16, 8, 2048, 768
    Wall, _ = wl.zero_heavy(fmt, f"t/zh/combine/{fmt}", E * N, K)
    Wall = Wall.reshape(-1)
    stride = wl.block_bytes(fmt, N, K)
    ids = wl.moe_ids(f"t/zh/combine/ids/{B}", B, T, E)
    w = wl.router_weights(f"t/zh/combine/w/{B}", B, T)
    x = wl.zero_heavy(fmt, f"t/zh/combine/{fmt}/x/{B}", 1, K, B=B * T)[1].reshape(B, T, K)
    out = qmv.qmv_moe_combine(fmt, dev(torch, Wall), stride, E, N, K, dev(torch, ids), dev(torch, w), dev(torch, x))
    torch.cuda.synchronize()
    ref, S = oracle.moe_combine(fmt, Wall, stride, E, N, K, ids, w, x_slots=x)
    bound = (1e-4 + 16 * 2.0 ** -24) * S + 1e-6 * np.abs(w).sum(axis=1, keepdims=True) + 1e-30
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= bound), (fmt, B, float((err / bound).max()))
