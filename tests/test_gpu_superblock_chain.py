"""qmv_chain and qmv_chain_noalloc with Q4_K and Q6_K stages through the C
ABI on an MI355X.  These formats run a chain's stages as launches of their
own (stream order in place of the stage barriers), each run of up to 4
stages that read one x with one width as one launch over their
concatenated rows.  Every output is bitwise the batch-1 entry point's on
the same stage, and within the bound of the oracle.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


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


def entry(qmv, fmt):
    return qmv.qmv_q4_k if fmt == "q4_k" else qmv.qmv_q6_k


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k"])
@pytest.mark.parametrize("K", [2048, 4096])
@pytest.mark.parametrize("noalloc", [False, True])
def test_superblock_chain_decode_levels(env, fmt, K, noalloc):
    """q, k, v on one x (row counts 512, 37, 65: at 2048 columns the 2-row
    tiles straddle the matrices), then o on q's output (a waiting stage),
    then gate and up on o's output, then down on gate's output: every
    output bitwise the batch-1 entry point's, within the oracle's bound,
    and the chain deterministic over two calls."""
    torch, qmv = env
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    shapes = {"q": (512, K), "k": (37, K), "v": (65, K), "o": (K, 512), "gate": (512, K), "up": (300, K),
              "down": (K, 512)}
    Ws = {m: wl.quant_weights(fmt, f"t/sbchain/{fmt}/{m}/{K}", *shapes[m]) for m in names}
    Wd = {m: dev(torch, Ws[m]) for m in names}
    x = dev(torch, wl.activations(f"t/sbchain/x/{K}", 1, K).reshape(-1))
    ys = {m: torch.full((shapes[m][0],), float("nan"), dtype=torch.float32, device="cuda:0") for m in names}
    inputs = {"q": x, "k": x, "v": x, "o": ys["q"], "gate": ys["o"], "up": ys["o"], "down": ys["gate"]}
    waits = {"o", "gate", "down"}
    stages = [(Wd[m], shapes[m][0], shapes[m][1], inputs[m], ys[m], m in waits) for m in names]
    say(f"sb chain {fmt} K={K} noalloc={noalloc}")
    runs = []
    for rep in range(2):
        if noalloc:
            qmv.qmv_chain_noalloc(fmt, stages)
        else:
            ws = torch.zeros(qmv.CHAIN_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
            qmv.qmv_chain(fmt, stages, ws)
        torch.cuda.synchronize()
        runs.append({m: ys[m].clone() for m in names})
    for m in names:
        assert torch.equal(runs[0][m].view(torch.int32), runs[1][m].view(torch.int32)), m
    f = entry(qmv, fmt)
    for m in names:
        N, Kc = shapes[m]
        ref = f(Wd[m], N, Kc, inputs[m])
        torch.cuda.synchronize()
        assert torch.equal(ys[m].view(torch.int32), ref.reshape(-1).view(torch.int32)), (fmt, K, m)
        yr, S = oracle.matvec(fmt, Ws[m], N, Kc, inputs[m].cpu().numpy().reshape(1, -1))
        assert_tol(ys[m].cpu().numpy().reshape(1, -1), yr, S, (fmt, K, m))
