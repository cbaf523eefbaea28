"""The streaming decode kernel behind qmv_chain (stages of whole 2048-column
windows, 16-byte aligned W and x): every stage against the oracle on its own
input (as the chain computed it), bitwise determinism over repeated calls,
and the workspace's error word staying 0.

Shapes: decode-dependent layers of the 8B set (q||k||v, o, gate||up, down at
4096 and 14336 columns, then an lm_head), levels with fewer rows than
workgroups, ragged row counts, window counts that do not divide the 14
compute waves (3 and 5 windows: the waves change window from item to item),
four-matrix levels, and more levels than one launch holds."""
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


def _check(y, yr, S, what):
    err = np.abs(np.asarray(y, dtype=np.float64) - yr)
    tol = 1e-4 * S + 1e-6
    assert np.all(err <= tol), (what, int((err > tol).sum()), float((err / tol).max()))


def _run_and_check(env, fmt, stages, host_W, reps=2, sample_above=20000):
    """Runs the chain `reps` times: outputs bitwise equal across calls, the
    error word 0, and each stage within the bound of the oracle on its own
    input (rows sampled for stages above sample_above rows)."""
    torch, qmv = env
    ws = torch.zeros(qmv.CHAIN_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    first = None
    for rep in range(reps):
        for st in stages:
            st[4].fill_(float("nan"))
        qmv.qmv_chain(fmt, stages, ws)
        torch.cuda.synchronize()
        assert int(ws.view(torch.int32)[2].item()) == 0, "barrier timed out"
        if first is None:
            first = [st[4].clone() for st in stages]
        else:
            for i, st in enumerate(stages):
                assert torch.equal(st[4].view(torch.int32), first[i].view(torch.int32)), (fmt, rep, i)
    for i, (W, N, K, x, y, _) in enumerate(stages):
        xin = x.cpu().numpy()[None]
        rows = None
        if N > sample_above:
            rows = np.unique(np.concatenate([np.arange(32), np.arange(N - 32, N),
                                             np.random.default_rng(N).choice(N, 2048, replace=False)]))
        yr, S = oracle.matvec(fmt, host_W[i], N, K, xin, rows=rows)
        got = y.cpu().numpy()
        _check((got if rows is None else got[rows])[None], yr, S, (fmt, i, N, K))


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_stream_llama8b_layers(env, fmt):
    """Two 8B-shaped decode layers and an lm_head: q, k, v read the layer
    input; o reads q; gate and up read o; down reads gate; the next layer
    reads down; the lm_head (16384 x 4096 here) reads the last down."""
    torch, qmv = env
    H, F = 4096, 14336
    mats = {"q": (H, H), "k": (1024, H), "v": (1024, H), "o": (H, H), "gate": (F, H), "up": (F, H), "down": (H, F)}
    Wh = {m: wl.quant_weights(fmt, f"t/dec/{fmt}/{m}", N, K) for m, (N, K) in mats.items()}
    Wd = {m: torch.from_numpy(w).to("cuda:0") for m, w in Wh.items()}
    Whead = wl.quant_weights(fmt, f"t/dec/{fmt}/head", 16384, H)
    h = torch.from_numpy(wl.activations(f"t/dec/{fmt}/h", 1, H)).to("cuda:0")[0]
    stages, host = [], []
    for layer in range(2):
        y = {m: torch.empty(N, device="cuda:0") for m, (N, _) in mats.items()}
        for m, x, wait in [("q", h, 1), ("k", h, 0), ("v", h, 0), ("o", y["q"], 1), ("gate", y["o"], 1),
                           ("up", y["o"], 0), ("down", y["gate"], 1)]:
            N, K = mats[m]
            stages.append((Wd[m], N, K, x, y[m], wait))
            host.append(Wh[m])
        h = y["down"]
    yh = torch.empty(16384, device="cuda:0")
    stages.append((torch.from_numpy(Whead).to("cuda:0"), 16384, H, h, yh, 1))
    host.append(Whead)
    print(f"decode stream {fmt}: {len(stages)} stages", flush=True)
    _run_and_check(env, fmt, stages, host)


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_stream_odd_shapes(env, fmt):
    """Levels of 1, 5, 255, 257 and 300 rows (fewer than, and ragged against,
    the workgroups), 3 and 5 windows per row (6144 and 10240 columns), a
    four-matrix level, a shared-input stage after it without a wait, and a
    dependent run of 40 small stages (more levels than one launch)."""
    torch, qmv = env
    dev = "cuda:0"
    rng = np.random.default_rng(3)
    stages, host = [], []

    def add(N, K, x, wait, tag):
        W = wl.quant_weights(fmt, f"t/dec/odd/{fmt}/{tag}", N, K)
        y = torch.empty(N, device=dev)
        stages.append((torch.from_numpy(W).to(dev), N, K, x, y, wait))
        host.append(W)
        return y

    x6 = torch.from_numpy(wl.activations(f"t/dec/odd/{fmt}/x6", 1, 6144)).to(dev)[0]
    a = add(257, 6144, x6, 0, "a")
    add(1, 6144, x6, 0, "b")
    add(5, 6144, x6, 0, "c")
    add(300, 6144, x6, 0, "d")                # four matrices in one level
    add(255, 6144, x6, 0, "e")                # same x, no wait: the next level
    x10 = torch.from_numpy(wl.activations(f"t/dec/odd/{fmt}/x10", 1, 10240)).to(dev)[0]
    b = add(6144, 10240, x10, 1, "f")         # 5 windows per row
    c = add(2048, 6144, b, 1, "g")            # reads f's output (3 windows)
    cur = c
    for i in range(40):
        cur = add(2048 if i % 3 else 37, 2048, cur if i % 3 != 1 else c, 1, f"r{i}")
        if cur.numel() != 2048:
            cur = c
    print(f"decode stream odd {fmt}: {len(stages)} stages", flush=True)
    _run_and_check(env, fmt, stages, host, reps=3)
    assert a.numel() == 257 and rng is not None


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_decode_stream_zero_heavy(env, fmt):
    """Rows mostly of zero weights, large activations on them (the accuracy
    edge case) through the streaming kernel: two levels at 4096 columns,
    the second waiting."""
    torch, qmv = env
    dev = "cuda:0"
    W1, x = wl.zero_heavy(fmt, f"t/dec/zh/{fmt}/1", 700, 4096)
    W2, _ = wl.zero_heavy(fmt, f"t/dec/zh/{fmt}/2", 300, 4096)
    xd = torch.from_numpy(x).to(dev)[0]
    y1 = torch.empty(700, device=dev)
    y2 = torch.empty(300, device=dev)
    stages = [(torch.from_numpy(W1).to(dev), 700, 4096, xd, y1, 0),
              (torch.from_numpy(W2).to(dev), 300, 4096, xd, y2, 1)]
    _run_and_check(env, fmt, stages, [W1, W2])
