"""Q6_K super-blocks (256 weights in 210 bytes) through the C ABI on an
MI355X, against the oracle.

Float matvec: |y_gpu - y| <= 1e-4 * S + 1e-6 per output (S = sum_j |w_ij x_j|)
against the fp64 dequantize-then-dot oracle, on encoded Gaussian weights,
random super-block bytes (random codes, int8 scales and fp16 d over their
whole range) and the zero-heavy rows.  Super-blocks start 2 (mod 4) bytes
into W at every other index and rows of an odd number of super-blocks
alternate that parity: both occur in every shape below.  Shapes span every lane
split of the kernel (8 / 16 / 32 / 64 lanes per row, from 4 to 568 groups
of 64 weights), rows in ragged counts against the workgroups, and the
8B-shaped layer matrices at full size with sampled rows.  Dequantization is
bitwise the oracle's values (exact in fp32); 16-bit activations
give bitwise the fp32 call on the widened values; a column is bitwise the
same at every batch width and over repeated calls.  The matrix-core path is
checked the same way: against the oracle on the shapes above, random bytes
and zero-heavy rows, bitwise position- and width-independent columns,
16-bit activations.
"""
import functools
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from tests import hand_blocks as hb

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


def random_super_blocks(seed, N, K):
    """Random bytes with a finite fp16 d over the whole range (subnormals
    included)."""
    g = np.random.default_rng(seed)
    ns = K // 256
    raw = g.integers(0, 256, size=(N, ns, 210), dtype=np.uint8)
    h = (g.integers(0, 2, size=(N, ns)) << 15) | (g.integers(0, 31, size=(N, ns)) << 10) | \
        g.integers(0, 1024, size=(N, ns))
    raw[..., 208] = h & 0xFF
    raw[..., 209] = h >> 8
    return raw.reshape(N, -1)


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("kind", ["encoded", "random_bytes", "zero_heavy"])
def test_q6k_dequant_bit_exact(env, kind):
    torch, qmv = env
    N, K = 37, 768
    say(f"q6_k dequant {kind} {N}x{K}")
    if kind == "encoded":
        W = wl.quant_weights("q6_k", "t/q6k/deq", N, K)
    elif kind == "random_bytes":
        W = random_super_blocks(11, N, K)
    else:
        W, _ = wl.zero_heavy("q6_k", "t/q6k/deq/zh", N, K)
    ref = oracle.dequant("q6_k", W, N, K).astype(np.float32)
    got = qmv.qmv_dequant("q6_k", dev(torch, W), N, K)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ hand super-blocks
@pytest.mark.parametrize("spec", [s for s in hb.load()["super_blocks"] if s["fmt"] == "q6_k"],
                         ids=lambda s: s["id"])
def test_q6k_hand_super_blocks(env, spec):
    torch, qmv = env
    blk = hb.super_block_bytes(spec)
    x = hb.x_vec256(spec["x"])[None, :]
    y = qmv.qmv_q6_k(dev(torch, blk), 1, 256, dev(torch, x))
    torch.cuda.synchronize()
    assert float(y[0, 0]) == float(np.float32(float(spec["y"]))), (spec["id"], float(y[0, 0]))


# ------------------------------------------------------------------ shapes
# (rows, columns): 1..4 super-blocks per row (8 / 16 lanes per row, 768
# columns with a half-idle last step), 5 (1280 columns), 8 and 16 (32 / 64
# lanes), 12 (16 lanes), 56 = 14336 columns (224 groups: 32 lanes, 7
# steps), 142 = 36352 columns (64 lanes, a ragged ninth step), 150 = 38400
# columns (the LDS limit: one activation row per pass).
SHAPES = [(1, 256), (7, 512), (37, 768), (130, 1024), (9, 1280), (257, 2048), (61, 3072), (65, 4096), (300, 4096),
          (5, 14336), (33, 36352), (3, 38400), (2100, 4096)]


@pytest.mark.parametrize("B", [1, 2, 3, 5, 8])
def test_q6k_shapes_encoded(env, B):
    torch, qmv = env
    for N, K in SHAPES:
        say(f"q6_k B={B} {N}x{K}")
        W = wl.quant_weights("q6_k", f"t/q6k/{N}x{K}", N, K)
        x = wl.activations(f"t/q6k/x/{K}/{B}", B, K)
        y = qmv.qmv_q6_k(dev(torch, W), N, K, dev(torch, x))
        torch.cuda.synchronize()
        yr, S = oracle.matvec("q6_k", W, N, K, x)
        assert_tol(y.cpu().numpy(), yr, S, (N, K, B))


def test_q6k_random_super_blocks(env):
    """Random codes, int8 scales and fp16 d over their whole range
    (subnormals included), activations over many binades."""
    torch, qmv = env
    g = np.random.default_rng(23)
    for N, K, B in [(64, 1024, 1), (19, 4096, 3), (300, 2048, 8), (33, 1280, 2)]:
        say(f"q6_k random bytes B={B} {N}x{K}")
        W = random_super_blocks(1000 + K, N, K)
        x = (g.standard_normal((B, K)) * np.exp(g.uniform(-6, 6, size=(B, K)))).astype(np.float32)
        y = qmv.qmv_q6_k(dev(torch, W), N, K, dev(torch, x))
        torch.cuda.synchronize()
        yr, S = oracle.matvec("q6_k", W, N, K, x)
        assert_tol(y.cpu().numpy(), yr, S, (N, K, B))


@pytest.mark.parametrize("B", [1, 4])
def test_q6k_zero_heavy(env, B):
    """Rows of mostly exact-zero weights under large activations: the per
    output bound holds (no offset is folded out of a sum)."""
    torch, qmv = env
    for N, K in [(700, 4096), (300, 14336), (9, 512)]:
        say(f"q6_k zero-heavy B={B} {N}x{K}")
        W, x = wl.zero_heavy("q6_k", f"t/q6k/zh/{N}x{K}", N, K, B=B)
        y = qmv.qmv_q6_k(dev(torch, W), N, K, dev(torch, x))
        torch.cuda.synchronize()
        yr, S = oracle.matvec("q6_k", W, N, K, x)
        assert_tol(y.cpu().numpy(), yr, S, (N, K, B))


def test_q6k_columns_equal_batch1_and_deterministic(env):
    """The FMA kernel: every column bitwise its batch-1 result."""
    torch, qmv = env
    N, K = 1000, 4096
    W = dev(torch, wl.quant_weights("q6_k", "t/q6k/det", N, K))
    x = dev(torch, wl.activations("t/q6k/det/x", 8, K))
    ref = [qmv.qmv_q6_k(W, N, K, x[b]).reshape(-1) for b in range(8)]
    for B in (2, 3, 5, 8):
        say(f"q6_k columns B={B}")
        for rep in range(2):
            y = qmv.qmv_matvec_path("q6_k", W, N, K, x[:B], qmv.PATH_FMA)
            torch.cuda.synchronize()
            for b in range(B):
                assert torch.equal(y[b].view(torch.int32), ref[b].view(torch.int32)), (B, b, rep)


def test_q6k_strided_and_unaligned_activations(env):
    """ldx > n_cols (x rows not 16-byte aligned: the scalar staging), y rows
    strided; outputs past n_rows untouched."""
    torch, qmv = env
    N, K, B = 129, 2048, 3
    W = wl.quant_weights("q6_k", "t/q6k/str", N, K)
    xbig = wl.activations("t/q6k/str/x", B, K + 1)
    xt = dev(torch, xbig)[:, :K]
    y = torch.zeros((B, N + 3), dtype=torch.float32, device="cuda:0")
    qmv.qmv_q6_k(dev(torch, W), N, K, xt, y=y[:, :N])
    torch.cuda.synchronize()
    yr, S = oracle.matvec("q6_k", W, N, K, xbig[:, :K])
    assert_tol(y[:, :N].cpu().numpy(), yr, S)
    assert np.all(y[:, N:].cpu().numpy() == 0)


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_q6k_x16_equal_widened_fp32(env, kind):
    torch, qmv = env
    for N, K in [(37, 768), (65, 4096), (5, 14336), (2100, 4096)]:
        W = wl.quant_weights("q6_k", f"t/q6k/{N}x{K}", N, K)
        Wd = dev(torch, W)
        for B in (1, 2, 8):
            say(f"q6_k x16 {kind} B={B} {N}x{K}")
            x = wl.activations(f"t/q6k/x16/{K}/{B}", B, K)
            xh = dev(torch, x).to(torch.float16 if kind == "f16" else torch.bfloat16)
            xw = xh.float()
            for path in (qmv.PATH_AUTO, qmv.PATH_FMA):
                y16 = qmv.qmv_matvec_xt("q6_k", Wd, N, K, xh, path)
                y32 = qmv.qmv_matvec_path("q6_k", Wd, N, K, xw, path)
                torch.cuda.synchronize()
                assert torch.equal(y16.view(torch.int32), y32.view(torch.int32)), (N, K, B, path)
            yr, S = oracle.matvec("q6_k", W, N, K, xw.cpu().numpy())
            assert_tol(y16.cpu().numpy(), yr, S, (kind, N, K, B))


@functools.lru_cache(maxsize=None)
def _layer_weights(name, N, K):
    return wl.quant_weights("q6_k", f"t/q6k/l8b/{name}", N, K)


@pytest.mark.parametrize("B", [1, 8])
def test_q6k_llama8b_layer_set(env, B):
    """The 8B layer matrices at full size (q, k, v, o, gate, up, down), rows
    sampled for the oracle: the first and last 32 rows and 512 more."""
    torch, qmv = env
    for name, N, K in wl.LLAMA8B_LAYER:
        say(f"q6_k llama8b {name} {N}x{K} B={B}")
        W = _layer_weights(name, N, K)
        x = wl.activations(f"t/q6k/l8b/x/{K}/{B}", B, K)
        y = qmv.qmv_q6_k(dev(torch, W), N, K, dev(torch, x))
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([np.arange(32), np.arange(N - 32, N),
                                         np.random.default_rng(N + K).choice(N, 512, replace=False)]))
        yr, S = oracle.matvec("q6_k", W, N, K, x, rows=rows)
        assert_tol(y.cpu().numpy()[:, rows], yr, S, (name, B))


# ------------------------------------------------------------------ matrix cores
MMA_SHAPES = [(1, 256), (37, 768), (130, 1024), (257, 2048), (65, 4096), (300, 4096), (5, 14336), (33, 36352),
              (2100, 4096)]


@pytest.mark.parametrize("B", [2, 3, 5, 8])
def test_q6k_mfma_shapes(env, B):
    """The matrix-core path (scales folded into two exact bf16 pieces of
    the codes) against the oracle; the automatic path too, bitwise the result of
    the family it chooses."""
    torch, qmv = env
    for N, K in MMA_SHAPES:
        say(f"q6_k mfma B={B} {N}x{K}")
        W = wl.quant_weights("q6_k", f"t/q6k/{N}x{K}", N, K)
        Wd = dev(torch, W)
        x = wl.activations(f"t/q6k/mx/{K}/{B}", B, K)
        xd = dev(torch, x)
        y = qmv.qmv_matvec_path("q6_k", Wd, N, K, xd, qmv.PATH_MFMA)
        ya = qmv.qmv_q6_k(Wd, N, K, xd)
        torch.cuda.synchronize()
        yr, S = oracle.matvec("q6_k", W, N, K, x)
        assert_tol(y.cpu().numpy(), yr, S, (N, K, B))
        assert_tol(ya.cpu().numpy(), yr, S, ("auto", N, K, B))
        # the automatic choice (per shape and batch) runs one of the two
        # families: bitwise its result
        yf = qmv.qmv_matvec_path("q6_k", Wd, N, K, xd, qmv.PATH_FMA)
        torch.cuda.synchronize()
        assert (torch.equal(y.view(torch.int32), ya.view(torch.int32))
                or torch.equal(yf.view(torch.int32), ya.view(torch.int32))), (N, K, B)


def test_q6k_mfma_random_and_zero_heavy(env):
    """Random super-block bytes (d over the whole fp16 range, int8 scales
    and codes at their extremes) and zero-heavy rows on the matrix cores."""
    torch, qmv = env
    g = np.random.default_rng(29)
    for N, K, B in [(64, 1024, 3), (300, 2048, 8), (19, 4096, 2)]:
        say(f"q6_k mfma random bytes B={B} {N}x{K}")
        W = random_super_blocks(2000 + K, N, K)
        x = (g.standard_normal((B, K)) * np.exp(g.uniform(-6, 6, size=(B, K)))).astype(np.float32)
        y = qmv.qmv_matvec_path("q6_k", dev(torch, W), N, K, dev(torch, x), qmv.PATH_MFMA)
        torch.cuda.synchronize()
        yr, S = oracle.matvec("q6_k", W, N, K, x)
        assert_tol(y.cpu().numpy(), yr, S, ("random", N, K, B))
    for N, K, B in [(700, 4096, 3), (300, 14336, 8), (9, 512, 4)]:
        say(f"q6_k mfma zero-heavy B={B} {N}x{K}")
        W, x = wl.zero_heavy("q6_k", f"t/q6k/mzh/{N}x{K}", N, K, B=B)
        y = qmv.qmv_matvec_path("q6_k", dev(torch, W), N, K, dev(torch, x), qmv.PATH_MFMA)
        torch.cuda.synchronize()
        yr, S = oracle.matvec("q6_k", W, N, K, x)
        assert_tol(y.cpu().numpy(), yr, S, ("zero-heavy", N, K, B))


def test_q6k_mfma_columns_independent_and_x16(env):
    """On the matrix cores a column gives bitwise the same result at every
    width 2..8 and position, over repeated calls; f16/bf16 activations give
    bitwise the fp32 call on the widened values."""
    torch, qmv = env
    N, K = 1000, 4096
    Wd = dev(torch, wl.quant_weights("q6_k", "t/q6k/mdet", N, K))
    x = dev(torch, wl.activations("t/q6k/mdet/x", 8, K))
    full = qmv.qmv_matvec_path("q6_k", Wd, N, K, x, qmv.PATH_MFMA)
    for B in (2, 3, 5, 8):
        for off in (0, 8 - B):
            y = qmv.qmv_matvec_path("q6_k", Wd, N, K, x[off:off + B], qmv.PATH_MFMA)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int32), full[off:off + B].view(torch.int32)), (B, off)
    for kind in ("f16", "bf16"):
        xh = x.to(torch.float16 if kind == "f16" else torch.bfloat16)
        y16 = qmv.qmv_matvec_xt("q6_k", Wd, N, K, xh, qmv.PATH_MFMA)
        y32 = qmv.qmv_matvec_path("q6_k", Wd, N, K, xh.float(), qmv.PATH_MFMA)
        torch.cuda.synchronize()
        assert torch.equal(y16.view(torch.int32), y32.view(torch.int32)), kind
