"""Parity of the HIP library with the oracle, on an MI355X.

Float paths: |y_gpu - y| <= 1e-4 * S + 1e-6 per output, S = sum_j |w_ij x_j|
(the accuracy bound of the matvec contract), against the fp64
dequantize-then-dot oracle.  Dequantized values and the int8 requant path:
bit-exact.  Inputs come from the seeded generators in workloads/, with the
shapes and distributions of the five workloads (small cases that span several
tiles and a ragged tail, then the full sizes, sampled rows where the oracle
would be slow).  All calls go through the C ABI via the Python binding.
"""
import functools
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from tests import hand_blocks as hb

pytestmark = pytest.mark.gpu

FMTS = ["q8_0", "q4_0", "q4_1"]


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


def gpu_matvec(env, fmt, W, N, K, x):
    torch, qmv = env
    f = {"q8_0": qmv.qmv_q8_0, "q4_0": qmv.qmv_q4_0, "q4_1": qmv.qmv_q4_1}[fmt]
    y = f(dev(torch, W), N, K, dev(torch, x))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_tol(y, yr, S, what=""):
    err = np.abs(y.astype(np.float64) - yr)
    tol = 1e-4 * S + 1e-6
    bad = err > tol
    assert not np.any(bad), (what, int(bad.sum()), float((err / tol).max()))
    return float((err / tol).max())


def random_blocks(seed, fmt, N, K):
    """Stored bytes with random codes and random finite fp16 scales
    (subnormals included)."""
    g = np.random.default_rng(seed)
    bb = wl.BLOCK_BYTES[fmt]
    raw = g.integers(0, 256, size=(N, K // 32, bb), dtype=np.uint8)
    for off in ([0] if fmt != "q4_1" else [0, 2]):
        e = g.integers(0, 31, size=(N, K // 32))
        f = g.integers(0, 1024, size=(N, K // 32))
        s = g.integers(0, 2, size=(N, K // 32))
        h = (s << 15) | (e << 10) | f
        raw[..., off] = h & 0xFF
        raw[..., off + 1] = h >> 8
    return raw.reshape(N, -1)


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("kind", ["encoded", "random_bytes"])
def test_dequant_bit_exact(env, fmt, kind):
    torch, qmv = env
    N, K = 37, 320          # 10 blocks per row: both block parities in every row
    say(f"dequant {fmt} {kind} {N}x{K}")
    if kind == "encoded":
        W = wl.quant_weights(fmt, f"t/deq/{fmt}", N, K)
    else:
        W = random_blocks(101, fmt, N, K)
    ref = oracle.dequant(fmt, W, N, K).astype(np.float32)
    got = qmv.qmv_dequant(fmt, dev(torch, W), N, K)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ hand blocks
@pytest.mark.parametrize("spec", hb.load()["blocks"], ids=lambda s: s["id"])
def test_hand_blocks(env, spec):
    blk = hb.block_bytes(spec)
    x = hb.x_vec(spec["x"])[None, :]
    y = gpu_matvec(env, spec["fmt"], blk, 1, 32, x)
    assert float(y[0, 0]) == float(np.float32(float(spec["y"]))), (spec["id"], y[0, 0])


# ------------------------------------------------------------------ small shapes
SMALL = [(1, 32), (7, 64), (37, 96), (130, 1024), (257, 768), (65, 4096), (5, 14336), (300, 2048),
         (33, 1056), (9, 35424)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [1, 2, 3, 5, 8])
def test_small_shapes(env, fmt, B):
    for N, K in SMALL:
        say(f"small {fmt} B={B} {N}x{K}")
        W = wl.quant_weights(fmt, f"t/small/{N}x{K}", N, K)
        x = wl.activations(f"t/small/x/{K}/{B}", B, K)
        y = gpu_matvec(env, fmt, W, N, K, x)
        yr, S = oracle.matvec(fmt, W, N, K, x)
        assert_tol(y, yr, S, (fmt, B, N, K))


@pytest.mark.parametrize("fmt", FMTS)
def test_random_byte_blocks(env, fmt):
    """Arbitrary stored bytes (any codes, any finite scale)."""
    N, K, B = 41, 1024, 3
    W = random_blocks(7, fmt, N, K)
    x = wl.activations("t/rb/x", B, K)
    y = gpu_matvec(env, fmt, W, N, K, x)
    yr, S = oracle.matvec(fmt, W, N, K, x)
    assert_tol(y, yr, S, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_contiguous_path_equals_per_block_path(env, fmt):
    """Rows of whole 64-block steps with 16-byte aligned W take the
    contiguous-chunk kernel where it is chosen; the same bytes at a 4-byte
    offset take the per-block kernel.  Same lane mapping and arithmetic:
    bitwise equal, and both within the bound of the oracle.  The shapes
    reach each launch choice: >= 8192 rows (Q8_0, 8 waves), >= 256 blocks
    per row (16 waves), the LDS fallbacks to 8 waves (30720 columns, loop
    staging) and 4 waves (32768 columns), Q4 rows of < 256 blocks (the
    per-block kernel with two rows per lane, aligned or not), and ragged
    row counts."""
    torch, qmv = env
    f = _chain_fn(qmv, fmt)
    for N, K in [(8193, 2048), (2100, 4096), (5, 8192), (129, 14336), (3, 30720), (2, 32768), (40000, 2048)]:
        W = wl.quant_weights(fmt, f"t/contig/{N}x{K}", N, K)
        x = wl.activations(f"t/contig/x/{K}", 1, K)
        Wd, xd = dev(torch, W), dev(torch, x)
        buf = torch.zeros(W.size + 16, dtype=torch.uint8, device="cuda:0")
        Wo = buf[4:4 + W.size]
        Wo.copy_(Wd.reshape(-1))
        assert Wd.data_ptr() % 16 == 0 and Wo.data_ptr() % 16 == 4
        y_c = f(Wd, N, K, xd[0])
        y_b = f(Wo, N, K, xd[0])
        torch.cuda.synchronize()
        assert torch.equal(y_c.view(torch.int32), y_b.view(torch.int32)), (N, K)
        yr, S = oracle.matvec(fmt, W, N, K, x)
        assert_tol(y_c.cpu().numpy(), yr, S, (fmt, N, K))

@pytest.mark.parametrize("fmt", FMTS)
def test_one_hot_columns_exact(env, fmt):
    """FMA kernels: x = e_j gives y_i = DEQ(W)_ij exactly (all other products
    are 0; Q4_1 weights are dequantized with one rounding, d*c + m, before
    the dot), at batch 8 and batch 1, on random bytes and scales."""
    torch, qmv = env
    N, K, B = 50, 1024, 8
    W = random_blocks(3, fmt, N, K)
    cols = [0, 1, 31, 32, 33, 511, 1000, 1023]
    x = np.zeros((B, K), dtype=np.float32)
    for b, j in enumerate(cols):
        x[b, j] = 1.0
    Wd, xd = dev(torch, W), dev(torch, x)
    y = qmv.qmv_matvec_path(fmt, Wd, N, K, xd, qmv.PATH_FMA).cpu().numpy()
    y1 = gpu_matvec(env, fmt, W, N, K, x[:1])
    deq = oracle.dequant(fmt, W, N, K).astype(np.float32)
    for b, j in enumerate(cols):
        assert np.array_equal(y[b], deq[:, j]), (fmt, j)
    assert np.array_equal(y1[0], deq[:, cols[0]])


@pytest.mark.parametrize("fmt", FMTS)
def test_batch_columns_equal_batch1_and_deterministic(env, fmt):
    """The FMA kernels give every batch column bitwise the batch-1 result;
    the entry point's own choice (the matrix-core kernel at this batch) is
    deterministic and within the bound."""
    torch, qmv = env
    N, K = 300, 4096
    W = wl.quant_weights(fmt, "t/b1/W", N, K)
    x = wl.activations("t/b1/x", 8, K)
    Wd, xd = dev(torch, W), dev(torch, x)
    y8 = qmv.qmv_matvec_path(fmt, Wd, N, K, xd, qmv.PATH_FMA)
    for b in range(8):
        y1 = qmv.qmv_matvec_path(fmt, Wd, N, K, xd[b:b + 1], qmv.PATH_FMA)
        assert torch.equal(y1[0].view(torch.int32), y8[b].view(torch.int32)), b
    ya = gpu_matvec(env, fmt, W, N, K, x)
    yb = gpu_matvec(env, fmt, W, N, K, x)
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32))
    yr, S = oracle.matvec(fmt, W, N, K, x)
    assert_tol(ya, yr, S, fmt)
    assert_tol(y8.cpu().numpy(), yr, S, fmt)


def test_strided_activations(env):
    torch, qmv = env
    N, K, B = 70, 2048, 3
    W = wl.quant_weights("q4_1", "t/str/W", N, K)
    xbig = wl.activations("t/str/x", B, K + 40)
    x = xbig[:, :K]
    xt = dev(torch, xbig)[:, :K]
    y = torch.zeros((B, N + 5), dtype=torch.float32, device="cuda:0")
    qmv.qmv_q4_1(dev(torch, W), N, K, xt, y=y[:, :N])
    torch.cuda.synchronize()
    yr, S = oracle.matvec("q4_1", W, N, K, x)
    assert_tol(y[:, :N].cpu().numpy(), yr, S)
    assert np.all(y[:, N:].cpu().numpy() == 0)     # nothing written beyond ldy's row


# ------------------------------------------------------------------ matrix-core path
# n_cols multiples of 256 (whole 8-block steps); row counts with ragged
# 16-row tiles; 8192 and 30720 columns need several activation chunks in
# LDS at batch 8 (and 30720 at every width).
MFMA_SHAPES = [(1, 256), (7, 512), (37, 768), (130, 1024), (65, 4096), (5, 14336), (300, 2048),
               (17, 2304), (33, 8192), (3, 30720), (1000, 4096)]


def mfma_matvec(env, fmt, Wd, N, K, xd, path=2):
    torch, qmv = env
    y = qmv.qmv_matvec_path(fmt, Wd, N, K, xd, path)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [2, 3, 4, 7, 8])
def test_mfma_path_small_shapes(env, fmt, B):
    torch, qmv = env
    for N, K in MFMA_SHAPES:
        say(f"mfma {fmt} B={B} {N}x{K}")
        W = wl.quant_weights(fmt, f"t/small/{N}x{K}", N, K)
        x = wl.activations(f"t/small/x/{K}/{B}", B, K)
        y = mfma_matvec(env, fmt, dev(torch, W), N, K, dev(torch, x)).cpu().numpy()
        yr, S = oracle.matvec(fmt, W, N, K, x)
        assert_tol(y, yr, S, (fmt, B, N, K))


@pytest.mark.parametrize("fmt", FMTS)
def test_auto_path_rows_beyond_fma_staging(env, fmt):
    """36608 columns: one activation row does not fit the FMA kernels' LDS
    staging (at most 36384), so batch 1 is refused, and at batch 2..8 the
    automatic choice takes the matrix cores (bitwise the forced path, within
    the bound of the oracle) whatever the shape rule prefers."""
    torch, qmv = env
    N, K = 40, 36608
    W = wl.quant_weights(fmt, f"t/long/{N}x{K}", N, K)
    Wd = dev(torch, W)
    with pytest.raises(qmv.QmvError):
        qmv.qmv_matvec_path(fmt, Wd, N, K, dev(torch, wl.activations("t/long/x1", 1, K)), qmv.PATH_AUTO)
    for B in (2, 3, 8):
        say(f"long rows {fmt} B={B}")
        x = wl.activations(f"t/long/x/{B}", B, K)
        xd = dev(torch, x)
        ya = mfma_matvec(env, fmt, Wd, N, K, xd, qmv.PATH_AUTO)
        ym = mfma_matvec(env, fmt, Wd, N, K, xd, qmv.PATH_MFMA)
        assert torch.equal(ya.view(torch.int32), ym.view(torch.int32)), (fmt, B)
        yr, S = oracle.matvec(fmt, W, N, K, x)
        assert_tol(ya.cpu().numpy(), yr, S, (fmt, B))


@pytest.mark.parametrize("fmt", FMTS)
def test_mfma_path_random_bytes_and_scales(env, fmt):
    """Arbitrary codes and finite fp16 scales (subnormal to 65504), and
    activations over many binades: the split into two bf16 pieces keeps the
    bound."""
    torch, _ = env
    N, K, B = 45, 2048, 8
    W = random_blocks(17, fmt, N, K)
    g = np.random.default_rng(5)
    x = (g.standard_normal((B, K)) * np.exp2(g.integers(-30, 30, size=(B, K)))).astype(np.float32)
    y = mfma_matvec(env, fmt, dev(torch, W), N, K, dev(torch, x)).cpu().numpy()
    yr, S = oracle.matvec(fmt, W, N, K, x)
    assert_tol(y, yr, S, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_mfma_path_one_hot_exact(env, fmt):
    """x = e_j: hi = 1, lo = 0, one code times 1 in the dot, so y_i = DEQ(W)_ij
    exactly."""
    torch, _ = env
    N, K, B = 50, 1024, 8
    W = random_blocks(3, fmt, N, K)
    cols = [0, 1, 31, 32, 33, 511, 1000, 1023]
    x = np.zeros((B, K), dtype=np.float32)
    for b, j in enumerate(cols):
        x[b, j] = 1.0
    y = mfma_matvec(env, fmt, dev(torch, W), N, K, dev(torch, x)).cpu().numpy()
    deq64 = oracle.dequant(fmt, W, N, K)
    deq = deq64.astype(np.float32)
    exact = deq.astype(np.float64) == deq64
    for b, j in enumerate(cols):
        if fmt != "q4_1":
            assert np.array_equal(y[b], deq[:, j]), (fmt, j)
        else:
            # d (c - k) + mu with mu = m + d k rounded once: exact wherever
            # d c + m is exact in fp32 (every stored block whose value bits
            # span <= 24), else within one ulp of it (random scales here)
            e = exact[:, j]
            assert np.array_equal(y[b][e], deq[e, j]), (fmt, j)
            ulp = np.spacing(np.abs(deq[~e, j]))
            assert np.all(np.abs(y[b][~e].astype(np.float64) - deq64[~e, j]) <= ulp), (fmt, j)


@pytest.mark.parametrize("fmt", FMTS)
def test_mfma_path_columns_independent_and_deterministic(env, fmt):
    """A column's result depends on its own activations only: bitwise the same
    at any batch width 2..8 and position, and run to run."""
    torch, _ = env
    N, K = 300, 4096
    W = wl.quant_weights(fmt, "t/b1/W", N, K)
    Wd = dev(torch, W)
    x = wl.activations("t/b1/x", 8, K)
    xd = dev(torch, x)
    y8 = mfma_matvec(env, fmt, Wd, N, K, xd)
    y8b = mfma_matvec(env, fmt, Wd, N, K, xd)
    assert torch.equal(y8.view(torch.int32), y8b.view(torch.int32))
    for b in range(8):
        pair = dev(torch, np.stack([x[(b + 3) % 8], x[b]]))
        y2 = mfma_matvec(env, fmt, Wd, N, K, pair)
        assert torch.equal(y2[1].view(torch.int32), y8[b].view(torch.int32)), b
    y5 = mfma_matvec(env, fmt, Wd, N, K, xd[3:8])
    assert torch.equal(y5.view(torch.int32), y8[3:8].view(torch.int32))
    yr, S = oracle.matvec(fmt, W, N, K, x)
    assert_tol(y8.cpu().numpy(), yr, S, fmt)


def test_mfma_path_strided(env):
    torch, qmv = env
    N, K, B = 70, 2048, 3
    W = wl.quant_weights("q4_0", "t/str/W0", N, K)
    xbig = wl.activations("t/str/x", B, K + 40)
    xt = dev(torch, xbig)[:, :K]
    y = torch.zeros((B, N + 5), dtype=torch.float32, device="cuda:0")
    qmv.qmv_matvec_path("q4_0", dev(torch, W), N, K, xt, qmv.PATH_MFMA, y=y[:, :N])
    torch.cuda.synchronize()
    yr, S = oracle.matvec("q4_0", W, N, K, xbig[:, :K])
    assert_tol(y[:, :N].cpu().numpy(), yr, S)
    assert np.all(y[:, N:].cpu().numpy() == 0)


# ------------------------------------------------------------------ 16-bit activations
def _x16(torch, x, kind):
    """x (float32 numpy) rounded to fp16 / bf16 on the device, and the exact
    fp32 widening of those values."""
    t = dev(torch, x).to(torch.float16 if kind == "f16" else torch.bfloat16)
    return t, t.float()


X16_SHAPES = [(1, 32), (37, 96), (130, 1024), (65, 4096), (5, 14336), (300, 2048), (33, 1056), (2100, 4096)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_x16_activations_equal_widened_fp32(env, fmt, kind):
    """16-bit activations give bitwise the result of the fp32 call on the
    exactly widened activations, on every kernel family, and are within the
    bound of the oracle run on those widened values."""
    torch, qmv = env
    for N, K in X16_SHAPES:
        W = wl.quant_weights(fmt, f"t/small/{N}x{K}", N, K)
        Wd = dev(torch, W)
        for B in (1, 2, 3, 8):
            say(f"x16 {fmt} {kind} B={B} {N}x{K}")
            x = wl.activations(f"t/x16/{K}/{B}", B, K)
            xh, xw = _x16(torch, x, kind)
            for path in (qmv.PATH_AUTO, qmv.PATH_FMA, qmv.PATH_MFMA):
                if path == qmv.PATH_MFMA and (B == 1 or K % 256):
                    continue
                y16 = qmv.qmv_matvec_xt(fmt, Wd, N, K, xh, path)
                y32 = qmv.qmv_matvec_path(fmt, Wd, N, K, xw, path)
                torch.cuda.synchronize()
                assert torch.equal(y16.view(torch.int32), y32.view(torch.int32)), (N, K, B, path)
            yr, S = oracle.matvec(fmt, W, N, K, xw.cpu().numpy())
            assert_tol(y16.cpu().numpy(), yr, S, (fmt, kind, N, K, B))


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_x16_unaligned_and_strided(env, kind):
    """x at a 2-byte offset (element-wise staging, no matrix cores) and an
    odd row stride; fp16 subnormals and extreme values survive widening."""
    torch, qmv = env
    N, K, B = 70, 2048, 3
    W = wl.quant_weights("q4_1", "t/str/W", N, K)
    Wd = dev(torch, W)
    x = wl.activations("t/x16s/x", B, K + 7)
    # fp16: subnormal, smallest normal and largest values; bf16: far outside
    # the fp16 range (the block dot sum_j c_j x_j must stay finite in fp32)
    x[0, :5] = [6.0e-8, -6.1e-5, 65504.0, -3.0e30 if kind == "bf16" else -60000.0, 1e-30 if kind == "bf16" else 1e-7]
    dt = torch.float16 if kind == "f16" else torch.bfloat16
    big = torch.zeros(B * (K + 7) + 1, dtype=dt, device="cuda:0")
    xv = big[1:].view(B, K + 7)[:, :K]                  # 2-byte aligned only, ldx = K + 7
    xv.copy_(dev(torch, x[:, :K]).to(dt))
    assert xv.data_ptr() % 4 == 2
    # the fp32 reference with the same layout (4-byte offset, ldx = K + 7):
    # neither takes the matrix-core kernel
    big32 = torch.zeros(B * (K + 7) + 1, dtype=torch.float32, device="cuda:0")
    xw = big32[1:].view(B, K + 7)[:, :K]
    xw.copy_(xv.float())
    for path in (qmv.PATH_AUTO, qmv.PATH_FMA):
        y16 = qmv.qmv_matvec_xt("q4_1", Wd, N, K, xv, path)
        y32 = qmv.qmv_matvec_path("q4_1", Wd, N, K, xw, path)
        torch.cuda.synchronize()
        assert torch.equal(y16.view(torch.int32), y32.view(torch.int32)), path
    yr, S = oracle.matvec("q4_1", W, N, K, xv.float().cpu().numpy())
    assert_tol(y16.cpu().numpy(), yr, S)
    with pytest.raises(qmv.QmvError):
        qmv.qmv_matvec_xt("q4_1", Wd, N, K, xv, qmv.PATH_MFMA)


# ------------------------------------------------------------------ full sizes
@functools.lru_cache(maxsize=None)
def _float_weights(tag, N, K):
    return wl.weights_f32(tag, N, K)


def _encoded(fmt, tag, N, K):
    return wl.ENCODERS[fmt](_float_weights(tag, N, K))


def _sample_rows(N, n, seed):
    g = np.random.default_rng(seed)
    r = set(g.choice(N, size=min(n, N), replace=False).tolist()) | {0, N - 1}
    return np.array(sorted(r), dtype=np.int64)


def test_config_q8_0_1024(env):
    """Q8_0 1024 x 1024, batch 1, all rows."""
    N = K = 1024
    W = wl.quant_weights("q8_0", "cfg0/W", N, K)
    x = wl.activations("cfg0/x", 1, K)
    y = gpu_matvec(env, "q8_0", W, N, K, x)
    yr, S = oracle.matvec("q8_0", W, N, K, x)
    r = assert_tol(y, yr, S)
    say(f"cfg0 max err/tol {r:.3g}")


@pytest.mark.parametrize("fmt,batches", [("q8_0", (1,)), ("q4_0", (1, 2, 4, 8)), ("q4_1", (1, 2, 4, 8))])
def test_llama8b_layer_set(env, fmt, batches):
    """One 8B layer set + lm_head at full size (all layers share the shapes)."""
    torch, qmv = env
    mats = wl.LLAMA8B_LAYER + [wl.LLAMA8B_LM_HEAD]
    worst = 0.0
    for name, N, K in mats:
        W = _encoded(fmt, f"llama8b/{name}", N, K)
        Wd = dev(torch, W)
        for B in batches:
            say(f"llama8b {fmt} {name} {N}x{K} B={B}")
            x = wl.activations(f"llama8b/x/{name}/{B}", B, K)
            f = {"q8_0": qmv.qmv_q8_0, "q4_0": qmv.qmv_q4_0, "q4_1": qmv.qmv_q4_1}[fmt]
            y = f(Wd, N, K, dev(torch, x))
            torch.cuda.synchronize()
            y = y.cpu().numpy()
            full = (B == 1 and fmt == "q8_0" and name != "lm_head")
            rows = None if full else _sample_rows(N, 1024, N + B)
            yr, S = oracle.matvec(fmt, W, N, K, x, rows=rows)
            yy = y if rows is None else y[:, rows]
            worst = max(worst, assert_tol(yy, yr, S, (fmt, name, B)))
        del Wd
    say(f"llama8b {fmt} max err/tol {worst:.3g}")


# ------------------------------------------------------------------ int8 requant
def gpu_i8(env, W, x, mult, shift):
    torch, qmv = env
    y = qmv.qmv_i8_requant(dev(torch, W), dev(torch, x), dev(torch, mult), dev(torch, shift))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_int8_qwen06b_shapes_bit_exact(env):
    """Every Qwen3-0.6B-shaped matrix, uniform int8 W and x, mult in
    [2^30, 2^31), shift 0..20; bit-exact."""
    mats = wl.QWEN06B_LAYER + [wl.QWEN06B_LM_HEAD]
    for name, N, K in mats:
        say(f"int8 {name} {N}x{K}")
        W = wl.int8_uniform(f"qwen/W/{name}", (N, K))
        x = wl.int8_uniform(f"qwen/x/{name}", (1, K))
        mult, shift = wl.requant_params(f"qwen/ms/{name}", N)
        y = gpu_i8(env, W, x, mult, shift)
        _, yr = oracle.matvec_i8(W, x, mult, shift)
        assert np.array_equal(y, yr), name


def test_int8_calibrated_shift_and_batch(env):
    """Shifts chosen so outputs do not saturate (exercises the rounding
    paths), batch 1..8, a ragged row count."""
    N, K = 1000, 3072
    W = wl.int8_uniform("qwen/cal/W", (N, K))
    g = np.random.default_rng(5)
    mult = g.integers(1 << 30, 1 << 31, size=N).astype(np.int32)
    sigma = 127 * 127 / np.sqrt(3) * np.sqrt(K) / np.sqrt(3)
    # smallest e with 3 sigma * mult / 2^31 / 2^e <= 127
    e = np.ceil(np.log2(3 * sigma * mult.astype(np.float64) / 2 ** 31 / 127)).astype(np.int32)
    shift = np.clip(e, 0, 31).astype(np.int32)
    for B in (1, 2, 3, 8):
        x = wl.int8_uniform(f"qwen/cal/x/{B}", (B, K))
        y = gpu_i8(env, W, x, mult, shift)
        _, yr = oracle.matvec_i8(W, x, mult, shift)
        assert np.array_equal(y, yr), B
        sat = np.mean((yr == 127) | (yr == -128))
        assert sat < 0.05


def test_int8_edges(env):
    """x and W at -128, negative and extreme multipliers, shifts 0 and 31,
    the largest n_cols, tiny shapes."""
    g = np.random.default_rng(8)
    for N, K in [(1, 16), (5, 48), (67, 1040), (3, 131056)]:
        say(f"int8 edge {N}x{K}")
        W = g.integers(-128, 128, size=(N, K), dtype=np.int8)
        W[0, :] = -128
        x = g.integers(-128, 128, size=(2, K), dtype=np.int8)
        x[0, :] = -128
        mult = g.integers(-(1 << 31), 1 << 31, size=N, dtype=np.int64).astype(np.int32)
        mult[0] = -(1 << 31)
        shift = g.integers(0, 32, size=N).astype(np.int32)
        shift[0] = 0
        if N > 1:
            shift[-1] = 31
        y = gpu_i8(env, W, x, mult, shift)
        _, yr = oracle.matvec_i8(W, x, mult, shift)
        assert np.array_equal(y, yr), (N, K)


def test_int8_pipelined_shapes(env):
    """The pipelined int8 form (n_cols a multiple of 1024, batch x n_cols <=
    32 KB) on what the Qwen3-0.6B shapes do not reach: tall ragged matrices
    (four rows per group, N % 4 != 0) at batch 1, 3 and 8 with and without
    a table, long rows (32 steps per row), single rows, odd row counts with
    two rows per group and the activations in registers (batch 1, 1..4
    steps per row), batch 1 at 5 steps (staged activations), and the sizes
    on either side of the LDS limit (batch 8 at 4096 columns: pipelined; at
    5120: the per-segment kernel); bit-exact against the oracle."""
    torch, qmv = env
    g = np.random.default_rng(21)
    lut = wl.int8_table("lut/random")
    for N, K, B in [(16387, 1024, 1), (16387, 1024, 3), (20001, 2048, 8), (513, 32768, 1), (1, 1024, 2),
                    (1, 1024, 1), (5, 2048, 1), (3, 3072, 1), (777, 4096, 1), (16383, 1024, 1), (77, 5120, 1),
                    (777, 4096, 8), (777, 5120, 8)]:
        say(f"int8 pipelined {N}x{K} B={B}")
        W = g.integers(-128, 128, size=(N, K), dtype=np.int8)
        x = g.integers(-128, 128, size=(B, K), dtype=np.int8)
        mult = g.integers(-(1 << 31), 1 << 31, size=N, dtype=np.int64).astype(np.int32)
        shift = g.integers(0, 32, size=N).astype(np.int32)
        Wd, xd, md, sd = dev(torch, W), dev(torch, x), dev(torch, mult), dev(torch, shift)
        y = qmv.qmv_i8_requant(Wd, xd, md, sd)
        yl = qmv.qmv_i8_requant_lut(Wd, xd, md, sd, dev(torch, lut))
        torch.cuda.synchronize()
        _, yr = oracle.matvec_i8(W, x, mult, shift)
        assert np.array_equal(y.cpu().numpy(), yr), (N, K, B)
        assert np.array_equal(yl.cpu().numpy(), lut[yr.astype(np.int64) + 128]), (N, K, B, "lut")


# ------------------------------------------------------------------ MoE
@functools.lru_cache(maxsize=None)
def _moe_experts(kind, N, K, E=wl.MOE_EXPERTS):
    W = wl.quant_weights("q4_0", f"moe/{kind}", E * N, K)
    return W.reshape(-1)


def gpu_moe(env, fmt, Wall, stride, E, N, K, ids, x):
    torch, qmv = env
    y = qmv.qmv_moe(fmt, dev(torch, Wall), stride, E, N, K, dev(torch, ids), dev(torch, x))
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("B", [1, 2, 3, 4, 8])
def test_moe_30b_a3b_shapes(env, B):
    """128 Q4_0 experts, top-8 distinct ids per token; gate/up 768x2048 with
    one input per token, down 2048x768 with one input per (token, slot)."""
    E, T = wl.MOE_EXPERTS, wl.MOE_TOPK
    H, F = wl.MOE_HIDDEN, wl.MOE_FFN
    ids = wl.moe_ids(f"moe/ids/{B}", B, T, E)
    for kind, N, K in [("gate", F, H), ("down", H, F)]:
        say(f"moe {kind} B={B}")
        Wall = _moe_experts(kind, N, K)
        stride = wl.block_bytes("q4_0", N, K)
        if kind == "gate":
            x = wl.activations(f"moe/x/{kind}/{B}", B, K)
            yr, S = oracle.moe("q4_0", Wall, stride, E, N, K, ids, x)
        else:
            x = wl.activations(f"moe/x/{kind}/{B}", B * T, K).reshape(B, T, K)
            yr, S = oracle.moe("q4_0", Wall, stride, E, N, K, ids, None, x_slots=x)
        y = gpu_moe(env, "q4_0", Wall, stride, E, N, K, ids, x)
        assert_tol(y, yr, S, (kind, B))


@pytest.mark.parametrize("case", ["shared", "disjoint", "duplicates", "many_dup"])
def test_moe_routing_edge_cases(env, case):
    E, N, K = 16, 96, 512
    fmt = "q4_0"
    per = wl.block_bytes(fmt, N, K)
    stride = per + 64
    Wq = wl.quant_weights(fmt, "moe/edge/W", E * N, K).reshape(E, per)
    Wall = np.zeros((E, stride), dtype=np.uint8)
    Wall[:, :per] = Wq
    Wall = Wall.reshape(-1)
    if case == "shared":
        ids = np.tile(np.array([3, 1, 4, 15], dtype=np.int32), (8, 1))
    elif case == "disjoint":
        ids = np.arange(16, dtype=np.int32).reshape(8, 2)
    elif case == "duplicates":
        ids = np.array([[2, 2, 5], [5, 2, 2]], dtype=np.int32)
    else:                      # one expert used by 12 pairs: two groups of <= 8
        ids = np.full((4, 3), 7, dtype=np.int32)
    B, T = ids.shape
    x = wl.activations(f"moe/edge/x/{case}", B * T, K).reshape(B, T, K)
    y = gpu_moe(env, fmt, Wall, stride, E, N, K, ids, x)
    yr, S = oracle.moe(fmt, Wall, stride, E, N, K, ids, None, x_slots=x)
    assert_tol(y, yr, S, case)
    # each pair equals the plain single-expert matvec of its expert, bitwise
    torch, qmv = env
    for b in range(B):
        for s in range(T):
            e = int(ids[b, s])
            y1 = gpu_matvec(env, fmt, Wq[e], N, K, x[b, s][None])
            assert np.array_equal(y1[0].view(np.uint32), y[b, s].view(np.uint32))


@pytest.mark.parametrize("case", ["dup_invalid", "long_rows", "unaligned_slots"])
def test_moe_batch1_paths(env, case):
    """One token: its pairs run as separate grid rows of the dense kernel
    (no grouping; a duplicated id streams that expert twice, the second time
    mostly from cache), or, when the activations cannot be staged
    straight-line (rows of > 16384 columns, or slot strides that break
    16-byte alignment), through the grouping kernel.  Either way each valid pair equals the single-expert dense call
    bitwise, invalid ids give NaN, and the result is within the bound."""
    torch, qmv = env
    fmt = "q4_1"
    E = 5
    if case == "dup_invalid":
        N, K, ids, slot_pad = 200, 2048, np.array([[3, 3, 9, -1, 0, 3]], dtype=np.int32), 0
    elif case == "long_rows":
        N, K, ids, slot_pad = 40, 16416, np.array([[1, 4, 1]], dtype=np.int32), 0
    else:
        N, K, ids, slot_pad = 64, 768, np.array([[2, 0, 2, 4]], dtype=np.int32), 1
    per = wl.block_bytes(fmt, N, K)
    Wq = wl.quant_weights(fmt, f"moe/b1/{case}", E * N, K).reshape(E, per)
    Wall = Wq.reshape(-1)
    T = ids.shape[1]
    xs = wl.activations(f"moe/b1/x/{case}", T, K)
    ld = K + slot_pad                     # slot stride in floats
    xbuf = np.zeros((T, ld), dtype=np.float32)
    xbuf[:, :K] = xs
    xd = torch.from_numpy(xbuf.reshape(-1)).to("cuda:0")
    Wd, idsd = dev(torch, Wall), dev(torch, ids)
    yd = torch.full((T * N,), float("nan"), device="cuda:0")
    rc = qmv.lib().qmv_moe(qmv.FORMATS[fmt], Wd.data_ptr(), per, E, N, K, idsd.data_ptr(), 1, T, xd.data_ptr(),
                           T * ld, ld, yd.data_ptr(), None)
    assert rc == 0, qmv.last_error()
    torch.cuda.synchronize()
    y = yd.cpu().numpy().reshape(1, T, N)
    valid = (ids >= 0) & (ids < E)
    assert np.all(np.isnan(y[~valid]))
    for s in range(T):
        if not valid[0, s]:
            continue
        e = int(ids[0, s])
        y1 = gpu_matvec(env, fmt, Wq[e], N, K, xs[s][None])
        assert np.array_equal(y1[0].view(np.uint32), y[0, s].view(np.uint32)), (case, s)
        yr, S = oracle.matvec(fmt, Wq[e], N, K, xs[s][None])
        assert_tol(y[0, s][None], yr, S, (case, s))


@pytest.mark.parametrize("fmt", FMTS)
def test_moe_formats_and_invalid_ids(env, fmt):
    E, N, K = 5, 70, 256
    per = wl.block_bytes(fmt, N, K)
    Wall = wl.quant_weights(fmt, f"moe/fmt/{fmt}", E * N, K).reshape(-1)
    ids = np.array([[0, 4], [9, 1], [4, -1]], dtype=np.int32)
    x = wl.activations(f"moe/fmt/x/{fmt}", 3, K)
    y = gpu_moe(env, fmt, Wall, per, E, N, K, ids, x)
    valid = (ids >= 0) & (ids < E)
    assert np.all(np.isnan(y[~valid]))
    ids_ok = np.where(valid, ids, 0).astype(np.int32)
    yr, S = oracle.moe(fmt, Wall, per, E, N, K, ids_ok, x)
    assert_tol(y[valid], yr[valid], S[valid], fmt)


# ------------------------------------------------------------------ chain
def _chain_fn(qmv, fmt):
    return {"q8_0": qmv.qmv_q8_0, "q4_0": qmv.qmv_q4_0, "q4_1": qmv.qmv_q4_1}[fmt]


@pytest.mark.parametrize("fmt", FMTS)
def test_chain_independent_stages(env, fmt):
    """Stages that do not wait: each equals the batch-1 entry point bitwise
    (>= 64 blocks per row) or the oracle within the bound (shorter rows)."""
    torch, qmv = env
    shapes = [(300, 4096), (1024, 2048), (77, 14336), (130, 1024), (40, 768), (2000, 4096)]
    ws = torch.zeros(qmv.CHAIN_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    stages, keep = [], []
    for i, (N, K) in enumerate(shapes):
        W = wl.quant_weights(fmt, f"t/chain/{N}x{K}", N, K)
        x = wl.activations(f"t/chain/x/{i}", 1, K)
        Wd, xd = dev(torch, W), dev(torch, x)
        yd = torch.full((N,), float("nan"), device="cuda:0")
        stages.append((Wd, N, K, xd[0], yd, 0))
        keep.append((W, x, N, K))
    qmv.qmv_chain(fmt, stages, ws)
    torch.cuda.synchronize()
    assert int(ws.view(torch.int32)[2].item()) == 0
    for (Wd, N, K, xd, yd, _), (W, x, _, _) in zip(stages, keep):
        y = yd.cpu().numpy()
        if K >= 2048:
            ref = _chain_fn(qmv, fmt)(Wd, N, K, xd)
            torch.cuda.synchronize()
            assert np.array_equal(y.view(np.uint32), ref.cpu().numpy()[0].view(np.uint32)), (N, K)
        yr, S = oracle.matvec(fmt, W, N, K, x)
        assert_tol(y[None], yr, S, (fmt, N, K))


@pytest.mark.parametrize("fmt", ["q8_0", "q4_1"])
def test_chain_dependent_stages(env, fmt):
    """x of stage s+1 is y of stage s (square 2048 x 2048 layers, more stages
    than one launch holds; whole 2048-column windows, so the streaming
    decode kernel runs it): every stage within the bound of the oracle on
    its own input, bitwise the same over repeated calls (deterministic, and
    the workspace's barrier words stay consistent), and within the bound of
    sequential batch-1 calls."""
    torch, qmv = env
    N = K = 2048
    n_stages = 70
    Ws = [dev(torch, wl.quant_weights(fmt, f"t/chain/dep/{i % 5}", N, K)) for i in range(n_stages)]
    x0 = dev(torch, wl.activations("t/chain/dep/x", 1, K))[0]
    ys = [torch.empty(N, device="cuda:0") for _ in range(n_stages)]
    stages = [(Ws[i], N, K, x0 if i == 0 else ys[i - 1], ys[i], 1) for i in range(n_stages)]
    ws = torch.zeros(qmv.CHAIN_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    ref = []
    cur = x0
    for i in range(n_stages):
        cur = _chain_fn(qmv, fmt)(Ws[i], N, K, cur)[0]
        ref.append(cur)
    torch.cuda.synchronize()
    first = None
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        qmv.qmv_chain(fmt, stages, ws)
        torch.cuda.synchronize()
        assert int(ws.view(torch.int32)[2].item()) == 0
        if first is None:
            first = [y.clone() for y in ys]
        for i in range(n_stages):
            assert torch.equal(ys[i].view(torch.int32), first[i].view(torch.int32)), (rep, i)
    # the oracle on every stage's own input (as the chain computed it)
    Wh = {}
    for i in range(n_stages):
        key = i % 5
        if key not in Wh:
            Wh[key] = Ws[i].cpu().numpy()
        xin = (x0 if i == 0 else ys[i - 1]).cpu().numpy()[None]
        yr, S = oracle.matvec(fmt, Wh[key], N, K, xin)
        assert_tol(ys[i].cpu().numpy()[None], yr, S, (fmt, i))
    # the sequential batch-1 calls, stage by stage on the chain's inputs
    for i in range(n_stages):
        xin = x0 if i == 0 else ys[i - 1]
        r = _chain_fn(qmv, fmt)(Ws[i], N, K, xin)[0].cpu().numpy()
        yr, S = oracle.matvec(fmt, Wh[i % 5], N, K, xin.cpu().numpy()[None])
        err = np.abs(ys[i].cpu().numpy().astype(np.float64) - r)
        assert np.all(err <= 2 * (1e-4 * S[0] + 1e-6)), (fmt, i)
    last = first[-1].cpu().numpy()
    assert np.isfinite(last).all() and np.abs(last).max() > 1e-3   # the chain did not decay or blow up


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_chain_decode_pattern(env, fmt):
    """Decode-shaped dependencies over 12 layers (72 stages, two launches):
    q and k read the layer input, o reads q, gate and up read o, down reads
    up and is the next layer's input.  k and up do not wait: they read an
    output of the chain that the barrier of the stage before them (q, gate)
    already made visible.  Every output equals the sequential batch-1 calls
    bitwise."""
    torch, qmv = env
    H, F = 2048, 5632
    mats = {"q": (H, H), "k": (512, H), "o": (H, H), "gate": (F, H), "up": (F, H), "down": (H, F)}
    Wd = {(m, v): dev(torch, wl.quant_weights(fmt, f"t/chain/dec/{m}/{v}", N, K))
          for m, (N, K) in mats.items() for v in range(2)}
    h0 = dev(torch, wl.activations("t/chain/dec/h", 1, H))[0]
    stages, outs = [], []
    h = h0
    for layer in range(12):
        y = {m: torch.full((N,), float("nan"), device="cuda:0") for m, (N, _) in mats.items()}
        W = {m: Wd[(m, layer % 2)] for m in mats}
        stages += [(W["q"], H, H, h, y["q"], 1), (W["k"], 512, H, h, y["k"], 0),
                   (W["o"], H, H, y["q"], y["o"], 1), (W["gate"], F, H, y["o"], y["gate"], 1),
                   (W["up"], F, H, y["o"], y["up"], 0), (W["down"], H, F, y["up"], y["down"], 1)]
        outs.append(y)
        h = y["down"]
    ws = torch.zeros(qmv.CHAIN_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    qmv.qmv_chain(fmt, stages, ws)
    torch.cuda.synchronize()
    assert int(ws.view(torch.int32)[2].item()) == 0
    f = _chain_fn(qmv, fmt)
    for i, (W, N, K, x, y, _) in enumerate(stages):
        ref = f(W, N, K, x)[0]        # x as the chain computed it: checks each stage on its own input
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), i
    # the oracle on the last layer's six stages, each on its own input
    for i in range(len(stages) - 6, len(stages)):
        W, N, K, x, y, _ = stages[i]
        yr, S = oracle.matvec(fmt, W.cpu().numpy(), N, K, x.cpu().numpy()[None])
        assert_tol(y.cpu().numpy()[None], yr, S, (fmt, i))
    last = outs[-1]["down"].cpu().numpy()
    assert np.isfinite(last).all() and np.abs(last).max() > 1e-3


@pytest.mark.parametrize("fmt", FMTS)
def test_chain_shared_input_groups(env, fmt):
    """Stages that read one x and do not wait: up to 4 run as one matvec over
    their concatenated rows (the launch the grouped batch-1 decode step
    times for q||k||v and gate||up), more through the streaming decode
    kernel (whole 2048-column windows) or, with a misaligned W, the
    per-stage chain kernel.  Every output is checked against the oracle
    within the bound (all rows, or 1024 sampled rows plus both ends of each
    matrix of the 8B gate||up group); outside the streaming kernel each
    also equals the batch-1 entry point on its own matrix bitwise (>= 64
    blocks per row)."""
    torch, qmv = env
    f = _chain_fn(qmv, fmt)
    ws = torch.zeros(qmv.CHAIN_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    groups = {
        # the 8B decode groups: q||k||v and gate||up at 4096 columns
        "qkv_8b": [(4096, 4096), (1024, 4096), (1024, 4096)],
        "gate_up_8b": [(14336, 4096), (14336, 4096)],
        "gate_up": [(3000, 2048), (3000, 2048)],
        "five": [(300, 2048), (77, 2048), (1, 2048), (513, 2048), (64, 2048)],
        "misaligned": [(700, 2048), (129, 2048)],
        # > 8192 rows: Q4 takes two rows per wave step; a row pair straddles
        # the two matrices and the last pair has one row
        "big_odd": [(5001, 2048), (4000, 2048)],
    }
    for gname, shapes in groups.items():
        say(f"chain group {fmt} {gname}")
        K = shapes[0][1]
        xh = wl.activations(f"t/chain/grp/{gname}/x", 1, K)
        x = dev(torch, xh)[0]
        stages, mats = [], []
        for i, (N, _) in enumerate(shapes):
            Wh = wl.quant_weights(fmt, f"t/chain/grp/{gname}/{i}", N, K)
            W = dev(torch, Wh).reshape(-1)
            if gname == "misaligned" and i == 1:
                buf = torch.zeros(W.numel() + 16, dtype=torch.uint8, device="cuda:0")
                buf[4:4 + W.numel()].copy_(W)
                W = buf[4:4 + W.numel()]
            y = torch.full((N,), float("nan"), device="cuda:0")
            stages.append((W, N, K, x, y, 0))
            mats.append((W, N, Wh))
        qmv.qmv_chain(fmt, stages, ws)
        torch.cuda.synchronize()
        assert int(ws.view(torch.int32)[2].item()) == 0
        for (W, N, Wh), st in zip(mats, stages):
            got = st[4].cpu().numpy()
            if N > 4096:
                rows = np.unique(np.concatenate([np.arange(64), np.arange(N - 64, N),
                                                 np.random.default_rng(N).choice(N, size=1024, replace=False)]))
                yr, S = oracle.matvec(fmt, Wh, N, K, xh, rows=rows)
                assert_tol(got[rows][None], yr, S, (gname, N))
            else:
                yr, S = oracle.matvec(fmt, Wh, N, K, xh)
                assert_tol(got[None], yr, S, (gname, N))
            if gname == "five":
                continue        # five stages of whole windows: the streaming decode kernel (oracle only)
            ref = f(W, N, K, x)[0]
            torch.cuda.synchronize()
            assert torch.equal(st[4].view(torch.int32), ref.view(torch.int32)), (gname, N)


# ------------------------------------------------------------------ fused steps
def silu_table(s_in, s_out):
    """An int8 SiLU table of the frozen-table kind, written out here from the
    closed form (example data for the table step, which itself only looks
    entries up): entry v + 128 = clamp(round(SiLU(v s_in) / s_out))."""
    v = np.arange(-128, 128, dtype=np.float64) * s_in
    r = v / (1.0 + np.exp(-v)) / s_out
    return np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -128, 127).astype(np.int8)


def test_int8_lut_bit_exact(env):
    """The requant output through a frozen table: a SiLU table, a random
    table and the identity (which must equal qmv_i8_requant); Qwen3-0.6B
    gate shape, batch 1..8, a ragged shape; bit-exact."""
    torch, qmv = env
    tables = {"silu": silu_table(1 / 16, 1 / 16), "random": wl.int8_table("lut/random"),
              "identity": (np.arange(256) - 128).astype(np.int8)}
    assert tables["silu"][128 + 16] == 12 and tables["silu"][128 - 16] == -4 and tables["silu"][128] == 0
    for (N, K), B in [((3072, 1024), 1), ((3072, 1024), 8), ((77, 1040), 3)]:
        W = wl.int8_uniform(f"lut/W/{N}", (N, K))
        x = wl.int8_uniform(f"lut/x/{N}/{B}", (B, K))
        g = np.random.default_rng(N)
        mult = g.integers(1 << 30, 1 << 31, size=N).astype(np.int32)
        sigma = 127 * 127 / 3 * np.sqrt(K)
        shift = np.clip(np.ceil(np.log2(3 * sigma * mult / 2 ** 31 / 127)), 0, 31).astype(np.int32)
        Wd, xd, md, sd = dev(torch, W), dev(torch, x), dev(torch, mult), dev(torch, shift)
        plain = qmv.qmv_i8_requant(Wd, xd, md, sd)
        for name, lut in tables.items():
            say(f"int8 lut {name} {N}x{K} B={B}")
            y = qmv.qmv_i8_requant_lut(Wd, xd, md, sd, dev(torch, lut))
            torch.cuda.synchronize()
            _, yr = oracle.matvec_i8_lut(W, x, mult, shift, lut)
            assert np.array_equal(y.cpu().numpy(), yr), (name, N, B)
            if name == "identity":
                assert torch.equal(y, plain)


def swiglu_bound(h, g, u, Sg, Su):
    """|h_gpu - h| for h = SiLU(g) u from fp32 g, u within the matvec bound
    (tg, tu): |SiLU'| <= 1.1, so |dh| <= 1.1 tg (|u| + tu) + (|SiLU(g)| +
    1.1 tg) tu, plus the fp32 epilogue (a few ulps of h)."""
    tg, tu = 1e-4 * Sg + 1e-6, 1e-4 * Su + 1e-6
    sg = np.abs(g / (1.0 + np.exp(-g)))
    return 1.1 * tg * (np.abs(u) + tu) + (sg + 1.1 * tg) * tu + 2.0 ** -20 * np.abs(h) + 1e-30


def gpu_swiglu(env, fmt, Wall, stride, E, F, K, ids, x):
    torch, qmv = env
    h = qmv.qmv_moe_swiglu(fmt, dev(torch, Wall), stride, E, F, K, dev(torch, ids), dev(torch, x))
    torch.cuda.synchronize()
    return h.cpu().numpy()


@pytest.mark.parametrize("B", [1, 2, 8])
def test_moe_swiglu_30b_a3b(env, B):
    """128 Q4_0 experts of gate||up 1536 x 2048, top-8 per token: h against
    the fp64 oracle within the propagated bound, and the gate and up sums
    bitwise those of qmv_moe on the same experts."""
    torch, qmv = env
    E, T, H, F = wl.MOE_EXPERTS, wl.MOE_TOPK, wl.MOE_HIDDEN, wl.MOE_FFN
    gate = wl.quant_weights("q4_0", "moe/gate", E * F, H).reshape(E, -1)
    up = wl.quant_weights("q4_0", "moe/up", E * F, H).reshape(E, -1)
    Wall = np.concatenate([gate, up], axis=1).reshape(-1)
    stride = 2 * wl.block_bytes("q4_0", F, H)
    ids = wl.moe_ids(f"moe/swiglu/ids/{B}", B, T, E)
    x = wl.activations(f"moe/swiglu/x/{B}", B, H)
    say(f"moe swiglu B={B}")
    h = gpu_swiglu(env, "q4_0", Wall, stride, E, F, H, ids, x)
    rows = np.sort(np.random.default_rng(B).choice(F, size=96, replace=False))
    hr, g, u, Sg, Su = oracle.moe_swiglu("q4_0", Wall, stride, E, F, H, ids, x, rows=rows)
    err = np.abs(h[:, :, rows].astype(np.float64) - hr)
    assert np.all(err <= swiglu_bound(hr, g, u, Sg, Su)), float((err / swiglu_bound(hr, g, u, Sg, Su)).max())
    # the gate and up sums are qmv_moe's: h == SiLU(g32) * u32 up to the epilogue's rounding
    y = gpu_moe(env, "q4_0", Wall, stride, E, 2 * F, H, ids, x).astype(np.float64)
    g32, u32 = y[:, :, :F], y[:, :, F:]
    href = g32 / (1.0 + np.exp(-g32)) * u32
    assert np.all(np.abs(h - href) <= 2.0 ** -21 * np.abs(href) + 1e-37)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", ["dup_invalid", "strided", "long_rows"])
def test_moe_swiglu_edges(env, fmt, case):
    """Duplicated and invalid ids (NaN rows), per-slot inputs with an odd
    stride, rows of 16416 columns (looping stager); all rows against the
    oracle."""
    torch, qmv = env
    E = 5
    if case == "dup_invalid":
        F, K, ids, pad = 40, 1024, np.array([[3, 3, 9], [0, -1, 3]], dtype=np.int32), 0
    elif case == "strided":
        F, K, ids, pad = 72, 768, np.array([[2, 0, 4, 1], [4, 4, 1, 0]], dtype=np.int32), 1
    else:
        F, K, ids, pad = 24, 16416, np.array([[1, 4]], dtype=np.int32), 0
    B, T = ids.shape
    per = wl.block_bytes(fmt, 2 * F, K)
    Wall = wl.quant_weights(fmt, f"moe/swiglu/{case}", E * 2 * F, K).reshape(-1)
    say(f"moe swiglu edge {fmt} {case}")
    if case == "strided":
        ld = K + pad
        xs = wl.activations(f"moe/swiglu/x/{case}", B * T, K).reshape(B, T, K)
        buf = np.zeros((B * T, ld), dtype=np.float32)
        buf[:, :K] = xs.reshape(B * T, K)
        hd = torch.empty((B, T, F), dtype=torch.float32, device="cuda:0")
        Wd, idsd, xd = dev(torch, Wall), dev(torch, ids), dev(torch, buf.reshape(-1))   # alive across the call
        rc = qmv.lib().qmv_moe_swiglu(qmv.FORMATS[fmt], Wd.data_ptr(), per, E, F, K, idsd.data_ptr(), B, T,
                                      xd.data_ptr(), T * ld, ld, hd.data_ptr(), None)
        assert rc == 0, qmv.last_error()
        torch.cuda.synchronize()
        h = hd.cpu().numpy()
        hr, g, u, Sg, Su = oracle.moe_swiglu(fmt, Wall, per, E, F, K, ids, None, x_slots=xs)
    else:
        x = wl.activations(f"moe/swiglu/x/{case}", B, K)
        h = gpu_swiglu(env, fmt, Wall, per, E, F, K, ids, x)
        valid = (ids >= 0) & (ids < E)
        assert np.all(np.isnan(h[~valid]))
        ids_ok = np.where(valid, ids, 0).astype(np.int32)
        hr, g, u, Sg, Su = oracle.moe_swiglu(fmt, Wall, per, E, F, K, ids_ok, x)
        h, hr, g, u, Sg, Su = (a[valid] for a in (h, hr, g, u, Sg, Su))
    err = np.abs(h.astype(np.float64) - hr)
    assert np.all(err <= swiglu_bound(hr, g, u, Sg, Su)), (case, float((err / swiglu_bound(hr, g, u, Sg, Su)).max()))


def combine_bound(S, w):
    """The combine's bound: the weighted matvec bounds plus the fp32
    multiply-add chain over at most 16 slots."""
    return (1e-4 + 16 * 2.0 ** -24) * S + 1e-6 * np.abs(w).sum(axis=1, keepdims=True) + 1e-30


def gpu_combine(env, fmt, Wall, stride, E, N, K, ids, w, x):
    torch, qmv = env
    out = qmv.qmv_moe_combine(fmt, dev(torch, Wall), stride, E, N, K, dev(torch, ids), dev(torch, w), dev(torch, x))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("B", [1, 2, 8])
def test_moe_combine_30b_a3b(env, B):
    """128 Q4_0 down experts 2048 x 768, one input per (token, slot), router
    weights summing to 1: against the fp64 oracle, and against the
    weighted sum of qmv_moe's per-slot outputs (the same per-slot sums)."""
    torch, qmv = env
    E, T, H, F = wl.MOE_EXPERTS, wl.MOE_TOPK, wl.MOE_HIDDEN, wl.MOE_FFN
    Wall = _moe_experts("down", H, F)
    stride = wl.block_bytes("q4_0", H, F)
    ids = wl.moe_ids(f"moe/combine/ids/{B}", B, T, E)
    w = wl.router_weights(f"moe/combine/w/{B}", B, T)
    x = wl.activations(f"moe/combine/x/{B}", B * T, F).reshape(B, T, F)
    say(f"moe combine B={B}")
    out = gpu_combine(env, "q4_0", Wall, stride, E, H, F, ids, w, x)
    ref, S = oracle.moe_combine("q4_0", Wall, stride, E, H, F, ids, w, x_slots=x)
    err = np.abs(out.astype(np.float64) - ref)
    assert np.all(err <= combine_bound(S, w)), float((err / combine_bound(S, w)).max())
    y = gpu_moe(env, "q4_0", Wall, stride, E, H, F, ids, x).astype(np.float64)
    mix = np.einsum("bs,bsn->bn", w.astype(np.float64), y)
    assert np.all(np.abs(out - mix) <= T * 2.0 ** -24 * np.einsum("bs,bsn->bn", np.abs(w), np.abs(y)) + 1e-37)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", ["one_hot_dup", "invalid", "chunked_slots", "token_inputs"])
def test_moe_combine_edges(env, fmt, case):
    """One-hot weights (out equals one slot's qmv_moe output bitwise),
    duplicated ids, an invalid id (the token's row becomes NaN), top_k 16 on
    rows of 16384 columns (slot vectors staged in several chunks, rows in
    several ranges), one input per token."""
    torch, qmv = env
    E = 6
    if case == "one_hot_dup":
        N, K, ids = 300, 1024, np.array([[2, 5, 2], [0, 0, 1]], dtype=np.int32)
    elif case == "invalid":
        N, K, ids = 96, 512, np.array([[1, 3], [7, 2], [4, 4]], dtype=np.int32)
    elif case == "chunked_slots":
        N, K, ids = 4200, 16384, np.array([[i % E for i in range(16)]], dtype=np.int32)
    else:
        N, K, ids = 128, 2048, np.array([[5, 1, 0, 3], [2, 2, 4, 1]], dtype=np.int32)
    B, T = ids.shape
    per = wl.block_bytes(fmt, N, K)
    Wall = wl.quant_weights(fmt, f"moe/combine/{case}", E * N, K).reshape(-1)
    w = wl.router_weights(f"moe/combine/w/{case}", B, T)
    say(f"moe combine edge {fmt} {case}")
    if case == "token_inputs":
        x = wl.activations(f"moe/combine/x/{case}", B, K)
        out = gpu_combine(env, fmt, Wall, per, E, N, K, ids, w, x)
        ref, S = oracle.moe_combine(fmt, Wall, per, E, N, K, ids, w, x_tokens=x)
    else:
        x = wl.activations(f"moe/combine/x/{case}", B * T, K).reshape(B, T, K)
        if case == "one_hot_dup":
            w = np.zeros((B, T), dtype=np.float32)
            w[0, 2] = 1.0
            w[1, 1] = 1.0
        out = gpu_combine(env, fmt, Wall, per, E, N, K, ids, w, x)
        if case == "invalid":
            valid = np.all((ids >= 0) & (ids < E), axis=1)
            assert np.all(np.isnan(out[~valid])) and not np.any(np.isnan(out[valid]))
            ids_ok = np.where((ids >= 0) & (ids < E), ids, 0).astype(np.int32)
            ref, S = oracle.moe_combine(fmt, Wall, per, E, N, K, ids_ok, w, x_slots=x)
            out, ref, S, w = out[valid], ref[valid], S[valid], w[valid]
        elif case == "chunked_slots":
            rows = np.sort(np.random.default_rng(3).choice(N, size=64, replace=False))
            rows[-1] = N - 1
            ref, S = oracle.moe_combine(fmt, Wall, per, E, N, K, ids, w, x_slots=x, rows=rows)
            out = out[:, rows]
        else:
            ref, S = oracle.moe_combine(fmt, Wall, per, E, N, K, ids, w, x_slots=x)
            y = gpu_moe(env, fmt, Wall, per, E, N, K, ids, x)
            assert np.array_equal(out[0].view(np.uint32), y[0, 2].view(np.uint32))
            assert np.array_equal(out[1].view(np.uint32), y[1, 1].view(np.uint32))
    err = np.abs(out.astype(np.float64) - ref)
    assert np.all(err <= combine_bound(S, w)), (case, float((err / combine_bound(S, w)).max()))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_moe_x16_equals_widened_fp32(env, fmt, kind):
    """qmv_moe_xt and qmv_moe_swiglu_xt with 16-bit activations equal, bitwise,
    qmv_moe / qmv_moe_swiglu on the exactly widened activations: the
    per-pair route (aligned activations of <= 16384 columns, any batch) and
    the grouping kernel (longer rows, x at a 2-byte offset), per-token and
    per-slot inputs, duplicated ids; within the bound of the oracle on the
    widened values."""
    torch, qmv = env
    E = 6
    cases = [("b1_tok", 1, 256, 2048, [[4, 1, 4, 0]], False, 0),
             ("b8_tok", 8, 96, 1024, None, False, 0),
             ("b3_slot", 3, 64, 768, [[0, 5, 2], [2, 2, 1], [5, 0, 3]], True, 0),
             ("b2_long", 2, 40, 16416, [[1, 3], [3, 5]], False, 0),
             ("b2_offset", 2, 72, 512, [[2, 0], [1, 2]], True, 1)]
    for name, B, N, K, ids, per_slot, off in cases:
        say(f"moe x16 {fmt} {kind} {name}")
        T = 4 if ids is None else len(ids[0])
        ids_np = wl.moe_ids(f"moe/x16/ids/{name}", B, T, E) if ids is None else np.array(ids, dtype=np.int32)
        Wall = wl.quant_weights(fmt, f"moe/x16/W/{name}", E * 2 * N, K).reshape(-1)
        per = wl.block_bytes(fmt, 2 * N, K)
        shape = (B, T, K) if per_slot else (B, K)
        x = wl.activations(f"moe/x16/x/{name}", int(np.prod(shape[:-1])), K).reshape(shape)
        xh, xw = _x16(torch, x, kind)
        if off:
            # the same values one element into a larger buffer: 2-byte aligned only
            buf = torch.zeros(xh.numel() + 1, dtype=xh.dtype, device="cuda:0")
            buf[1:] = xh.reshape(-1)
            xh = buf[1:].view(shape)
        Wd, idsd = dev(torch, Wall), dev(torch, ids_np)
        y16 = qmv.qmv_moe_xt(fmt, Wd, per, E, 2 * N, K, idsd, xh)
        y32 = qmv.qmv_moe(fmt, Wd, per, E, 2 * N, K, idsd, xw)
        h16 = qmv.qmv_moe_swiglu_xt(fmt, Wd, per, E, N, K, idsd, xh)
        h32 = qmv.qmv_moe_swiglu(fmt, Wd, per, E, N, K, idsd, xw)
        torch.cuda.synchronize()
        assert torch.equal(y16.view(torch.int32), y32.view(torch.int32)), name
        assert torch.equal(h16.view(torch.int32), h32.view(torch.int32)), name
        xw_np = xw.cpu().numpy()
        if per_slot:
            yr, S = oracle.moe(fmt, Wall, per, E, 2 * N, K, ids_np, None, x_slots=xw_np)
        else:
            yr, S = oracle.moe(fmt, Wall, per, E, 2 * N, K, ids_np, xw_np)
        assert_tol(y16.cpu().numpy(), yr, S, (fmt, kind, name))


@pytest.mark.parametrize("fmt", FMTS)
def test_fused_steps_degenerate_shapes(env, fmt):
    """The smallest shapes of the fused steps: one output row of one block
    (n_ff = 1 for SwiGLU, n_rows = 1 for the combine), top_k 1 and batch 1
    and 8; the one-slot combine is the weight times qmv_moe's output."""
    torch, qmv = env
    E, K = 3, 32
    for B, T in [(1, 1), (8, 1), (2, 3)]:
        say(f"fused degenerate {fmt} B={B} T={T}")
        ids = np.array([[(b + s) % E for s in range(T)] for b in range(B)], dtype=np.int32)
        Wsw = wl.quant_weights(fmt, f"deg/sw/{B}/{T}", E * 2, K).reshape(-1)
        per_sw = wl.block_bytes(fmt, 2, K)
        x = wl.activations(f"deg/x/{B}/{T}", B, K)
        h = gpu_swiglu(env, fmt, Wsw, per_sw, E, 1, K, ids, x)
        hr, g, u, Sg, Su = oracle.moe_swiglu(fmt, Wsw, per_sw, E, 1, K, ids, x)
        assert np.all(np.abs(h.astype(np.float64) - hr) <= swiglu_bound(hr, g, u, Sg, Su)), (B, T)
        # one-block experts at a stride rounded up to the ABI's 4-byte multiple
        per = wl.block_bytes(fmt, 1, K)
        per_dn = (per + 3) // 4 * 4
        Wdn = np.zeros((E, per_dn), dtype=np.uint8)
        Wdn[:, :per] = wl.quant_weights(fmt, f"deg/dn/{B}/{T}", E, K).reshape(E, per)
        Wdn = Wdn.reshape(-1)
        xs = wl.activations(f"deg/xs/{B}/{T}", B * T, K).reshape(B, T, K)
        w = wl.router_weights(f"deg/w/{B}/{T}", B, T)
        out = gpu_combine(env, fmt, Wdn, per_dn, E, 1, K, ids, w, xs)
        ref, S = oracle.moe_combine(fmt, Wdn, per_dn, E, 1, K, ids, w, x_slots=xs)
        assert np.all(np.abs(out.astype(np.float64) - ref) <= combine_bound(S, w)), (B, T)
        if T == 1:
            y = gpu_moe(env, fmt, Wdn, per_dn, E, 1, K, ids, xs)
            assert np.array_equal(out.view(np.uint32), (w * y[:, :, 0]).astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("nbytes,out_words", [(16, 256), (1 << 20, 256), ((1 << 20) + 48, 8 * 256 * 300),
                                              (64 << 20, 1 << 20)])
def test_stream_read_xor(env, nbytes, out_words):
    """The stream-read ceiling kernel reads every word exactly once: the XOR
    of what its threads write equals the XOR of the buffer (a word skipped
    or read twice changes it).  Unwritten output words stay zero."""
    torch, qmv = env
    say(f"stream_read {nbytes} bytes, {out_words} output words")
    buf = np.random.default_rng(nbytes % 1009).integers(0, 256, size=nbytes, dtype=np.uint8)
    out = torch.zeros(out_words, dtype=torch.int32, device="cuda:0")
    qmv.qmv_stream_read(dev(torch, buf), out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(buf.view(np.uint32))
