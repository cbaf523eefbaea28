"""Pins of the oracle to facts fixed outside it (CPU only).

Each pin is chosen so that a plausible mistake in the oracle fails it:
  * fp16 decoding: exhaustive over all 65536 patterns against numpy's
    IEEE binary16 (library routine);
  * byte layouts and nibble order: hand-computed blocks;
  * encoders + decoders together: quantize/dequantize round-trip bounds;
  * the fp64 dot: exact rational brute force on tiny matrices;
  * the integer requant: hand cases, closed forms and an independent
    big-integer mirror on edge and random pairs;
  * MoE: reduction to single-expert matvecs sliced independently in numpy;
  * the fused steps: the int8 table lookup against numpy indexing (identity
    and permutation tables), SiLU against scipy's logistic function and its
    odd-part identity, SwiGLU against the plain MoE oracle on the gate and
    up rows (a swapped gate/up or a row offset fails), the weighted combine
    against one-hot weights and numpy's einsum.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl
from tests import hand_blocks as hb

FMTS = ["q8_0", "q4_0", "q4_1"]


# ------------------------------------------------------------------ fp16
def test_f16_decode_exhaustive(oracle_lib):
    o = oracle_lib
    h = np.arange(65536, dtype=np.uint16)
    got = o.f16_to_f64(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros and infinities keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ------------------------------------------------------------------ hand blocks
@pytest.mark.parametrize("spec", hb.load()["blocks"], ids=lambda s: s["id"])
def test_hand_block(oracle_lib, spec):
    o = oracle_lib
    blk = hb.block_bytes(spec)
    x = hb.x_vec(spec["x"])
    y, S = o.matvec(spec["fmt"], blk, 1, 32, x[None, :])
    assert y[0, 0] == float(spec["y"]), (spec["id"], y[0, 0])
    # the same block through the full dequantizer
    w = o.dequant(spec["fmt"], blk, 1, 32)[0]
    assert float(np.dot(w, x.astype(np.float64))) == float(spec["y"])


def test_q4_nibble_order_distinguishes(oracle_lib):
    """HB12: element j is the low nibble of byte j, element j+16 its high
    nibble; the interleaved order would give a different value."""
    spec = [s for s in hb.load()["blocks"] if s["id"] == "HB12"][0]
    w = oracle_lib.dequant("q4_0", hb.block_bytes(spec), 1, 32)[0]
    assert np.array_equal(w[:16], np.arange(16) - 8.0)
    assert np.array_equal(w[16:], np.full(16, -8.0))


@pytest.mark.parametrize("spec", hb.load()["super_blocks"], ids=lambda s: s["id"])
def test_hand_super_block(oracle_lib, spec):
    """Q4_K (HB13-HB15) and Q6_K (HB16-HB18) super-blocks worked by hand:
    y of the oracle's matvec and of its dequantizer, and HB14's
    per-sub-block weights and 6-bit fields."""
    o = oracle_lib
    fmt = spec["fmt"]
    blk = hb.super_block_bytes(spec)
    x = hb.x_vec256(spec["x"])
    y, S = o.matvec(fmt, blk, 1, 256, x[None, :])
    assert y[0, 0] == float(spec["y"]), (spec["id"], y[0, 0])
    w = o.dequant(fmt, blk, 1, 256)[0]
    assert float(np.dot(w, x.astype(np.float64))) == float(spec["y"])
    if "w" in spec:
        for s in range(8):
            assert np.all(w[32 * s:32 * s + 32] == float(spec["w"][s])), (spec["id"], s)


def test_q4k_nibble_order_distinguishes(oracle_lib):
    """HB15: sub-block 2p takes the low nibbles of bytes 32p..32p+31 and
    sub-block 2p+1 their high nibbles; element by element."""
    spec = [s for s in hb.load()["super_blocks"] if s["id"] == "HB15"][0]
    w = oracle_lib.dequant("q4_k", hb.super_block_bytes(spec), 1, 256)[0]
    for p in range(4):
        i = np.arange(32)
        assert np.array_equal(w[64 * p:64 * p + 32], ((32 * p + i) & 15).astype(np.float64))
        assert np.array_equal(w[64 * p + 32:64 * p + 64], ((32 * p + i) >> 4).astype(np.float64))


def test_q6k_element_order(oracle_lib):
    """HB17 (ql[k] = k, qh[k] = k, d = 1, scales 1) element by element:
    w_e = c_e - 32 with c_e worked by hand from the layout reading."""
    spec = [s for s in hb.load()["super_blocks"] if s["id"] == "HB17"][0]
    w = oracle_lib.dequant("q6_k", hb.super_block_bytes(spec), 1, 256)[0]
    cases = {
        0: 0,            # h0 q0 l0: low nibble of ql[0] = 0, bits 0-1 of qh[0] = 0
        37: 5 + 16,      # h0 q1 l5: low nibble of ql[37] = 5, bits 2-3 of qh[5] = 1
        81: 1 + 16,      # h0 q2 l17: high nibble of ql[17] = 1, bits 4-5 of qh[17] = 1
        127: 3 + 0,      # h0 q3 l31: high nibble of ql[63] = 3, bits 6-7 of qh[31] = 0
        131: 3 + 48,     # h1 q0 l3: low nibble of ql[67] = 3, bits 0-1 of qh[35] = 3
        178: 2 + 0,      # h1 q1 l18: low nibble of ql[114] = 2, bits 2-3 of qh[50] = 0
        255: 7 + 0,      # h1 q3 l31: high nibble of ql[127] = 7, bits 6-7 of qh[63] = 0
    }
    for e, c in cases.items():
        assert w[e] == c - 32, (e, w[e], c)


def test_q6k_scale_per_16_weights(oracle_lib):
    """HB18 (d = -0.5, every code 63): weight e uses the signed scale
    sc[e / 16]; the sub-block boundaries 15 | 16 and 127 | 128 change it."""
    spec = [s for s in hb.load()["super_blocks"] if s["id"] == "HB18"][0]
    w = oracle_lib.dequant("q6_k", hb.super_block_bytes(spec), 1, 256)[0]
    sc = spec["sc"]
    for s_ in range(16):
        assert np.all(w[16 * s_:16 * s_ + 16] == -0.5 * sc[s_] * 31), s_
    assert w[15] == 1984.0 and w[16] == -1968.5 and w[127] == -124.0 and w[128] == 139.5


def test_q4k_rows_and_one_hot(oracle_lib):
    """Two-super-block rows of HB13 and HB14 in either order (row pitch 288
    bytes), one-hot x picks single weights, and a row subset equals the
    full run."""
    o = oracle_lib
    sbs = {s["id"]: hb.super_block_bytes(s) for s in hb.load()["super_blocks"]}
    W = np.stack([np.concatenate([sbs["HB13"], sbs["HB14"]]), np.concatenate([sbs["HB14"], sbs["HB13"]])])
    for j, want in [(0, [1.0, 94.25]), (256 + 32 * 7 + 5, [460.75, 16.0]), (256 + 64, [-15.5, 3.0])]:
        x = np.zeros((1, 512), dtype=np.float32)
        x[0, j] = 1
        y, _ = o.matvec("q4_k", W, 2, 512, x)
        assert list(y[0]) == want, (j, y)
    x = np.ones((1, 512), dtype=np.float32)
    y, _ = o.matvec("q4_k", W, 2, 512, x)
    assert list(y[0]) == [1792.0 + 33728.0] * 2
    y1, _ = o.matvec("q4_k", W, 2, 512, x, rows=np.array([1]))
    assert y1[0, 0] == y[0, 1]


# ------------------------------------------------------------------ round trip
def _blocks_f64(Wf):
    N, K = Wf.shape
    return Wf.astype(np.float64).reshape(N, K // 32, 32)


def _scale_bits(Wq, fmt, N, K, off=0):
    bb = wl.BLOCK_BYTES[fmt]
    raw = Wq.reshape(N, K // 32, bb)[..., off:off + 2].copy()
    return raw.view(np.float16)[..., 0].astype(np.float64)


def _test_weights():
    g = np.random.default_rng(1234)
    W = g.standard_normal((24, 256)) * 0.02
    W[0, :32] = 0.0                       # all-zero block
    W[1, :32] = g.standard_normal(32) * 1e-4   # subnormal (nonzero) fp16 scale
    W[1, 32:64] = g.standard_normal(32) * 1e-9 # scale underflows to fp16 zero
    W[2, :32] = 3.0                       # constant block
    W[3, :32] = -np.linspace(0, 1, 32)    # monotone, negative extreme
    W[4, 32:64] = np.linspace(-1, 1, 32)  # tie in |w| between ends (first wins)
    W[5, :32] = g.standard_normal(32) * 100.0
    return W.astype(np.float32)


def test_roundtrip_q8_0(oracle_lib):
    W = _test_weights()
    N, K = W.shape
    Wq = wl.encode_q8_0(W)
    deq = oracle_lib.dequant("q8_0", Wq, N, K).reshape(N, K // 32, 32)
    blk = _blocks_f64(W)
    d = np.abs(_scale_bits(Wq, "q8_0", N, K))[..., None]
    # every element is within half a step of the stored scale; the subnormal
    # fp16 scale may be rounded by up to 2^-25 relative to amax/127, which
    # can move the clipped extreme by at most 127 * 2^-25.
    slack = 127 * 2.0 ** -25
    assert np.all(np.abs(blk - deq) <= d / 2 + slack + 1e-300)
    # the largest-magnitude element maps to +-127 whenever the stored scale is
    # a normal fp16 number; a zero scale (all-zero block, or amax/127 below half the
    # smallest fp16 subnormal) stores all-zero codes
    q = Wq.reshape(N, K // 32, 34)[..., 2:].view(np.int8).astype(np.int64)
    amax_i = np.abs(blk).argmax(-1)
    qa = np.take_along_axis(np.abs(q), amax_i[..., None], -1)[..., 0]
    # (normal fp16 scale: |amax/d - 127| <= 127 * 2^-11 < 1/2)
    nz = d[..., 0] != 0
    normal = d[..., 0] >= 2.0 ** -14
    assert nz[1, 0] and not normal[1, 0] and not nz[1, 1] and not nz[0, 0]
    assert np.all(qa[normal] == 127)
    assert np.all(deq[~nz] == 0) and np.all(q[~nz] == 0)


def test_roundtrip_q4_0(oracle_lib):
    W = _test_weights()
    N, K = W.shape
    Wq = wl.encode_q4_0(W)
    deq = oracle_lib.dequant("q4_0", Wq, N, K).reshape(N, K // 32, 32)
    blk = _blocks_f64(W)
    d = np.abs(_scale_bits(Wq, "q4_0", N, K))[..., None]
    qs = Wq.reshape(N, K // 32, 18)[..., 2:]
    codes = np.concatenate([qs & 15, qs >> 4], axis=-1).astype(np.int64)
    err = np.abs(blk - deq)
    clipped = codes == 15
    normal = d >= 2.0 ** -14
    # unclipped codes: within half a step; clipped at 15 (w/d >= 7.5): within
    # one step plus the fp16 rounding slack of d (8 * 2^-11 relative).
    assert np.all(err[~clipped & np.broadcast_to(normal, err.shape)] <=
                  (d / 2 * np.ones_like(err))[~clipped & np.broadcast_to(normal, err.shape)] * (1 + 1e-12))
    bound_clip = d * (1 + 2.0 ** -8)
    assert np.all((err <= bound_clip * (1 + 1e-12))[np.broadcast_to(normal, err.shape)])
    # the signed extreme maps to code 0 (w_ext / d = -8)
    iext = np.abs(blk).argmax(-1)
    cext = np.take_along_axis(codes, iext[..., None], -1)[..., 0]
    nz = np.abs(blk).max(-1) > 0
    assert np.all(cext[nz & normal[..., 0]] == 0)
    # zero block: d = 0, codes 8, decodes to zeros
    assert np.all(deq[~nz] == 0)


def test_roundtrip_q4_1(oracle_lib):
    W = _test_weights()
    N, K = W.shape
    Wq = wl.encode_q4_1(W)
    deq = oracle_lib.dequant("q4_1", Wq, N, K).reshape(N, K // 32, 32)
    blk = _blocks_f64(W)
    d16 = _scale_bits(Wq, "q4_1", N, K, 0)
    m16 = _scale_bits(Wq, "q4_1", N, K, 2)
    mn, mx = blk.min(-1), blk.max(-1)
    d32 = (mx - mn) / 15.0
    qs = Wq.reshape(N, K // 32, 20)[..., 4:]
    codes = np.concatenate([qs & 15, qs >> 4], axis=-1)
    assert codes.max() <= 15
    bound = d16 / 2 + np.abs(mn - m16) + 15 * np.abs(d32 - d16)
    assert np.all(np.abs(blk - deq) <= bound[..., None] * (1 + 1e-9) + 1e-300)


def _q4k_affine(o, Wq, N, K):
    """Per sub-block (a, b) with DEQ = a c - b, probed through the oracle:
    the same super-blocks with every code 0 give -b, with every code 1 give
    a - b."""
    ns = K // 256
    sb = Wq.reshape(N, ns, 144)
    z = sb.copy()
    z[..., 16:] = 0x00
    one = sb.copy()
    one[..., 16:] = 0x11
    d0 = o.dequant("q4_k", z.reshape(N, -1), N, K).reshape(N, ns, 8, 32)[..., 0]
    d1 = o.dequant("q4_k", one.reshape(N, -1), N, K).reshape(N, ns, 8, 32)[..., 0]
    return d1 - d0, -d0


def test_roundtrip_q4_k(oracle_lib):
    """Encoder round trip: every weight within half a code step of its
    sub-block's grid {a c - b}, plus the distance by which it lies outside
    the grid's ends; Gaussian rows keep an rms error below a tenth of the
    weights' spread; the special rows (all-zero, constant, scale underflow)
    decode as expected."""
    g = np.random.default_rng(4321)
    N, K = 24, 512
    W = g.standard_normal((N, K)) * 0.02
    W[0, :256] = 0.0                        # all-zero super-block
    W[1, :32] = 3.0                         # constant positive sub-block
    W[2, 256:] = g.standard_normal(256) * 1e-9   # scales underflow to fp16 zero
    W[3, :256] = -np.abs(W[3, :256])        # all non-positive
    W[4, 256:] = np.abs(W[4, 256:])         # all non-negative: minimums 0
    W = W.astype(np.float32)
    Wq = wl.encode_q4_k(W)
    assert Wq.shape == (N, K // 256 * 144)
    deq = oracle_lib.dequant("q4_k", Wq, N, K).reshape(N, K // 256, 8, 32)
    a, b = _q4k_affine(oracle_lib, Wq, N, K)
    w = W.astype(np.float64).reshape(N, K // 256, 8, 32)
    lo, hi = -b, 15 * a - b
    outside = np.maximum(0, np.maximum(w - hi[..., None], lo[..., None] - w))
    assert np.all(np.abs(w - deq) <= a[..., None] / 2 * (1 + 1e-9) + outside + 1e-300)
    assert np.all(deq[0, 0] == 0) and np.all(deq[2, 1] == 0)
    assert np.all(b[4, 1] == 0)
    gauss = np.ones(N, dtype=bool)
    gauss[:5] = False
    rms = np.sqrt(np.mean((w[gauss] - deq[gauss]) ** 2))
    assert rms < 0.1 * 0.02, rms


def test_roundtrip_q6_k(oracle_lib):
    """Q6_K encoder round trip: every weight within half a code step of its
    sub-block's grid d sc (c - 32) (no clipping: the extreme maps to +-31
    up to the rounding of sc and d); Gaussian rows keep an rms error below
    a twentieth of the weights' spread; all-zero and underflowing
    super-blocks decode to zero."""
    g = np.random.default_rng(4322)
    N, K = 24, 512
    W = g.standard_normal((N, K)) * 0.02
    W[0, :256] = 0.0
    W[1, 256:] = g.standard_normal(256) * 1e-12
    W[2, :16] = 5.0                        # constant sub-block beside small ones
    W = W.astype(np.float32)
    Wq = wl.encode_q6_k(W)
    assert Wq.shape == (N, K // 256 * 210)
    deq = oracle_lib.dequant("q6_k", Wq, N, K).reshape(N, K // 256, 16, 16)
    # the step of each sub-block, probed through the oracle: every code 33
    # (signed 1) gives d * sc
    probe = Wq.reshape(N, K // 256, 210).copy()
    probe[..., 0:128] = 0x11
    probe[..., 128:192] = 0xAA
    step = oracle_lib.dequant("q6_k", probe.reshape(N, -1), N, K).reshape(N, K // 256, 16, 16)[..., 0]
    w = W.astype(np.float64).reshape(N, K // 256, 16, 16)
    lo, hi = -32 * step, 31 * step
    outside = np.maximum(0, np.maximum(w - hi[..., None], lo[..., None] - w))
    assert np.all(np.abs(w - deq) <= step[..., None] / 2 * (1 + 1e-9) + outside + 1e-300)
    assert np.all(deq[0, 0] == 0) and np.all(deq[1, 1] == 0)
    rms = np.sqrt(np.mean((w[3:] - deq[3:]) ** 2))
    assert rms < 0.05 * 0.02, rms


def test_zero_heavy_q6_k_is_exact_zero(oracle_lib):
    N, K = 12, 1024
    Wq, x = wl.zero_heavy("q6_k", "t/pins/zh6", N, K, B=2)
    deq = oracle_lib.dequant("q6_k", Wq, N, K)
    small = (np.arange(K) % 16) == 15
    assert np.all(deq[:, ~small] == 0) and np.count_nonzero(deq[:, small]) > 0


def test_zero_heavy_q4_k_is_exact_zero(oracle_lib):
    """The zero-heavy Q4_K rows decode to exactly 0 off the sparse columns
    (d sc k - dmin sc k with dmin = d) and carry the activations' 1e3 / 1e-3
    split."""
    N, K = 12, 1024
    Wq, x = wl.zero_heavy("q4_k", "t/pins/zh", N, K, B=2)
    deq = oracle_lib.dequant("q4_k", Wq, N, K)
    small = (np.arange(K) % 16) == 15
    assert np.all(deq[:, ~small] == 0) and np.count_nonzero(deq[:, small]) > 0
    assert np.all(np.abs(x[:, small]) < 0.1) and np.median(np.abs(x[:, ~small])) > 100


# ------------------------------------------------------------------ exact brute force
def _random_blocks(g, fmt, N, K):
    """Random stored bytes with finite, varied scales (random codes)."""
    bb = wl.BLOCK_BYTES[fmt]
    raw = g.integers(0, 256, size=(N, K // 32, bb), dtype=np.uint8)
    # finite fp16 scales: exponent field 0..30 (includes subnormals)
    for off in ([0] if fmt != "q4_1" else [0, 2]):
        e = g.integers(0, 31, size=(N, K // 32))
        f = g.integers(0, 1024, size=(N, K // 32))
        s = g.integers(0, 2, size=(N, K // 32))
        h = (s << 15) | (e << 10) | f
        raw[..., off] = h & 0xFF
        raw[..., off + 1] = h >> 8
    return raw.reshape(N, -1)


def _exact_dequant(fmt, blkbytes):
    """Exact rational DEQ of one block, written from the layout directly."""
    def f16(lo, hi):
        return Fraction(float(np.array([lo | (hi << 8)], dtype=np.uint16).view(np.float16)[0]))
    b = [int(v) for v in blkbytes]
    if fmt == "q8_0":
        d = f16(b[0], b[1])
        return [d * (v - 256 if v >= 128 else v) for v in b[2:34]]
    if fmt == "q4_0":
        d = f16(b[0], b[1])
        return [d * ((b[2 + j] & 15) - 8) for j in range(16)] + \
               [d * ((b[2 + j] >> 4) - 8) for j in range(16)]
    d, m = f16(b[0], b[1]), f16(b[2], b[3])
    return [d * (b[4 + j] & 15) + m for j in range(16)] + \
           [d * (b[4 + j] >> 4) + m for j in range(16)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K", [32, 64])
def test_matvec_exact_rational(oracle_lib, fmt, K):
    g = np.random.default_rng(77 + K)
    N, B = 4, 3
    Wq = _random_blocks(g, fmt, N, K)
    x = (g.standard_normal((B, K)) * np.exp(g.uniform(-8, 8, size=(B, K)))).astype(np.float32)
    y, S = oracle_lib.matvec(fmt, Wq, N, K, x)
    bb = wl.BLOCK_BYTES[fmt]
    rows = Wq.reshape(N, K // 32, bb)
    for i in range(N):
        w = sum((_exact_dequant(fmt, rows[i, k]) for k in range(K // 32)), [])
        for b in range(B):
            exact = sum(wi * Fraction(float(xi)) for wi, xi in zip(w, x[b]))
            sabs = sum(abs(wi * Fraction(float(xi))) for wi, xi in zip(w, x[b]))
            err = abs(Fraction(y[b, i]) - exact)
            assert err <= Fraction(K) * Fraction(2) ** -52 * sabs, (fmt, i, b)
            assert abs(Fraction(S[b, i]) - sabs) <= Fraction(K) * Fraction(2) ** -52 * sabs


def _random_super_blocks(g, N, K):
    """Random Q4_K bytes with finite fp16 d and dmin (subnormals included)."""
    raw = g.integers(0, 256, size=(N, K // 256, 144), dtype=np.uint8)
    for off in (0, 2):
        h = (g.integers(0, 2, size=(N, K // 256)) << 15) | (g.integers(0, 31, size=(N, K // 256)) << 10) | \
            g.integers(0, 1024, size=(N, K // 256))
        raw[..., off] = h & 0xFF
        raw[..., off + 1] = h >> 8
    return raw.reshape(N, -1)


def _exact_dequant_q4k(sb):
    """Exact rational DEQ of one Q4_K super-block, from the layout reading:
    the 6-bit fields are read bit by bit out of the 96-bit field area."""
    sb = [int(v) for v in sb]

    def f16(lo, hi):
        return Fraction(float(np.array([lo | (hi << 8)], dtype=np.uint16).view(np.float16)[0]))

    d, dmin = f16(sb[0], sb[1]), f16(sb[2], sb[3])
    fb = sb[4:16]

    def bits(byte, lo, n):
        return (fb[byte] >> lo) & ((1 << n) - 1)

    out = []
    for s in range(8):
        if s < 4:
            sc, mn = bits(s, 0, 6), bits(s + 4, 0, 6)
        else:
            sc = bits(s + 4, 0, 4) | (bits(s - 4, 6, 2) << 4)
            mn = bits(s + 4, 4, 4) | (bits(s, 6, 2) << 4)
        for i in range(32):
            q = sb[16 + 32 * (s // 2) + i]
            c = (q >> 4) if s % 2 else (q & 15)
            out.append(d * sc * c - dmin * mn)
    return out


def _random_super_blocks_q6k(g, N, K):
    """Random Q6_K bytes with a finite fp16 d (subnormals included)."""
    raw = g.integers(0, 256, size=(N, K // 256, 210), dtype=np.uint8)
    h = (g.integers(0, 2, size=(N, K // 256)) << 15) | (g.integers(0, 31, size=(N, K // 256)) << 10) | \
        g.integers(0, 1024, size=(N, K // 256))
    raw[..., 208] = h & 0xFF
    raw[..., 209] = h >> 8
    return raw.reshape(N, -1)


def _exact_dequant_q6k(sb):
    """Exact rational DEQ of one Q6_K super-block, from the layout reading:
    the 6-bit codes reassembled as a bit string (4 low bits from the ql
    area, 2 high bits from the qh area)."""
    sb = [int(v) for v in sb]
    d = Fraction(float(np.array([sb[208] | (sb[209] << 8)], dtype=np.uint16).view(np.float16)[0]))
    out = []
    for e in range(256):
        half, rem = divmod(e, 128)
        quarter, l = divmod(rem, 32)
        byte = sb[64 * half + 32 * (quarter % 2) + l]
        nib = (byte >> 4) if quarter >= 2 else (byte & 15)
        top = (sb[128 + 32 * half + l] >> (2 * quarter)) & 3
        scale = sb[192 + e // 16]
        scale = scale - 256 if scale >= 128 else scale
        out.append(d * scale * ((top << 4 | nib) - 32))
    return out


@pytest.mark.parametrize("K", [256, 512])
def test_matvec_exact_rational_q6k(oracle_lib, K):
    """Random Q6_K super-blocks: the oracle's DEQ is exact, and its double
    sums are within (K+1) ulps (relative to sum |w x|) of the exact
    rational matvec."""
    g = np.random.default_rng(311 + K)
    N, B = 3, 2
    Wq = _random_super_blocks_q6k(g, N, K)
    x = (g.standard_normal((B, K)) * np.exp(g.uniform(-8, 8, size=(B, K)))).astype(np.float32)
    y, S = oracle_lib.matvec("q6_k", Wq, N, K, x)
    deq = oracle_lib.dequant("q6_k", Wq, N, K)
    rows = Wq.reshape(N, K // 256, 210)
    for i in range(N):
        w = sum((_exact_dequant_q6k(rows[i, k]) for k in range(K // 256)), [])
        for j in range(K):
            assert deq[i, j] == w[j], (i, j)      # exact in double
        for b in range(B):
            exact = sum(wi * Fraction(float(xi)) for wi, xi in zip(w, x[b]))
            sabs = sum(abs(wi * Fraction(float(xi))) for wi, xi in zip(w, x[b]))
            err = abs(Fraction(y[b, i]) - exact)
            assert err <= Fraction(K + 1) * Fraction(2) ** -52 * sabs, (i, b)


@pytest.mark.parametrize("K", [256, 512])
def test_matvec_exact_rational_q4k(oracle_lib, K):
    """Random super-blocks: the oracle's double sums are within K ulps
    (relative to sum |w x|) of the exact rational matvec, and its DEQ
    rounds the exact weight once at most."""
    g = np.random.default_rng(99 + K)
    N, B = 3, 2
    Wq = _random_super_blocks(g, N, K)
    x = (g.standard_normal((B, K)) * np.exp(g.uniform(-8, 8, size=(B, K)))).astype(np.float32)
    y, S = oracle_lib.matvec("q4_k", Wq, N, K, x)
    deq = oracle_lib.dequant("q4_k", Wq, N, K)
    rows = Wq.reshape(N, K // 256, 144)
    for i in range(N):
        w = sum((_exact_dequant_q4k(rows[i, k]) for k in range(K // 256)), [])
        for j in range(K):
            assert deq[i, j] == float(w[j]), (i, j)      # float() rounds to nearest
        for b in range(B):
            exact = sum(wi * Fraction(float(xi)) for wi, xi in zip(w, x[b]))
            sabs = sum(abs(wi * Fraction(float(xi))) for wi, xi in zip(w, x[b]))
            err = abs(Fraction(y[b, i]) - exact)
            assert err <= Fraction(K + 1) * Fraction(2) ** -52 * sabs, (i, b)


@pytest.mark.parametrize("fmt", FMTS)
def test_one_hot_selects_column(oracle_lib, fmt):
    g = np.random.default_rng(5)
    N, K = 6, 96
    Wq = _random_blocks(g, fmt, N, K)
    deq = oracle_lib.dequant(fmt, Wq, N, K)
    x = np.eye(K, dtype=np.float32)[[0, 31, 32, 47, 95]]
    y, _ = oracle_lib.matvec(fmt, Wq, N, K, x)
    assert np.array_equal(y, deq[:, [0, 31, 32, 47, 95]].T)


def test_row_subset_matches_full(oracle_lib):
    g = np.random.default_rng(9)
    N, K = 10, 64
    Wq = _random_blocks(g, "q4_1", N, K)
    x = g.standard_normal((2, K)).astype(np.float32)
    y, S = oracle_lib.matvec("q4_1", Wq, N, K, x)
    rows = np.array([9, 0, 4])
    y2, S2 = oracle_lib.matvec("q4_1", Wq, N, K, x, rows=rows)
    assert np.array_equal(y[:, rows], y2) and np.array_equal(S[:, rows], S2)


# ------------------------------------------------------------------ integer path
from oracle import py_int  # noqa: E402

I32MIN, I32MAX = -(1 << 31), (1 << 31) - 1


def test_hand_integer_cases(oracle_lib):
    o = oracle_lib
    cases = {c["id"]: c for c in hb.load()["integer"]}
    c = cases["HB8"]
    W = np.full((1, c["K"]), c["w"], dtype=np.int8)
    x = np.full((1, c["K"]), c["x"], dtype=np.int8)
    acc, y = o.matvec_i8(W, x, [c["mult"]], [c["shift"]])
    assert acc[0, 0] == c["acc"] and y[0, 0] == c["y"]
    assert o.srdhm(c["acc"], c["mult"]) == c["srdhm"] == py_int.srdhm(c["acc"], c["mult"])
    c = cases["HB9"]
    for a, e in zip(c["a"], c["expect"]):
        assert o.srdhm(a, c["srdhm_b"]) == e == py_int.srdhm(a, c["srdhm_b"])
    c = cases["HB10"]
    for v, e in zip(c["x"], c["expect"]):
        assert o.rdbpot(v, c["rdbpot_e"]) == e == py_int.rdbpot(v, c["rdbpot_e"])
    c = cases["HB11"]
    for a, s, e in zip(c["acc"], c["srdhm"], c["y"]):
        assert o.srdhm(a, c["mult"]) == s
        assert o.requant(a, c["mult"], c["shift"]) == e == py_int.requant(a, c["mult"], c["shift"])


def test_srdhm_closed_forms(oracle_lib):
    o = oracle_lib
    g = np.random.default_rng(3)
    for a in list(g.integers(I32MIN, I32MAX, size=2000)) + [I32MIN, I32MAX, 0, -1, 1]:
        a = int(a)
        # b = 2^30: a/2 rounded, ties up
        assert o.srdhm(a, 1 << 30) == (a + 1) // 2
        # b = 2^31 - 1 is the identity on (-2^30, 2^30]
        if -(1 << 30) < a <= (1 << 30):
            assert o.srdhm(a, I32MAX) == a
    assert o.srdhm(-(1 << 30), I32MAX) == -(1 << 30) + 1
    assert o.srdhm(I32MIN, I32MIN) == I32MAX
    assert o.srdhm(I32MIN, I32MAX) == I32MIN + 1
    assert o.srdhm(0, I32MIN) == 0


def test_rdbpot_closed_forms(oracle_lib):
    o = oracle_lib
    g = np.random.default_rng(4)
    for v in list(g.integers(I32MIN, I32MAX, size=1000)) + [I32MIN, I32MAX, 0, -1, 1]:
        v = int(v)
        assert o.rdbpot(v, 0) == v
        for e in (1, 7, 20, 31):
            # exact division when divisible
            q = o.rdbpot(v, e)
            assert abs(Fraction(v, 1 << e) - q) <= Fraction(1, 2)
            if v % (1 << e) == 0:
                assert q == v >> e
    # exhaustive small range against the rational definition
    for v in range(-70, 71):
        for e in range(0, 6):
            r = Fraction(v, 1 << e)
            exp = int(abs(r) + Fraction(1, 2)) * (1 if r >= 0 else -1)
            assert o.rdbpot(v, e) == exp


def test_requant_c_vs_bigint_mirror(oracle_lib):
    o = oracle_lib
    g = np.random.default_rng(11)
    edge = [I32MIN, I32MIN + 1, -(1 << 30) - 1, -(1 << 30), -(1 << 30) + 1, -2, -1, 0, 1, 2,
            (1 << 30) - 1, 1 << 30, (1 << 30) + 1, I32MAX - 1, I32MAX]
    for a in edge:
        for b in edge:
            assert o.srdhm(a, b) == py_int.srdhm(a, b), (a, b)
        for e in range(32):
            assert o.rdbpot(a, e) == py_int.rdbpot(a, e), (a, e)
    A = g.integers(I32MIN, I32MAX, size=20000, endpoint=True)
    Bm = g.integers(1 << 30, I32MAX, size=20000, endpoint=True)
    E = g.integers(0, 32, size=20000)
    for a, b, e in zip(A.tolist(), Bm.tolist(), E.tolist()):
        assert o.requant(a, b, e) == py_int.requant(a, b, e)
        assert o.srdhm(a, -b) == py_int.srdhm(a, -b)


def test_matvec_i8_small_vs_mirror(oracle_lib):
    g = np.random.default_rng(12)
    N, K, B = 7, 48, 2
    W = g.integers(-127, 128, size=(N, K), dtype=np.int8)
    x = g.integers(-128, 128, size=(B, K), dtype=np.int8)
    mult = g.integers(1 << 30, 1 << 31, size=N).astype(np.int32)
    shift = g.integers(0, 21, size=N).astype(np.int32)
    acc, y = oracle_lib.matvec_i8(W, x, mult, shift)
    for b in range(B):
        a2, y2 = py_int.matvec_i8(W.tolist(), x[b].tolist(), mult.tolist(), shift.tolist())
        assert acc[b].tolist() == a2 and y[b].tolist() == y2


def test_matvec_i8_overflow_reported(oracle_lib):
    W = np.full((1, 1 << 18), -128, dtype=np.int8)
    x = np.full((1, 1 << 18), -128, dtype=np.int8)
    with pytest.raises(OverflowError):
        oracle_lib.matvec_i8(W, x, [1 << 30], [0])


# ------------------------------------------------------------------ MoE
def test_moe_reduces_to_single_expert_matvecs(oracle_lib):
    o = oracle_lib
    g = np.random.default_rng(21)
    E, N, K, B, T = 5, 8, 64, 3, 2
    per = N * (K // 32) * 18
    stride = per + 36                       # padded experts
    Wall = g.integers(0, 256, size=E * stride, dtype=np.uint8)
    for e in range(E):
        Wall[e * stride:e * stride + per] = _random_blocks(g, "q4_0", N, K).reshape(-1)
    ids = np.array([[4, 1], [1, 0], [2, 4]], dtype=np.int32)
    xt = g.standard_normal((B, K)).astype(np.float32)
    xs = g.standard_normal((B, T, K)).astype(np.float32)
    y1, _ = o.moe("q4_0", Wall, stride, E, N, K, ids, xt)
    y2, _ = o.moe("q4_0", Wall, stride, E, N, K, ids, None, x_slots=xs)
    for b in range(B):
        for s in range(T):
            e = ids[b, s]
            We = Wall[e * stride:e * stride + per]
            r1, _ = o.matvec("q4_0", We, N, K, xt[b:b + 1])
            r2, _ = o.matvec("q4_0", We, N, K, xs[b, s][None])
            assert np.array_equal(y1[b, s], r1[0]) and np.array_equal(y2[b, s], r2[0])
    with pytest.raises(ValueError):
        o.moe("q4_0", Wall, stride, E, N, K, np.array([[5, 0]], dtype=np.int32), xt[:1])


# ------------------------------------------------------------------ fused steps
def test_matvec_i8_lut_identity_and_permutation(oracle_lib):
    o = oracle_lib
    g = np.random.default_rng(31)
    N, K, B = 9, 64, 3
    W = g.integers(-127, 128, size=(N, K), dtype=np.int8)
    x = g.integers(-127, 128, size=(B, K), dtype=np.int8)
    mult = g.integers(1 << 30, 1 << 31, size=N).astype(np.int32)
    shift = g.integers(8, 16, size=N).astype(np.int32)
    acc, y = o.matvec_i8(W, x, mult, shift)
    ident = (np.arange(256) - 128).astype(np.int8)
    acc2, y2 = o.matvec_i8_lut(W, x, mult, shift, ident)
    assert np.array_equal(acc, acc2) and np.array_equal(y, y2)
    perm = g.permutation(256).astype(np.int64) - 128
    perm = perm.astype(np.int8)
    _, y3 = o.matvec_i8_lut(W, x, mult, shift, perm)
    assert np.array_equal(y3, perm[y.astype(np.int64) + 128])
    assert len(np.unique(y)) > 3          # the case spans several table entries


def test_silu_library_and_identities(oracle_lib):
    from scipy.special import expit
    o = oracle_lib
    assert o.silu(0.0) == 0.0
    for z in [-30.0, -5.5, -1.0, -0.125, 0.3, 1.0, 2.0, 7.25, 40.0]:
        assert abs(o.silu(z) - z * expit(z)) <= 4e-16 * max(1.0, abs(z)), z
        # silu(z) - silu(-z) = z (sigma(z) + sigma(-z) = 1)
        assert abs((o.silu(z) - o.silu(-z)) - z) <= 4e-16 * max(1.0, abs(z)), z
    assert o.silu(800.0) == 800.0 and o.silu(-800.0) == 0.0


def _moe_case(g, fmt, E, rows, K, pad=0):
    per = wl.block_bytes(fmt, rows, K)
    stride = per + pad
    Wall = np.zeros(E * stride, dtype=np.uint8)
    for e in range(E):
        Wall[e * stride:e * stride + per] = _random_blocks(g, fmt, rows, K).reshape(-1)
    return Wall, per, stride


@pytest.mark.parametrize("fmt", FMTS)
def test_moe_swiglu_reduces_to_gate_and_up_matvecs(oracle_lib, fmt):
    from scipy.special import expit
    o = oracle_lib
    g = np.random.default_rng(41)
    E, F, K = 4, 6, 64
    Wall, per, stride = _moe_case(g, fmt, E, 2 * F, K, pad=20)
    ids = np.array([[3, 1], [1, 2]], dtype=np.int32)
    x = g.standard_normal((2, K)).astype(np.float32)
    h, gg, uu, Sg, Su = o.moe_swiglu(fmt, Wall, stride, E, F, K, ids, x)
    y, S = o.moe(fmt, Wall, stride, E, 2 * F, K, ids, x)
    assert np.array_equal(gg, y[:, :, :F]) and np.array_equal(uu, y[:, :, F:])
    assert np.array_equal(Sg, S[:, :, :F]) and np.array_equal(Su, S[:, :, F:])
    ref = y[:, :, :F] * expit(y[:, :, :F]) * y[:, :, F:]
    assert np.allclose(h, ref, rtol=1e-14, atol=1e-300)
    swapped = y[:, :, F:] * expit(y[:, :, F:]) * y[:, :, :F]
    assert not np.allclose(h, swapped, rtol=1e-6)
    rows = np.array([5, 0, 2], dtype=np.int64)
    hr = o.moe_swiglu(fmt, Wall, stride, E, F, K, ids, x, rows=rows)[0]
    assert np.array_equal(hr, h[:, :, rows])


def test_moe_swiglu_hand_case(oracle_lib):
    """One Q8_0 expert, F = 1, K = 32: gate row q_0 = 3, up row q_1 = -2,
    d = 1, so g = 3 x_0 and u = -2 x_1 exactly."""
    from scipy.special import expit
    o = oracle_lib
    blk = np.zeros((2, 34), dtype=np.uint8)
    blk[:, 1] = 0x3C                      # d = 1.0 (fp16 0x3C00)
    blk[0, 2] = 3
    blk[1, 3] = np.uint8(256 - 2)
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0], x[0, 1] = 0.75, 1.5
    h, gg, uu, _, _ = o.moe_swiglu("q8_0", blk.reshape(-1), 68, 1, 1, 32, np.zeros((1, 1), np.int32), x)
    assert gg[0, 0, 0] == 2.25 and uu[0, 0, 0] == -3.0
    assert abs(h[0, 0, 0] - 2.25 * expit(2.25) * -3.0) <= 1e-15


@pytest.mark.parametrize("fmt", FMTS)
def test_moe_combine_one_hot_and_einsum(oracle_lib, fmt):
    o = oracle_lib
    g = np.random.default_rng(51)
    E, N, K, B, T = 5, 7, 96, 3, 4
    Wall, per, stride = _moe_case(g, fmt, E, N, K)
    ids = np.array([[0, 4, 2, 1], [3, 3, 0, 4], [2, 1, 0, 3]], dtype=np.int32)
    xs = g.standard_normal((B, T, K)).astype(np.float32)
    y, S = o.moe(fmt, Wall, stride, E, N, K, ids, None, x_slots=xs)
    for s in range(T):
        w = np.zeros((B, T), dtype=np.float32)
        w[:, s] = 1.0
        out, So = o.moe_combine(fmt, Wall, stride, E, N, K, ids, w, x_slots=xs)
        assert np.array_equal(out, y[:, s]) and np.array_equal(So, S[:, s])
    w = g.random((B, T)).astype(np.float32)
    w[1, 2] = -0.5                        # a negative weight counts by magnitude in S
    out, So = o.moe_combine(fmt, Wall, stride, E, N, K, ids, w, x_slots=xs)
    w64 = w.astype(np.float64)
    assert np.allclose(out, np.einsum("bs,bsn->bn", w64, y), rtol=1e-13, atol=1e-13)
    assert np.allclose(So, np.einsum("bs,bsn->bn", np.abs(w64), S), rtol=1e-13)
    xt = g.standard_normal((B, K)).astype(np.float32)
    out_t, _ = o.moe_combine(fmt, Wall, stride, E, N, K, ids, w, x_tokens=xt)
    yt, _ = o.moe(fmt, Wall, stride, E, N, K, ids, xt)
    assert np.allclose(out_t, np.einsum("bs,bsn->bn", w64, yt), rtol=1e-13, atol=1e-13)
