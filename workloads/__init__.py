"""Seeded synthetic inputs for the block-quantized matvec path.

This module is the one place both sides draw their inputs from: the tests
feed the same arrays to the oracle and to the HIP library, and bench.py uses
it for the timed workload.  It holds no part of the matvec arithmetic (no
decoding, no dot products, no requantization); it only draws random numbers
and encodes them into the stored block formats, as the input recipe says:

* float weights W ~ N(0, 0.02^2), encoded per 32-weight row block:
    Q8_0  d = fp16(max|w| / 127),         q = round(w / d) in [-127, 127]
    Q4_0  d = fp16(w_ext / -8) with w_ext the signed element of largest
          magnitude (first on ties),      c = clamp(round(w / d) + 8, 0, 15)
    Q4_1  d = fp16((max - min) / 15), m = fp16(min),
                                          c = clamp(round((w - m) / d), 0, 15)
  "round" is round-half-away-from-zero against the stored fp16 scale; the
  fp16 conversion is numpy's IEEE round-to-nearest-even.
    Q4_K  per 256-weight super-block of eight 32-weight sub-blocks s:
          lo_s = min(0, min w), step_s = (max w - lo_s) / 15;
          d = fp16(max_s step_s / 63), dmin = fp16(max_s (-lo_s) / 63),
          sc_s = clamp(round(step_s / d), 0, 63),
          mn_s = clamp(round(-lo_s / dmin), 0, 63),
          c = clamp(round((w + dmin mn_s) / (d sc_s)), 0, 15)
          (a zero scale gives zero fields).
    Q6_K  per 256-weight super-block of sixteen 16-weight sub-blocks s:
          t_s = max|w| / 31, d = fp16(max_s t_s / 127),
          sc_s = clamp(round(t_s / d), 0, 127),
          c = clamp(round(w / (d sc_s)), -32, 31) + 32 (a zero scale gives
          c = 32, the code of 0).
* activations x ~ N(0, 1) float32;
* int8 weights / activations uniform in [-127, 127]; per-row requant
  multipliers uniform in [2^30, 2^31 - 1] and shifts uniform in [0, 20];
* MoE expert ids: per token, top_k distinct ids uniform without replacement;
  router weights per token drawn from a flat Dirichlet (positive, summing
  to 1 over the token's top_k slots);
* an int8 lookup table: 256 entries uniform in [-128, 127];
* "zero-heavy" rows (an edge case of the stored formats, not a workload):
  blocks whose weights are exactly zero except on a sparse set of columns,
  with activations of magnitude ~1e3 on the zero weights and ~1e-3 on the
  others, so that sum_j |w_j x_j| is tiny next to sum_j |x_j|.  Q8_0 codes
  0, Q4_0 codes 8, Q4_1 codes k with d*k + m = 0 exactly (d with few
  significant bits and m = -d*k, both exact in fp16), Q4_K codes k_s with
  dmin = d and mn_s = sc_s k_s (d sc_s k_s - dmin mn_s = 0 exactly), Q6_K
  code 32 (signed code 0).

Byte layouts (ggml-compatible, little-endian): Q8_0 = [d:fp16][q:int8 x32];
Q4_0 = [d:fp16][qs:16 bytes], element j<16 in the low nibble of qs[j] and
element j+16 in its high nibble; Q4_1 = [d:fp16][m:fp16][qs:16 bytes];
Q4_K = [d:fp16][dmin:fp16][b:12 bytes of 6-bit sc_s, mn_s][q:128 bytes],
sub-block 2p in the low nibbles of q[32p..32p+31] and 2p+1 in their high
nibbles (the packing of b is the one the oracle's reading states);
Q6_K = [ql:128 bytes][qh:64 bytes][sc:16 x int8][d:fp16], code e = 128h +
32q + l with its low 4 bits in ql[64h + 32(q mod 2) + l] (low nibble for
q < 2, high for q >= 2) and its high 2 bits at bits 2q of qh[32h + l].

Seeds: numpy PCG64 seeded with the first 8 bytes (little-endian) of
SHA-256("qmv/<tag>").
"""
import hashlib

import numpy as np

BLOCK_BYTES = {"q8_0": 34, "q4_0": 18, "q4_1": 20}   # per 32 weights
SUPER_BLOCK = {"q4_k": (256, 144), "q6_k": (256, 210)}   # (weights, bytes)


def row_bytes(fmt, K):
    """Stored bytes of one row of K weights."""
    if fmt in SUPER_BLOCK:
        w, b = SUPER_BLOCK[fmt]
        assert K % w == 0, (fmt, K)
        return K // w * b
    assert K % 32 == 0, (fmt, K)
    return K // 32 * BLOCK_BYTES[fmt]


def seed_for(tag: str) -> int:
    h = hashlib.sha256(("qmv/" + tag).encode()).digest()
    return int.from_bytes(h[:8], "little")


def rng(tag: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_for(tag)))


# ---------------------------------------------------------------- draws
def weights_f32(tag, N, K, std=0.02):
    return (rng(tag).standard_normal((N, K), dtype=np.float32) * np.float32(std))


def activations(tag, B, K):
    return rng(tag).standard_normal((B, K), dtype=np.float32)


def int8_uniform(tag, shape):
    return rng(tag).integers(-127, 128, size=shape, dtype=np.int8)


def requant_params(tag, N, shift_max=20):
    g = rng(tag)
    mult = g.integers(1 << 30, (1 << 31), size=N, dtype=np.int64).astype(np.int32)
    shift = g.integers(0, shift_max + 1, size=N, dtype=np.int32)
    return mult, shift


def moe_ids(tag, batch, top_k, n_experts):
    g = rng(tag)
    return np.stack([g.choice(n_experts, size=top_k, replace=False)
                     for _ in range(batch)]).astype(np.int32)


def router_weights(tag, batch, top_k):
    return rng(tag).dirichlet(np.ones(top_k), size=batch).astype(np.float32)


def int8_table(tag):
    return rng(tag).integers(-128, 128, size=256, dtype=np.int8)


# ---------------------------------------------------------------- encoders
def _round_half_away(v):
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def _f16(v):
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16)


def _nibbles_to_bytes(c):
    """c: [..., 32] codes 0..15 -> [..., 16] bytes, low nibble = c[j],
    high nibble = c[j+16]."""
    c = c.astype(np.uint8)
    return (c[..., :16] | (c[..., 16:] << 4)).astype(np.uint8)


def encode_q8_0(Wf):
    """float [N, K] -> uint8 [N, K/32*34]."""
    Wf = np.asarray(Wf)
    N, K = Wf.shape
    assert K % 32 == 0
    blk = Wf.reshape(N, K // 32, 32).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    d16 = _f16(amax / 127.0)
    d = d16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(d != 0, np.clip(_round_half_away(blk / d), -127, 127), 0)
    out = np.empty((N, K // 32, 34), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(N, K // 32, 2)
    out[..., 2:] = q.astype(np.int8).view(np.uint8)
    return out.reshape(N, -1)


def encode_q4_0(Wf):
    """float [N, K] -> uint8 [N, K/32*18] (signed-extreme scale)."""
    Wf = np.asarray(Wf)
    N, K = Wf.shape
    assert K % 32 == 0
    blk = Wf.reshape(N, K // 32, 32).astype(np.float64)
    idx = np.abs(blk).argmax(axis=-1)[..., None]          # first on ties
    wext = np.take_along_axis(blk, idx, axis=-1)[..., 0]
    d16 = _f16(wext / -8.0)
    d = d16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.where(d != 0, np.clip(_round_half_away(blk / d) + 8, 0, 15), 8)
    out = np.empty((N, K // 32, 18), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(N, K // 32, 2)
    out[..., 2:] = _nibbles_to_bytes(c)
    return out.reshape(N, -1)


def encode_q4_1(Wf):
    """float [N, K] -> uint8 [N, K/32*20] (scale + minimum)."""
    Wf = np.asarray(Wf)
    N, K = Wf.shape
    assert K % 32 == 0
    blk = Wf.reshape(N, K // 32, 32).astype(np.float64)
    mn = blk.min(axis=-1)
    mx = blk.max(axis=-1)
    d16 = _f16((mx - mn) / 15.0)
    m16 = _f16(mn)
    d = d16.astype(np.float64)[..., None]
    m = m16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.where(d != 0, np.clip(_round_half_away((blk - m) / d), 0, 15), 0)
    out = np.empty((N, K // 32, 20), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(N, K // 32, 2)
    out[..., 2:4] = m16.view(np.uint8).reshape(N, K // 32, 2)
    out[..., 4:] = _nibbles_to_bytes(c)
    return out.reshape(N, -1)


def _pack_q4k(d16, dmin16, sc, mn, c):
    """Fields -> uint8 [..., 144]: d16, dmin16 [...] fp16; sc, mn [..., 8]
    in 0..63; c [..., 256] codes 0..15 in weight order."""
    sc = sc.astype(np.uint8)
    mn = mn.astype(np.uint8)
    b = np.empty(sc.shape[:-1] + (12,), dtype=np.uint8)
    b[..., 0:4] = (sc[..., 0:4] & 63) | ((sc[..., 4:8] >> 4) << 6)
    b[..., 4:8] = (mn[..., 0:4] & 63) | ((mn[..., 4:8] >> 4) << 6)
    b[..., 8:12] = (sc[..., 4:8] & 15) | ((mn[..., 4:8] & 15) << 4)
    cs = c.astype(np.uint8).reshape(c.shape[:-1] + (4, 2, 32))   # [pair][lo/hi][i]
    q = (cs[..., 0, :] | (cs[..., 1, :] << 4)).reshape(c.shape[:-1] + (128,))
    lead = d16.shape
    return np.concatenate([d16.view(np.uint8).reshape(lead + (2,)), dmin16.view(np.uint8).reshape(lead + (2,)),
                           b, q], axis=-1)


def encode_q4_k(Wf):
    """float [N, K] -> uint8 [N, K/256*144] (super-blocks of 6-bit
    sub-block scales and minimums)."""
    Wf = np.asarray(Wf)
    N, K = Wf.shape
    assert K % 256 == 0
    ns = K // 256
    sub = Wf.reshape(N, ns, 8, 32).astype(np.float64)
    lo = np.minimum(sub.min(axis=-1), 0.0)
    step = (sub.max(axis=-1) - lo) / 15.0
    d16 = _f16(step.max(axis=-1) / 63.0)
    dmin16 = _f16((-lo).max(axis=-1) / 63.0)
    d = d16.astype(np.float64)[..., None]
    dmin = dmin16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d != 0, np.clip(_round_half_away(step / d), 0, 63), 0)
        mn = np.where(dmin != 0, np.clip(_round_half_away(-lo / dmin), 0, 63), 0)
        ds = (d * sc)[..., None]
        dm = (dmin * mn)[..., None]
        c = np.where(ds != 0, np.clip(_round_half_away((sub + dm) / ds), 0, 15), 0)
    return _pack_q4k(d16, dmin16, sc, mn, c.reshape(N, ns, 256)).reshape(N, ns * 144)


def _pack_q6k(d16, sc, c):
    """Fields -> uint8 [..., 210]: d16 [...] fp16; sc [..., 16] int8
    values; c [..., 256] codes 0..63 in weight order."""
    lead = d16.shape
    c = c.astype(np.uint8).reshape(lead + (2, 4, 32))          # [half][quarter][l]
    low, high = c & 15, c >> 4
    ql = np.concatenate([low[..., 0, :] | (low[..., 2, :] << 4), low[..., 1, :] | (low[..., 3, :] << 4)],
                        axis=-1).reshape(lead + (128,))
    qh = (high[..., 0, :] | (high[..., 1, :] << 2) | (high[..., 2, :] << 4) | (high[..., 3, :] << 6)).reshape(
        lead + (64,))
    return np.concatenate([ql, qh, sc.astype(np.int8).view(np.uint8), d16.view(np.uint8).reshape(lead + (2,))],
                          axis=-1)


def encode_q6_k(Wf):
    """float [N, K] -> uint8 [N, K/256*210] (signed 6-bit codes, int8
    scales per 16 weights)."""
    Wf = np.asarray(Wf)
    N, K = Wf.shape
    assert K % 256 == 0
    ns = K // 256
    sub = Wf.reshape(N, ns, 16, 16).astype(np.float64)
    t = np.abs(sub).max(axis=-1) / 31.0
    d16 = _f16(t.max(axis=-1) / 127.0)
    d = d16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d != 0, np.clip(_round_half_away(t / d), 0, 127), 0)
        ds = (d * sc)[..., None]
        q = np.where(ds != 0, np.clip(_round_half_away(sub / ds), -32, 31), 0)
    return _pack_q6k(d16, sc, (q + 32).reshape(N, ns, 256)).reshape(N, ns * 210)


ENCODERS = {"q8_0": encode_q8_0, "q4_0": encode_q4_0, "q4_1": encode_q4_1, "q4_k": encode_q4_k,
            "q6_k": encode_q6_k}


def quant_weights(fmt, tag, N, K, std=0.02, chunk_rows=8192):
    """Draw W ~ N(0, std^2) [N, K] and encode it; chunked to bound memory.

    The draw is one PCG64 stream, so the bytes do not depend on chunk_rows."""
    enc = ENCODERS[fmt]
    g = rng(tag)
    out = np.empty((N, row_bytes(fmt, K)), dtype=np.uint8)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        w = g.standard_normal((r1 - r0, K), dtype=np.float32) * np.float32(std)
        out[r0:r1] = enc(w)
    return out


# ---------------------------------------------------------------- shapes
# 8B Llama-shaped layer set: hidden 4096, GQA 32q/8kv x head_dim 128,
# SwiGLU intermediate 14336; lm_head 128256 x 4096; 32 layers.
LLAMA8B_LAYER = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096),
                 ("o", 4096, 4096), ("gate", 14336, 4096), ("up", 14336, 4096),
                 ("down", 4096, 14336)]
LLAMA8B_LM_HEAD = ("lm_head", 128256, 4096)
LLAMA8B_LAYERS = 32

# Qwen3-0.6B-shaped int8 layers (hidden 1024, 16q/8kv x 128, FFN 3072,
# tied lm_head over vocab 151936); 28 layers.
QWEN06B_LAYER = [("q", 2048, 1024), ("k", 1024, 1024), ("v", 1024, 1024),
                 ("o", 1024, 2048), ("gate", 3072, 1024), ("up", 3072, 1024),
                 ("down", 1024, 3072)]
QWEN06B_LM_HEAD = ("lm_head", 151936, 1024)
QWEN06B_LAYERS = 28

# 30B-A3B-style MoE experts: hidden 2048, 128 experts, top-8, expert
# gate/up 768 x 2048 and down 2048 x 768, 48 layers, Q4_0.
MOE_HIDDEN, MOE_FFN, MOE_EXPERTS, MOE_TOPK, MOE_LAYERS = 2048, 768, 128, 8, 48


def block_bytes(fmt, N, K):
    return N * row_bytes(fmt, K)


def zero_heavy(fmt, tag, N, K, B=1, every=16):
    """Stored bytes [N][row bytes] and activations [B][K] float32 of the
    zero-heavy kind (module docstring): column j carries nonzero codes only
    when j % every == every - 1 (the "small" columns)."""
    g = rng(tag)
    nb = K // 32
    small = (np.arange(K) % every) == every - 1
    x = g.standard_normal((B, K)).astype(np.float32)
    x *= np.where(small, np.float32(1e-3), np.float32(1e3))
    if fmt == "q6_k":
        ns = K // 256
        e = g.integers(-10, 3, size=(N, ns))
        d16 = np.ldexp(1.0 + g.integers(0, 8, size=(N, ns)) / 8.0, e).astype(np.float16)
        sc = g.integers(-128, 128, size=(N, ns, 16))
        codes = np.full((N, K), 32, dtype=np.int64)
        codes[:, small] = g.integers(0, 64, size=(N, int(small.sum())))
        return _pack_q6k(d16, sc, codes.reshape(N, ns, 256)).reshape(N, ns * 210), x
    if fmt == "q4_k":
        ns = K // 256
        e = g.integers(-10, 3, size=(N, ns))
        d16 = np.ldexp(1.0 + g.integers(0, 8, size=(N, ns)) / 8.0, e).astype(np.float16)   # <= 4 bits
        sc = g.integers(1, 5, size=(N, ns, 8))
        k = np.minimum(g.integers(0, 16, size=(N, ns, 8)), 63 // sc)
        codes = np.repeat(k, 32, axis=2).reshape(N, K)
        codes[:, small] = g.integers(0, 16, size=(N, int(small.sum())))
        out = _pack_q4k(d16, d16, sc, sc * k, codes.reshape(N, ns, 256))
        return out.reshape(N, ns * 144), x
    e = g.integers(-10, 3, size=(N, nb))
    frac = g.integers(0, 8, size=(N, nb))
    mag = np.ldexp(1.0 + frac / 8.0, e)                     # <= 4 significant bits
    if fmt == "q8_0":
        codes = np.zeros((N, K), dtype=np.int64)
        codes[:, small] = g.integers(-127, 128, size=(N, int(small.sum())))
        d = (mag * np.where(g.integers(0, 2, size=(N, nb)) == 1, -1.0, 1.0)).astype(np.float16)
        out = np.zeros((N, nb, 34), dtype=np.uint8)
        out[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
        out[:, :, 2:] = codes.astype(np.int8).view(np.uint8).reshape(N, nb, 32)
        return out.reshape(N, nb * 34), x
    if fmt == "q4_0":
        codes = np.full((N, K), 8, dtype=np.int64)
        codes[:, small] = g.integers(0, 16, size=(N, int(small.sum())))
        d = (mag * np.where(g.integers(0, 2, size=(N, nb)) == 1, -1.0, 1.0)).astype(np.float16)
        hdr = d.view(np.uint8).reshape(N, nb, 2)
        bb = 18
    else:
        k = g.integers(0, 16, size=(N, nb))
        codes = np.repeat(k, 32, axis=1)
        codes[:, small] = g.integers(0, 16, size=(N, int(small.sum())))
        d = mag.astype(np.float16)
        m = (-(mag * k)).astype(np.float16)                # exact: <= 8 significant bits
        assert np.all(m.astype(np.float64) == -(mag * k))
        hdr = np.concatenate([d.view(np.uint8).reshape(N, nb, 2), m.view(np.uint8).reshape(N, nb, 2)], axis=2)
        bb = 20
    c = codes.reshape(N, nb, 32).astype(np.uint8)
    qs = (c[:, :, :16] | (c[:, :, 16:] << 4)).astype(np.uint8)
    out = np.concatenate([hdr, qs], axis=2)
    assert out.shape[2] == bb
    return out.reshape(N, nb * bb), x
