"""Builds the hand-computed blocks of tests/golden/hand_blocks.json."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_blocks.json")


def load():
    with open(GOLDEN) as f:
        return json.load(f)


def _u16(h):
    v = int(h, 16)
    return [v & 0xFF, v >> 8]


def block_bytes(spec):
    fmt = spec["fmt"]
    if fmt == "q8_0":
        codes = np.zeros(32, dtype=np.int64)
        c = spec["codes"]
        if c == "j-16":
            codes = np.arange(32) - 16
        elif c.startswith("e0:"):
            codes[0] = int(c[3:])
        else:
            raise ValueError(c)
        return np.array(_u16(spec["d"]) + [int(v) & 0xFF for v in codes], dtype=np.uint8)
    qs = np.zeros(16, dtype=np.int64)
    q = spec["qs"]
    if q.startswith("all:"):
        qs[:] = int(q[4:], 16)
    elif q == "j|(15-j)<<4":
        j = np.arange(16)
        qs = j | ((15 - j) << 4)
    elif q == "j":
        qs = np.arange(16)
    elif q.startswith("e0:"):
        qs[0] = int(q[3:])  # low nibble of byte 0 = element 0
    else:
        raise ValueError(q)
    head = _u16(spec["d"]) + (_u16(spec["m"]) if fmt == "q4_1" else [])
    return np.array(head + [int(v) for v in qs], dtype=np.uint8)


def x_vec(kind):
    if kind == "ones":
        return np.ones(32, dtype=np.float32)
    if kind == "ramp":
        return np.arange(32, dtype=np.float32)
    if kind == "e0":
        x = np.zeros(32, dtype=np.float32)
        x[0] = 1
        return x
    raise ValueError(kind)


def _bytes_of(spec, n):
    if isinstance(spec, list):
        assert len(spec) == n
        return [v & 0xFF for v in spec]
    if spec.startswith("all:"):
        return [int(spec[4:], 0) & 0xFF] * n
    if spec == "k":
        return list(range(n))
    raise ValueError(spec)


def super_block_bytes(spec):
    """The stored bytes of a super-block spec: 144 for Q4_K, 210 for Q6_K."""
    if spec["fmt"] == "q6_k":
        out = _bytes_of(spec["ql"], 128) + _bytes_of(spec["qh"], 64) + _bytes_of(spec["sc"], 16) + _u16(spec["d"])
        assert len(out) == 210
        return np.array(out, dtype=np.uint8)
    q = spec["q"]
    if q.startswith("all:"):
        qs = [int(q[4:], 16)] * 128
    elif q == "k":
        qs = list(range(128))
    else:
        raise ValueError(q)
    out = _u16(spec["d"]) + _u16(spec["dmin"]) + list(spec["b"]) + qs
    assert len(out) == 144
    return np.array(out, dtype=np.uint8)


def x_vec256(kind):
    if kind == "ones":
        return np.ones(256, dtype=np.float32)
    if kind == "ramp":
        return np.arange(256, dtype=np.float32)
    raise ValueError(kind)
