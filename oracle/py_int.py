"""Independent big-integer mirror of the integer requant semantics.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Written separately
from ``qmv_oracle.c`` in exact rational arithmetic, from the readings of the
two functions that "Blue -- porting zen-nano (Qwen3-0.6B) to deterministic
on-chain inference" names in its "Quantization recipe":

* SaturatingRoundingDoublingHighMul(a, b): a*b / 2^31 rounded to the nearest
  integer, ties toward +infinity; the one overflowing input pair
  (-2^31, -2^31) saturates to 2^31 - 1.
* RoundingDivideByPOT(x, e): x / 2^e rounded to nearest, ties away from zero.
* The int8 result saturates to [-128, 127].
"""
from fractions import Fraction
import math

INT32_MIN = -(1 << 31)
INT32_MAX = (1 << 31) - 1


def srdhm(a: int, b: int) -> int:
    if a == INT32_MIN and b == INT32_MIN:
        return INT32_MAX
    v = Fraction(a * b, 1 << 31)
    return math.floor(v + Fraction(1, 2))


def rdbpot(x: int, e: int) -> int:
    v = Fraction(x, 1 << e)
    mag = math.floor(abs(v) + Fraction(1, 2))
    return mag if v >= 0 else -mag


def sat8(v: int) -> int:
    return max(-128, min(127, v))


def requant(acc: int, mult: int, shift: int) -> int:
    return sat8(rdbpot(srdhm(acc, mult), shift))


def matvec_i8(W, x, mult, shift):
    """Tiny-size int8 matvec with requant, pure Python loops.

    W: list of rows of ints, x: list of ints; returns (acc list, y list)."""
    acc = [sum(int(w) * int(v) for w, v in zip(row, x)) for row in W]
    return acc, [requant(a, int(m), int(s)) for a, m, s in zip(acc, mult, shift)]
