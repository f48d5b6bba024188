"""The FP8 append's quotient sequence in exact arithmetic (CPU).

The FP8 append kernel computes x / s without a division per element:
q0 = RN(x * r) with r = RN(1/s), then twice q <- RN(q + RN(x - s * q) * r)
with fused multiply-adds, keeping q0 when |q0| is outside [2^-100, 2^100).
Here every float32 operation of that sequence is carried out exactly
(fractions) and rounded once to float32, nearest-even, and the result must
equal the correctly rounded quotient RN(x / s) -- the value the cache
encoding is defined on ("Quantizing the KV cache", FP8 KV cache: each value
divided by its per-head scale) -- wherever the FP8 code could depend on it.
Inputs include values a few units from every E4M3 rounding midpoint times the
scale, where a single reciprocal product would round to the wrong code."""

import math
import random
from fractions import Fraction as Fr

import numpy as np


def rn32(v):
    """Nearest-even float32 of an exact rational (float32 subnormals kept)."""
    if v == 0:
        return 0.0
    sign = -1.0 if v < 0 else 1.0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    ulp = Fr(2) ** (max(e, -126) - 23)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and n % 2 == 1):
        n += 1
    r = n * ulp
    if r >= Fr(2) ** 128:
        return sign * math.inf
    return sign * float(r)


def quotient_by_recip(x, s, r):
    """The kernel's sequence, each float32 operation rounded once."""
    q0 = rn32(Fr(x) * Fr(r))
    if not math.isfinite(q0) or not (2.0 ** -100 <= abs(q0) < 2.0 ** 100):
        return q0
    q = q0
    for _ in range(2):
        e = rn32(-Fr(q) * Fr(s) + Fr(x))
        q = rn32(Fr(e) * Fr(r) + Fr(q))
    return q


def e4m3_grid():
    vals = [m / 512 for m in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if not (e == 15 and m == 7):
                vals.append((1 + m / 8) * 2.0 ** (e - 7))
    return vals


def f32(v):
    return float(np.float32(v))


def bf16(v):
    """A bfloat16-valued float (float32 with the low 16 bits cleared)."""
    bits = np.array([np.float32(v)]).view(np.uint32) & np.uint32(0xFFFF0000)
    return float(bits.view(np.float32)[0])


def test_quotient_equals_correctly_rounded():
    rng = random.Random(20261202)
    grid = e4m3_grid()
    mids = [(a + b) / 2 for a, b in zip(grid, grid[1:])]
    checked = 0
    for trial in range(3000):
        kind = trial % 3
        amax = bf16(rng.lognormvariate(0, 3))
        s = f32(amax / 448.0)
        r = rn32(Fr(1) / Fr(s))
        if not (2.0 ** -60 <= r <= 2.0 ** 60):
            continue
        if kind == 0:       # bfloat16-valued inputs
            x = bf16(rng.gauss(0, 1) * amax / 3)
        elif kind == 1:     # a few units from an FP8 midpoint after division
            x = f32(rng.choice(mids) * s * rng.choice([1, -1]))
            for _ in range(rng.randint(0, 3)):
                x = float(np.nextafter(np.float32(x), np.float32(rng.choice([math.inf, 0.0]))))
        else:               # any magnitude
            x = f32(rng.uniform(-1, 1) * 2.0 ** rng.randint(-140, 127))
        want = rn32(Fr(x) / Fr(s))
        got = quotient_by_recip(x, s, r)
        if abs(want) < 2.0 ** -100 or abs(want) >= 2.0 ** 99 or not math.isfinite(want):
            # outside the refined range only the FP8 code must agree: a signed
            # zero below, the saturated maximum above
            assert math.copysign(1, got) == math.copysign(1, want)
            assert (abs(got) < 2.0 ** -90) == (abs(want) < 2.0 ** -90)
            continue
        assert got == want, (x, s, got, want)
        checked += 1
    assert checked > 2000
