"""Constructed Q8_1 blocks whose s field tells one rounding from two.

s = d * sum(q) is an fp32 product that is then rounded to binary16.  For the
blocks built here the exact product rounds to binary16 differently in one step
than through fp32 first, so a quantiser that fuses the two roundings fails.
Found by search in exact rational arithmetic; nothing here runs the layer.
"""
from fractions import Fraction

import numpy as np

from test_oracle_pins import rn16, rn32  # noqa: E402


def double_rounding_blocks(n: int = 8, seed: int = 3):
    rng = np.random.default_rng(seed)
    out = []
    tries = 0
    while len(out) < n and tries < 200000:
        tries += 1
        amax = np.float32(rng.uniform(0.05, 40.0))
        d = rn32(Fraction(float(amax)) / 127)
        if d == 0:
            continue
        total = int(rng.integers(-4064, 4065))
        p = d * total
        if p == 0 or rn16(rn32(p)) == rn16(p):
            continue
        # 31 codes plus the amax element (+127) summing to total
        rest = total - 127
        if abs(rest) > 31 * 127:
            continue
        q = np.full(31, rest // 31, dtype=np.int64)
        q[: rest - int(q.sum())] += 1
        if np.abs(q).max() > 127:
            continue
        v = np.empty(32, np.float32)
        v[0] = amax
        v[1:] = [np.float32(float(rn32(int(c) * d))) for c in q]
        # the construction must reproduce q exactly under the definition
        qq = [0 if d == 0 else int(np.sign(float(rn32(Fraction(float(x)) / d))) *
                                   np.floor(abs(float(rn32(Fraction(float(x)) / d))) + 0.5)) for x in v]
        if sum(qq) != total or qq[0] != 127:
            continue
        out.append(v)
    return np.stack(out)
