"""Pins of the CPU oracle to facts fixed outside it.

Every check here compares the oracle with something it does not compute
itself: IEEE 754 bit patterns, hand-derived golden blocks, exact rational
arithmetic, brute-force integer sums, library sorts, closed forms and
invariants of the layer.  A plausible slip in the oracle (a dropped term, a
wrong sign or index, a swapped operand, the wrong rounding mode) fails at least
one of them.
"""
import dataclasses
import json
import math
import os
from fractions import Fraction

import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- exact helpers
def _parse(s):
    """'127*2^-20', '2^-24', '1 + 3*2^-11', '1365 * 2^-12' -> Fraction (tiny grammar)."""
    s = s.replace(" ", "")
    if s in ("inf", "-inf"):
        return s
    total = Fraction(0)
    s = s.replace("^-", "^m")
    for term in s.replace("-", "+-").split("+"):
        if not term:
            continue
        neg = term.startswith("-")
        term = term.lstrip("-")
        val = Fraction(1)
        for f in term.split("*"):
            if "^" in f:
                b, e = f.split("^")
                val *= Fraction(int(b)) ** int(e.replace("m", "-"))
            else:
                val *= Fraction(f)
        total += -val if neg else val
    return total


def _binade(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def rn(fr: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Round a rational to the nearest value with mant_bits significand bits (ties to even),
    gradual underflow below 2^emin.  Overflow is not modelled."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = max(_binade(a), emin)
    q = Fraction(2) ** (e - (mant_bits - 1))
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * q


def rn32(fr):
    return rn(Fraction(fr), 24, -126)


def rn16(fr):
    return rn(Fraction(fr), 11, -14)


def half_away(fr: Fraction) -> int:
    a = abs(fr)
    n = int(math.floor(a + Fraction(1, 2)))
    return -n if fr < 0 else n


def q8_1_exact(v32: np.ndarray):
    """Q8_1 of a float32 block from the definition, in exact rational arithmetic."""
    vals = [Fraction(float(x)) for x in v32]
    amax = max(abs(x) for x in vals)
    d = rn32(amax / 127)
    q = [0 if d == 0 else half_away(rn32(x / d)) for x in vals]
    s = rn32(d * sum(q))
    return d, s, q


# ------------------------------------------------------------------ binary16
def test_f16_decode_ieee_patterns(orc):
    g = json.load(open(os.path.join(GOLD, "f16_patterns.json")))
    for c in g["cases"]:
        bits = int(c["bits"], 16)
        got = orc.f16_decode(bits)
        if c["value"] == "inf":
            assert got == math.inf
        else:
            assert Fraction(got) == _parse(c["value"]), c


def test_f16_encode_ieee_rounding(orc):
    g = json.load(open(os.path.join(GOLD, "f16_patterns.json")))
    for c in g["cases"]:
        if c["value"] == "inf":
            continue
        assert orc.f16_encode(float(_parse(c["value"]))) == int(c["bits"], 16), c
    for c in g["rounding"]["cases"]:
        v = _parse(c["value"]) if "^" in c["value"] else Fraction(c["value"])
        assert orc.f16_encode(float(v)) == int(c["bits"], 16), c


def test_f16_roundtrip_all_patterns(orc):
    for h in range(0, 1 << 16, 7):
        e = (h >> 10) & 31
        if e == 31 and (h & 1023):
            continue  # NaN
        assert orc.f16_encode(orc.f16_decode(h)) == h


def test_f16_encode_matches_numpy(orc):
    """numpy's double -> binary16 conversion is a correctly rounded library routine."""
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(2000) * 10.0 ** rng.integers(-9, 5, 2000),
        (np.arange(-300, 300) + 0.5) * 2.0 ** -24,     # subnormal ties
        1.0 + (np.arange(0, 64) + 0.5) * 2.0 ** -10,    # normal ties
        [65504.0, 65519.0, 65520.0, 1e6, -65520.0]])
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    for v, r in zip(vals, ref):
        assert orc.f16_encode(float(v)) == int(r), v


def test_f16_encode_exact_rational(orc):
    rng = np.random.default_rng(8)
    for v in rng.standard_normal(300) * 1e-3:
        assert Fraction(orc.f16_decode(orc.f16_encode(float(v)))) == rn16(Fraction(float(v)))


# ---------------------------------------------------------------- Q8_1 blocks
def _golden_q8_1():
    g = json.load(open(os.path.join(GOLD, "quant_blocks.json")))
    for c in g["q8_1"]:
        if "fill" in c:
            v = np.full(32, float(_parse(c["fill"])), dtype=np.float32)
            q = np.full(32, c["q_all"], dtype=np.int8)
        else:
            v = np.zeros(c["pad_zero_to"], dtype=np.float32)
            v[:len(c["v"])] = [float(_parse(s)) for s in c["v"]]
            q = np.zeros(32, dtype=np.int8)
            q[:len(c["q"])] = c["q"]
        yield c, v, q


def test_q8_1_golden_blocks(orc):
    for c, v, q in _golden_q8_1():
        blk = orc.quantize_q8_1(v)[0]
        assert (int(blk[0]) | int(blk[1]) << 8) == int(c["d16"], 16), c["name"]
        assert (int(blk[2]) | int(blk[3]) << 8) == int(c["s16"], 16), c["name"]
        assert np.array_equal(blk[4:].view(np.int8), q), c["name"]


def _check_exact(orc, v):
    blk = orc.quantize_q8_1(v)[0]
    d, s, q = q8_1_exact(v)
    assert np.array_equal(blk[4:].view(np.int8).astype(int), np.array(q)), v
    assert Fraction(orc.f16_decode(int(blk[0]) | int(blk[1]) << 8)) == rn16(d)
    assert Fraction(orc.f16_decode(int(blk[2]) | int(blk[3]) << 8)) == rn16(s)


def test_q8_1_exact_rational_random(orc):
    rng = np.random.default_rng(11)
    for scale in (1.0, 1e-3, 30.0, 2.0 ** -18):
        for _ in range(40):
            _check_exact(orc, (rng.standard_normal(32) * scale).astype(np.float32))


def test_q8_1_true_divide_not_reciprocal(orc):
    """Blocks where v * (1/d) and v / d round to different integers: the oracle must take the
    correctly rounded divide."""
    rng = np.random.default_rng(12)
    found = 0
    for _ in range(4000):
        amax = np.float32(rng.uniform(0.5, 8.0))
        d = rn32(Fraction(float(amax)) / 127)
        inv = rn32(1 / d)
        n = int(rng.integers(1, 126))
        centre = rn32((n + Fraction(1, 2)) * d)
        for k in range(-3, 4):
            v = np.float32(float(centre))
            v = np.nextafter(v, np.float32(np.inf) if k > 0 else np.float32(-np.inf), dtype=np.float32) \
                if k else v
            for _ in range(abs(k) - 1):
                v = np.nextafter(v, np.float32(np.inf) if k > 0 else np.float32(-np.inf), dtype=np.float32)
            if half_away(rn32(Fraction(float(v)) / d)) != half_away(rn32(Fraction(float(v)) * inv)):
                blk = np.zeros(32, np.float32)
                blk[0] = amax
                blk[1] = v
                _check_exact(orc, blk)
                found += 1
        if found >= 5:
            break
    assert found >= 5


def test_q8_1_invariants(orc):
    rng = np.random.default_rng(13)
    v = (rng.standard_normal((64, 32)) * rng.uniform(0.01, 10, (64, 1))).astype(np.float32)
    blk = orc.quantize_q8_1(v.reshape(-1)).reshape(64, 36)
    for b in range(64):
        q = blk[b, 4:].view(np.int8).astype(np.int64)
        assert np.abs(q).max() == 127
        assert abs(int(q[np.argmax(np.abs(v[b]))])) == 127
        assert np.all((q == 0) | (np.sign(q) == np.sign(v[b])))
        d = float(np.float32(np.abs(v[b]).max()) / np.float32(127))
        assert np.all(np.abs(v[b] - d * q) <= 0.5 * d * (1 + 1e-6))
    # power-of-two scaling leaves q unchanged and scales d exactly
    b2 = orc.quantize_q8_1((v[:8] * np.float32(4.0)).reshape(-1)).reshape(8, 36)
    assert np.array_equal(b2[:, 4:], blk[:8, 4:])
    for b in range(8):
        assert orc.f16_decode(int(b2[b, 0]) | int(b2[b, 1]) << 8) == pytest.approx(
            4 * orc.f16_decode(int(blk[b, 0]) | int(blk[b, 1]) << 8), rel=2 ** -10)


# ------------------------------------------------------------------ block dots
def _rand_q8_0(rng, n):
    b = np.zeros((n, 34), np.uint8)
    d = (np.abs(rng.standard_normal(n)) * 0.02 / 127).astype(np.float16).view(np.uint16)
    b[:, 0] = d & 0xFF
    b[:, 1] = d >> 8
    b[:, 2:] = rng.integers(-127, 128, (n, 32)).astype(np.int8).view(np.uint8)
    return b


def _rand_q4_0(rng, n):
    b = np.zeros((n, 18), np.uint8)
    d = (np.abs(rng.standard_normal(n)) * 0.02 / 8).astype(np.float16).view(np.uint16)
    b[:, 0] = d & 0xFF
    b[:, 1] = d >> 8
    b[:, 2:] = rng.integers(0, 256, (n, 16)).astype(np.uint8)
    return b


def _rand_q8_1(orc, rng, n):
    return orc.quantize_q8_1(rng.standard_normal(32 * n).astype(np.float32)).reshape(n, 36)


def test_isum_q8_0_bruteforce(orc):
    rng = np.random.default_rng(21)
    w = _rand_q8_0(rng, 200)
    a = _rand_q8_1(orc, rng, 200)
    for i in range(200):
        ref = int(np.dot(w[i, 2:].view(np.int8).astype(np.int64), a[i, 4:].view(np.int8).astype(np.int64)))
        assert orc.isum(8, w[i], a[i]) == ref
    # extremes: |isum| reaches 32 * 127 * 127
    w1 = w[0].copy(); w1[2:] = np.uint8(127)
    a1 = a[0].copy(); a1[4:] = np.uint8(127)
    assert orc.isum(8, w1, a1) == 516128
    a1[4:] = np.int8(-127).view(np.uint8)
    assert orc.isum(8, w1, a1) == -516128


def test_isum_q4_0_golden_nibble_order(orc):
    g = json.load(open(os.path.join(GOLD, "quant_blocks.json")))
    for c in g["q4_0"]:
        w = np.zeros(18, np.uint8)
        d = int(c["d16"], 16)
        w[0], w[1] = d & 0xFF, d >> 8
        w[2:] = int(c["rest"], 16)
        if c["bytes"]:
            w[2] = int(c["bytes"], 16)
        a = np.zeros(36, np.uint8)
        a[4:] = (np.arange(32) + 1).astype(np.int8).view(np.uint8)
        assert orc.isum(2, w, a) == c["isum"], c["name"]


def test_isum_q4_0_bruteforce(orc):
    rng = np.random.default_rng(22)
    w = _rand_q4_0(rng, 200)
    a = _rand_q8_1(orc, rng, 200)
    for i in range(200):
        codes = np.concatenate([w[i, 2:] & 0x0F, w[i, 2:] >> 4]).astype(np.int64) - 8
        ref = int(np.dot(codes, a[i, 4:].view(np.int8).astype(np.int64)))
        assert orc.isum(2, w[i], a[i]) == ref


def _q5_1_block(c):
    w = np.zeros(24, np.uint8)
    d, m = int(c["d16"], 16), int(c["m16"], 16)
    w[0], w[1], w[2], w[3] = d & 0xFF, d >> 8, m & 0xFF, m >> 8
    w[4:8] = np.frombuffer(bytes.fromhex(c["qh"]), np.uint8)
    w[8:] = np.frombuffer(bytes.fromhex(c["qs"]), np.uint8)
    return w


def test_q5_1_golden_blocks(orc):
    """Hand-derived Q5_1 blocks: bit and nibble order of the codes, the little-endian qh, and
    the min term, which multiplies the Q8_1 block's stored s (not d_a * sum(q_a))."""
    g = json.load(open(os.path.join(GOLD, "quant_blocks.json")))
    assert len(g["q5_1"]) == 7
    for c in g["q5_1"]:
        w = _q5_1_block(c)
        a = np.zeros(36, np.uint8)
        ad, as_ = int(c["a_d16"], 16), int(c["a_s16"], 16)
        a[0], a[1], a[2], a[3] = ad & 0xFF, ad >> 8, as_ & 0xFF, as_ >> 8
        a[4:] = (np.arange(32) + 1).astype(np.int8).view(np.uint8)
        assert orc.isum(7, w, a) == c["isum"], c["name"]
        y = orc.matvec(7, w, 1, 1, a)
        assert y[0] == np.float32(c["y"]), (c["name"], y[0])


def _rand_q5_1(rng, n):
    b = np.zeros((n, 24), np.uint8)
    d = (np.abs(rng.standard_normal(n)) * 0.02 / 16).astype(np.float16).view(np.uint16)
    m = (-np.abs(rng.standard_normal(n)) * 0.01).astype(np.float16).view(np.uint16)
    b[:, 0], b[:, 1] = d & 0xFF, d >> 8
    b[:, 2], b[:, 3] = m & 0xFF, m >> 8
    b[:, 4:] = rng.integers(0, 256, (n, 20)).astype(np.uint8)
    return b


def test_isum_q5_1_bruteforce(orc):
    """The integer part against numpy bit arithmetic on random blocks."""
    rng = np.random.default_rng(24)
    w = _rand_q5_1(rng, 200)
    a = _rand_q8_1(orc, rng, 200)
    for i in range(200):
        qh = int.from_bytes(bytes(w[i, 4:8]), "little")
        nib = np.concatenate([w[i, 8:] & 0x0F, w[i, 8:] >> 4]).astype(np.int64)
        hi = np.array([(qh >> j) & 1 for j in range(32)], np.int64)
        ref = int(np.dot(nib | (hi << 4), a[i, 4:].view(np.int8).astype(np.int64)))
        assert orc.isum(7, w[i], a[i]) == ref


def test_q5_1_row_is_dequantised_dot_with_the_stored_s(orc):
    """A Q5_1 row equals the fp64 dot of the dequantised weights (d*q + m) with the Q8_1
    activations when the activation sum is taken as each block's stored s: the d*q part is
    exact per block and the m part is m * s."""
    rng = np.random.default_rng(25)
    nblk = 10
    W = _rand_q5_1(rng, 3 * nblk)
    A = _rand_q8_1(orc, rng, nblk)
    y, isum = orc.matvec(7, W.reshape(-1), 3, nblk, A.reshape(-1), with_isum=True)
    for r in range(3):
        acc = 0.0
        for b in range(nblk):
            wb = W[r * nblk + b]
            da = orc.f16_decode(int(A[b, 0]) | int(A[b, 1]) << 8)
            sa = orc.f16_decode(int(A[b, 2]) | int(A[b, 3]) << 8)
            dw = orc.f16_decode(int(wb[0]) | int(wb[1]) << 8)
            mw = orc.f16_decode(int(wb[2]) | int(wb[3]) << 8)
            qa = A[b, 4:].view(np.int8).astype(np.int64)
            # d*q part: the dequantised codes times the dequantised activations, exact
            part = math.fsum((orc.dequant_weight(7, wb, j) - mw) * da * int(qa[j]) for j in range(32))
            assert part == dw * da * isum[r, b]
            # the stored s is d * sum(q_a) (fp32 d, rounded to binary16), not the float sum
            assert sa == pytest.approx(da * int(qa.sum()), rel=2 ** -9, abs=2 ** -24)
            acc += part + mw * sa
        assert y[r] == np.float32(acc)


def _q4_k_superblock(d16=0, dmin16=0, scales="00" * 12, qs=()):
    sb = np.zeros(144, np.uint8)
    sb[0], sb[1], sb[2], sb[3] = d16 & 0xFF, d16 >> 8, dmin16 & 0xFF, dmin16 >> 8
    sb[4:16] = np.frombuffer(bytes.fromhex(scales), np.uint8)
    for i, v in qs:
        sb[16 + i] = v
    return sb


def test_q4_k_golden_superblocks(orc):
    """Hand-derived Q4_K super-blocks: the 6-bit scale and min unpacking of sub-blocks below
    and above 4, the nibble order of the codes, and one row value whose min term takes the
    activation block's code sum."""
    g = json.load(open(os.path.join(GOLD, "quant_blocks.json")))
    for c in g["q4_k"]:
        sb = _q4_k_superblock(scales=c["scales"])
        assert orc.q4_k_scale_min(sb, c["b"]) == (c["scale"], c["min"]), c["name"]
    c = g["q4_k_codes"]
    sb = _q4_k_superblock(qs=[(c["qs_byte"], int(c["value"], 16))])
    a = np.zeros(36, np.uint8)
    a[4:] = (np.arange(32) + 1).astype(np.int8).view(np.uint8)
    assert orc.isum_q4_k(sb, 2, a) == c["isum_b2"]
    assert orc.isum_q4_k(sb, 3, a) == c["isum_b3"]
    assert orc.isum_q4_k(sb, 0, a) == 0 and orc.isum_q4_k(sb, 1, a) == 0
    c = g["q4_k_row"]
    sb = _q4_k_superblock(int(c["d16"], 16), int(c["dmin16"], 16), c["scales"],
                          [(c["qs_byte"], int(c["value"], 16))])
    act = np.zeros((8, 36), np.uint8)
    ad = int(c["a_d16"], 16)
    act[c["active_block"], 0], act[c["active_block"], 1] = ad & 0xFF, ad >> 8
    act[c["active_block"], 4:] = (np.arange(32) + 1).astype(np.int8).view(np.uint8)
    y = orc.matvec(12, sb, 1, 8, act.reshape(-1))
    assert y[0] == np.float32(c["y"])


def _rand_q4_k(rng, n):
    sb = rng.integers(0, 256, (n, 144)).astype(np.uint8)
    d = (np.abs(rng.standard_normal(n)) * 0.02 / 512).astype(np.float16).view(np.uint16)
    dm = (np.abs(rng.standard_normal(n)) * 0.02 / 128).astype(np.float16).view(np.uint16)
    sb[:, 0], sb[:, 1], sb[:, 2], sb[:, 3] = d & 0xFF, d >> 8, dm & 0xFF, dm >> 8
    return sb


def test_q4_k_bruteforce_and_dequantised_dot(orc):
    """Integer sums against numpy bit arithmetic, and each sub-block's contribution equal,
    exactly, to the fp64 dot of the dequantised weights d*scale*q - dmin*min with the
    dequantised activations; the row sums the sub-blocks in order."""
    rng = np.random.default_rng(26)
    n = 6
    W = _rand_q4_k(rng, 2 * n)
    A = _rand_q8_1(orc, rng, 8 * n)
    y = orc.matvec(12, W.reshape(-1), 2, 8 * n, A.reshape(-1))
    for r in range(2):
        acc = 0.0
        for b in range(8 * n):
            sb = W[r * n + b // 8]
            j = b % 8
            sbytes = sb[4:16].astype(np.int64)
            if j < 4:
                sc, mn = sbytes[j] & 63, sbytes[j + 4] & 63
            else:
                sc = (sbytes[j + 4] & 15) | (sbytes[j - 4] >> 6) << 4
                mn = (sbytes[j + 4] >> 4) | (sbytes[j] >> 6) << 4
            assert orc.q4_k_scale_min(sb, j) == (sc, mn)
            nib = sb[16 + 32 * (j // 2):16 + 32 * (j // 2) + 32].astype(np.int64)
            q = (nib >> 4) if j % 2 else (nib & 15)
            qa = A[b, 4:].view(np.int8).astype(np.int64)
            assert orc.isum_q4_k(sb, j, A[b]) == int(np.dot(q, qa))
            da = orc.f16_decode(int(A[b, 0]) | int(A[b, 1]) << 8)
            part = math.fsum(orc.dequant_weight(12, sb, 32 * j + i) * da * int(qa[i]) for i in range(32))
            d = orc.f16_decode(int(sb[0]) | int(sb[1]) << 8)
            dmin = orc.f16_decode(int(sb[2]) | int(sb[3]) << 8)
            assert part == d * sc * da * int(np.dot(q, qa)) - dmin * mn * da * int(qa.sum())
            acc += part
        assert y[r] == np.float32(acc)


def test_q5_k_golden_fifth_bits(orc):
    """Hand-derived Q5_K codes: the fifth bit of element i of sub-block b is bit b of qh byte
    i, on top of the Q4_K nibble order."""
    g = json.load(open(os.path.join(GOLD, "quant_blocks.json")))
    c = g["q5_k_codes"]
    sb = np.zeros(176, np.uint8)
    sb[16 + c["qh_byte"]] = int(c["qh"], 16)
    sb[48 + c["qs_byte"]] = int(c["qs"], 16)
    a = np.zeros(36, np.uint8)
    a[4:] = (np.arange(32) + 1).astype(np.int8).view(np.uint8)
    for b in (2, 3, 4, 5):
        assert orc.isum_q5_k(sb, b, a) == c[f"isum_b{b}"], b
    assert orc.isum_q5_k(sb, 0, a) == 0


def test_q5_k_bruteforce_and_dequantised_dot(orc):
    """Q5_K integer sums against numpy bit arithmetic, and the sub-block contribution equal,
    exactly, to the dequantised fp64 dot; the row sums the sub-blocks in order."""
    rng = np.random.default_rng(27)
    n = 4
    W = rng.integers(0, 256, (2 * n, 176)).astype(np.uint8)
    d = (np.abs(rng.standard_normal(2 * n)) * 0.02 / 1024).astype(np.float16).view(np.uint16)
    dm = (np.abs(rng.standard_normal(2 * n)) * 0.02 / 128).astype(np.float16).view(np.uint16)
    W[:, 0], W[:, 1], W[:, 2], W[:, 3] = d & 0xFF, d >> 8, dm & 0xFF, dm >> 8
    A = _rand_q8_1(orc, rng, 8 * n)
    y = orc.matvec(13, W.reshape(-1), 2, 8 * n, A.reshape(-1))
    for r in range(2):
        acc = 0.0
        for b in range(8 * n):
            sb = W[r * n + b // 8]
            j = b % 8
            sc, mn = orc.q4_k_scale_min(sb, j)
            nib = sb[48 + 32 * (j // 2):48 + 32 * (j // 2) + 32].astype(np.int64)
            q = ((nib >> 4) if j % 2 else (nib & 15)) | ((sb[16:48].astype(np.int64) >> j) & 1) << 4
            qa = A[b, 4:].view(np.int8).astype(np.int64)
            assert orc.isum_q5_k(sb, j, A[b]) == int(np.dot(q, qa))
            da = orc.f16_decode(int(A[b, 0]) | int(A[b, 1]) << 8)
            part = math.fsum(orc.dequant_weight(13, sb, 32 * j + i) * da * int(qa[i]) for i in range(32))
            dd = orc.f16_decode(int(sb[0]) | int(sb[1]) << 8)
            dmin = orc.f16_decode(int(sb[2]) | int(sb[3]) << 8)
            assert part == dd * sc * da * int(np.dot(q, qa)) - dmin * mn * da * int(qa.sum())
            acc += part
        assert y[r] == np.float32(acc)


def _q3_k_superblock(d16=0, scales="00" * 12, qs=(), hmask=()):
    sb = np.zeros(110, np.uint8)
    for i, v in hmask:
        sb[i] = v
    for i, v in qs:
        sb[32 + i] = v
    sb[96:108] = np.frombuffer(bytes.fromhex(scales), np.uint8)
    sb[108], sb[109] = d16 & 0xFF, d16 >> 8
    return sb


def test_q3_k_golden_superblocks(orc):
    """Hand-derived Q3_K super-blocks: the 6-bit signed sub-block scales (low nibbles of
    bytes 0..7 for sub-blocks below 8, high nibbles above, top bits from bytes 8..11), the
    code order (two bits in qs, the high bit in hmask, minus 4), the two scaled halves of a
    block, and one row value."""
    g = json.load(open(os.path.join(GOLD, "quant_blocks.json")))
    for c in g["q3_k"]:
        sb = _q3_k_superblock(scales=c["scales"])
        assert orc.q3_k_scale(sb, c["i"]) == c["scale"], c["name"]
    c = g["q3_k_codes"]
    sb = _q3_k_superblock(scales=c["scales"], qs=[(c["qs_byte"], int(c["qs"], 16))],
                          hmask=[(c["hmask_byte"], int(c["hmask"], 16))])
    assert orc.q3_k_code(sb, c["element"]) == c["code"]
    assert orc.q3_k_code(sb, 0) == c["zero_code"]
    a = np.zeros(36, np.uint8)
    a[4:] = (np.arange(32) + 1).astype(np.int8).view(np.uint8)
    assert orc.isum_q3_k(sb, 6, a) == c["isum_b6"]
    assert orc.isum_q3_k(sb, 1, a) == c["isum_b1"]
    c = g["q3_k_row"]
    sb = _q3_k_superblock(int(c["d16"], 16), c["scales"], [(c["qs_byte"], int(c["qs"], 16))],
                          [(c["hmask_byte"], int(c["hmask"], 16))])
    act = np.zeros((8, 36), np.uint8)
    ad = int(c["a_d16"], 16)
    act[c["active_block"], 0], act[c["active_block"], 1] = ad & 0xFF, ad >> 8
    act[c["active_block"], 4:] = (np.arange(32) + 1).astype(np.int8).view(np.uint8)
    y = orc.matvec(11, sb, 1, 8, act.reshape(-1))
    assert y[0] == np.float32(c["y"])


def test_q3_k_bruteforce_and_dequantised_dot(orc):
    """Q3_K codes and scales against numpy bit arithmetic over whole super-blocks, integer
    block sums against the numpy dot, and each block's contribution equal, exactly, to the
    fp64 dot of the dequantised weights d * scale * code with the dequantised activations."""
    rng = np.random.default_rng(28)
    n = 4
    W = rng.integers(0, 256, (2 * n, 110)).astype(np.uint8)
    d = (np.abs(rng.standard_normal(2 * n)) * 0.02 / 128).astype(np.float16).view(np.uint16)
    W[:, 108], W[:, 109] = d & 0xFF, d >> 8
    A = _rand_q8_1(orc, rng, 8 * n)
    y = orc.matvec(11, W.reshape(-1), 2, 8 * n, A.reshape(-1))
    e = np.arange(256)
    half, j, l = e // 128, (e % 128) // 32, e % 32
    for r in range(2):
        acc = 0.0
        for sbi in range(n):
            sb = W[r * n + sbi]
            s = sb[96:108].astype(np.int64)
            i = np.arange(16)
            lo = np.where(i < 8, s[i % 8] & 15, s[i % 8] >> 4)
            sc = (lo | ((s[8 + i % 4] >> (2 * (i // 4))) & 3) << 4) - 32
            code = ((sb[32 + 32 * half + l].astype(np.int64) >> (2 * j)) & 3) \
                + 4 * ((sb[l].astype(np.int64) >> (4 * half + j)) & 1) - 4
            assert [orc.q3_k_scale(sb, k) for k in range(16)] == list(sc)
            assert [orc.q3_k_code(sb, k) for k in range(256)] == list(code)
            dd = orc.f16_decode(int(sb[108]) | int(sb[109]) << 8)
            for b in range(8):
                a = A[sbi * 8 + b]
                qa = a[4:].view(np.int8).astype(np.int64)
                ref = int(sc[2 * b] * np.dot(code[32 * b:32 * b + 16], qa[:16])
                          + sc[2 * b + 1] * np.dot(code[32 * b + 16:32 * b + 32], qa[16:]))
                assert orc.isum_q3_k(sb, b, a) == ref
                da = orc.f16_decode(int(a[0]) | int(a[1]) << 8)
                part = math.fsum(orc.dequant_weight(11, sb, 32 * b + k) * da * int(qa[k])
                                 for k in range(32))
                assert part == dd * da * ref
                acc += part
        assert y[r] == np.float32(acc)


# -------------------------------------------------------------------- NVFP4
def _nvfp4_gold():
    return json.load(open(os.path.join(GOLD, "nvfp4.json")))


def test_nvfp4_e2m1_value_table(orc):
    """Every FP4 E2M1 code decodes to the published value table (sign bit 3)."""
    g = _nvfp4_gold()
    for c in range(16):
        v = orc.e2m1(c)
        assert v == g["e2m1"][c] and math.copysign(1.0, v) == math.copysign(1.0, g["e2m1"][c]), c


def test_nvfp4_e4m3_values(orc):
    """E4M3 scale bytes: zero, subnormals, the smallest normal, a mantissa, the largest finite,
    a negative, and NaN at 0x7F / 0xFF."""
    for e in _nvfp4_gold()["e4m3"]:
        assert orc.e4m3(int(e["byte"], 16)) == e["value"], e
    assert math.isnan(orc.e4m3(0x7F)) and math.isnan(orc.e4m3(0xFF))


def _nvfp4_act(orc, case):
    """The Q8_1 activation block of a golden case (d, the codes, and s = d * sum(q) in binary16)."""
    j = np.arange(32)
    q = (j - 16) if case["act_q"].startswith("q_j = j - 16") else np.where(j < 16, j + 1, 1)
    a = np.zeros(36, dtype=np.uint8)
    d16 = int(case["act_d"], 16)
    a[0], a[1] = d16 & 0xFF, d16 >> 8
    s16 = orc.f16_encode(orc.f16_decode(d16) * float(q.sum()))
    a[2], a[3] = s16 & 0xFF, s16 >> 8
    a[4:] = q.astype(np.int8).view(np.uint8)
    return a


def test_nvfp4_golden_blocks(orc):
    """Hand-derived blocks pin the nibble order (2i low, 2i + 1 high), the per-half scales,
    the sign bit, a subnormal scale, the half sums of 2 * e2m1 * q_a, the tap packing (half 0
    in the low 16 bits) and the tensor scale."""
    for case in _nvfp4_gold()["blocks"]:
        w = np.array([int(b, 16) for b in case["block"].split()], dtype=np.uint8)
        a = _nvfp4_act(orc, case)
        h0, h1 = case["isum_half"]
        assert orc.isum_nvfp4_half(w, a, 0) == h0, case["name"]
        assert orc.isum_nvfp4_half(w, a, 1) == h1, case["name"]
        y, tap = orc.row_dot_nvfp4(w, a, 1, case["tensor_scale"], with_isum=True)
        assert y == np.float32(case["dot"]), (case["name"], y)
        assert int(tap[0]) == np.int32(np.uint32((h0 & 0xFFFF) | ((h1 & 0xFFFF) << 16))), case["name"]
        for j, v in case["dequant"].items():
            assert orc.dequant_weight(40, w, int(j)) == v, (case["name"], j)


def test_nvfp4_bruteforce_and_dequantised_dot(orc):
    """Random rows: the half sums equal brute force over the golden E2M1 table and the
    canonical nibble order; per block the fp64 dot of the dequantised weights (E2M1 x E4M3)
    and activations is exact and equals the integer path; the row is their sum in block
    order times the tensor scale, rounded once."""
    table = np.array(_nvfp4_gold()["e2m1"])
    rng = np.random.default_rng(41)
    nblk, rows = 9, 4
    W = rng.integers(0, 256, size=(rows * nblk, 18), dtype=np.uint8)
    W[:, :2] = ((5 + rng.integers(0, 5, size=(rows * nblk, 2))) << 3 | rng.integers(0, 8, size=(rows * nblk, 2))).astype(np.uint8)
    A = _rand_q8_1(orc, rng, nblk)
    ts = 0.0037
    for r in range(rows):
        row = W[r * nblk:(r + 1) * nblk]
        y, tap = orc.row_dot_nvfp4(row.reshape(-1), A.reshape(-1), nblk, ts, with_isum=True)
        acc = 0.0
        for b in range(nblk):
            wb, a = row[b], A[b]
            codes = np.stack([wb[2:] & 0x0F, wb[2:] >> 4], axis=1).reshape(-1)   # element order
            qa = a[4:].view(np.int8).astype(np.int64)
            halves = [int(np.dot((2 * table[codes[16 * h:16 * h + 16]]).astype(np.int64),
                                 qa[16 * h:16 * h + 16])) for h in (0, 1)]
            assert orc.isum_nvfp4_half(wb, a, 0) == halves[0]
            assert orc.isum_nvfp4_half(wb, a, 1) == halves[1]
            assert int(tap[b]) == np.int32(np.uint32((halves[0] & 0xFFFF) | ((halves[1] & 0xFFFF) << 16)))
            da = orc.f16_decode(int(a[0]) | int(a[1]) << 8)
            part = math.fsum(orc.dequant_weight(40, wb, j) * da * int(qa[j]) for j in range(32))
            assert part == da * (orc.e4m3(int(wb[0])) * halves[0] + orc.e4m3(int(wb[1])) * halves[1]) / 2
            acc += part
        assert y == np.float32(acc * ts)


@pytest.mark.parametrize("fmt", [8, 2])
def test_dequantised_fp64_dot_equals_int_path_per_block(orc, fmt):
    """Per block, the fp64 dot of the dequantised weights and activations is exact and equals
    d_w * d_a * isum; the row sums them in block order."""
    rng = np.random.default_rng(23 + fmt)
    nblk = 12
    W = (_rand_q8_0 if fmt == 8 else _rand_q4_0)(rng, 5 * nblk)
    A = _rand_q8_1(orc, rng, nblk)
    y, isum = orc.matvec(fmt, W.reshape(-1), 5, nblk, A.reshape(-1), with_isum=True)
    for r in range(5):
        acc = 0.0
        for b in range(nblk):
            wb = W[r * nblk + b]
            da = orc.f16_decode(int(A[b, 0]) | int(A[b, 1]) << 8)
            deq = [orc.dequant_weight(fmt, wb, j) * (da * int(np.int8(A[b, 4 + j]))) for j in range(32)]
            blk = math.fsum(deq)
            dw = orc.f16_decode(int(wb[0]) | int(wb[1]) << 8)
            assert blk == dw * da * isum[r, b]          # exact, no tolerance
            # the dequantised values themselves: d * q (Q8_0) or d * (c - 8) (Q4_0)
            if fmt == 8:
                assert orc.dequant_weight(fmt, wb, 5) == dw * int(np.int8(wb[2 + 5]))
            else:
                assert orc.dequant_weight(fmt, wb, 20) == dw * ((int(wb[2 + 4]) >> 4) - 8)
            acc += blk
        assert y[r] == np.float32(acc)


# -------------------------------------------------------------------- router
def _wl(**kw):
    from quantized_moe_expert_softmax_amd.synth import Workload
    base = dict(name="pin", hidden=64, n_experts=8, top_k=3, n_ff=64, tokens=5, seed=5)
    base.update(kw)
    return Workload(**base)


def _topk_bruteforce(l, k, allowed):
    idx = [e for e in range(len(l)) if allowed[e]]
    order = sorted(idx, key=lambda e: (-l[e], e))   # library sort: larger logit first, ties lower id
    return order[:k]


def test_router_logits_topk_softmax(orc, synth):
    w = _wl(n_experts=16, top_k=4)
    rng = np.random.default_rng(31)
    Wr = (rng.standard_normal((16, 64)) / np.sqrt(512)).astype(np.float32)
    br = rng.standard_normal(16).astype(np.float32)
    for t in range(20):
        x = rng.standard_normal(64).astype(np.float32)
        ids, wt, l = orc.route_token(w, x, Wr, br)
        ref_l = Wr.astype(np.float64) @ x.astype(np.float64) + br.astype(np.float64)
        assert np.allclose(l, ref_l, rtol=0, atol=1e-13)
        assert list(ids) == _topk_bruteforce(l, 4, [1] * 16)
        ex = np.exp(l[ids] - l[ids].max())
        assert np.allclose(wt, ex / ex.sum(), rtol=1e-6, atol=0)
        assert abs(float(np.sum(wt.astype(np.float64))) - 1.0) < 4e-7
        assert np.all(np.diff(wt) <= 0)


def test_router_ties_go_to_lower_index(orc):
    w = _wl(n_experts=8, top_k=3)
    Wr = np.zeros((8, 64), np.float32)
    Wr[5] = 1.0
    Wr[2] = 1.0
    Wr[6] = 0.5
    x = np.ones(64, np.float32)
    ids, wt, _ = orc.route_token(w, x, Wr)
    assert list(ids) == [2, 5, 6]
    assert wt[0] == wt[1]


def test_router_k1_and_k_equals_e(orc):
    rng = np.random.default_rng(33)
    Wr = rng.standard_normal((8, 64)).astype(np.float32)
    x = rng.standard_normal(64).astype(np.float32)
    ids, wt, l = orc.route_token(_wl(top_k=1), x, Wr)
    assert ids[0] == int(np.argmax(l)) and wt[0] == 1.0
    ids, wt, l = orc.route_token(_wl(top_k=8), x, Wr)
    full = np.exp(l - l.max()) / np.exp(l - l.max()).sum()
    assert sorted(ids) == list(range(8))
    assert np.allclose(wt, full[ids], rtol=1e-6)


def test_router_zero_input_uniform(orc):
    w = _wl(top_k=3)
    ids, wt, l = orc.route_token(w, np.zeros(64, np.float32), np.ones((8, 64), np.float32))
    assert list(ids) == [0, 1, 2]
    assert np.all(wt == np.float32(1.0 / 3.0))


def test_router_group_limit_bruteforce(orc):
    """Group-limited routing on tiny E by enumerating group choices."""
    import itertools
    rng = np.random.default_rng(34)
    E, G, TG, k = 12, 4, 2, 3
    w = _wl(n_experts=E, top_k=k, n_groups=G, topk_groups=TG)
    for trial in range(30):
        perm = rng.permutation(E)
        groups = (perm // (E // G)).astype(np.int32)       # non-contiguous labels
        Wr = rng.standard_normal((E, 64)).astype(np.float32)
        x = rng.standard_normal(64).astype(np.float32)
        ids, wt, l = orc.route_token(w, x, Wr, None, groups)
        gmax = [max(l[e] for e in range(E) if groups[e] == g) for g in range(G)]
        # the chosen groups are the set of TG groups with the largest maxima (ties: lower ids)
        best = max(itertools.combinations(range(G), TG),
                   key=lambda c: (sorted([gmax[g] for g in c], reverse=True), [-g for g in c]))
        allowed = [groups[e] in best for e in range(E)]
        assert list(ids) == _topk_bruteforce(l, k, allowed)
        assert all(groups[e] in best for e in ids)


# ---------------------------------------------------------------- expert FFN
def _blob_from_rows(rows_blocks):
    return np.concatenate([r.reshape(-1) for r in rows_blocks]).astype(np.uint8)


def _q8_0_row(nblk, entries):
    """A Q8_0 row with d = 1.0 and the given {element: q} entries."""
    b = np.zeros((nblk, 34), np.uint8)
    b[:, 0], b[:, 1] = 0x00, 0x3C
    for j, q in entries.items():
        b[j // 32, 2 + j % 32] = np.uint8(np.int8(q))
    return b


def test_swiglu_closed_form_gate_first(orc):
    """g and u set to exact known values: h = g / (1 + e^-g) * u, gate first."""
    w = _wl(hidden=32, n_ff=32, n_experts=1, top_k=1)
    act = np.zeros((1, 36), np.uint8)
    act[0, 1] = 0x3C                       # d = 1
    act[0, 4] = 2                          # x_0 = 2
    gate = [_q8_0_row(1, {0: 1 + r % 3}) for r in range(32)]      # g_r = 2 * (1 + r % 3)
    up = [_q8_0_row(1, {0: -(r % 5)}) for r in range(32)]         # u_r = -2 * (r % 5)
    down = [_q8_0_row(1, {r: 1}) for r in range(32)]              # y_r = hq_r * d_h
    blob = _blob_from_rows(gate + up + down)
    r = orc.expert_ffn(w, blob, act)
    for i in range(32):
        g, u = 2.0 * (1 + i % 3), -2.0 * (i % 5)
        assert r["h"][i] == np.float32(g / (1.0 + math.exp(-g)) * u)
    # down with an identity: y_r = f16(d_h) * q_r, the dequantised Q8_1(h)
    d_h = orc.f16_decode(int(r["hq"][0, 0]) | int(r["hq"][0, 1]) << 8)
    assert np.array_equal(r["y"], (d_h * r["hq"][0, 4:].view(np.int8).astype(np.float64)).astype(np.float32))


def test_silu_zero_gate(orc):
    w = _wl(hidden=32, n_ff=32, n_experts=1, top_k=1)
    act = np.zeros((1, 36), np.uint8)
    act[0, 1], act[0, 4] = 0x3C, 3
    gate = [_q8_0_row(1, {}) for _ in range(32)]                  # g = 0 -> silu(0) = 0
    up = [_q8_0_row(1, {0: 7}) for _ in range(32)]
    down = [_q8_0_row(1, {0: 1}) for _ in range(32)]
    r = orc.expert_ffn(w, _blob_from_rows(gate + up + down), act)
    assert np.all(r["h"] == 0) and np.all(r["y"] == 0)


def _layer_inputs(synth, w, batch=0):
    return synth.gen_layer(w, batch)


def test_identical_experts_independent_of_routing(orc, synth):
    w = _wl(hidden=64, n_experts=6, top_k=3, n_ff=64, tokens=6)
    inp = _layer_inputs(synth, w)
    one = synth.gen_expert(w, 0)
    experts = np.tile(one, w.n_experts)
    out, taps = orc.layer_forward(w, inp["x"], inp["router_w"], experts=experts, taps=("xq", "ids"))
    for t in range(w.tokens):
        y = orc.expert_ffn(w, one, taps["xq"][t])["y"]
        assert np.allclose(out[t], y, rtol=1e-6, atol=1e-7 * np.abs(y).max())
    assert len({tuple(r) for r in taps["ids"]}) > 1       # routing really differed


def test_zero_weights_and_zero_input(orc, synth):
    w = _wl(tokens=4)
    inp = _layer_inputs(synth, w)
    zero = inp["experts"].copy()
    bb = w.block_bytes
    zb = zero.reshape(-1, bb)
    zb[:, 2:] = 0
    out, _ = orc.layer_forward(w, inp["x"], inp["router_w"], experts=zero)
    assert np.all(out == 0)
    out, taps = orc.layer_forward(w, np.zeros_like(inp["x"]), inp["router_w"],
                                  experts=inp["experts"], taps=("ids", "weights"))
    assert np.all(out == 0)
    assert np.all(taps["ids"] == np.arange(w.top_k)) and np.all(taps["weights"] == np.float32(1 / 3))


def test_token_list_matches_full_run(orc, synth):
    w = _wl(tokens=7)
    inp = _layer_inputs(synth, w)
    full, _ = orc.layer_forward(w, inp["x"], inp["router_w"], experts=inp["experts"], nthreads=3)
    part, _ = orc.layer_forward(w, inp["x"], inp["router_w"], experts=inp["experts"], tokens=[6, 2])
    assert np.array_equal(part, full[[6, 2]])


def _dequant_rows(orc, fmt, blocks, rows, nblk, tensor_scale=1.0):
    bb = 34 if fmt == 8 else 18
    B = blocks.reshape(rows * nblk, bb)
    if fmt == 40:
        table = np.array(_nvfp4_gold()["e2m1"])
        codes = np.stack([B[:, 2:] & 0x0F, B[:, 2:] >> 4], axis=2).reshape(rows * nblk, 32)
        sc = np.array([[orc.e4m3(int(b)) for b in blk[:2]] for blk in B])
        return (tensor_scale * np.repeat(sc, 16, axis=1) * table[codes]).reshape(rows, nblk * 32)
    d = B[:, :2].copy().view(np.float16).astype(np.float64).reshape(-1)
    if fmt == 8:
        q = B[:, 2:].view(np.int8).astype(np.float64)
    else:
        q = np.concatenate([B[:, 2:] & 0x0F, B[:, 2:] >> 4], axis=1).astype(np.float64) - 8
    return (d[:, None] * q).reshape(rows, nblk * 32)


@pytest.mark.parametrize("latent,fmt", [(0, 8), (0, 2), (64, 8), (64, 2), (0, 40), (64, 40)])
def test_layer_close_to_unquantised_float_layer(orc, synth, latent, fmt):
    """Sanity band: the quantised layer is within activation-quantisation error (about 1e-2
    relative) of the same layer in float64 with unquantised activations.  Catches transposed
    operands, a swapped gate/up, a missing combine weight."""
    w = _wl(hidden=128, n_experts=8, top_k=2, n_ff=96, tokens=6, latent=latent, expert_fmt=fmt,
            n_groups=4 if latent else 0, topk_groups=2 if latent else 0, seed=9)
    inp = _layer_inputs(synth, w)
    if latent:
        # At these small widths the latent chain's values are ~1e-5, where the binary16 Q8_1
        # scale is subnormal and keeps only a bit or two; x * 32 puts them where the full-size
        # layers put them (y_lat ~ 1e-2).
        inp["x"] = inp["x"] * np.float32(32.0)
    out, taps = orc.layer_forward(w, inp["x"], inp["router_w"], groups=inp["groups"],
                                  experts=inp["experts"], D=inp["D"], U=inp["U"],
                                  taps=("ids", "weights"))
    H, F, kin = w.hidden, w.n_ff, w.k_in
    eb = w.expert_bytes
    x = inp["x"].astype(np.float64)
    if latent:
        Dm = _dequant_rows(orc, 8, inp["D"], latent, H // 32)
        Um = _dequant_rows(orc, 8, inp["U"], H, latent // 32)
    ref = np.zeros((w.tokens, H))
    for t in range(w.tokens):
        a = Dm @ x[t] if latent else x[t]
        acc = np.zeros(kin)
        for j, e in enumerate(taps["ids"][t]):
            blob = inp["experts"][e * eb:(e + 1) * eb]
            bb = w.block_bytes
            n_gu = F * (kin // 32) * bb
            n_dn = kin * (F // 32) * bb
            ts = blob[2 * n_gu + n_dn:2 * n_gu + n_dn + 12].view("<f4").astype(np.float64) \
                if fmt == 40 else np.ones(3)
            G = _dequant_rows(orc, fmt, blob[:n_gu], F, kin // 32, ts[0])
            Uu = _dequant_rows(orc, fmt, blob[n_gu:2 * n_gu], F, kin // 32, ts[1])
            Dn = _dequant_rows(orc, fmt, blob[2 * n_gu:2 * n_gu + n_dn], kin, F // 32, ts[2])
            g, u = G @ a, Uu @ a
            acc += float(taps["weights"][t, j]) * (Dn @ (g / (1 + np.exp(-g)) * u))
        ref[t] = Um @ acc if latent else acc
    rel = np.sqrt(np.mean((out - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))
    assert 1e-4 < rel < 5e-2, rel


def test_latent_selection_dense(orc, synth):
    """D selecting the first L hidden units with d = 1, q = 1 makes z the dequantised Q8_1(x)
    prefix exactly."""
    w = _wl(hidden=128, n_experts=4, top_k=2, n_ff=64, tokens=3, latent=64, seed=4)
    inp = _layer_inputs(synth, w)
    D = np.zeros((64, 4, 34), np.uint8)
    D[:, :, 1] = 0x3C
    for r in range(64):
        D[r, r // 32, 2 + r % 32] = 1
    out, taps = orc.layer_forward(w, inp["x"], inp["router_w"], experts=inp["experts"],
                                  D=D.reshape(-1), U=inp["U"], taps=("xq", "z"))
    for t in range(3):
        xq = taps["xq"][t]
        deq = np.concatenate([orc.f16_decode(int(b[0]) | int(b[1]) << 8) * b[4:].view(np.int8).astype(np.float64)
                              for b in xq])
        assert np.array_equal(taps["z"][t], deq[:64].astype(np.float32))


def test_latent_selection_dense_q4_0(orc, synth):
    """Q4_0 D and U as selections (d = 1, code 9 = +1 on the diagonal, code 8 = 0
    elsewhere; low nibble = element j, high nibble = element j + 16): z is the
    dequantised Q8_1(x) prefix and out is the dequantised Q8_1(y_lat) followed
    by zeros, exactly."""
    H, L = 128, 64
    w = _wl(hidden=H, n_experts=4, top_k=2, n_ff=64, tokens=3, latent=L, seed=5,
            dense_fmt=synth.Q4_0)
    inp = _layer_inputs(synth, w)

    def selection(rows, nblk):
        m = np.full((rows, nblk, 18), 0x88, np.uint8)
        m[:, :, 0] = 0x00
        m[:, :, 1] = 0x3C
        for r in range(min(rows, nblk * 32)):
            p = r % 32
            m[r, r // 32, 2 + p % 16] = 0x89 if p < 16 else 0x98
        return m.reshape(-1)

    out, taps = orc.layer_forward(w, inp["x"], inp["router_w"], experts=inp["experts"],
                                  D=selection(L, H // 32), U=selection(H, L // 32),
                                  taps=("xq", "z", "ylq"))

    def deq(q8_1_blocks):
        return np.concatenate([orc.f16_decode(int(b[0]) | int(b[1]) << 8)
                               * b[4:].view(np.int8).astype(np.float64) for b in q8_1_blocks])

    for t in range(3):
        assert np.array_equal(taps["z"][t], deq(taps["xq"][t])[:L].astype(np.float32))
        want = np.zeros(H, np.float32)
        want[:L] = deq(taps["ylq"][t]).astype(np.float32)
        assert np.array_equal(out[t], want)


def test_oracle_refuses_bad_groups(orc, synth):
    w = _wl(n_experts=8, top_k=3, n_groups=4, topk_groups=1)   # 1 group of 2 < k = 3
    inp = _layer_inputs(synth, dataclasses.replace(w, n_groups=0, topk_groups=0))
    with pytest.raises(ValueError):
        orc.layer_forward(w, inp["x"], inp["router_w"], groups=np.arange(8, dtype=np.int32) // 2,
                          experts=inp["experts"])


def test_q8_1_s_is_rounded_twice(orc):
    """s is rounded to fp32 and then to binary16; blocks where one rounding differs."""
    import quant_cases
    blocks = quant_cases.double_rounding_blocks(6)
    assert len(blocks) == 6
    for v in blocks:
        _check_exact(orc, v)


# ------------------------------------------- the oracle downstream of given intermediates
@pytest.mark.parametrize("latent", [0, 64])
def test_given_own_intermediates_reproduce_the_layer(orc, synth, latent):
    """Given its own ids and Q8_1 vectors, the oracle returns its own output bit for bit."""
    w = _wl(hidden=128, n_experts=8, top_k=3, n_ff=64, tokens=5, latent=latent,
            n_groups=4 if latent else 0, topk_groups=2 if latent else 0, seed=12)
    inp = _layer_inputs(synth, w)
    names = ("ids", "weights", "hq") + (("zq", "ylq") if latent else ())
    ref, t = orc.layer_forward(w, inp["x"], inp["router_w"], groups=inp["groups"],
                               experts=inp["experts"], D=inp["D"], U=inp["U"], taps=names)
    given = {n: t[n] for n in ("ids", "zq", "hq", "ylq") if n in t}
    out, t2 = orc.layer_forward(w, inp["x"], inp["router_w"], groups=inp["groups"],
                                experts=inp["experts"], D=inp["D"], U=inp["U"], taps=names,
                                given=given)
    assert np.array_equal(out, ref)
    for n in names:
        assert np.array_equal(t2[n], t[n]), n


def test_given_ids_take_the_softmax_of_their_own_logits(orc, synth):
    """Given experts (any order, not the top-k) get weights exp(l_j) / sum exp(l_i) over
    their own logits, and the output is their weighted sum: here checked against
    expert_ffn of each and an exact-rational softmax of the fp64 logits."""
    w = _wl(hidden=128, n_experts=8, top_k=3, n_ff=64, tokens=3, seed=13)
    inp = _layer_inputs(synth, w)
    ids = np.array([[7, 0, 4], [1, 2, 3], [5, 6, 0]], dtype=np.int32)
    out, t = orc.layer_forward(w, inp["x"], inp["router_w"], experts=inp["experts"],
                               taps=("ids", "weights", "logits", "xq"), given=dict(ids=ids))
    assert np.array_equal(t["ids"], ids)
    eb = w.expert_bytes
    for i in range(3):
        l = t["logits"][i][ids[i]]
        ex = np.exp(l - l.max())
        assert np.allclose(t["weights"][i], ex / ex.sum(), rtol=2e-7, atol=0)
        ys = np.stack([orc.expert_ffn(w, inp["experts"][e * eb:(e + 1) * eb], t["xq"][i])["y"]
                       for e in ids[i]]).astype(np.float64)
        comb = (t["weights"][i].astype(np.float64)[:, None] * ys).sum(0)
        assert np.allclose(out[i], comb, rtol=0, atol=1e-6 * np.abs(comb).max())
    with pytest.raises(ValueError):                 # a repeated expert is refused
        orc.layer_forward(w, inp["x"], inp["router_w"], experts=inp["experts"],
                          given=dict(ids=np.array([[1, 1, 2]] * 3, dtype=np.int32)))


def test_given_hq_enters_the_down_projection(orc, synth):
    """One code of a given Q8_1(h) moved by +1 moves that expert's y by exactly
    d_h * d_w[r] * q_w[r, e] in every down row r (Q8_0), nothing else."""
    w = _wl(hidden=64, n_experts=4, top_k=1, n_ff=64, tokens=1, seed=14)
    inp = _layer_inputs(synth, w)
    _, t = orc.layer_forward(w, inp["x"], inp["router_w"], experts=inp["experts"],
                             taps=("ids", "hq", "y"))
    hq = t["hq"].copy()                               # [1][1][F/32][36]
    b, e = 1, 5
    q = hq[0, 0, b, 4 + e].view(np.int8)
    assert abs(int(q)) < 127
    hq[0, 0, b, 4 + e] = np.array([int(q) + 1], dtype=np.int8).view(np.uint8)[0]
    _, t2 = orc.layer_forward(w, inp["x"], inp["router_w"], experts=inp["experts"],
                              taps=("y",), given=dict(hq=hq))
    eid = int(t["ids"][0, 0])
    eb = w.expert_bytes
    down = inp["experts"][eid * eb:(eid + 1) * eb][2 * w.n_ff * (w.hidden // 32) * 34:]
    D = down.reshape(w.hidden, w.n_ff // 32, 34)
    dw = D[:, b, :2].copy().view(np.float16).astype(np.float64).reshape(-1)
    qw = D[:, b, 2 + e].view(np.int8).astype(np.float64)
    dh = float(hq[0, 0, b, :2].copy().view(np.float16)[0])
    delta = t2["y"][0, 0].astype(np.float64) - t["y"][0, 0].astype(np.float64)
    expect = dh * dw * qw
    assert np.allclose(delta, expect, rtol=0, atol=4 * np.spacing(np.abs(t["y"]).max()))
    assert np.any(expect != 0)
