"""Pins for the oracle's bf16 conversion, sigmoid and gate-product rounding.

Each reference here is computed a different way from the oracle's C code:
  * bf16 rounding: exact rational arithmetic (fractions.Fraction) against the
    enumerated grid of all finite bf16 values, ties broken by the even bit
    pattern -- the oracle instead scales by a power of two and rounds.
  * bf16 -> fp64: struct's IEEE binary32 decoding.
  * sigmoid: Python decimal at 40 significant digits for all 65,536 gates,
    plus hand-derived near-midpoint cases (tests/golden).
"""
import bisect
import math
import os
import random
import struct
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# All finite non-negative bf16 values, ascending with the bit pattern.
_POS_BITS = list(range(0x0000, 0x7F80))


def _bits_to_float(b: int) -> float:
    return struct.unpack(">f", struct.pack(">I", (b & 0xFFFF) << 16))[0]


_POS_VALS = [Fraction(_bits_to_float(b)) for b in _POS_BITS]
_MAX_FINITE = _POS_VALS[-1]
_OVERFLOW_AT = _MAX_FINITE + (Fraction(2) ** 128 - _MAX_FINITE) / 2  # midpoint to 2^128


def grid_round(x) -> int:
    """bf16 bits nearest to the exact rational value of x, ties to even bits."""
    if isinstance(x, float):
        if math.isnan(x):
            return 0x7FC0
        if math.isinf(x):
            return 0x7F80 if x > 0 else 0xFF80
    fx = Fraction(x)
    neg = fx < 0 or (isinstance(x, float) and fx == 0 and math.copysign(1.0, x) < 0)
    a = abs(fx)
    sign = 0x8000 if neg else 0
    if a >= _OVERFLOW_AT:
        return sign | 0x7F80
    i = bisect.bisect_left(_POS_VALS, a)
    if i < len(_POS_VALS) and _POS_VALS[i] == a:
        return sign | _POS_BITS[i]
    if i == len(_POS_VALS):  # between max finite and the overflow midpoint
        return sign | _POS_BITS[-1]
    lo, hi = i - 1, i
    dlo, dhi = a - _POS_VALS[lo], _POS_VALS[hi] - a
    if dlo < dhi:
        pick = lo
    elif dhi < dlo:
        pick = hi
    else:
        pick = lo if _POS_BITS[lo] % 2 == 0 else hi
    return sign | _POS_BITS[pick]


def _edge_doubles():
    vals = [0.0, -0.0, 1.0, -1.0, 2.0 ** -126, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135,
            2.0 ** -134 * (1 + 2 ** -40), 2.0 ** -134 * (1 - 2 ** -40), 1e-45, 5e-324,
            float(_MAX_FINITE), float(_OVERFLOW_AT), float(_OVERFLOW_AT) * (1 - 2 ** -52),
            float(_OVERFLOW_AT) * (1 + 2 ** -52), 3.0e38, 1e300, -1e300]
    # exact midpoints between neighbouring bf16 values, and one fp64 ulp either side
    rng = random.Random(7)
    for b in [0x0001, 0x0002, 0x007F, 0x0080, 0x0081, 0x3F00, 0x3F7F, 0x3F80, 0x3F81,
              0x4000, 0x7F00, 0x7F7E] + [rng.randrange(0x0001, 0x7F7F) for _ in range(300)]:
        m = (_POS_VALS[b] + _POS_VALS[b + 1]) / 2
        fm = float(m)
        assert Fraction(fm) == m
        vals += [fm, -fm, math.nextafter(fm, math.inf), math.nextafter(fm, -math.inf)]
    return vals


def test_bf16_rne_edges():
    xs = _edge_doubles()
    got = oracle.bf16_rne(np.array(xs))
    for x, g in zip(xs, got):
        assert int(g) == grid_round(x), (x, hex(int(g)), hex(grid_round(x)))


def test_bf16_rne_random_wide_range():
    rng = np.random.default_rng(123)
    mant = rng.uniform(1.0, 2.0, 20000)
    exps = rng.integers(-150, 130, 20000)
    xs = np.ldexp(mant, exps) * np.where(rng.random(20000) < 0.5, -1.0, 1.0)
    got = oracle.bf16_rne(xs)
    for x, g in zip(xs.tolist(), got.tolist()):
        assert g == grid_round(x), (x, hex(g), hex(grid_round(x)))


def test_bf16_rne_nan_inf():
    got = oracle.bf16_rne(np.array([math.inf, -math.inf, math.nan]))
    assert got[0] == 0x7F80 and got[1] == 0xFF80
    assert (got[2] & 0x7F80) == 0x7F80 and (got[2] & 0x007F) != 0


def test_bf16_value_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    v = oracle.bf16_value(bits)
    for b in range(65536):
        ref = _bits_to_float(b)
        if math.isnan(ref):
            assert math.isnan(v[b])
        else:
            assert v[b] == ref and math.copysign(1.0, v[b]) == math.copysign(1.0, ref), hex(b)


def _decimal_sigmoid_bits(b: int) -> int:
    g = _bits_to_float(b)
    if math.isnan(g):
        return 0x7FC0
    if g == math.inf:
        return 0x3F80
    if g == -math.inf:
        return 0x0000
    if g < -200.0:   # sigmoid < e^-200 < 2^-134: rounds to +0
        return 0x0000
    if g > 200.0:    # 1 - sigmoid < e^-200: rounds to 1.0
        return 0x3F80
    with localcontext() as ctx:
        ctx.prec = 40
        s = Decimal(1) / (Decimal(1) + (-Decimal(g)).exp())
    return grid_round(Fraction(s))


@pytest.mark.parametrize("part", range(4))
def test_sigmoid_table_exhaustive_vs_decimal(part):
    table = oracle.sigmoid_table()
    lo, hi = part * 16384, (part + 1) * 16384
    for b in range(lo, hi):
        ref = _decimal_sigmoid_bits(b)
        got = int(table[b])
        if ref == 0x7FC0:
            assert (got & 0x7F80) == 0x7F80 and (got & 0x7F) != 0, hex(b)
        else:
            assert got == ref, (hex(b), hex(got), hex(ref))


def _golden_sigmoid_rows():
    rows = []
    with open(os.path.join(GOLDEN, "sigmoid_bf16_near_midpoint.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((int(parts[0], 16), parts[1], int(parts[2], 16)))
    return rows


@pytest.mark.parametrize("gate_bits,gate_text,sigma_bits", _golden_sigmoid_rows())
def test_sigmoid_golden(gate_bits, gate_text, sigma_bits):
    if gate_text not in ("+inf", "-inf"):
        assert _bits_to_float(gate_bits) == float(gate_text)
    assert oracle.sigmoid_bf16(gate_bits) == sigma_bits


def test_gate_output_product_rounding():
    rng = random.Random(11)
    pats = [0x0000, 0x8000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F00, 0x7F7F, 0xFF7F, 0x3400]
    pats += [rng.randrange(0, 0x7F80) | (rng.randrange(2) << 15) for _ in range(3000)]
    sig = [0x3F00, 0x3F80, 0x3F7F, 0x0001, 0x0000, 0x3EFF, 0x2F80]
    sig += [rng.randrange(0, 0x3F81) for _ in range(30)]
    for ob in pats:
        for sb in sig:
            ref = grid_round(Fraction(_bits_to_float(ob)) * Fraction(_bits_to_float(sb)))
            if _bits_to_float(ob) * _bits_to_float(sb) == 0 and (ob ^ sb) & 0x8000:
                ref = 0x8000  # signed zero of the exact product
            assert oracle.gate_output(ob, sb) == ref, (hex(ob), hex(sb))


def test_gate_zero_halves_and_gate_40_is_identity():
    # sigma_b(0) = 0.5 exactly, so out = Ob / 2 exactly for normal Ob;
    # sigma_b(40) = 1.0, so out = Ob.
    s0 = oracle.sigmoid_bf16(0x0000)
    s40 = oracle.sigmoid_bf16(0x4220)
    assert s0 == 0x3F00 and s40 == 0x3F80
    for ob in list(range(0x0100, 0x7F80, 97)) + list(range(0x8100, 0xFF80, 89)):
        assert oracle.gate_output(ob, s40) == ob
        assert oracle.gate_output(ob, s0) == ob - 0x0080  # exponent minus one
