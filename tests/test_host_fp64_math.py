"""The table-driven fp64 exp and log of the score and selection kernels,
restated step by step in Python (each fused multiply-add rounded once, via
exact rationals) and checked against 50-digit references: the error bounds
the kernel comments state, and the exact points they rely on.  CPU only."""
import math
import random
import struct
from decimal import Decimal, getcontext
from fractions import Fraction as F

import pytest

getcontext().prec = 50


def fma(a, b, c):
    return float(F(a) * F(b) + F(c))


def bits(x):
    return struct.unpack("<Q", struct.pack("<d", x))[0]


def dbl(b):
    return struct.unpack("<d", struct.pack("<Q", b & (2**64 - 1)))[0]


# log_ge1: x = 2^k m, c = m cut to 7 fractional bits, r = (m - c) / c,
# log x = k ln2 + log c + log1p(r) (degree-7 Taylor polynomial)
LOG_INV = [1.0 / (1.0 + t / 128.0) for t in range(128)]
LOG_C = [math.log1p(t / 128.0) for t in range(128)]
LN2_HI, LN2_LO = 0.6931471803691238, 1.9082149292705877e-10


def log_ge1(x):
    b = bits(x)
    hx, lx = b >> 32, b & 0xFFFFFFFF
    k = (hx >> 20) - 1023
    hm = (hx & 0x000FFFFF) | 0x3FF00000
    m, c = dbl((hm << 32) | lx), dbl((hm & 0xFFFFE000) << 32)
    j = (hx >> 13) & 127
    r = (m - c) * LOG_INV[j]
    q = fma(1.0 / 7.0, r, -1.0 / 6.0)
    for cf in (1.0 / 5.0, -0.25, 1.0 / 3.0, -0.5, 1.0):
        q = fma(q, r, cf)
    return fma(float(k), LN2_HI, fma(float(k), LN2_LO, LOG_C[j] + q * r))


# exp_neg: x = k ln2/64 + r, exp(x) = 2^(k>>6) tab[k&63] exp(r) (degree 5)
EXP_TAB = [2.0 ** (j / 64.0) for j in range(64)]


def exp_neg(x):
    xc = max(x, -700.0)
    k = float(round(xc * 92.33248261689366))   # rint (ties to even) as the kernel's v_rndne
    r = fma(-k, 0.010830424695086549, xc)
    r = fma(-k, 1.162596423439437e-12, r)
    p = fma(r, 1.0 / 120.0, 1.0 / 24.0)
    for cf in (1.0 / 6.0, 0.5, 1.0, 1.0):
        p = fma(p, r, cf)
    ki = int(k)
    v = EXP_TAB[ki & 63] * p
    return dbl(bits(v) + ((ki >> 6) << 52))


def test_ln2_split_and_table_points():
    assert F(LN2_HI) + F(LN2_LO) - F(Decimal(2).ln()) < F(1, 2**80)
    # ln2 head has 21 trailing zero bits: k * head is exact for |k| < 2^21
    assert bits(LN2_HI) & ((1 << 21) - 1) == 0
    assert log_ge1(1.0) == 0.0
    for e in range(1, 4):
        assert log_ge1(2.0 ** e) == fma(float(e), LN2_HI, float(e) * LN2_LO)


def test_log_ge1_error_on_1_to_8():
    rnd = random.Random(7)
    xs = [1.0 + 2**-52, 2.0 - 2**-52, 7.999999999999999] + [rnd.uniform(1.0, 8.0) for _ in range(3000)]
    xs += [1.0 + rnd.random() * 1e-3 for _ in range(500)]
    worst = max(abs(F(log_ge1(x)) - F(Decimal(x).ln())) for x in xs)
    assert worst < F(4, 10**16), float(worst)


def test_exp_neg_error_and_floor():
    rnd = random.Random(11)
    xs = [0.0, -1e-300, -0.5, -math.log(2) / 128] + [-rnd.expovariate(0.2) for _ in range(3000)]
    for x in xs:
        if x < -690:
            continue
        ref = F(Decimal(x).exp())
        assert abs(F(exp_neg(x)) - ref) <= ref * F(5, 10**16), x
    assert exp_neg(0.0) == 1.0
    # below -700 (and -inf) the result is exp(-700), a normal number that no
    # sum of at least 1 notices
    lo = exp_neg(-700.0)
    assert exp_neg(-800.0) == lo and exp_neg(float("-inf")) == lo
    assert 0.0 < lo < 1e-300 and 1.0 + 4096 * lo == 1.0


@pytest.mark.parametrize("x", [1.5, 3.25, 6.0])
def test_log_exp_roundtrip(x):
    assert abs(exp_neg(-log_ge1(x)) * x - 1.0) < 1e-15
