"""Pins for the oracle's bf16 rounding, GEMM, SwiGLU and error metric (CPU only)."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import BFP4, BFP8


def _exact_bf16(v: float) -> Fraction:
    """Round a float to 8 significant bits (ties to even) in exact rationals."""
    f = Fraction(v)
    if f == 0:
        return f
    sign = -1 if f < 0 else 1
    a = abs(f)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    e = max(e, -126)                        # subnormal range: fixed quantum 2**-133
    q = Fraction(2) ** (e - 7)
    t = abs(f) / q
    lo = math.floor(t)
    rem = t - lo
    n = lo + 1 if (rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1)) else lo
    return sign * n * q


def test_bf16_round_known_values():
    r = oracle.bf16_round(np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8 + 2 ** -30),
                                    2 ** -133, 1.5 * 2 ** -133, 2.5 * 2 ** -133, 0.0, -0.0]))
    assert r.tolist()[:4] == [1.0, 1.0, 1 + 2 ** -6, -(1 + 2 ** -7)]
    assert r.tolist()[4:7] == [2 ** -133, 2 * 2 ** -133, 2 * 2 ** -133]
    assert np.signbit(r[8]) and r[7] == 0


def test_bf16_round_vs_exact_rationals():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-140, 100, 3000))
    # include exact ties
    v[:200] = (rng.integers(1, 512, 200) + 0.5) * np.exp2(rng.integers(-20, 20, 200) - 8)
    r = oracle.bf16_round(v)
    for a, b in zip(v, r):
        assert Fraction(float(b)) == _exact_bf16(float(a))


def test_bf16_round_matches_input_generator_on_fp32():
    # the input generator's own fp32 -> bf16 rounding and the oracle's agree on fp32 values
    rng = np.random.default_rng(9)
    x = rng.standard_normal(20000).astype(np.float32)
    a = synth.bf16_values(synth.bf16_bits(x)).astype(np.float64)
    b = oracle.bf16_round(x.astype(np.float64))
    assert np.array_equal(a, b)


def _tiny_case(rng, fmt, m, n, k):
    w = (rng.standard_normal((n, k)) * 0.3).astype(np.float32)
    exp, code = oracle.encode(w, fmt)
    wd = oracle.decode(exp, code, fmt, n, k)
    xb = synth.bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    return oracle.bf16_to_f64(xb), wd


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
def test_gemm_tiny_vs_exact_rationals(fmt):
    rng = np.random.default_rng(21 + fmt)
    for m, n, k in ((1, 3, 16), (2, 8, 64), (2, 5, 48)):
        x, w = _tiny_case(rng, fmt, m, n, k)
        y = oracle.gemm(x, w)
        nrm = oracle.normaliser(x, w)
        for i in range(m):
            for j in range(n):
                exact = sum(Fraction(float(x[i, t])) * Fraction(float(w[j, t])) for t in range(k))
                # fp64 summation of exact products: error far below 1e-12 of the abs sum
                assert abs(Fraction(float(y[i, j])) - exact) <= Fraction(1, 10 ** 12) * Fraction(float(nrm[i, j])) + Fraction(0)
                absum = sum(abs(Fraction(float(x[i, t])) * Fraction(float(w[j, t]))) for t in range(k))
                assert abs(Fraction(float(nrm[i, j])) - absum) <= Fraction(1, 10 ** 12) * absum


def test_gemm_one_hot_is_exact():
    rng = np.random.default_rng(4)
    n, k = 16, 128
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    exp, code = oracle.encode(w, BFP8)
    wd = oracle.decode(exp, code, BFP8, n, k)
    x = np.zeros((1, k))
    x[0, 37] = -1.625
    y = oracle.gemm(x, wd)
    assert np.array_equal(y[0], -1.625 * wd[:, 37])


def test_gemm_orientation():
    # y[m][n] = sum_k x[m][k] w[n][k]; a transposed operand would fail on this shape
    x = np.array([[1.0, 2.0, 3.0]])
    w = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 1.0]])
    assert oracle.gemm(x, w).tolist() == [[1.0, 3.0]]


def test_silu_and_swiglu():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    g = np.array([50.0, 700.0, -700.0, -3.0, 0.7, 2.0])
    s = oracle.silu(g)
    assert abs(s[0] - 50.0) < 1e-15 * 50
    assert s[1] == 700.0 and s[2] < 0 and abs(s[2] - (-700.0 * math.exp(-700.0))) <= 1e-15 * abs(s[2])
    for gv, sv in zip(g[3:], s[3:]):
        assert abs(sv - gv / (1.0 + math.exp(-gv))) <= 1e-15 * abs(gv)
    u = np.array([2.0, -1.0, 0.5, 1.0, 1.0, 3.0])
    assert np.allclose(oracle.swiglu(g, u), s * u, rtol=0, atol=0)
    assert oracle.linalg.sigmoid(np.array([0.0]))[0] == 0.5
    # closed forms at g = +-ln 3, where e^-g is 1/3 or 3: silu(ln 3) = (3/4) ln 3,
    # silu(-ln 3) = -(1/4) ln 3 (a sign slip in the exponent swaps the two)
    l3 = math.log(3.0)
    s3 = oracle.silu(np.array([l3, -l3]))
    assert abs(s3[0] - 0.75 * l3) <= 4e-16 * l3 and abs(s3[1] + 0.25 * l3) <= 4e-16 * l3


# logistic function values from 50-digit decimal arithmetic (1 / (1 + e^-z)), i.e. the
# constants e/(1+e), 1/(1+e^2), ... of mathematical tables, not the oracle's own formula
_SIGMOID_TABLE = {
    1.0: 0.73105857863000487925,
    2.0: 0.88079707797788244406,
    -2.0: 0.11920292202211755594,
    0.5: 0.62245933120185456464,
    -40.0: 4.2483542552915889773e-18,
}


def test_sigmoid_pins():
    """The shared-expert gate sigma(z) = 1 / (1 + e^-z): closed forms that a sign slip
    (1 / (1 + e^z)), a missing term or a swapped branch fails."""
    sig = oracle.linalg.sigmoid
    for z, want in _SIGMOID_TABLE.items():
        got = sig(np.array([z]))[0]
        assert abs(got - want) <= 2.3e-16 * want, (z, got, want)
    # sigma(ln k) = k / (k + 1) (e^-ln k = 1/k), on both sides of zero
    for k in range(2, 12):
        z = math.log(k)
        got = sig(np.array([z, -z]))
        assert abs(got[0] - k / (k + 1)) <= 4e-16 and abs(got[1] - 1 / (k + 1)) <= 4e-16 / (k + 1) * k
    # limits: sigma(40) rounds to 1 in fp64, sigma(-40) = e^-40 (1 - e^-40 + ...) and never 0
    assert sig(np.array([40.0]))[0] == 1.0
    assert abs(sig(np.array([-40.0]))[0] - math.exp(-40.0)) <= 1e-15 * math.exp(-40.0)
    assert sig(np.array([-745.0]))[0] > 0.0 and sig(np.array([800.0]))[0] == 1.0
    # strictly increasing with sigma(z) > 1/2 for z > 0
    z = np.linspace(-30, 30, 2001)
    v = sig(z)
    assert np.all(np.diff(v) > 0) and np.all(v[z > 0] > 0.5) and np.all(v[z < 0] < 0.5)


def test_normaliser_hand_case():
    """sum_k |x_ik| |w_jk|, worked by hand."""
    x = np.array([[1.0, -2.0], [0.5, 0.0]])
    w = np.array([[3.0, 4.0], [-1.0, 0.5]])
    assert np.array_equal(oracle.normaliser(x, w), np.array([[11.0, 2.0], [1.5, 0.5]]))


def test_bf16_to_f64_known_patterns():
    """bf16 bit patterns with known values: 1, -2, the smallest subnormal 2^-133, the largest
    finite (2 - 2^-7) 2^127, +inf, -0."""
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x7F80, 0x8000], dtype=np.uint16)
    v = oracle.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 2.0 ** -133
    assert v[3] == (2.0 - 2.0 ** -7) * 2.0 ** 127 and math.isinf(v[4]) and v[4] > 0
    assert v[5] == 0.0 and math.copysign(1.0, v[5]) < 0


def test_rel_err_zero_normaliser():
    r = oracle.rel_err(np.array([0.0, 1.0, 2.0]), np.array([0.0, 0.5, 2.0]), np.array([0.0, 0.0, 4.0]))
    assert r[0] == 0.0 and math.isinf(r[1]) and r[2] == 0.0


def test_greedy_pick_hand_cases():
    nan, inf = math.nan, math.inf
    rows = [
        ([1.0, 3.0, 3.0, 2.0], 1),        # tie: first column
        ([1.0, nan, 5.0, nan], 1),        # NaN above every number, first NaN
        ([-inf, -inf, -inf], 0),          # all equal
        ([-0.0, 0.0], 0),                 # -0 equals +0
        ([-1.0, 0.0, -0.0], 1),
        ([-2.0, -1.0, -1.5], 1),          # all negative
        ([7.0], 0),                       # one column
        ([0.0, inf, 1e308, inf], 1),
    ]
    for vals, want in rows:
        idx, val = oracle.greedy_pick(np.array([vals]))
        assert idx[0] == want, (vals, idx[0])
        assert (math.isnan(val[0]) and math.isnan(vals[want])) or val[0] == vals[want]
    # rows are independent, dtype kept
    idx, val = oracle.greedy_pick(np.array([[0.0, 2.0], [5.0, 1.0]], dtype=np.float32))
    assert idx.tolist() == [1, 0] and val.dtype == np.float32


def test_greedy_pick_vs_brute_force_and_numpy():
    # small integer values: many ties; NaNs sprinkled in some rows
    rng = np.random.default_rng(3)
    for trial in range(200):
        n = int(rng.integers(1, 12))
        y = rng.integers(-2, 3, size=(3, n)).astype(np.float64)
        if trial % 4 == 0:
            y[rng.integers(0, 3), rng.integers(0, n)] = math.nan
        idx, val = oracle.greedy_pick(y)
        for i in range(3):
            # definition by sorting: order columns by (NaN first, value descending, index ascending)
            order = sorted(range(n), key=lambda j: (0 if math.isnan(y[i, j]) else 1,
                                                    0.0 if math.isnan(y[i, j]) else -y[i, j], j))
            assert idx[i] == order[0]
            # numpy's argmax follows the same rule (first maximum, first NaN)
            assert idx[i] == int(np.argmax(y[i]))
