"""Pins of the hyper-connection stream average (oracle.hc): the float64 ->
bfloat16 rounding against exact rational rounding (ties, values a float32
intermediate would collapse onto a tie, carries, subnormals, -0); the average
against rational brute force, the identity at one stream, constant and
permuted streams."""
import bisect
from fractions import Fraction
import math

import numpy as np

import oracle
from oracle import hc
from workloads import synth


# every finite non-negative bf16 value, increasing with the bit pattern
_POS = [Fraction(float(v)) for v in
        oracle.widen(np.arange(0x7F80, dtype=np.uint16), "bf16")]


def _round_bf16_exact(x: Fraction) -> int:
    """Correctly rounded bf16 bits of a rational (ties to even), by bisection
    over the bit patterns (finite inputs inside the bf16 range)."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    lo = bisect.bisect_right(_POS, a) - 1       # largest bf16 magnitude <= a
    if _POS[lo] == a:
        return sign | lo
    hi = lo + 1
    dl, dh = a - _POS[lo], _POS[hi] - a
    pick = lo if dl < dh else hi if dh < dl else (lo if lo % 2 == 0 else hi)
    return sign | pick


def test_f64_to_bf16_matches_exact_rounding():
    rng = np.random.default_rng(1)
    vals = []
    # exact ties between neighbouring bf16 values, and points just off a tie by
    # less than a float32 step (a float32 round-to-nearest would land on the tie)
    for e in (-130, -126, -20, 0, 7, 100):
        for m in (0, 1, 0x3F, 0x7E):
            lo = Fraction(128 + m, 128) * Fraction(2) ** e
            step = Fraction(1, 128) * Fraction(2) ** e
            tie = lo + step / 2
            vals += [tie, tie + step * Fraction(1, 2 ** 40), tie - step * Fraction(1, 2 ** 40),
                     lo, lo + step * Fraction(1, 3)]
    vals += [Fraction(float(v)) for v in rng.standard_normal(60) * np.exp(rng.uniform(-30, 30, 60))]
    vals += [Fraction(2) ** -133, Fraction(3) * Fraction(2) ** -135, Fraction(255, 256)]
    xs = np.array([float(v) for v in vals])
    got = hc.f64_to_bf16_bits(xs)
    for v, x, g in zip(vals, xs, got):
        want = _round_bf16_exact(Fraction(float(x)))
        assert int(g) == want, (v, x, hex(int(g)), hex(want))
    # carries into the exponent and -0
    assert hc.f64_to_bf16_bits(np.array([1.99999999999])).tolist() == [0x4000]
    assert hc.f64_to_bf16_bits(np.array([-0.0])).tolist() == [0x8000]


def test_average_matches_rational_brute_force():
    rng = np.random.default_rng(2)
    for n_streams in (2, 3, 4, 5, 7):
        streams = [synth.to_bf16_bits((rng.standard_normal((3, 9))
                                       * np.exp(rng.uniform(-8, 8, (3, 9)))).astype(np.float32))
                   for _ in range(n_streams)]
        got = hc.hc_average(streams, "bf16")
        vals = [oracle.widen(s, "bf16") for s in streams]
        for r in range(3):
            for h in range(9):
                exact = sum(Fraction(float(v[r, h])) for v in vals) / n_streams
                assert int(got[r, h]) == _round_bf16_exact(exact), (n_streams, r, h)


def test_one_stream_constant_and_permuted_streams():
    rng = np.random.default_rng(3)
    x = synth.to_bf16_bits(rng.standard_normal((5, 64)).astype(np.float32))
    assert np.array_equal(hc.hc_average([x], "bf16"), x)
    assert np.array_equal(hc.hc_average([x, x, x], "bf16"), x)
    streams = [synth.to_bf16_bits(rng.standard_normal((5, 64)).astype(np.float32)) for _ in range(4)]
    a = hc.hc_average(streams, "bf16")
    # a permutation only reorders exact float64 additions of bf16 values here
    assert np.array_equal(a, hc.hc_average(streams[::-1], "bf16"))
    f = [rng.standard_normal((4, 8)).astype(np.float32) for _ in range(3)]
    want = ((f[0].astype(np.float64) + f[1] + f[2]) / 3).astype(np.float32)
    assert np.array_equal(hc.hc_average(f, "f32"), want)


def test_average_of_two_is_exact_midpoint_when_representable():
    # x and x + 2 ulp: the midpoint x + 1 ulp is a bf16 value
    x = np.array([0x3F80, 0xC0A0, 0x0100], dtype=np.uint16)
    y = x + np.uint16(2)
    assert hc.hc_average([x, y], "bf16").tolist() == (x + np.uint16(1)).tolist()
    assert math.isclose(float(oracle.widen(hc.hc_average([x[:1], y[:1]], "bf16"), "bf16")[0]),
                        1.0 + 2 ** -7)
