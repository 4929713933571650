"""Pins of the fp8 weight oracle (oracle.fp8): the E4M3 decode against hand
values of the format, its structure and torch's float8_e4m3fn; the fp8 LM head
and fc against exact rational brute force on tiny shapes, against the
(separately pinned) bf16 definitions when the scale is 1, and under
power-of-two scales; and the synthetic quantisation recipe's error bound."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import fp8
from workloads import synth

torch = pytest.importorskip("torch")


def test_e4m3_hand_values():
    # sign | exponent (bias 7) | mantissa, per the E4M3 field layout
    cases = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0x3C: 1.5, 0x7E: 448.0,
             0xFE: -448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
             0x0F: 1.875 * 2.0 ** -6, 0x77: 240.0, 0x78: 256.0, 0xB8: -1.0}
    for code, v in cases.items():
        assert fp8.e4m3_value(code) == v, hex(code)
    assert np.signbit(fp8.e4m3_value(0x80)) and fp8.e4m3_value(0x80) == 0.0
    assert np.isnan(fp8.e4m3_value(0x7F)) and np.isnan(fp8.e4m3_value(0xFF))


def test_e4m3_structure():
    t = fp8.E4M3_TABLE
    assert np.sum(np.isnan(t)) == 2
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                  # codes 0..126 increase
    assert np.array_equal(t[0x80:0xFF], -pos)        # the sign bit negates
    assert pos.max() == fp8.E4M3_MAX
    # spacing: 2^-9 among subnormals and the first binade, then doubling per binade
    gaps = np.diff(pos)
    assert np.all(gaps[:15] == 2.0 ** -9)
    for e in range(1, 15):
        assert np.all(gaps[8 * e: 8 * e + 7] == 2.0 ** (e - 10))


def test_e4m3_matches_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.decode_e4m3(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.signbit(got[~both_nan]), np.signbit(ref[~both_nan]))


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38                     # no NaN codes
    return c


def _f32(x) -> np.float32:
    return np.float32(float(x))


def test_lm_head_fp8_brute_force():
    rng = np.random.default_rng(11)
    M, H, V = 3, 7, 5                                 # non-square: a transpose fails
    hid = synth.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    q = _rand_codes(rng, (V, H))
    s = (rng.random(V) * 3 + 0.1).astype(np.float32)
    got = fp8.lm_head_fp8(hid, q, s, "bf16")
    x = oracle.widen(hid, "bf16")
    for m in range(M):
        for v in range(V):
            acc = sum(Fraction(float(x[m, h])) * Fraction(fp8.e4m3_value(q[v, h]))
                      for h in range(H))
            assert got[m, v] == _f32(acc * Fraction(float(s[v]))), (m, v)


def test_fuse_fc_fp8_brute_force():
    rng = np.random.default_rng(12)
    T, rows, H = 3, 4, 6
    taps = [synth.to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
            for _ in range(T)]
    q = _rand_codes(rng, (H, T * H))
    s = (rng.random(H) + 0.5).astype(np.float32)
    got = fp8.fuse_fc_fp8(taps, q, s, "bf16")
    for m in range(rows):
        for o in range(H):
            acc = Fraction(0)
            for t in range(T):
                xt = oracle.widen(taps[t], "bf16")
                for h in range(H):
                    acc += Fraction(float(xt[m, h])) * Fraction(fp8.e4m3_value(q[o, t * H + h]))
            assert got[m, o] == _f32(acc * Fraction(float(s[o]))), (m, o)


def test_unit_scale_reduces_to_the_bf16_definitions():
    # every E4M3 value is a bfloat16 value, so with scale 1 the fp8 weight is a
    # bf16 weight and the fp8 results must equal the bf16 definitions exactly
    finite = fp8.E4M3_TABLE[np.isfinite(fp8.E4M3_TABLE)]
    as_bf16 = oracle.widen(oracle.f32_to_bf16_bits(finite.astype(np.float32)), "bf16")
    assert np.array_equal(as_bf16, finite)
    rng = np.random.default_rng(13)
    H, V, T, rows = 64, 300, 5, 9
    hid = synth.to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
    lm_q = _rand_codes(rng, (V, H))
    lm_bf16 = oracle.f32_to_bf16_bits(fp8.decode_e4m3(lm_q).astype(np.float32))
    assert np.array_equal(fp8.lm_head_fp8(hid, lm_q, np.ones(V, np.float32), "bf16"),
                          oracle.lm_head(hid, lm_bf16, "bf16"))
    taps = [synth.to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
            for _ in range(T)]
    fc_q = _rand_codes(rng, (H, T * H))
    fc_bf16 = oracle.f32_to_bf16_bits(fp8.decode_e4m3(fc_q).astype(np.float32))
    assert np.array_equal(fp8.fuse_fc_fp8(taps, fc_q, np.ones(H, np.float32), "bf16"),
                          oracle.fuse_fc(taps, fc_bf16, "bf16"))


def test_power_of_two_scales_scale_the_result_exactly():
    rng = np.random.default_rng(14)
    H, V = 32, 40
    hid = synth.to_bf16_bits(rng.standard_normal((2, H)).astype(np.float32))
    q = _rand_codes(rng, (V, H))
    e = rng.integers(-6, 7, size=V)
    s = (2.0 ** e).astype(np.float32)
    base = fp8.lm_head_fp8(hid, q, np.ones(V, np.float32), "bf16")
    assert np.array_equal(fp8.lm_head_fp8(hid, q, s, "bf16"), base * s[None, :])


def test_nan_codes_and_bad_scales_are_rejected():
    hid = synth.to_bf16_bits(np.ones((1, 4), np.float32))
    q = np.full((2, 4), 0x38, np.uint8)
    q[1, 2] = 0xFF
    with pytest.raises(ValueError):
        fp8.lm_head_fp8(hid, q, np.ones(2, np.float32), "bf16")
    with pytest.raises(ValueError):
        fp8.lm_head_fp8(hid, q[:1], np.ones(2, np.float32), "bf16")
    with pytest.raises(ValueError):
        fp8.decode_e4m3(q.astype(np.int32))


def test_quantisation_recipe_error_bound():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((50, 333)).astype(np.float32) * np.exp(rng.standard_normal((50, 1)))
    x[7] = 0.0
    q, s = synth.quantize_e4m3_rows(x)
    assert q.dtype == np.uint8 and s.dtype == np.float32
    assert s[7] == 1.0 and np.all(q[7] == 0)
    back = fp8.decode_e4m3(q) * s.astype(np.float64)[:, None]
    live = np.arange(50) != 7
    # the largest magnitude of every row lands on +-448
    assert np.all(np.max(np.abs(fp8.decode_e4m3(q[live])), axis=1) == 448.0)
    # normal range: within half a step (2^-4 relative); subnormal range: half of 2^-9 * scale
    err = np.abs(back - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)
