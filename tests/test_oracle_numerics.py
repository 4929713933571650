"""Pins of the oracle's number-format helpers (bfloat16 widening and rounding)."""
import numpy as np
import pytest
import torch

from oracle import reference as ref


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0),
    (0xBF80, -1.0),
    (0x4049, 3.140625),
    (0x3F81, 1.0 + 2.0 ** -7),
    (0x0001, 2.0 ** -133),                 # smallest subnormal
    (0x0080, 2.0 ** -126),                 # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
    (0x0000, 0.0),
])
def test_widen_bf16_hand_values(bits, value):
    got = ref.widen(np.array([bits], dtype=np.uint16), "bf16")[0]
    assert got == value


def test_widen_negative_zero_keeps_sign():
    got = ref.widen(np.array([0x8000], dtype=np.uint16), "bf16")[0]
    assert got == 0.0 and np.signbit(got)


def test_widen_f32_exact():
    x = np.array([1.0000001, -3.5e-40, 3.4e38], dtype=np.float32)
    assert np.array_equal(ref.widen(x, "f32"), x.astype(np.float64))


@pytest.mark.parametrize("f32bits,bf16bits", [
    (0x3F800000, 0x3F80),   # 1.0 exact
    (0x3F808000, 0x3F80),   # 1 + 2^-8: exact half-way, lower is even -> down
    (0x3F818000, 0x3F82),   # 1 + 3*2^-8: half-way, upper is even -> up
    (0x3F808001, 0x3F81),   # just above half-way -> up
    (0x3F807FFF, 0x3F80),   # just below half-way -> down
    (0xBF808000, 0xBF80),   # negative mirror of the tie
    (0xBF818000, 0xBF82),
    (0x3FFF8000, 0x4000),   # tie with carry into the exponent: 1.99609375.. -> 2.0
    (0x00000001, 0x0000),   # tiny subnormal rounds to +0
    (0x80000000, 0x8000),   # -0 stays -0
])
def test_bf16_rne_hand_values(f32bits, bf16bits):
    got = ref.f32_to_bf16_bits(np.array([_f32(f32bits)], dtype=np.float32))[0]
    assert int(got) == bf16bits


def test_bf16_rne_matches_torch_conversion():
    """Special case that reduces to a library routine: torch's CPU float->bf16 cast is RNE."""
    g = np.random.default_rng(7)
    x = g.standard_normal(200_000).astype(np.float32) * np.float32(37.0)
    # plus constructed exact ties: low half exactly 0x8000
    ties = (g.integers(0x0080, 0x7F00, 5000, dtype=np.uint32) << 16) | 0x8000
    x = np.concatenate([x, ties.astype(np.uint32).view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ref.f32_to_bf16_bits(x), want)


def test_bf16_rounding_rejects_non_finite():
    with pytest.raises(ValueError):
        ref.f32_to_bf16_bits(np.array([np.inf], dtype=np.float32))


def test_round_to_f32_is_rne():
    # 1 + 2^-24 is half-way between 1 and 1 + 2^-23: ties to even -> 1
    assert ref.round_to_f32(np.array([1.0 + 2.0 ** -24]))[0] == np.float32(1.0)
    assert ref.round_to_f32(np.array([1.0 + 3 * 2.0 ** -24]))[0] == np.float32(1.0 + 2.0 ** -22)
