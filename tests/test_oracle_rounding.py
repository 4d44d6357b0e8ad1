"""Pins of the oracle's bfloat16 rounding (oracle.round_bf16): fp64 -> fp32 ->
bfloat16, each step round to nearest with ties to even, returned as bit
patterns.  It is the expected value of the merged bf16 weight, so a wrong tie
rule, truncation or a lost carry must fail here.

Known answers are written as fp32 bit patterns and their correctly rounded
bfloat16 patterns (IEEE 754 round-to-nearest-even, worked by hand below), and
the function is checked against two independent implementations on random
finite inputs: torch's float32 -> bfloat16 cast and the input generator's
integer rounding."""

import numpy as np
import torch

import oracle as O
from workloads import f32_to_bf16_bits


def _from_bits(u32):
    return np.asarray(u32, dtype=np.uint32).view(np.float32).astype(np.float64)


# fp32 pattern -> bf16 pattern.  The low 16 bits are what rounding drops: 0x8000
# is exactly half a bf16 step (a tie), below rounds down, above rounds up.
KNOWN = [
    (0x3F800000, 0x3F80),  # 1.0 exact
    (0x3F808000, 0x3F80),  # 1 + 2^-8: tie, 0x3F80 is even -> down
    (0x3F818000, 0x3F82),  # 1 + 3*2^-8: tie, 0x3F81 is odd -> up to 0x3F82
    (0x3F80C000, 0x3F81),  # 1 + 3*2^-9: three quarters of a step -> up
    (0x3F804000, 0x3F80),  # 1 + 2^-9: a quarter of a step -> down
    (0x3F807FFF, 0x3F80),  # just below the tie -> down
    (0x3F808001, 0x3F81),  # just above the tie -> up
    (0xBF808000, 0xBF80),  # -(1 + 2^-8): negative tie, even -> magnitude down
    (0xBF818000, 0xBF82),  # negative tie, odd -> magnitude up
    (0x3FFF8000, 0x4000),  # 1.9921875 + half step: odd mantissa 0x7F rounds up and carries into the exponent
    (0x7F7F8000, 0x7F80),  # largest bf16 + half step: the tie rounds to even = infinity
    (0x7F7F7FFF, 0x7F7F),  # just below that tie stays finite
    (0x00000000, 0x0000),  # +0
    (0x80000000, 0x8000),  # -0
    (0x00080000, 0x0008),  # subnormal 2^-130 is exact in bf16
    (0x00018000, 0x0002),  # subnormal tie, 0x0001 is odd -> up
]


def test_known_fp32_patterns():
    src = np.array([k for k, _ in KNOWN], dtype=np.uint32)
    want = np.array([v for _, v in KNOWN], dtype=np.uint16)
    np.testing.assert_array_equal(O.round_bf16(_from_bits(src)), want)


def test_fp64_inputs_round_through_fp32():
    # The merged weight is formed in fp32 and then rounded, so an fp64 value is
    # first rounded to fp32.  1 + 2^-8 + 2^-30 is above the bf16 tie in fp64,
    # but 2^-30 is below half an fp32 step at 1 (2^-24), so its fp32 value is
    # the tie 1 + 2^-8, which rounds to even: 0x3F80.  A direct fp64 -> bf16
    # rounding would give 0x3F81.
    x = np.array([1.0 + 2.0**-8 + 2.0**-30, 1.0 + 2.0**-8 + 2.0**-20, -(1.0 + 2.0**-8 + 2.0**-30)])
    np.testing.assert_array_equal(O.round_bf16(x), np.array([0x3F80, 0x3F81, 0xBF80], dtype=np.uint16))


def test_matches_independent_roundings_on_random_values():
    rng = np.random.default_rng(2024)
    u = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    u = u[np.isfinite(f)]
    f = u.view(np.float32)
    got = O.round_bf16(f.astype(np.float64))
    np.testing.assert_array_equal(got, f32_to_bf16_bits(f))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    # values of the size a merged weight holds, where every exponent path is common
    w = rng.standard_normal(1 << 18) * 0.02
    ref = torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.round_bf16(w), ref)
