"""Pins of the oracle's bfloat16 rounding (CPU only).

The oracle's ``round_bf16`` is written from the format definition; here it is pinned
against values the format fixes by hand and against torch's float32 -> bfloat16
conversion (a library routine), which rounds to nearest even.
"""

import numpy as np
import pytest
import torch

from oracle.numerics import BF16_MAX, round_bf16, round_f32, rounder


def test_hand_values():
    # spacing of bfloat16 just above 1 is 2**-7
    assert round_bf16(1.0 + 2.0**-8) == 1.0  # exact tie -> even (1.0)
    assert round_bf16(1.0 + 3 * 2.0**-8) == 1.0 + 2.0**-6  # tie between ...01 and ...10 -> even
    assert round_bf16(1.0 + 2.0**-8 + 2.0**-20) == 1.0 + 2.0**-7  # just above the tie
    assert round_bf16(-(1.0 + 2.0**-8 + 2.0**-20)) == -(1.0 + 2.0**-7)
    assert round_bf16(3.0) == 3.0 and round_bf16(0.0) == 0.0
    assert round_bf16(BF16_MAX) == BF16_MAX
    assert round_bf16(2.0**128) == np.inf  # beyond the largest finite value
    assert round_bf16(2.0**-133) == 2.0**-133  # smallest subnormal
    assert round_bf16(2.0**-135) == 0.0  # below half of it
    assert round_bf16(1.0 / 3.0) == 0.333984375  # 0x3EAB


def test_matches_torch_conversion():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(200_000) * 10.0 ** rng.integers(-30, 30, 200_000),
        rng.standard_normal(50_000).astype(np.float32),
    ]).astype(np.float32)
    # exact ties: bf16 values plus half a spacing
    base = torch.from_numpy(rng.standard_normal(50_000).astype(np.float32)).to(torch.bfloat16)
    b = base.float().numpy()
    spacing = 2.0 ** (np.floor(np.log2(np.abs(b))) - 7)
    ties = (b + 0.5 * spacing).astype(np.float32)
    vals = np.concatenate([vals, ties[np.abs(ties) > 0]])
    want = torch.from_numpy(vals).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = round_bf16(vals.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_idempotent_and_monotone():
    rng = np.random.default_rng(2)
    v = np.sort(rng.standard_normal(10_000))
    r = round_bf16(v)
    np.testing.assert_array_equal(round_bf16(r), r)
    assert np.all(np.diff(r) >= 0)


def test_f32_and_rounder():
    v = np.array([1.0 + 2.0**-30, 0.1])
    np.testing.assert_array_equal(round_f32(v), np.float32(v).astype(np.float64))
    assert rounder("f64")(v)[0] == v[0]
    with pytest.raises(ValueError):
        rounder("fp8")
