"""Pins of the oracle's FP8 E4M3 rounding (oracle.paged.round_fp8_e4m3), the
storage format of page mean/variance when they are kept in 8 bits.  Checked
against the format's own code table (every code decoded from its sign,
exponent and mantissa fields), the ties-to-even rule at every midpoint,
saturation, hand-worked values, and PyTorch's float8_e4m3fn conversion."""

import numpy as np
import pytest
import torch

import oracle

R = oracle.paged.round_fp8_e4m3


def code_values():
    """Value of every non-NaN code: exponent field 0 is subnormal (m * 2^-9),
    otherwise (1 + m/8) * 2^(e-7); the code S.1111.111 is NaN."""
    out = {}
    for s in (0, 1):
        for e in range(16):
            for m in range(8):
                if e == 15 and m == 7:
                    continue
                v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
                out[(s << 7) | (e << 3) | m] = -v if s else v
    return out


def test_code_table_shape():
    vals = code_values()
    assert len(vals) == 254
    pos = sorted({v for v in vals.values() if v > 0})
    assert pos[0] == 2.0 ** -9 and pos[-1] == 448.0 and len(pos) == 126


def test_every_code_value_is_a_fixed_point():
    v = np.array(list(code_values().values()))
    np.testing.assert_array_equal(R(v), v)


def test_midpoints_round_to_the_even_code():
    vals = code_values()
    pos = sorted((v, c) for c, v in vals.items() if v > 0 and c < 128)
    pos = [(0.0, 0)] + pos
    for (v0, c0), (v1, c1) in zip(pos[:-1], pos[1:]):
        mid = 0.5 * (v0 + v1)
        want = v0 if c0 % 2 == 0 else v1
        assert R(np.array([mid]))[0] == want, (v0, v1)
        assert R(np.array([-mid]))[0] == -want
        eps = (v1 - v0) * 1e-6
        assert R(np.array([mid - eps]))[0] == v0
        assert R(np.array([mid + eps]))[0] == v1


@pytest.mark.parametrize("x,want", [
    (1.0625, 1.0),            # midpoint of 1 and 1.125: even mantissa 0
    (1.1875, 1.25),           # midpoint of 1.125 and 1.25: even mantissa 2
    (0.2, 0.203125),          # 1.625 * 2^-3
    (-3.3, -3.25),            # 1.625 * 2^1
    (447.0, 448.0),           # rounds to the largest finite value
    (464.0, 448.0),           # midpoint to the (reserved) next code: saturates
    (1e6, 448.0),
    (-1e30, -448.0),
    (2.0 ** -10, 0.0),        # half the smallest subnormal: ties to zero
    (3 * 2.0 ** -10, 2.0 ** -8),   # 1.5 subnormal steps: ties to 2 steps
    (0.0146, 0.013671875),          # just below 2^-6: subnormal grid (7.475 steps -> 7 * 2^-9)
    (0.0146484375, 0.015625),       # 7.5 steps: ties to 8 * 2^-9 = 2^-6, the smallest normal
])
def test_worked_values(x, want):
    assert R(np.array([x]))[0] == want


def test_nan_and_signed_zero():
    out = R(np.array([np.nan, -0.0, 0.0]))
    assert np.isnan(out[0])
    assert out[1] == 0.0 and np.signbit(out[1]) and not np.signbit(out[2])


def test_matches_torch_float8_e4m3fn_in_range():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-14, 6.5, 200000))
    x = x.astype(np.float32).astype(np.float64)
    x = x[np.abs(x) < 448.0]
    want = torch.from_numpy(x).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(R(x), want)
