"""Oracle pins for the number formats (CPU only).

E2M1 is pinned to the OCP Microscaling v1.0 value table and to a brute-force
nearest-value search in exact rational arithmetic; E4M3 to torch's
independent float8_e4m3fn conversion and to the 448 bound that the
BitDecoding-FP4 config's probability_environment allows for tau; E8M0 to its
power-of-two definition.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


# OCP MX v1.0, FP4 E2M1 element values for magnitude codes 0..7
OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_grid_matches_ocp_table():
    vals = F.e2m1_value(np.arange(16, dtype=np.uint8))
    assert list(vals[:8]) == OCP_E2M1
    assert list(-vals[8:]) == OCP_E2M1
    assert F.E2M1_MAX == 6.0


def _brute_e2m1(x: Fraction, s: Fraction) -> int:
    """Nearest grid point to |x|/s by exhaustive search; ties to the even code."""
    if s == 0:
        return 0
    r = abs(x) / s
    best = None
    for m, g in enumerate(OCP_E2M1):
        d = abs(r - Fraction(g))
        key = (d, m % 2)          # smaller distance, then even code
        if best is None or key < best[0]:
            best = (key, m)
    return best[1]


def _e4m3_values():
    return [float(v) for v in F.e4m3_value(np.arange(0x7F, dtype=np.uint8))]


def test_e2m1_encode_matches_bruteforce_dense_and_ties():
    scales = [0.0, 2.0 ** -9, 3 * 2.0 ** -9, 2.0 ** -6, 0.875, 1.0, 1.375, 6.5, 448.0]
    ks = np.arange(-520, 521)                       # r = k/64 covers [-8.1, 8.1]
    for s in scales:
        s32 = np.float32(s)
        x = (ks.astype(np.float64) / 64.0 * s).astype(np.float32)
        got = F.e2m1_encode(x, s32)
        for xi, gi in zip(x, got):
            want = _brute_e2m1(Fraction(float(xi)), Fraction(float(s32)))
            if s == 0:
                assert gi == 0
                continue
            assert (gi & 7) == want, (s, xi, gi, want)
            assert (gi >> 3) == (1 if np.signbit(xi) else 0)


def test_e2m1_encode_random_against_bruteforce():
    rng = np.random.default_rng(1)
    vals = _e4m3_values()[1:]
    for _ in range(2000):
        s = np.float32(vals[rng.integers(len(vals))])
        x = np.float32(rng.standard_normal() * float(s) * 4)
        got = int(F.e2m1_encode(np.array([x]), s)[0])
        assert (got & 7) == _brute_e2m1(Fraction(float(x)), Fraction(float(s)))


def test_e2m1_tie_points_round_to_even_code():
    s = np.float32(1.0)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    assert list(F.e2m1_encode(ties, s)) == [0, 2, 2, 4, 4, 6, 6]
    assert list(F.e2m1_encode(-ties, s)) == [8, 10, 10, 12, 12, 14, 14]
    assert list(F.e2m1_encode(np.array([6.0, 7.0, 1e30], np.float32), s)) == [7, 7, 7]


def test_e4m3_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    mine = F.e4m3_value(np.arange(256, dtype=np.uint8))
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(t[~nan], mine[~nan])
    assert F.e4m3_value(np.uint8(0x7E)) == 448.0
    assert np.isnan(F.e4m3_value(np.uint8(0x7F)))


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    vals = np.array(_e4m3_values())
    mids = (vals[1:] + vals[:-1]) / 2                     # exact ties
    x = np.concatenate([
        vals, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
        np.nextafter(mids.astype(np.float32), np.float32(1e9)),
        np.exp(rng.uniform(np.log(1e-5), np.log(447.0), 20000)),
        [0.0, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 1e-30],
    ]).astype(np.float32)
    x = x[x <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(x), ref)


def test_e4m3_saturates_at_448():
    # 448 is the largest finite E4M3 value, the upper bound the config allows tau
    x = np.array([448.0, 450.0, 464.0, 470.0, 1e6, 3e38], dtype=np.float32)
    assert list(F.e4m3_encode(x)) == [0x7E] * 6
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([-1.0], np.float32))


def test_e8m0_powers_of_two():
    c = np.arange(255, dtype=np.uint8)
    assert np.array_equal(F.e8m0_value(c), 2.0 ** (c.astype(np.float64) - 127))
    assert F.e8m0_value(np.uint8(127)) == 1.0
    assert np.isnan(F.e8m0_value(np.uint8(255)))


def test_bf16_widening_is_exact():
    x = np.array([1.0, -2.5, 3.140625, 1e-20], dtype=np.float32)
    u = (x.view(np.uint32) >> 16).astype(np.uint16)
    back = F.bf16_to_f32(u)
    ref = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(back, ref)
