"""Pins of the oracle's number-format codecs against torch's CPU casts (an
independent implementation) and against the formats' defining properties."""

import numpy as np
import pytest
import torch

from oracle import codecs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_bf16_decode_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all((ours == ref) | both_nan)
    # the sign bit is kept for zeros
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_bf16_encode_matches_torch_on_random_and_ties():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0),
        rng.standard_normal(1000).astype(np.float32) * np.float32(1e-38),   # subnormals
        np.float32([0.0, -0.0, 1.0, -1.0, 3.3895314e38, -3.3895314e38, np.inf, -np.inf]),
    ]).astype(np.float32)
    # exact midpoints between neighbouring bf16 values: the low 16 bits are 0x8000
    mids = (rng.integers(0x0080, 0x7F00, 5000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, mids, -mids])
    ours = codecs.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # ties go to the even neighbour
    assert codecs.f32_to_bf16_bits(np.uint32([0x3F808000]).view(np.float32))[0] == 0x3F80
    assert codecs.f32_to_bf16_bits(np.uint32([0x3F818000]).view(np.float32))[0] == 0x3F82


def test_bf16_nan_stays_nan():
    out = codecs.f32_to_bf16_bits(np.float32([np.nan]))
    assert np.isnan(codecs.bf16_bits_to_f64(out))[0]


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all((ours == ref) | both_nan)
    assert np.nanmax(ours) == 448.0 and np.nanmin(ours) == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert np.count_nonzero(np.isnan(ours)) == 2                  # no infinities, one NaN per sign


def test_e4m3_every_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = codecs.e4m3_bits_to_f64(codes).astype(np.float32)
    assert np.array_equal(codecs.f32_to_e4m3_bits(vals), codes)


def test_e4m3_midpoints_round_to_even():
    pos = np.arange(0x00, 0x7E, dtype=np.uint8)                   # 0 .. just below 448
    lo = codecs.e4m3_bits_to_f64(pos)
    hi = codecs.e4m3_bits_to_f64(pos + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)  # midpoints are float32-exact
    got = codecs.f32_to_e4m3_bits(mid)
    even = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    assert np.array_equal(got, even)
    assert np.array_equal(codecs.f32_to_e4m3_bits(-mid), even | 0x80)


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    v = np.concatenate([
        rng.standard_normal(300_000) * 60.0,
        rng.standard_normal(20_000) * 0.01,                       # subnormal region
        rng.uniform(-448, 448, 20_000),
    ]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    ours = codecs.f32_to_e4m3_bits(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates():
    v = np.float32([448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3e38, np.inf, -500.0, -np.inf])
    got = codecs.f32_to_e4m3_bits(v)
    assert np.array_equal(got, np.uint8([0x7E] * 8 + [0xFE] * 2))
    assert codecs.f32_to_e4m3_bits(np.float32([np.nan]))[0] == 0x7F


def _exact_bf16_round(v):
    """Nearest bf16 value to a float64, ties to even, by exact rational
    comparison of the two bf16 neighbours obtained by truncation."""
    from fractions import Fraction
    u = np.float64(v).view(np.uint64)
    lo = (u & ~np.uint64((1 << 45) - 1)).view(np.float64)         # toward zero
    step = np.uint64(1 << 45)
    hi = (u & ~np.uint64((1 << 45) - 1)) + step
    hi = hi.view(np.float64)
    fv, flo, fhi = Fraction(float(v)), Fraction(float(lo)), Fraction(float(hi))
    dlo, dhi = abs(fv - flo), abs(fhi - fv)
    if dlo < dhi:
        return float(lo)
    if dhi < dlo:
        return float(hi)
    lo_even = ((np.float64(lo).view(np.uint64) >> np.uint64(45)) & np.uint64(1)) == 0
    return float(lo) if lo_even else float(hi)


def test_round_to_bf16_exact_on_random_float64():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-20, 20, 3000),
                        -rng.standard_normal(1000)])
    got = codecs.round_to_bf16(v)
    ref = np.array([_exact_bf16_round(a) for a in v])
    assert np.array_equal(got, ref)


def test_round_to_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal(100_000) * 5).astype(np.float32)
    mids = (rng.integers(0x0080, 0x7F00, 5000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, mids, -mids])
    got = codecs.round_to_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
