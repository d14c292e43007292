"""Pins for the oracle's number formats (CPU only)."""
from fractions import Fraction
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_values(name):
    vals = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            vals.append(float(line))
    return vals


def test_e2m1_grid_matches_golden():
    # eight magnitudes per sign (the pages' count), values from the E2M1 bit layout
    assert list(F.E2M1_MAG) == _golden_values("e2m1_magnitudes.txt")
    assert len(F.E2M1_MAG) == 8


def test_e2m1_decode_all_codes():
    codes = np.arange(16, dtype=np.uint8)
    v = F.e2m1_decode(codes)
    assert list(v[:8]) == list(F.E2M1_MAG)
    assert list(v[8:]) == [-m for m in F.E2M1_MAG]


def _interesting_e2m1_inputs():
    pts = []
    grid = [0, .5, 1, 1.5, 2, 3, 4, 6]
    mids = [(a + b) / 2 for a, b in zip(grid, grid[1:])]
    for p in grid + mids + [6.5, 7, 8, 100, 1e30]:
        p32 = np.float32(p)
        pts += [p32, np.nextafter(p32, np.float32(np.inf)), np.nextafter(p32, np.float32(0))]
    pts = np.array(pts, dtype=np.float32)
    return np.concatenate([pts, -pts])


def test_e2m1_encode_matches_threshold_rule_on_edges():
    v = _interesting_e2m1_inputs()
    got = F.e2m1_encode(v)
    want = [exact.e2m1_code_by_thresholds(Fraction(float(x)), bool(np.signbit(x))) for x in v]
    assert list(got) == want


def test_e2m1_encode_matches_threshold_rule_dense():
    # every float32 in [0, 8) with a 2**-12 step plus random magnitudes
    rng = np.random.default_rng(1)
    v = np.concatenate([np.arange(0, 8, 2.0 ** -12, dtype=np.float32),
                        rng.uniform(-10, 10, 20000).astype(np.float32)])
    got = F.e2m1_encode(v)
    want = [exact.e2m1_code_by_thresholds(Fraction(float(x)), bool(np.signbit(x))) for x in v]
    assert list(got) == want


def test_e2m1_ties_go_to_even_code():
    # hand-listed: midpoint -> code
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, c in cases.items():
        assert F.e2m1_encode(np.float32(v)) == c, v
        assert F.e2m1_encode(np.float32(-v)) == (8 | c), v


def test_e2m1_signed_zero_and_saturation():
    assert F.e2m1_encode(np.float32(-0.0)) == 0x8
    assert F.e2m1_encode(np.float32(0.0)) == 0x0
    assert F.e2m1_encode(np.float32(-0.1)) == 0x8
    assert F.e2m1_encode(np.float32(1e9)) == 0x7
    assert F.e2m1_encode(np.float32(-1e9)) == 0xF


def test_e4m3_table_structure():
    vals = F.E4M3_POS
    assert len(vals) == 127 and vals[0] == 0 and vals[-1] == 448.0
    assert vals[1] == 2.0 ** -9            # smallest subnormal
    assert vals[8] == 2.0 ** -6            # smallest normal
    assert np.all(np.diff(vals) > 0)
    assert F.e4m3_decode(np.uint8(0x7F)) != F.e4m3_decode(np.uint8(0x7F))   # NaN


def test_e4m3_encode_matches_torch_cast():
    # torch's float32 -> float8_e4m3fn cast rounds to nearest even; on [0, 448]
    # it is a library reference for the encoder
    vals = F.E4M3_POS
    mids = (vals[1:] + vals[:-1]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)),
                          np.nextafter(pts, np.float32(0))])
    rng = np.random.default_rng(2)
    pts = np.concatenate([pts, rng.uniform(0, 448, 50000).astype(np.float32),
                          np.exp2(rng.uniform(-14, 8.8, 50000)).astype(np.float32)])
    pts = pts[(pts >= 0) & (pts <= 448)]
    want = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode_nonneg(pts)
    assert np.array_equal(got, want)


def test_e4m3_encode_saturates_and_matches_exact_rule():
    assert F.e4m3_encode_nonneg(np.float32(448)) == 0x7E
    assert F.e4m3_encode_nonneg(np.float32(1e6)) == 0x7E
    assert F.e4m3_encode_nonneg(np.float32(2.0 ** -10)) == 0          # tie -> 0 (even)
    assert F.e4m3_encode_nonneg(np.float32(3 * 2.0 ** -10)) == 2      # tie 1|2 -> 2
    for u in [1.0625, 1.1875, 0.01, 300.0, 447.9, 2.0 ** -9 * 1.5]:
        assert F.e4m3_encode_nonneg(np.float32(u)) == exact.e4m3_round(Fraction(float(np.float32(u))))


def test_bf16_round_matches_torch_on_float32():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 100,
                        np.exp2(rng.uniform(-120, 120, 10000)).astype(np.float32),
                        np.array([0, -0.0, 1, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 65504], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f64_to_bf16_bits(x.astype(np.float64)), want)


def test_bf16_round_from_float64_is_single_rounding():
    # just above a bf16 midpoint: a float32 detour would land on the midpoint
    # and round to even (down); one rounding from float64 goes up
    x = 1.0 + 2 ** -8 + 2 ** -40
    assert F.round_to_bf16(np.float64(x)) == 1.0 + 2 ** -7
    assert float(np.float64(np.float32(x))) == 1.0 + 2 ** -8
    rng = np.random.default_rng(4)
    xs = rng.standard_normal(2000) * np.exp2(rng.integers(-30, 30, 2000))
    got = F.round_to_bf16(xs)
    want = [float(exact.to_bf16(Fraction(float(v)))) for v in xs]
    assert list(got) == want


def test_bits_roundtrip():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    assert np.array_equal(F.f64_to_bf16_bits(v[fin]), bits[fin])
