"""Pins for the oracle's element formats (E2M1 codes, E4M3 scales, BF16).

Pinned against: the format facts on the PACT blog's FAQ (golden fixture), the
value set implied by each bit layout, torch's independent float8_e4m3fn and
bfloat16 conversions, and brute-force nearest-value search in exact rationals.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import _exact as ex

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def fmt():
    with open(os.path.join(GOLD, "nvfp4_format.json")) as f:
        return json.load(f)


def test_e2m1_value_set(fmt):
    mags = [oracle.e2m1_value(c) for c in range(8)]
    assert mags == fmt["e2m1_magnitudes"]
    for c in range(8):
        assert oracle.e2m1_value(c | 8) == -mags[c]
    assert np.signbit(oracle.e2m1_value(8))  # code 8 is -0


def test_e4m3_matches_torch_decode_all_bytes(fmt):
    bytes_ = torch.arange(256, dtype=torch.uint8)
    ref = bytes_.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for b in range(256):
        v = oracle.e4m3_value(b)
        if np.isnan(ref[b]):
            assert np.isnan(v), b
        else:
            assert v == ref[b], (b, v, ref[b])
    for key, val in fmt["e4m3_landmarks"].items():
        assert oracle.e4m3_value(int(key, 16)) == val
    finite_nonneg = [b for b in range(128) if not np.isnan(oracle.e4m3_value(b))]
    assert len(finite_nonneg) == 127 and max(oracle.e4m3_value(b) for b in finite_nonneg) == 448.0


def test_roundtrip_encode_decode():
    for c in range(8):
        assert oracle.e2m1_encode_mag(oracle.e2m1_value(c)) == c
    for b in range(127):
        assert oracle.e4m3_encode(oracle.e4m3_value(b)) == b


def _float_grid_around(points, n_ulps=3):
    out = set()
    for p in points:
        f = np.float32(p)
        out.add(float(f))
        lo = hi = f
        for _ in range(n_ulps):
            lo = np.nextafter(lo, np.float32(-np.inf))
            hi = np.nextafter(hi, np.float32(np.inf))
            out.add(float(lo))
            out.add(float(hi))
    return sorted(v for v in out if v >= 0)


def test_e2m1_rounding_brute_force():
    mags = ex.E2M1_MAGS
    mids = [(a + b) / 2 for a, b in zip(mags, mags[1:])]
    pts = [float(m) for m in mags] + [float(m) for m in mids] + [6.5, 7.0, 100.0, 1e30]
    rng = np.random.default_rng(1)
    pts += list(rng.uniform(0, 7, 2000))
    for r in _float_grid_around(pts):
        want = ex.nearest_even(Fraction(r), mags)
        assert oracle.e2m1_encode_mag(r) == want, r
    # closed-form thresholds (ties to the even code)
    assert [oracle.e2m1_encode_mag(t) for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)] == \
        [0, 2, 2, 4, 4, 6, 6]


def test_e4m3_rounding_brute_force_and_torch():
    vals = ex.E4M3_VALS
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    pts = [float(v) for v in vals] + [float(m) for m in mids] + [2.0 ** -10, 2.0 ** -11, 460.0,
                                                                 464.0, 1000.0, 3e38]
    grid = _float_grid_around(pts, 2)
    for t in grid:
        want = ex.nearest_even(Fraction(t), vals)
        assert oracle.e4m3_encode(t) == want, t
    # torch's own round-to-nearest-even cast agrees inside the finite range
    inside = np.array([t for t in grid if t <= 448.0], np.float32)
    tref = torch.from_numpy(inside).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(t)) for t in inside], np.uint8)
    np.testing.assert_array_equal(got, tref)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    # add exact ties: low half == 0x8000 with odd and even kept parts
    ties = (rng.integers(0, 2 ** 16, 2000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    bits = np.concatenate([bits, ties])
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.0e38)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(v) for v in f], np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_operand_products_exact_in_bf16_and_f16():
    """Every (E2M1 value) x (E4M3 scale) is exact in BF16 and in FP16, so a GEMM
    may feed decoded operands to BF16 or FP16 matrix units without rounding."""
    for c in range(16):
        for b in range(127):
            p = Fraction(oracle.e2m1_value(c)) * Fraction(oracle.e4m3_value(b))
            assert ex.rnbf16(p) == p
            if p != 0:
                assert abs(p) >= Fraction(1, 2 ** 10) and abs(p) <= 2688
            # FP16: 11 significant bits, min normal 2^-14 (all products are normal)
            assert ex.round_to_binary(p, 11, -14) == p
