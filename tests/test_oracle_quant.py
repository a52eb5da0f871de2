"""Pins for the oracle's row quantizer Q (NVFP4: 16 E2M1 + one E4M3 scale, plus
a per-row FP32 scale; simolm.com PACT blog, FAQ).

Pinned against: exact round trips of rows built to be representable, exact
ties, invariants that hold for every input, an exact-rational model run by
brute force on small rows, and the 4.5-bit storage fact from the blog's FAQ.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from nvfp4_gemm_amd import synth
from tests import _exact as ex

GOLD = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def representable_row(rng, nblocks, k, ties=False):
    """A row whose quantization is known in closed form: row scale d = 2^k
    (one element equals 2688 * 2^k), block b has E4M3 scale s_b and contains a
    +-6 element, every element is (E2M1 value) * s_b * 2^k.  With ties=True
    some elements sit exactly on an E2M1 rounding midpoint instead."""
    codes = rng.integers(0, 16, size=nblocks * 16)
    scale_bytes = rng.integers(0x20, 0x7E, size=nblocks)  # normal scales
    top = rng.integers(nblocks)
    scale_bytes[top] = 0x7E
    for b in range(nblocks):
        j = 16 * b + rng.integers(16)
        codes[j] = 7 | (8 if rng.random() < 0.5 else 0)
    vals = np.array([E2M1[c & 7] * (-1 if c & 8 else 1) for c in codes], np.float64)
    expect_codes = codes.copy()
    if ties:
        mids = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]
        for j in range(0, nblocks * 16, 3):
            if (codes[j] & 7) == 7:
                continue
            mv, want = mids[rng.integers(len(mids))]
            neg = rng.random() < 0.5
            vals[j] = -mv if neg else mv
            expect_codes[j] = want | (8 if neg else 0)
    sc = np.array([oracle.e4m3_value(int(b)) for b in scale_bytes])
    x = vals * np.repeat(sc, 16) * 2.0 ** k
    return x, expect_codes, scale_bytes


@pytest.mark.parametrize("k", [-20, -3, 0, 5])
@pytest.mark.parametrize("ties", [False, True])
def test_exact_roundtrip_of_representable_rows(k, ties):
    rng = np.random.default_rng(100 + k + (7 if ties else 0))
    rows, nb = 6, 8
    X = np.zeros((rows, nb * 16))
    C = np.zeros((rows, nb * 16), np.uint8)
    S = np.zeros((rows, nb), np.uint8)
    for i in range(rows):
        X[i], C[i], S[i] = representable_row(rng, nb, k, ties)
    xb = synth.to_bf16_bits(X)
    assert np.array_equal(synth.bf16_bits_to_f32(xb).astype(np.float64), X)  # exact in BF16
    for q in (oracle.quantize_bf16(xb), oracle.quantize_f32(X.astype(np.float32))):
        np.testing.assert_array_equal(ex.unpack_codes(q.codes), C)
        np.testing.assert_array_equal(q.scales, S)
        np.testing.assert_array_equal(q.d, np.float32(2.0 ** k))
        if not ties:
            np.testing.assert_array_equal(oracle.dequantize(q), X.astype(np.float32))


def test_zero_and_signed_zero_rows():
    x = np.zeros((3, 32), np.float32)
    x[1, ::2] = -0.0
    x[2, 5] = -1e-30  # forces a tiny nonzero row scale; stays finite
    q = oracle.quantize_f32(x)
    c = ex.unpack_codes(q.codes)
    assert q.d[0] == 0 and q.d[1] == 0
    assert np.all(q.scales[:2] == 0)
    assert np.all(c[0] == 0)
    np.testing.assert_array_equal(c[1], np.where(np.arange(32) % 2 == 0, 8, 0))
    assert c[2, 5] == 8 | 7  # the row's only nonzero element is its max: -6


def test_invariants_on_heavy_tailed_rows():
    rng = np.random.default_rng(3)
    x = synth.student_t_bf16(rng, (64, 1024), 3.0, 0.5)
    q = oracle.quantize_bf16(x)
    xf = synth.bf16_bits_to_f32(x)
    c = ex.unpack_codes(q.codes)
    b = oracle.operand_values(q)
    assert q.scales.max() <= 0x7E
    sc = np.array([oracle.e4m3_value(i) for i in range(256)], np.float64)
    for i in range(x.shape[0]):
        absx = np.abs(xf[i]).reshape(-1, 16)
        top_block = np.argmax(absx.max(axis=1))
        assert q.scales[i, top_block] == 0x7E  # the row's max block takes scale 448
        for blk in range(absx.shape[0]):
            s = q.scales[i, blk]
            if s >= 0x08:  # normal scale: the block max encodes as +-6
                jmax = np.argmax(absx[blk])
                assert (c[i, 16 * blk + jmax] & 7) == 7
        # per element: |x/S - decoded magnitude| within half the E2M1 step
        S = (sc[q.scales[i]] * np.float64(q.d[i])).repeat(16)
        r = np.abs(xf[i].astype(np.float64)) / S
        mag = np.abs(b[i].astype(np.float64)) / sc[q.scales[i]].repeat(16)
        # half the gap to the neighbour on the side where x lies
        up = {0: .25, .5: .25, 1: .25, 1.5: .25, 2: .5, 3: .5, 4: 1., 6: 0.}
        dn = {0: 0., .5: .25, 1: .25, 1.5: .25, 2: .25, 3: .5, 4: .5, 6: 1.}
        half = np.where(r >= mag, [up[m] for m in mag], [dn[m] for m in mag])
        sat = (mag == 6) & ((r <= 6 * 17 / 16 * 1.001) | (q.scales[i].repeat(16) < 0x08))
        ok = (np.abs(r - mag) <= half * (1 + 1e-6)) | sat
        assert ok.all()
        np.testing.assert_array_equal(np.signbit(b[i]) | (b[i] == 0), np.signbit(xf[i]) | (b[i] == 0))


def test_brute_force_exact_model():
    rng = np.random.default_rng(4)
    cases = []
    for nu in (2.0, 4.0):
        cases.append(synth.student_t_bf16(rng, (3, 64), nu, 0.5))
    cases.append(synth.normal_bf16(rng, (3, 64), 1e-30))  # subnormal-range row scales
    cases.append(synth.normal_bf16(rng, (3, 64), 1e30))
    spread = rng.standard_normal((3, 64)) * np.exp2(rng.integers(-40, 40, (3, 64)))
    cases.append(synth.to_bf16_bits(spread))                 # wide block dynamic range
    for x in cases:
        q = oracle.quantize_bf16(x)
        c = ex.unpack_codes(q.codes)
        xf = synth.bf16_bits_to_f32(x)
        for i in range(x.shape[0]):
            codes, scales, d = ex.quantize_row_exact([float(v) for v in xf[i]])
            assert Fraction(float(q.d[i])) == d
            assert list(q.scales[i]) == scales
            assert list(c[i]) == codes


def test_fp32_inputs_brute_force():
    """Q on FP32 inputs with full 24-bit significands (the backward weight layout
    quantizes such values)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((4, 48)) * 0.02).astype(np.float32)
    q = oracle.quantize_f32(x)
    c = ex.unpack_codes(q.codes)
    for i in range(4):
        codes, scales, d = ex.quantize_row_exact([float(v) for v in x[i]])
        assert Fraction(float(q.d[i])) == d and list(q.scales[i]) == scales and list(c[i]) == codes


def test_storage_is_4p5_bits_per_element():
    with open(os.path.join(GOLD, "nvfp4_format.json")) as f:
        fmt = json.load(f)
    q = oracle.quantize_bf16(np.zeros((8, 4096), np.uint16))
    bits = 8 * (q.codes.nbytes + q.scales.nbytes) / (8 * 4096)
    assert bits == fmt["approx_bits_per_element"]
    assert q.codes.shape[1] * 2 // q.scales.shape[1] == fmt["elements_per_block"]
