"""Pins for the oracle's fused producers: RMSNorm -> quantize and
SiLU*mul -> quantize (simolm.com PACT blog, section "Method": quantization is
fused into the RMSNorm and SiLU-multiply kernels; the forward SiLU-multiply
reads BF16 and an NVFP4 copy of gate/up is kept for backward).

Pinned against: math.fsum (correctly rounded sums), closed forms for constant
and power-of-two rows, 50-digit mpmath evaluation of g/(1+exp(-g)) over all
65536 BF16 inputs, and torch's BF16 rounding for the final products.
"""
import math
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

import oracle
from nvfp4_gemm_amd import synth
from tests import _exact as ex


def test_sumsq_is_correctly_rounded():
    rng = np.random.default_rng(10)
    rows = [synth.student_t_bf16(rng, (3072,), 3.0, 0.5),
            synth.normal_bf16(rng, (1536,), 1.0),
            synth.to_bf16_bits(rng.standard_normal(2048) * np.exp2(rng.integers(-120, 120, 2048))),
            synth.to_bf16_bits(np.array([1e-38, 3e38, -2e-39, 1.0] * 4))]
    for x in rows:
        xf = synth.bf16_bits_to_f32(x).astype(np.float64)
        want = math.fsum(v * v for v in xf)  # squares are exact in binary64
        assert oracle.sumsq_bf16(x) == want


def test_rmsnorm_closed_forms():
    H = 256
    # constant rows c, eps = 0: rstd = RN32(1/|c|) computed exactly; y = bf16(c*rstd*gamma)
    for c in (1.0, -3.0, 0.15625, 1536.0, 2.0 ** -60):
        x = synth.to_bf16_bits(np.full((1, H), c))
        gamma = synth.to_bf16_bits(np.ones(H))
        y, yq, rstd = oracle.rmsnorm_quant(x, gamma, 0.0)
        cf = Fraction(float(synth.bf16_bits_to_f32(x)[0, 0]))
        ms = ex.rn64(ex.rn64(cf * cf * H) / H)
        mpmath.mp.dps = 60
        sq = mpmath.sqrt(mpmath.mpf(ms.numerator) / ms.denominator)
        want = ex.rn32(ex.rn64(1 / ex.rn64(_frac_of_mpf(sq))))
        assert Fraction(float(rstd[0])) == want
        if math.log2(abs(c)).is_integer():
            assert rstd[0] == 1 / abs(c)
            np.testing.assert_array_equal(synth.bf16_bits_to_f32(y), np.sign(c))


@pytest.mark.parametrize("eps", [1e-5, 1e-6])
def test_rmsnorm_against_high_precision(eps):
    rng = np.random.default_rng(11)
    x = synth.student_t_bf16(rng, (16, 512), 4.0, 0.5)
    gamma = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(512))
    y, yq, rstd = oracle.rmsnorm_quant(x, gamma, eps)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    gf = synth.bf16_bits_to_f32(gamma)
    for i in range(16):
        ss = math.fsum(v * v for v in xf[i])
        exact = 1 / mpmath.sqrt(mpmath.mpf(ss) / 512 + mpmath.mpf(np.float32(eps).item()))
        # the binary64 op chain is within a few binary64 ulps, so rstd is the
        # binary32 rounding of the exact value unless that is a near-tie
        assert abs(float(rstd[i]) - float(exact)) <= 0.5 * np.spacing(np.float32(rstd[i])) * (1 + 1e-6)
        t = (xf[i].astype(np.float32) * rstd[i]).astype(np.float32) * gf
        ref = torch.from_numpy(t.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
        np.testing.assert_array_equal(y[i], ref.view(np.uint16))
    # yq is Q applied to the BF16 output
    q2 = oracle.quantize_bf16(y)
    np.testing.assert_array_equal(yq.codes, q2.codes)
    np.testing.assert_array_equal(yq.scales, q2.scales)
    np.testing.assert_array_equal(yq.d, q2.d)
    # normalised rows have mean square ~1 before the gain
    ms = np.mean((synth.bf16_bits_to_f32(y) / gf) ** 2, axis=1)
    assert np.all(np.abs(ms - 1) < 0.02)


def _frac_of_mpf(v) -> Fraction:
    if v == 0:
        return Fraction(0)
    man, exp = mpmath.mpf(v).man_exp  # man_exp carries the magnitude only
    mag = Fraction(int(man)) * Fraction(2) ** int(exp)
    return -mag if v < 0 else mag


def _rn32_of_mpf(v) -> Fraction:
    return ex.rn32(_frac_of_mpf(v))


@pytest.fixture(scope="module")
def sigtab():
    return oracle.sigmoid_table()


def test_sigmoid_exhaustive_against_mpmath(sigtab):
    mpmath.mp.dps = 50
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g = synth.bf16_bits_to_f32(bits)
    for b in range(65536):
        gv = float(g[b])
        if not math.isfinite(gv):
            continue
        if gv == 0:
            assert sigtab[b] == 0 and np.signbit(sigtab[b]) == np.signbit(g[b])
            continue
        if gv < -120:
            assert sigtab[b] == 0 and np.signbit(sigtab[b])  # below the binary32 range
            continue
        if gv > 40:
            assert sigtab[b] == np.float32(gv)  # exp(-g) far below half an ulp
            continue
        gm = mpmath.mpf(gv)
        want = _rn32_of_mpf(gm / (1 + mpmath.exp(-gm)))
        assert Fraction(float(sigtab[b])) == want, (b, gv)


def test_silu_mul_products_and_stash(sigtab):
    rng = np.random.default_rng(12)
    g = synth.student_t_bf16(rng, (8, 256), 4.0, 0.5)
    u = synth.student_t_bf16(rng, (8, 256), 4.0, 0.5)
    h, hq, gq, uq = oracle.silu_mul_quant(g, u)
    prod = sigtab[g.astype(np.int64)] * synth.bf16_bits_to_f32(u)
    ref = torch.from_numpy(prod.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(h, ref.view(np.uint16))
    for q, src in ((hq, h), (gq, g), (uq, u)):
        q2 = oracle.quantize_bf16(src)
        np.testing.assert_array_equal(q.codes, q2.codes)
        np.testing.assert_array_equal(q.scales, q2.scales)
        np.testing.assert_array_equal(q.d, q2.d)
