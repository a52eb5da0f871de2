"""Pins of the oracle's nonlinear backward from the NVFP4 stash (simolm.com
PACT blog, section "Method", second bullet: the quantized RMSNorm output is
reused in backward, gate/up are kept in NVFP4 for backward).  Each check
compares against something other than the oracle's own arithmetic: a float64
evaluation, exact rational arithmetic, autograd of the forward function, or
the mathematics (identities, limits)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from nvfp4_gemm_amd import synth

torch = pytest.importorskip("torch")


def _f32(bits):
    return oracle.bf16_to_f32(np.asarray(bits, np.uint16))


def _finite_bf16():
    b = np.arange(65536, dtype=np.uint32)
    return b[((b >> 7) & 0xFF) != 0xFF]


def test_dsilu_table_against_float64():
    """silu'(g) = sigma(g) (1 + g (1 - sigma(g))) correctly rounded: within
    half an ulp (plus the float64 evaluation error) of a float64 evaluation
    for every finite BF16 input."""
    t = oracle.dsilu_table()
    b = _finite_bf16()
    g = _f32(b).astype(np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-g))
    ref = s * (1.0 + g * (1.0 - s))
    got = t[b].astype(np.float64)
    ulp = np.spacing(np.abs(got).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 0.5 * ulp + 1e-15 * np.abs(ref) + 1e-300)


def test_dsilu_exhaustive_against_mpmath():
    """silu'_32(g) = binary32 rounding of sigma(g)(1 + g(1 - sigma(g))) for
    every finite BF16 g, against 50-digit mpmath evaluation (100 digits when
    the 50-digit value lies within 1e-40 relative of a binary32 rounding
    midpoint); outside |g| <= 128 the value is 1 (g > 128: the excess over 1,
    about g e^-g, is far below half an ulp) or -0 (g < -128: about g e^g, far
    below the smallest subnormal)."""
    import math
    from fractions import Fraction

    import mpmath

    from tests import _exact as ex

    t = oracle.dsilu_table()

    def dsilu_mp(gv, dps):
        mpmath.mp.dps = dps
        gm = mpmath.mpf(gv)
        sg = 1 / (1 + mpmath.exp(-gm))
        return sg * (1 + gm * (1 - sg))

    def frac(v):
        if v == 0:
            return Fraction(0)
        man, exp = mpmath.mpf(v).man_exp
        mag = Fraction(int(man)) * Fraction(2) ** int(exp)
        return -mag if v < 0 else mag

    for b in _finite_bf16():
        gv = float(_f32(np.array([b]))[0])
        got = float(t[b])
        if gv > 128:
            assert got == 1.0, (hex(b), gv, got)
            continue
        if gv < -128:
            assert got == 0.0 and math.copysign(1.0, got) < 0, (hex(b), gv, got)
            continue
        v = frac(dsilu_mp(gv, 50))
        want = ex.rn32(v)
        # distance to the midpoints next to the rounded value, relative
        if want != 0:
            up = ex.rn32(want + abs(want) * Fraction(1, 2 ** 23))
            mids = [(want + up) / 2, want - (up - want) / 2]
            if min(abs(v - m) for m in mids) <= abs(want) * Fraction(1, 10 ** 40):
                want = ex.rn32(frac(dsilu_mp(gv, 100)))
        assert Fraction(got) == want, (hex(b), gv, got, float(want))


def test_dsilu_identities_and_limits():
    t = oracle.dsilu_table()
    assert t[0x0000] == 0.5 and t[0x8000] == 0.5           # silu'(+-0) = 1/2
    b = _finite_bf16()
    b = b[b < 0x8000]                                        # g >= 0
    # silu'(g) + silu'(-g) = 1 exactly in real arithmetic
    s = t[b].astype(np.float64) + t[b | 0x8000].astype(np.float64)
    assert np.max(np.abs(s - 1.0)) <= 2.0 ** -24 + 2.0 ** -25
    assert t[0x4300] == 1.0                                  # g = 128: 1 - 127 e^-128 rounds to 1
    assert t[0xC300] == 0.0 and np.signbit(t[0xC300])        # g = -128: about -127 e^-128, rounds to -0
    big = _f32(0x4010).item()                                # g = 2.25: silu' exceeds 1 for g > 1
    assert t[0x4010] > 1.0 and abs(t[0x4010] - (lambda s: s * (1 + big * (1 - s)))(1 / (1 + np.exp(-big)))) < 1e-6


def test_dot_exact_against_rationals():
    rng = np.random.default_rng(4)
    for n in (1, 7, 64, 333):
        a = synth.to_bf16_bits(rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n)))
        b = (rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n))).astype(np.float32)
        exact = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(_f32(a), b))
        assert oracle.dot_bf16_f32(a, b) == float(exact)     # Fraction -> float rounds to nearest even
    a = synth.to_bf16_bits(np.array([1.0, -1.0, 3.0, -3.0]))
    b = np.array([2.0 ** 100, 2.0 ** 100, 2.0 ** -100, 2.0 ** -100], np.float32)
    assert oracle.dot_bf16_f32(a, b) == 0.0                  # exact cancellation


def _stash(rng, rows, cols, scale=1.0):
    x = synth.to_bf16_bits(scale * rng.standard_t(4, (rows, cols)) * 0.5)
    return x, oracle.quantize_bf16(x)


def test_silu_mul_bwd_against_forward_derivative():
    """du = dh silu(g') and dg = dh u' silu'(g') on the BF16 values of the
    dequantized stash, against a float64 central difference of the forward
    silu(g) u; outputs within a BF16 rounding (plus the difference error)."""
    rng = np.random.default_rng(7)
    rows, cols = 5, 96
    _, gq = _stash(rng, rows, cols, 2.0)
    _, uq = _stash(rng, rows, cols)
    dh = synth.to_bf16_bits(rng.standard_normal((rows, cols)))
    dg, du, dgq, duq = oracle.silu_mul_bwd_quant(dh, gq, uq)
    g = _f32(synth.to_bf16_bits(oracle.dequantize(gq).astype(np.float64))).astype(np.float64)
    u = _f32(synth.to_bf16_bits(oracle.dequantize(uq).astype(np.float64))).astype(np.float64)
    d = _f32(dh).astype(np.float64)
    silu = lambda z: z / (1.0 + np.exp(-z))
    eps = 1e-6
    ref_dg = d * u * (silu(g + eps) - silu(g - eps)) / (2 * eps)
    ref_du = d * silu(g)
    for got, ref in ((dg, ref_dg), (du, ref_du)):
        gotf = _f32(got).astype(np.float64)
        assert np.all(np.abs(gotf - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-7 * (1 + np.abs(d * u)))
    # the quantized outputs are Q of the BF16 outputs (Q is pinned elsewhere)
    for q, x in ((dgq, dg), (duq, du)):
        r = oracle.quantize_bf16(x)
        assert np.array_equal(q.codes, r.codes) and np.array_equal(q.scales, r.scales) and np.array_equal(q.d, r.d)


def test_silu_mul_bwd_special_cases():
    rows, cols = 1, 16
    g = synth.to_bf16_bits(np.zeros((rows, cols)))
    u = synth.to_bf16_bits(np.full((rows, cols), 3.0))
    dh = synth.to_bf16_bits(np.full((rows, cols), 2.0))
    dg, du, _, _ = oracle.silu_mul_bwd_quant(dh, oracle.quantize_bf16(g), oracle.quantize_bf16(u))
    assert np.all(_f32(du) == 0.0)                           # silu(0) = 0
    assert np.all(_f32(dg) == 3.0)                           # 2 * 3 * silu'(0) = 3
    zero = synth.to_bf16_bits(np.zeros((rows, cols)))
    dg, du, dgq, _ = oracle.silu_mul_bwd_quant(zero, oracle.quantize_bf16(u), oracle.quantize_bf16(u))
    assert np.all(_f32(dg) == 0.0) and np.all(_f32(du) == 0.0) and np.all(dgq.d == 0.0)


def _rms_inputs(rng, rows, cols, eps=1e-5):
    x = synth.to_bf16_bits(rng.standard_t(4, (rows, cols)) * 0.5)
    gamma = synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(cols))
    _, yq, rstd = oracle.rmsnorm_quant(x, gamma, eps)
    dy = synth.to_bf16_bits(rng.standard_normal((rows, cols)))
    return yq, gamma, rstd, dy


def test_rmsnorm_bwd_against_autograd():
    """dx = rstd (g - x^ mean(g x^)), g = dy gamma, with x^ = deq(yq)/gamma:
    the input gradient of sum(dy * rmsnorm(x)) by float64 autograd at
    x = x^/rstd with the eps for which rstd is exact there."""
    rng = np.random.default_rng(11)
    rows, cols = 6, 128
    yq, gamma, rstd, dy = _rms_inputs(rng, rows, cols)
    dx, dxq = oracle.rmsnorm_bwd(dy, yq, gamma, rstd)
    y = oracle.dequantize(yq).astype(np.float64)
    gm = _f32(gamma).astype(np.float64)
    for i in range(rows):
        r = float(rstd[i])
        xh = y[i] / gm
        eps = (1.0 - np.mean(xh * xh)) / (r * r)
        x = torch.tensor(xh / r, dtype=torch.float64, requires_grad=True)
        out = x * torch.rsqrt(torch.mean(x * x) + eps) * torch.tensor(gm)
        (out * torch.tensor(_f32(dy[i]).astype(np.float64))).sum().backward()
        ref = x.grad.numpy()
        got = _f32(dx[i]).astype(np.float64)
        tol = 2.0 ** -8 * np.abs(ref) + 1e-5 * r * np.max(np.abs(_f32(dy[i])))
        assert np.all(np.abs(got - ref) <= tol), i
    r = oracle.quantize_bf16(dx)
    assert np.array_equal(dxq.codes, r.codes) and np.array_equal(dxq.scales, r.scales)


def test_rmsnorm_bwd_residual_and_zero():
    rng = np.random.default_rng(12)
    rows, cols = 3, 64
    yq, gamma, rstd, dy = _rms_inputs(rng, rows, cols)
    C = synth.to_bf16_bits(rng.standard_normal((rows, cols)))
    dx0, _ = oracle.rmsnorm_bwd(dy, yq, gamma, rstd)
    dxc, _ = oracle.rmsnorm_bwd(dy, yq, gamma, rstd, C)
    # dx with C differs from bf16(dx + C) by at most the two roundings
    a = _f32(dxc).astype(np.float64)
    b = _f32(dx0).astype(np.float64) + _f32(C).astype(np.float64)
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * (np.abs(b) + np.abs(_f32(dx0))) + 1e-30)
    zero = synth.to_bf16_bits(np.zeros((rows, cols)))
    dxz, dxq = oracle.rmsnorm_bwd(zero, yq, gamma, rstd)
    assert np.all(_f32(dxz) == 0.0) and np.all(dxq.d == 0.0)


def _lora_case(rng, M, N, K, r):
    x = synth.to_bf16_bits(rng.standard_t(4, (M, K)) * 0.5)
    xq = oracle.quantize_bf16(x)
    dY = synth.to_bf16_bits(rng.standard_normal((M, N)))
    A = synth.to_bf16_bits(0.02 * rng.standard_normal((r, K)))
    B = synth.to_bf16_bits(0.01 * rng.standard_normal((N, r)))
    return xq, dY, A, B


def test_lora_grads_against_autograd():
    """dA, dB of sum(dY * s (X^ A^T) B^T) by float64 autograd, X^ the BF16
    values of the dequantized stash; the oracle's BF16 intermediates stay
    within a BF16 rounding of it (relative to the gradient's scale)."""
    rng = np.random.default_rng(21)
    M, N, K, r, s = 40, 48, 64, 8, 2.0
    xq, dY, A, B = _lora_case(rng, M, N, K, r)
    dA, dB = oracle.lora_grads(xq, dY, A, B, s)
    X = torch.tensor(_f32(synth.to_bf16_bits(oracle.dequantize(xq).astype(np.float64))).astype(np.float64))
    tA = torch.tensor(_f32(A).astype(np.float64), requires_grad=True)
    tB = torch.tensor(_f32(B).astype(np.float64), requires_grad=True)
    loss = (torch.tensor(_f32(dY).astype(np.float64)) * (s * (X @ tA.T) @ tB.T)).sum()
    loss.backward()
    for got, ref in ((dA, tA.grad.numpy()), (dB, tB.grad.numpy())):
        assert np.max(np.abs(got - ref)) <= 2.0 ** -7 * np.max(np.abs(ref))


def test_lora_grads_zero_adapters():
    """B = 0 gives dA = 0 exactly (T' = 0); A = 0 gives dB = 0 exactly."""
    rng = np.random.default_rng(22)
    xq, dY, A, B = _lora_case(rng, 16, 32, 32, 4)
    zA = np.zeros_like(A)
    zB = np.zeros_like(B)
    dA, dB = oracle.lora_grads(xq, dY, A, zB, 2.0)
    assert np.all(dA == 0.0) and np.any(dB != 0.0)
    dA, dB = oracle.lora_grads(xq, dY, zA, B, 2.0)
    assert np.all(dB == 0.0) and np.any(dA != 0.0)
