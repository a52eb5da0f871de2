"""Pins for the oracle's cached weight layouts and NVFP4 GEMMs.

Layouts (simolm.com PACT blog, "Method", last bullet: forward and backward
NVFP4 weight layouts are rebuilt, transposed and re-quantized once, then
cached): pinned by a weight built so that both layouts are exact in closed
form, and by error bounds on random weights.

GEMMs (blog "Method", first bullet: FP32 accumulation, BF16 output, forward and
input-gradient; LoRA h = W0 x + B A x from the kongchang.com PEFT explainer):
pinned by float64 brute force within the FP32 summation bound, exact results
on small integer-valued cases, the LoRA identity (B = 0 reproduces the frozen
output) and the parameter-count closed form printed on the PEFT page.
"""
import json
import os

import numpy as np
import pytest

import oracle
from nvfp4_gemm_amd import synth
from tests import _exact as ex

GOLD = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E4M3 = np.array([oracle.e4m3_value(b) for b in range(127)])


def test_forward_layout_is_row_quantizer():
    rng = np.random.default_rng(20)
    W = synth.weight_bf16(rng, 64, 256)
    fwd, _ = oracle.build_weight_layouts(W)
    q = oracle.quantize_bf16(W)
    np.testing.assert_array_equal(fwd.codes, q.codes)
    np.testing.assert_array_equal(fwd.scales, q.scales)
    np.testing.assert_array_equal(fwd.d, q.d)


def test_both_layouts_exact_in_closed_form():
    """R[n,k] = E[n,k] * 448 * 2^P(n//16), with a +-6 in every 16-block of every
    row and column and every row holding E = +-6 in a P-maximal position:
    forward codes = E, scales 448, d = 2^P; backward codes = E^T, scale of
    block (k, nb) = 448 * 2^(P(nb) - Pmax), d = 2^Pmax."""
    rng = np.random.default_rng(21)
    N, K = 64, 96
    codes = rng.integers(0, 16, (N, K))
    codes[(np.arange(N)[:, None] % 16) == (np.arange(K)[None, :] % 16)] = 7  # +6 diagonal
    sign = np.where(codes & 8, -1.0, 1.0)
    E = E2M1[codes & 7] * sign
    P = rng.integers(-3, 4, N // 16)
    P[rng.integers(N // 16)] = 4
    Pmax = P.max()
    R = E * 448.0 * np.exp2(np.repeat(P, 16))[:, None]
    W = synth.to_bf16_bits(R)
    assert np.array_equal(synth.bf16_bits_to_f32(W), R.astype(np.float32))
    fwd, bwd = oracle.build_weight_layouts(W)
    np.testing.assert_array_equal(ex.unpack_codes(fwd.codes), codes)
    assert np.all(fwd.scales == 0x7E)
    np.testing.assert_array_equal(fwd.d, np.exp2(np.repeat(P, 16)).astype(np.float32))
    np.testing.assert_array_equal(ex.unpack_codes(bwd.codes), codes.T)
    want_scale = 448.0 * np.exp2(P - Pmax)
    got_scale = E4M3[bwd.scales]
    np.testing.assert_array_equal(got_scale, np.broadcast_to(want_scale, (K, N // 16)))
    np.testing.assert_array_equal(bwd.d, np.float32(2.0 ** Pmax))
    # the given-forward-layout path starts from the same point
    fwd2, bwd2 = oracle.build_weight_layouts(W_fwd=fwd)
    np.testing.assert_array_equal(bwd2.codes, bwd.codes)
    np.testing.assert_array_equal(bwd2.scales, bwd.scales)


def test_backward_layout_error_bound():
    rng = np.random.default_rng(22)
    W = synth.weight_bf16(rng, 128, 64)
    fwd, bwd = oracle.build_weight_layouts(W)
    R = oracle.dequantize(fwd).astype(np.float64)
    Rb = oracle.dequantize(bwd).astype(np.float64)
    # each element within half an E2M1 step of its block scale (6 at the top);
    # the row max block's E4M3 rounding adds at most 1/16 relative on top
    S = E4M3[bwd.scales].repeat(16, axis=1) * bwd.d[:, None].astype(np.float64)
    assert np.all(np.abs(Rb - R.T) <= S * 1.0 * (1 + 1e-6))
    assert np.all(bwd.scales.max(axis=1) == 0x7E)
    # relative Frobenius error of the round trip is that of a 4-bit format
    assert np.linalg.norm(Rb - R.T) / np.linalg.norm(R) < 0.2


def _dequant64(q):
    b = oracle.operand_values(q).astype(np.float64)
    return b, q.d.astype(np.float64)


def _bf16(x):
    return synth.bf16_bits_to_f32(x).astype(np.float64)


def _fwd_f64(xq, X, wq, A, B, s, C):
    """float64 model: exact frozen sum, BF16-rounded LoRA intermediate."""
    a, da = _dequant64(xq)
    b, db = _dequant64(wq)
    acc = a @ b.T
    y = acc * da[:, None] * db[None, :]
    absy = np.abs(a) @ np.abs(b).T * da[:, None] * db[None, :]
    if A is not None:
        T = _bf16(synth.to_bf16_bits(_bf16(X) @ _bf16(A).T))
        L = T @ _bf16(B).T
        y = y + s * L
        absy = absy + abs(s) * (np.abs(T) @ np.abs(_bf16(B)).T)
    if C is not None:
        y = y + _bf16(C)
        absy = absy + np.abs(_bf16(C))
    return y, absy


def _ulp_bf16(v):
    v = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(v)) - 7)


@pytest.mark.parametrize("M,N,K,r", [(5, 7, 48, 0), (9, 33, 160, 3), (17, 24, 64, 8)])
def test_gemm_fwd_brute_force_f64(M, N, K, r):
    li = synth.single_linear_inputs(M=M, N=N, K=K, r=max(r, 1), seed=M + N + K, act="t4")
    xq = oracle.quantize_bf16(li.X)
    wq = oracle.quantize_bf16(li.W)  # forward layout = Q over rows of W (N need not be 16k)
    rng = np.random.default_rng(23)
    C = synth.normal_bf16(rng, (M, N), 0.1)
    A, B = (li.A, li.B) if r else (None, None)
    Y = oracle.gemm_fwd(xq, li.X, wq, A, B, li.s, C)
    y64, absy = _fwd_f64(xq, li.X, wq, A, B, li.s, C)
    # sequential FP32: |err| <= gamma_n * sum|terms| (n = K + r + 4 roundings)
    n = K + max(r, 0) + 6
    gam = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
    bound = gam * absy + 0.5 * _ulp_bf16(y64) * 1.01 + 2.0 ** -140
    err = np.abs(_bf16(Y) - y64)
    assert np.all(err <= bound + 0.5 * _ulp_bf16(_bf16(Y))), np.max(err / bound)


def test_gemm_exact_when_sums_are_exact():
    """Small integer-valued operands: every partial sum is exact in FP32, so the
    result is the exact product rounded once to BF16."""
    rng = np.random.default_rng(24)
    M, N, K = 6, 10, 64
    codes_x = rng.integers(0, 16, (M, K))
    codes_w = rng.integers(0, 16, (N, K))
    xq = oracle.NVFP4(ex.pack_codes(codes_x), np.full((M, K // 16), 0x38, np.uint8),
                      np.ones(M, np.float32))  # scale byte 0x38 = 1.0
    wq = oracle.NVFP4(ex.pack_codes(codes_w), np.full((N, K // 16), 0x40, np.uint8),
                      np.full(N, 0.5, np.float32))  # scale byte 0x40 = 2.0
    Y = oracle.gemm_fwd(xq, None, wq)
    a = E2M1[codes_x & 7] * np.where(codes_x & 8, -1, 1)
    b = E2M1[codes_w & 7] * np.where(codes_w & 8, -1, 1) * 2.0
    want = synth.to_bf16_bits((a @ b.T) * 0.5)
    np.testing.assert_array_equal(Y, want)


def test_lora_identity_and_algebra():
    li = synth.single_linear_inputs(M=12, N=48, K=96, r=4, seed=3)
    xq = oracle.quantize_bf16(li.X)
    wq, wb = oracle.build_weight_layouts(li.W)
    Y0 = oracle.gemm_fwd(xq, li.X, wq)
    Yb0 = oracle.gemm_fwd(xq, li.X, wq, li.A, np.zeros_like(li.B), li.s)
    Ys0 = oracle.gemm_fwd(xq, li.X, wq, li.A, li.B, 0.0)
    np.testing.assert_array_equal(_bf16(Yb0), _bf16(Y0))  # values: +-0 compare equal
    np.testing.assert_array_equal(_bf16(Ys0), _bf16(Y0))
    # s B (A X) agrees with X (s B A)^T up to rounding
    Y = oracle.gemm_fwd(xq, li.X, wq, li.A, li.B, li.s)
    dW = li.s * _bf16(li.B) @ _bf16(li.A)
    lora = _bf16(li.X) @ dW.T
    diff = _bf16(Y) - _bf16(Y0)
    assert np.max(np.abs(diff - lora)) <= 0.02 * np.max(np.abs(lora)) + 4 * np.max(_ulp_bf16(_bf16(Y)))
    # dgrad identity too
    dyq = oracle.quantize_bf16(li.dY)
    G0 = oracle.gemm_dgrad(dyq, li.dY, wb)
    Gb0 = oracle.gemm_dgrad(dyq, li.dY, wb, li.A, np.zeros_like(li.B), li.s)
    np.testing.assert_array_equal(_bf16(Gb0), _bf16(G0))


@pytest.mark.parametrize("M,N,K,r", [(7, 48, 32, 0), (10, 64, 80, 5)])
def test_gemm_dgrad_brute_force_f64(M, N, K, r):
    li = synth.single_linear_inputs(M=M, N=N, K=K, r=max(r, 1), seed=7 + M)
    _, wb = oracle.build_weight_layouts(li.W)
    dyq = oracle.quantize_bf16(li.dY)
    A, B = (li.A, li.B) if r else (None, None)
    dX = oracle.gemm_dgrad(dyq, li.dY, wb, A, B, li.s)
    a, da = _dequant64(dyq)
    b, db = _dequant64(wb)
    y = (a @ b.T) * da[:, None] * db[None, :]
    absy = (np.abs(a) @ np.abs(b).T) * da[:, None] * db[None, :]
    if r:
        T = _bf16(synth.to_bf16_bits(_bf16(li.dY) @ _bf16(li.B)))  # [M, r]
        y = y + li.s * (T @ _bf16(li.A))
        absy = absy + abs(li.s) * (np.abs(T) @ np.abs(_bf16(li.A)))
    n = N + r + 6
    gam = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
    bound = gam * absy + 0.5 * _ulp_bf16(y) * 1.01 + 2.0 ** -140
    err = np.abs(_bf16(dX) - y)
    assert np.all(err <= bound + 0.5 * _ulp_bf16(_bf16(dX)))
    # the dgrad approximates dY . W of the original BF16 weights
    ref = _bf16(li.dY) @ _bf16(li.W)
    if r == 0:
        assert np.linalg.norm(_bf16(dX) - ref) / np.linalg.norm(ref) < 0.2


def test_rows_subset_matches_full():
    li = synth.single_linear_inputs(M=20, N=32, K=64, r=2, seed=9)
    xq = oracle.quantize_bf16(li.X)
    wq, _ = oracle.build_weight_layouts(li.W)
    full = oracle.gemm_fwd(xq, li.X, wq, li.A, li.B, li.s)
    rows = np.array([19, 0, 7])
    np.testing.assert_array_equal(oracle.gemm_fwd(xq, li.X, wq, li.A, li.B, li.s, rows=rows),
                                  full[rows])


def test_lora_parameter_count_closed_form():
    with open(os.path.join(GOLD, "lora_param_count.json")) as f:
        g = json.load(f)
    d, k, r = g["d"], g["k"], g["r"]
    full, lora = d * k, r * (d + k)
    assert abs(full / 1e6 - g["full_params_approx_millions"]) < 0.01
    assert abs(lora / 1e3 - g["lora_params_approx_thousands"]) < 0.1
    assert full / lora > g["min_compression"]
    # the shapes the oracle's LoRA term uses hold exactly r (d + k) parameters
    li = synth.single_linear_inputs(M=2, N=d // 64, K=k // 64, r=r)
    assert li.A.size + li.B.size == r * (d // 64 + k // 64)
