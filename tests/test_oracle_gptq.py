"""Pins for the oracle's NVFP4-adapted GPTQ (simolm.com PACT blog, "Method",
third bullet: offline calibration of the frozen weights by GPTQ adapted to
NVFP4 block scales, with statistics from reconstructed NVFP4 activations;
arXiv abstract of "PACT: NVFP4 Data-Flow LoRA Fine-Tuning on Consumer GPUs").

Pinned against:
  * a diagonal Hessian, where no error propagates and GPTQ is the plain
    quantizer (bit-exact);
  * the textbook optimal-brain-surgeon form of the same column sweep, written
    here independently: it updates the explicit inverse Hessian after every
    column instead of using its Cholesky factor, and applies every update
    column by column instead of in lazy batches;
  * invariance to the lazy-batch size and to which rows are quantized
    together (rows are independent);
  * dead inputs (all-zero activation columns) and the Hessian's definition
    by brute force;
  * the method's purpose: on correlated activations the layer output error
    ||(W - W^) X^T|| drops well below that of the plain quantizer.
"""
import numpy as np
import pytest

import oracle
from nvfp4_gemm_amd import synth
from tests import _exact as ex


def _case(N, K, n, seed, rank=16):
    rng = np.random.default_rng(seed)
    W = synth.weight_bf16(rng, N, K)
    X = synth.calibration_bf16(rng, n, K, rank=rank)
    xq = oracle.quantize_bf16(X)
    return W, xq


def _equal(a: oracle.NVFP4, b: oracle.NVFP4, what=""):
    np.testing.assert_array_equal(a.codes, b.codes, err_msg=what)
    np.testing.assert_array_equal(a.scales, b.scales, err_msg=what)
    np.testing.assert_array_equal(a.d.view(np.uint32), b.d.view(np.uint32), err_msg=what)


def test_hessian_brute_force():
    W, xq = _case(4, 32, 7, seed=1)
    H = oracle.gptq_hessian(xq)
    X = oracle.dequantize(xq).astype(np.float64)
    ref = np.zeros((32, 32))
    for t in range(7):
        for i in range(32):
            for j in range(32):
                ref[i, j] += X[t, i] * X[t, j]
    ref *= 2.0 / 7
    np.testing.assert_allclose(H, ref, rtol=1e-13, atol=0)
    assert np.array_equal(H, H.T)


def test_diagonal_hessian_is_plain_quantizer():
    rng = np.random.default_rng(2)
    N, K = 24, 256
    W = synth.weight_bf16(rng, N, K)
    H = np.diag(rng.uniform(0.5, 2.0, K))
    _equal(oracle.gptq_nvfp4(W, H), oracle.quantize_bf16(W), "diagonal H")


def _obs_reference(W, H, percdamp=0.01):
    """GPTQ's column sweep in its optimal-brain-surgeon form, per row: the
    inverse Hessian over the columns not yet quantized is kept explicitly and
    downdated after every column; every update applied at once."""
    N, K = W.shape
    Hd = np.array(H, dtype=np.float64, copy=True)
    dead = np.diag(Hd) == 0
    Hd[dead, dead] = 1.0
    Hd[np.arange(K), np.arange(K)] += percdamp * np.mean(np.diag(Hd))
    Hinv0 = np.linalg.inv(Hd)
    rtn = oracle.quantize_bf16(W)
    Wf = oracle.bf16_to_f32(W).astype(np.float64)
    Wf[:, dead] = 0.0
    codes = np.zeros((N, K), np.uint8)
    scales = np.zeros((N, K // 16), np.uint8)
    for n in range(N):
        Hinv = Hinv0.copy()
        w = Wf[n].copy()
        d = np.float32(rtn.d[n])
        D = np.float32(6) * d
        S = np.float32(0)
        for i in range(K):
            if i % 16 == 0:
                amax = np.max(np.abs(w[i:i + 16].astype(np.float32)))
                sb = oracle.e4m3_encode(float(amax / D)) if d != 0 else 0
                scales[n, i // 16] = sb
                S = np.float32(oracle.e4m3_value(sb)) * d
            wf = np.float32(w[i])
            mag = oracle.e2m1_encode_mag(float(np.abs(wf) / S)) if S != 0 else 0
            code = (8 if np.signbit(wf) else 0) | mag
            codes[n, i] = code
            q = oracle.e2m1_value(code) * oracle.e4m3_value(scales[n, i // 16]) * float(d)
            # optimal update of the remaining weights for the error at column i
            w[i + 1:] -= (w[i] - q) / Hinv[i, i] * Hinv[i, i + 1:]
            w[i] = q
            # remove column i from the inverse Hessian
            Hinv = Hinv - np.outer(Hinv[:, i], Hinv[i, :]) / Hinv[i, i]
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return oracle.NVFP4(packed, scales, rtn.d.copy())


@pytest.mark.parametrize("N,K,n,seed", [(5, 64, 200, 3), (3, 160, 120, 4), (4, 96, 40, 5)])
def test_matches_textbook_obs_sweep(N, K, n, seed):
    W, xq = _case(N, K, n, seed)
    H = oracle.gptq_hessian(xq)
    got = oracle.gptq_nvfp4(W, H, blocksize=32)
    _equal(got, _obs_reference(W, H), "GPTQ vs optimal-brain-surgeon sweep")
    assert not np.array_equal(got.codes, oracle.quantize_bf16(W).codes)  # errors did propagate


def test_lazy_batch_size_and_row_independence():
    W, xq = _case(40, 512, 600, seed=6)
    H = oracle.gptq_hessian(xq)
    ref = oracle.gptq_nvfp4(W, H, blocksize=128)
    for bs in (16, 48, 512):
        _equal(oracle.gptq_nvfp4(W, H, blocksize=bs), ref, f"blocksize {bs}")
    rows = np.array([3, 17, 39, 0])
    sub = oracle.gptq_nvfp4(W[rows], H, blocksize=128)
    _equal(sub, oracle.NVFP4(ref.codes[rows], ref.scales[rows], ref.d[rows]), "row subset")


def test_dead_input_columns():
    rng = np.random.default_rng(7)
    N, K, n = 8, 128, 300
    W = synth.weight_bf16(rng, N, K)
    X = synth.calibration_bf16(rng, n, K)
    X[:, 5] = 0
    X[:, 64:80] = 0          # a whole dead block
    xq = oracle.quantize_bf16(X)
    H = oracle.gptq_hessian(xq)
    assert H[5, 5] == 0 and np.all(np.diag(H)[64:80] == 0)
    q = oracle.gptq_nvfp4(W, H)
    c = ex.unpack_codes(q.codes)
    assert np.all(c[:, 5] == 0) and np.all(c[:, 64:80] == 0)
    assert np.all(q.scales[:, 4] == 0)  # block 64..79 quantizes zeros


def test_reduces_layer_output_error():
    W, xq = _case(64, 512, 2048, seed=8, rank=32)
    H = oracle.gptq_hessian(xq)
    Xh = oracle.dequantize(xq).astype(np.float64)
    Wf = oracle.bf16_to_f32(W).astype(np.float64)
    e_g = np.linalg.norm((Wf - oracle.dequantize(oracle.gptq_nvfp4(W, H))) @ Xh.T)
    e_r = np.linalg.norm((Wf - oracle.dequantize(oracle.quantize_bf16(W))) @ Xh.T)
    assert e_g < 0.85 * e_r, (e_g, e_r)
