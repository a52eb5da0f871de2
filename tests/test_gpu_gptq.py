"""GPU parity of the NVFP4-adapted GPTQ calibration (simolm.com PACT blog,
"Method", third bullet; arXiv abstract of "PACT: NVFP4 Data-Flow LoRA
Fine-Tuning on Consumer GPUs") against the oracle.

Both sides work in binary64 but sum in different orders (the Hessian's token
sums, the Cholesky factorization and inverse, the lazy-batch updates), so
their binary64 weights agree to about 1e-12 relative.  Every code and block
scale is decided in binary32 from those weights by the same rule, so a
decision can differ only where a weight lies within that distance of a
rounding boundary; the expected number of such cases over these tests is far
below one, and the tests require codes, scales and row scales to match bit
for bit.  The Hessian itself is compared within its summation error bound.
"""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_gemm_amd import pact as pb
from nvfp4_gemm_amd import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _case(N, K, n, seed, rank=32):
    rng = np.random.default_rng(seed)
    W = synth.weight_bf16(rng, N, K)
    X = synth.calibration_bf16(rng, n, K, rank=rank)
    return W, X


@pytest.mark.parametrize("n,K", [(37, 64), (1000, 256), (4096, 1024)])
def test_hessian_parity(n, K):
    _, X = _case(1, K, n, seed=n + K)
    xq = oracle.quantize_bf16(X)
    ref = oracle.gptq_hessian(xq)
    gxq = pb.pact_quantize_nvfp4(G.dev_bf16(X))
    H = pb.pact_gptq_hessian_nvfp4(gxq)
    # accumulate: a second batch (the same rows) doubles the sums
    H2 = pb.pact_gptq_hessian_nvfp4(gxq, H=H.clone(), accumulate=True)
    torch.cuda.synchronize()
    G.assert_nvfp4_equal(gxq, xq, "calibration rows")
    Xh = np.abs(oracle.dequantize(xq).astype(np.float64))
    bound = 4 * n * 2.0 ** -52 * (2.0 / n) * (Xh.T @ Xh) + 1e-300
    got = H.cpu().numpy()
    assert np.all(np.abs(got - ref) <= bound)
    assert np.all(np.abs(H2.cpu().numpy() - 2 * ref) <= 2 * bound)


@pytest.mark.parametrize("N,K,n,bs,dead", [(96, 256, 1024, 128, False), (70, 512, 800, 32, True),
                                           (130, 192, 300, 64, False)])
def test_gptq_parity_small(N, K, n, bs, dead):
    W, X = _case(N, K, n, seed=N + K)
    if dead:
        X[:, 7] = 0
        X[:, 128:144] = 0
    xq = oracle.quantize_bf16(X)
    ref = oracle.gptq_nvfp4(W, oracle.gptq_hessian(xq), blocksize=bs)
    H = pb.pact_gptq_hessian_nvfp4(pb.pact_quantize_nvfp4(G.dev_bf16(X)))
    got = pb.pact_gptq_nvfp4(G.dev_bf16(W), H, blocksize=bs)
    torch.cuda.synchronize()
    G.assert_nvfp4_equal(got, ref, f"GPTQ {N}x{K} bs {bs}")


def test_gptq_projection_size_to_layouts_and_gemm():
    """A 3B-shaped q projection (3072 x 3072) calibrated on 4096 synthetic
    tokens: sampled rows against the oracle (rows are independent), the
    transposed layout built from the calibrated forward layout bit-exact, a
    forward GEMM on it within the GEMM tolerance, and the calibration lowering
    the layer output error below the plain quantizer's."""
    N = K = 3072
    n = 4096
    W, X = _case(N, K, n, seed=5)
    xq = oracle.quantize_bf16(X)
    Href = oracle.gptq_hessian(xq)
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(1).integers(0, N, 40)]))
    ref_rows = oracle.gptq_nvfp4(W[rows], Href)
    gxq = pb.pact_quantize_nvfp4(G.dev_bf16(X))
    H = pb.pact_gptq_hessian_nvfp4(gxq)
    gW = G.dev_bf16(W)
    gf = pb.pact_gptq_nvfp4(gW, H)
    gf2, gb = pb.pact_build_weight_layouts(W_fwd_in=gf)
    torch.cuda.synchronize()
    hf = G.host_nvfp4(gf)
    G.assert_nvfp4_equal(oracle.NVFP4(hf.codes[rows], hf.scales[rows], hf.d[rows]), ref_rows, "GPTQ rows")
    _, ref_b = oracle.build_weight_layouts(W_fwd=hf)
    G.assert_nvfp4_equal(gb, ref_b, "W_bwd from the calibrated layout")
    G.assert_nvfp4_equal(gf2, hf, "W_fwd copy")
    # a forward GEMM on the calibrated layout
    mrows = np.arange(0, n, 97)
    Y = pb.pact_gemm_nvfp4_fwd(gxq, gf)
    torch.cuda.synchronize()
    Yref = oracle.gemm_fwd(xq, None, hf, rows=mrows)
    G.check_gemm_tolerance(G.host_bits(Y)[mrows], Yref, "fwd on the calibrated layout")
    # the calibration's purpose: a smaller layer output error than the plain quantizer's
    Xh = oracle.dequantize(xq)[::8].astype(np.float64)
    Wf = oracle.bf16_to_f32(W).astype(np.float64)
    e_g = np.linalg.norm((Wf - oracle.dequantize(hf)) @ Xh.T)
    e_r = np.linalg.norm((Wf - oracle.dequantize(oracle.quantize_bf16(W))) @ Xh.T)
    assert e_g < 0.9 * e_r, (e_g, e_r)
