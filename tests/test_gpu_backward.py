"""GPU parity of the nonlinear backward from the NVFP4 stash (simolm.com PACT
blog, section "Method", second bullet: the quantized RMSNorm output is reused
in backward; gate/up are kept in NVFP4 for backward): bit-exact BF16 outputs
and NVFP4 codes, scales and row scales against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_gemm_amd import pact as pb
from nvfp4_gemm_amd import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def test_dsilu32_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    want = oracle.dsilu_table()
    got = pb.pact_debug_dsilu32(torch.from_numpy(bits.view(np.int16).copy()).cuda()).cpu().numpy()
    bad = np.flatnonzero(finite & (got.view(np.uint32) != want.view(np.uint32)))
    assert bad.size == 0, [(hex(int(b)), float(got[b]), float(want[b])) for b in bad[:8]]


def _stash_gu(rng, rows, cols):
    g = synth.to_bf16_bits(rng.standard_t(4, (rows, cols)) * 1.5)
    u = synth.to_bf16_bits(rng.standard_t(4, (rows, cols)) * 0.5)
    _, _, gq, uq = oracle.silu_mul_quant(g, u)
    return gq, uq


@pytest.mark.parametrize("rows,cols", [(1, 16), (5, 48), (7, 1040), (64, 4096), (33, 8192), (9, 8960),
                                       (4, 9232), (3, 17408), (2, 25600)])
def test_silu_mul_bwd_parity(rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    gq, uq = _stash_gu(rng, rows, cols)
    dh = synth.to_bf16_bits(rng.standard_normal((rows, cols)))
    dg, du, dgq, duq = oracle.silu_mul_bwd_quant(dh, gq, uq)
    gdg, gdu, gdgq, gduq = pb.pact_silu_mul_bwd_quant_nvfp4(G.dev_bf16(dh), G.dev_nvfp4(gq), G.dev_nvfp4(uq))
    _, _, gdgq2, gduq2 = pb.pact_silu_mul_bwd_quant_nvfp4(G.dev_bf16(dh), G.dev_nvfp4(gq), G.dev_nvfp4(uq),
                                                          want_bf16=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(G.host_bits(gdg), dg)
    np.testing.assert_array_equal(G.host_bits(gdu), du)
    G.assert_nvfp4_equal(gdgq, dgq, "dgq")
    G.assert_nvfp4_equal(gduq, duq, "duq")
    G.assert_nvfp4_equal(gdgq2, dgq, "dgq (no BF16 outputs)")
    G.assert_nvfp4_equal(gduq2, duq, "duq (no BF16 outputs)")


def _rms_stash(rng, rows, cols, eps=1e-5):
    x = synth.to_bf16_bits(rng.standard_t(4, (rows, cols)) * 0.5)
    gamma = synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(cols))
    _, yq, rstd = oracle.rmsnorm_quant(x, gamma, eps)
    return yq, gamma, rstd


@pytest.mark.parametrize("rows,cols,with_c", [(1, 16, False), (5, 48, True), (7, 1040, False), (64, 2048, True),
                                              (33, 3072, True), (9, 1536, False), (4, 9232, True), (3, 17408, True)])
def test_rmsnorm_bwd_parity(rows, cols, with_c):
    rng = np.random.default_rng(rows * 11 + cols)
    yq, gamma, rstd = _rms_stash(rng, rows, cols)
    dy = synth.to_bf16_bits(rng.standard_normal((rows, cols)))
    C = synth.to_bf16_bits(rng.standard_normal((rows, cols))) if with_c else None
    dx, dxq = oracle.rmsnorm_bwd(dy, yq, gamma, rstd, C)
    args = (G.dev_bf16(dy), G.dev_nvfp4(yq), G.dev_bf16(gamma), torch.from_numpy(rstd).cuda())
    Cd = G.dev_bf16(C) if with_c else None
    gdx, gdxq = pb.pact_rmsnorm_bwd_nvfp4(*args, C=Cd)
    gdx2, _ = pb.pact_rmsnorm_bwd_nvfp4(*args, C=Cd, want_q=False)
    _, gdxq3 = pb.pact_rmsnorm_bwd_nvfp4(*args, C=Cd, want_dx=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(G.host_bits(gdx), dx)
    np.testing.assert_array_equal(G.host_bits(gdx2), dx)
    G.assert_nvfp4_equal(gdxq, dxq, "dxq")
    G.assert_nvfp4_equal(gdxq3, dxq, "dxq (no BF16 output)")


@pytest.mark.parametrize("cols", [3072, 9232])
def test_rmsnorm_bwd_edge_values(cols):
    """Edge values for the exact sum S = sum dy y' and x^ = y' / gamma: dy
    spanning up to 120 binades, subnormal dy, a lone outlier, zero and negative
    zero rows, sparse zeros; gamma with exact zeros (x^ = 0 there) and negative
    entries; with and without the residual; one wavefront per row (3072) and
    eight (9232), bit-exact against the oracle."""
    rng = np.random.default_rng(cols + 3)
    rows = 12
    x = synth.to_bf16_bits(rng.standard_t(4, (rows, cols)) * 0.5)
    g = 1.0 + 0.1 * rng.standard_normal(cols)
    g[rng.integers(0, cols, 40)] = 0.0
    g[rng.integers(0, cols, 40)] *= -1.0
    gamma = synth.to_bf16_bits(g)
    _, yq, rstd = oracle.rmsnorm_quant(x, gamma, 1e-5)
    d = rng.standard_normal((rows, cols))
    d[0] *= np.exp2(rng.integers(-60, 60, cols))        # wide exponent spread in every block
    d[1] *= 1e-39                                       # subnormal BF16 values
    d[2] = 0.0
    d[3] = -0.0
    d[4] *= 1e-3
    d[4, rng.integers(cols)] = 3e4                      # one outlier
    d[5, ::3] = 0.0                                     # sparse zeros
    d[6] *= np.exp2(rng.integers(-12, 13, cols))        # spread near the fast path's bound
    dy = synth.to_bf16_bits(d)
    C = synth.to_bf16_bits(rng.standard_normal((rows, cols)))
    for Cin in (None, C):
        dx, dxq = oracle.rmsnorm_bwd(dy, yq, gamma, rstd, Cin)
        gdx, gdxq = pb.pact_rmsnorm_bwd_nvfp4(G.dev_bf16(dy), G.dev_nvfp4(yq), G.dev_bf16(gamma),
                                              torch.from_numpy(rstd).cuda(),
                                              C=G.dev_bf16(Cin) if Cin is not None else None)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(G.host_bits(gdx), dx)
        G.assert_nvfp4_equal(gdxq, dxq, "dxq")


@pytest.mark.parametrize("shape", ["llama1b_layer", "llama3b_layer"])
def test_backward_layer_sizes_sampled_rows(shape):
    """At the layer workloads' full sizes ([M, I] for SiLU, [M, H] for RMSNorm)
    the kernels run in their real launch configuration; the oracle checks a
    sample of rows (rows are independent)."""
    S = synth.LAYERS[shape]
    M, H, I = S.tokens, S.hidden, S.inter
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, M - 1], np.arange(3, M, max(1, M // 16))]))
    gq, uq = _stash_gu(rng, M, I)
    dh = synth.to_bf16_bits(rng.standard_normal((M, I)))
    gdg, gdu, gdgq, gduq = pb.pact_silu_mul_bwd_quant_nvfp4(G.dev_bf16(dh), G.dev_nvfp4(gq), G.dev_nvfp4(uq))
    yq, gamma, rstd = _rms_stash(rng, M, H)
    dy = synth.to_bf16_bits(rng.standard_normal((M, H)))
    C = synth.to_bf16_bits(rng.standard_normal((M, H)))
    gdx, gdxq = pb.pact_rmsnorm_bwd_nvfp4(G.dev_bf16(dy), G.dev_nvfp4(yq), G.dev_bf16(gamma),
                                          torch.from_numpy(rstd).cuda(), C=G.dev_bf16(C))
    torch.cuda.synchronize()
    sub = lambda q: oracle.NVFP4(q.codes[rows], q.scales[rows], q.d[rows])
    dg, du, dgq, duq = oracle.silu_mul_bwd_quant(dh[rows], sub(gq), sub(uq))
    np.testing.assert_array_equal(G.host_bits(gdg)[rows], dg)
    np.testing.assert_array_equal(G.host_bits(gdu)[rows], du)
    G.assert_nvfp4_equal(sub(G.host_nvfp4(gdgq)), dgq, "dgq")
    G.assert_nvfp4_equal(sub(G.host_nvfp4(gduq)), duq, "duq")
    dx, dxq = oracle.rmsnorm_bwd(dy[rows], sub(yq), gamma, rstd[rows], C[rows])
    np.testing.assert_array_equal(G.host_bits(gdx)[rows], dx)
    G.assert_nvfp4_equal(sub(G.host_nvfp4(gdxq)), dxq, "dxq")


def test_backward_empty():
    """Zero rows: nothing is launched and nothing is written (the C ABI called
    with valid buffers and rows = 0)."""
    import ctypes
    L = pb.lib()
    buf = torch.full((1, 32), 7.0, dtype=torch.bfloat16, device="cuda")
    dst = torch.full((1, 32), 3.0, dtype=torch.bfloat16, device="cuda")
    gam = torch.ones(32, dtype=torch.bfloat16, device="cuda")
    rst = torch.ones(4, device="cuda")
    q, out = pb.NVFP4Tensor.empty(1, 32), pb.NVFP4Tensor.empty(1, 32)
    out.row_scale.fill_(5.0)
    dq = pb.pact_nvfp4(q.codes.data_ptr(), q.scales.data_ptr(), q.row_scale.data_ptr(), 0, 32)
    do = pb.pact_nvfp4(out.codes.data_ptr(), out.scales.data_ptr(), out.row_scale.data_ptr(), 0, 32)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    assert L.pact_silu_mul_bwd_quant_nvfp4(ptr(buf), 32, ctypes.byref(dq), ctypes.byref(dq), 0, 32, ptr(dst),
                                           ptr(dst), 32, ctypes.byref(do), ctypes.byref(do), None) == 0
    assert L.pact_rmsnorm_bwd_nvfp4(ptr(buf), 32, ctypes.byref(dq), ptr(gam), ptr(rst), None, 32, 0, 32,
                                    ptr(dst), 32, ctypes.byref(do), None) == 0
    torch.cuda.synchronize()
    assert torch.all(dst == 3.0) and torch.all(out.row_scale == 5.0)
