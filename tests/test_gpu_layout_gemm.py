"""GPU parity of the cached weight layouts (bit-exact) and of the NVFP4 GEMMs
with the BF16 LoRA term (within |d| <= 2 ulp_bf16 + 1e-3 max_row|ref| and a
relative Frobenius error <= 4e-3) against the oracle.  (simolm.com PACT blog,
"Method": NVFP4 GEMMs forward and input-gradient, FP32 accumulate, BF16 out;
cached forward/backward layouts; BF16 adapters.)"""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_gemm_amd import pact as pb
from nvfp4_gemm_amd import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(16, 16), (64, 96), (48, 80), (80, 272), (512, 2048),
                                 (2048, 512), (1024, 3072)])
def test_weight_layouts_parity(N, K):
    rng = np.random.default_rng(N + K)
    W = synth.weight_bf16(rng, N, K)
    f, b = oracle.build_weight_layouts(W)
    gf, gb = pb.pact_build_weight_layouts(G.dev_bf16(W))
    gf2, gb2 = pb.pact_build_weight_layouts(W_fwd_in=G.dev_nvfp4(f))
    torch.cuda.synchronize()
    G.assert_nvfp4_equal(gf, f, "W_fwd")
    G.assert_nvfp4_equal(gb, b, "W_bwd")
    G.assert_nvfp4_equal(gf2, f, "W_fwd copy")
    G.assert_nvfp4_equal(gb2, b, "W_bwd from given forward layout")


def _lora(li, r):
    if r == 0:
        return None, None, None
    return li.A[:r], li.B[:, :r], pb.LoRA(G.dev_bf16(li.A[:r]), G.dev_bf16(li.B[:, :r]), li.s)


def _run_pair(M, N, K, r, seed, with_c, act="t4", rows=None, s=2.0):
    li = synth.single_linear_inputs(M=M, N=N, K=K, r=max(r, 1), s=s, seed=seed, act=act, outliers=True)
    A, B, lora = _lora(li, r)
    rng = np.random.default_rng(seed + 1)
    C = synth.normal_bf16(rng, (M, N), 0.5) if with_c else None
    Cd = synth.normal_bf16(rng, (M, K), 0.5) if with_c else None
    xq = oracle.quantize_bf16(li.X)
    f, b = oracle.build_weight_layouts(li.W)
    dyq = oracle.quantize_bf16(li.dY)
    Y = oracle.gemm_fwd(xq, li.X, f, A, B, li.s, C, rows=rows)
    dX = oracle.gemm_dgrad(dyq, li.dY, b, A, B, li.s, Cd, rows=rows)
    gf, gb = pb.pact_build_weight_layouts(G.dev_bf16(li.W))
    gxq = pb.pact_quantize_nvfp4(G.dev_bf16(li.X))
    gdyq = pb.pact_quantize_nvfp4(G.dev_bf16(li.dY))
    gY = pb.pact_gemm_nvfp4_fwd(gxq, gf, X=G.dev_bf16(li.X), lora=lora,
                                C=G.dev_bf16(C) if with_c else None)
    gdX = pb.pact_gemm_nvfp4_dgrad(gdyq, gb, dY=G.dev_bf16(li.dY), lora=lora,
                                   C=G.dev_bf16(Cd) if with_c else None)
    torch.cuda.synchronize()
    G.assert_nvfp4_equal(gxq, xq, "Xq")
    gYh, gdXh = G.host_bits(gY), G.host_bits(gdX)
    if rows is not None:
        gYh, gdXh = gYh[rows], gdXh[rows]
    G.check_gemm_tolerance(gYh, Y, f"fwd {M}x{N}x{K} r{r}")
    G.check_gemm_tolerance(gdXh, dX, f"dgrad {M}x{N}x{K} r{r}")
    return li, gY, gdX


@pytest.mark.parametrize("M,N,K,r,with_c", [
    (1, 16, 16, 0, False), (5, 48, 32, 3, True), (64, 64, 128, 8, False),
    (130, 208, 272, 16, True), (300, 528, 1040, 32, False), (257, 1024, 512, 8, True),
    (64, 1552, 208, 5, False)])
def test_gemm_small_full(M, N, K, r, with_c):
    _run_pair(M, N, K, r, seed=M + N + K + r, with_c=with_c)


def test_single_linear_workload_full():
    """The single NVFP4 LoRA linear workload in full: X [256,512], W [1024,512],
    r = 8, s = 2, dY [256,1024], seed 0, N(0,1) activations."""
    li = synth.single_linear_inputs(**{k: v for k, v in synth.SINGLE_LINEAR.items()
                                       if k in ("M", "N", "K", "r", "seed")})
    xq = oracle.quantize_bf16(li.X)
    f, b = oracle.build_weight_layouts(li.W)
    dyq = oracle.quantize_bf16(li.dY)
    Y = oracle.gemm_fwd(xq, li.X, f, li.A, li.B, li.s)
    dX = oracle.gemm_dgrad(dyq, li.dY, b, li.A, li.B, li.s)
    lora = pb.LoRA(G.dev_bf16(li.A), G.dev_bf16(li.B), li.s)
    gf, gb = pb.pact_build_weight_layouts(G.dev_bf16(li.W))
    gY = pb.pact_gemm_nvfp4_fwd(pb.pact_quantize_nvfp4(G.dev_bf16(li.X)), gf, X=G.dev_bf16(li.X), lora=lora)
    gdX = pb.pact_gemm_nvfp4_dgrad(pb.pact_quantize_nvfp4(G.dev_bf16(li.dY)), gb, dY=G.dev_bf16(li.dY),
                                   lora=lora)
    torch.cuda.synchronize()
    G.assert_nvfp4_equal(gf, f, "W_fwd")
    G.assert_nvfp4_equal(gb, b, "W_bwd")
    G.check_gemm_tolerance(G.host_bits(gY), Y, "fwd")
    G.check_gemm_tolerance(G.host_bits(gdX), dX, "dgrad")


@pytest.mark.parametrize("M,N,K,r", [(1024, 2048, 2048, 16), (1024, 8192, 2048, 16),
                                     (2048, 3072, 8192, 32), (4096, 256, 1536, 16),
                                     (2048, 6144, 512, 16), (2304, 6160, 528, 8),
                                     (4096, 2048, 4096, 16), (4500, 4208, 576, 8)])
def test_gemm_layer_sizes_sampled_rows(M, N, K, r):
    """Projection shapes of the layer workloads in the kernel's real launch
    configuration; the oracle checks a sample of rows (first, last, strided)."""
    rows = np.unique(np.concatenate([[0, 1, M - 1], np.arange(7, M, max(1, M // 24))]))
    _run_pair(M, N, K, r, seed=3, with_c=True, rows=rows)


@pytest.mark.parametrize("M,N,K,r", [(1024, 512, 2048, 16), (1024, 2048, 8192, 16), (1000, 528, 2048, 8),
                                     (256, 512, 1024, 8), (1000, 528, 2048, 5), (1024, 512, 2048, 48)])
def test_gemm_split_k(M, N, K, r):
    """Shapes whose launch plan splits K across workgroups (FP32 partials
    summed in split order by a second kernel), including ragged M and N and
    ranks that are not multiples of 8 or exceed 32."""
    assert max(pb.pact_debug_gemm_plan(M, N, K, r)[1], pb.pact_debug_gemm_plan(M, K, N, r, True)[1]) > 1
    rows = np.unique(np.concatenate([[0, 1, M - 1], np.arange(5, M, max(1, M // 24))]))
    _run_pair(M, N, K, r, seed=17, with_c=True, rows=rows)


def test_gemm_split_k_workspace_fallback():
    """A workspace holding only the LoRA-down product runs the GEMM in one
    pass; both paths meet the tolerance and each is deterministic."""
    M, N, K, r = 1024, 512, 2048, 16
    assert pb.pact_debug_gemm_plan(M, N, K, r)[1] > 1
    li = synth.single_linear_inputs(M=M, N=N, K=K, r=r, seed=23, act="t4", outliers=True)
    A, B, lora = _lora(li, r)
    rows = np.unique(np.concatenate([[0, M - 1], np.arange(3, M, 41)]))
    xq = oracle.quantize_bf16(li.X)
    f, _ = oracle.build_weight_layouts(li.W)
    Y = oracle.gemm_fwd(xq, li.X, f, A, B, li.s, None, rows=rows)
    gf, _ = pb.pact_build_weight_layouts(G.dev_bf16(li.W))
    gxq = pb.pact_quantize_nvfp4(G.dev_bf16(li.X))
    X = G.dev_bf16(li.X)
    full = torch.empty((pb.pact_gemm_workspace(M, N, K, r),), dtype=torch.uint8, device="cuda")
    small = torch.empty((M * 16 * 2,), dtype=torch.uint8, device="cuda")  # the [M][16] BF16 product only
    assert small.numel() < full.numel()
    outs = [pb.pact_gemm_nvfp4_fwd(gxq, gf, X=X, lora=lora, ws=w) for w in (full, small, full, small)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[3])
    for o, name in ((outs[0], "split"), (outs[1], "one pass")):
        G.check_gemm_tolerance(G.host_bits(o)[rows], Y, f"fwd {name}")


def test_lora_identity_and_alias():
    """B = 0 reproduces the frozen-only output; C may alias Y."""
    M, N, K, r = 96, 160, 256, 16
    li = synth.single_linear_inputs(M=M, N=N, K=K, r=r, seed=11)
    gf, gb = pb.pact_build_weight_layouts(G.dev_bf16(li.W))
    xq = pb.pact_quantize_nvfp4(G.dev_bf16(li.X))
    X = G.dev_bf16(li.X)
    y0 = pb.pact_gemm_nvfp4_fwd(xq, gf)
    zero = pb.LoRA(G.dev_bf16(li.A), torch.zeros((N, r), dtype=torch.bfloat16, device="cuda"), li.s)
    yb0 = pb.pact_gemm_nvfp4_fwd(xq, gf, X=X, lora=zero)
    c = G.dev_bf16(synth.normal_bf16(np.random.default_rng(2), (M, N), 1.0))
    ref_c = pb.pact_gemm_nvfp4_fwd(xq, gf, C=c.clone())
    alias = c.clone()
    pb.pact_gemm_nvfp4_fwd(xq, gf, C=alias, Y=alias)
    y0b = pb.pact_gemm_nvfp4_fwd(xq, gf)
    torch.cuda.synchronize()
    assert torch.equal(y0.float(), yb0.float())
    assert torch.equal(ref_c, alias)
    assert torch.equal(y0, y0b)  # deterministic
