"""GPU parity of the kernel variants that the layer workloads do not select:
every (wavefronts per row, blocks per lane) shape of the five row kernels, and
the GEMM, LoRA-down and LoRA-gradient variants that the launch plans choose
only for other shapes (long K, K not a multiple of 64, rank-64 input
gradients at 2048 rows, rank-32 LoRA-down at 3072 rows, LoRA gradients of
ranks 32-64 and of wide outputs at 4096 rows).  Where a host-side plan
diagnostic exists, each case first asserts the variant it is meant to reach,
so that a plan change which leaves a variant untested fails here.  The bars
are the other tests' (simolm.com PACT blog, "Method": NVFP4 operands with
per-16 E4M3 scales, FP32 accumulation, BF16 adapters): quantized outputs and
BF16 results of the row kernels bit-exact, GEMMs within the GEMM tolerance,
LoRA gradients within their bound (tests/_gpu.py)."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_gemm_amd import pact as pb
from nvfp4_gemm_amd import synth
from tests import _gpu as G
from tests.test_gpu_layout_gemm import _run_pair
from tests.test_gpu_lora_grads import _case as grads_case

pytestmark = pytest.mark.gpu

# Row widths of 64, 100, 192, 200, 500, 700, 1000, 1500 and 2000 blocks of 16:
# together they select every launch shape of the five row kernels (several
# with a partly filled last chunk of 64 blocks).
WIDTHS = [1024, 1600, 3072, 3200, 8000, 11200, 16000, 24000, 32000]


def _rows(M, n=16, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, M - 1], rng.integers(0, M, n)])).astype(np.int64)


@pytest.mark.parametrize("cols", WIDTHS)
def test_row_kernel_shapes(cols):
    """Five rows (a ragged last row group where a workgroup holds four) through
    all five row kernels at one width: quantize, RMSNorm-quantize,
    SiLU-multiply-quantize, and the two backward kernels on the forward's own
    NVFP4 outputs."""
    rows = 5
    rng = np.random.default_rng(cols)
    x = synth.student_t_bf16(rng, (rows, cols), 3.0, 0.5)
    gq_x = pb.pact_quantize_nvfp4(G.dev_bf16(x))
    gamma = synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(cols))
    y, yq, rstd = oracle.rmsnorm_quant(x, gamma, 1e-5)
    gy, gyq, grstd = pb.pact_rmsnorm_quant_nvfp4(G.dev_bf16(x), G.dev_bf16(gamma), 1e-5)
    g = synth.student_t_bf16(rng, (rows, cols), 4.0, 1.5)
    u = synth.student_t_bf16(rng, (rows, cols), 4.0, 0.5)
    h, hq, gq, uq = oracle.silu_mul_quant(g, u)
    gh, ghq, ggq, guq = pb.pact_silu_mul_quant_nvfp4(G.dev_bf16(g), G.dev_bf16(u))
    dh = synth.to_bf16_bits(rng.standard_normal((rows, cols)))
    dg, du, dgq, duq = oracle.silu_mul_bwd_quant(dh, gq, uq)
    gdg, gdu, gdgq, gduq = pb.pact_silu_mul_bwd_quant_nvfp4(G.dev_bf16(dh), G.dev_nvfp4(gq), G.dev_nvfp4(uq))
    dy = synth.to_bf16_bits(rng.standard_normal((rows, cols)))
    C = synth.to_bf16_bits(rng.standard_normal((rows, cols)))
    dx, dxq = oracle.rmsnorm_bwd(dy, yq, gamma, rstd, C)
    gdx, gdxq = pb.pact_rmsnorm_bwd_nvfp4(G.dev_bf16(dy), G.dev_nvfp4(yq), G.dev_bf16(gamma),
                                          torch.from_numpy(rstd).cuda(), C=G.dev_bf16(C))
    torch.cuda.synchronize()
    G.assert_nvfp4_equal(gq_x, oracle.quantize_bf16(x), f"quantize {cols}")
    np.testing.assert_array_equal(grstd.cpu().numpy().view(np.uint32), rstd.view(np.uint32))
    np.testing.assert_array_equal(G.host_bits(gy), y)
    G.assert_nvfp4_equal(gyq, yq, f"rmsnorm yq {cols}")
    np.testing.assert_array_equal(G.host_bits(gh), h)
    G.assert_nvfp4_equal(ghq, hq, f"hq {cols}")
    G.assert_nvfp4_equal(ggq, gq, f"gq {cols}")
    G.assert_nvfp4_equal(guq, uq, f"uq {cols}")
    np.testing.assert_array_equal(G.host_bits(gdg), dg)
    np.testing.assert_array_equal(G.host_bits(gdu), du)
    G.assert_nvfp4_equal(gdgq, dgq, f"dgq {cols}")
    G.assert_nvfp4_equal(gduq, duq, f"duq {cols}")
    np.testing.assert_array_equal(G.host_bits(gdx), dx)
    G.assert_nvfp4_equal(gdxq, dxq, f"dxq {cols}")


@pytest.mark.parametrize("M,N,K,r,plan", [
    (4096, 4096, 12288, 16, (1, 1)),  # 256x256 with 4 wavefronts and register decode, whole K (long K)
    (4096, 2048, 24576, 16, (1, 2)),  # the same kernel with K split over two workgroups, separate LoRA-down
    (2048, 768, 1024, 16, (2, 4)),    # 256x128 tiles, K split four ways, LoRA-down fused into the split launch
    (256, 256, 96, 16, (2, 1)),       # 256x128 tiles on K = 96 (not a multiple of 64)
])
def test_gemm_kernel_variants(M, N, K, r, plan):
    """Forward plans asserted, then forward and input gradient (whose own
    plans differ) against the oracle on sampled rows."""
    assert pb.pact_debug_gemm_plan(M, N, K, r)[:2] == plan
    _run_pair(M, N, K, r, seed=M + K + r, with_c=True, rows=_rows(M) if M > 1024 else None)


def test_lora_down_gather_four_rank_groups():
    """Input gradient at 2048 rows, r = 64: the LoRA-down kernel that gathers
    the strided rank rows, with four rank groups."""
    M, N, K, r = 2048, 1024, 2048, 64
    assert pb.pact_debug_lora_down_plan(M, K, N, r, dgrad=True) == (4, [(4, 1, 16)])
    _run_pair(M, N, K, r, seed=73, with_c=False, rows=_rows(M, seed=1))


def test_lora_down_pipe_two_rank_groups_one_row_group():
    """Forward at 3072 rows, r = 32: the pipelined LoRA-down with two rank
    groups and one row group per wavefront (two row groups start at 4096)."""
    M, N, K, r = 3072, 2048, 2048, 32
    assert pb.pact_debug_lora_down_plan(M, N, K, r) == (2, [(2, 1, 8)])
    _run_pair(M, N, K, r, seed=79, with_c=True, rows=_rows(M, seed=2))


@pytest.mark.parametrize("M,N,K,r", [
    (3072, 1024, 2048, 32),  # NVFP4 LoRA-down: 2 rank groups, 1 row group per wavefront
    (4096, 4096, 1024, 48),  # 3 rank groups, 2 row groups; dB over 4096 columns in 256-column blocks, 2 rank tiles
    (4096, 8192, 512, 64),   # 4 rank groups, 2 row groups (4 wavefronts); 256-column blocks, 2 rank tiles
    (4096, 4096, 256, 16),   # 256-column blocks, 1 rank tile
])
def test_lora_grads_variants(M, N, K, r):
    """LoRA weight gradients in the launch shapes the layer workloads (ranks
    16 and 32, outputs up to 3072 wide at 8192 rows or 8192 wide at 1024)
    do not select."""
    xq, dY, A, B = grads_case(M, N, K, r, seed=M + N + r)
    dA, dB = oracle.lora_grads(xq, dY, A, B, 2.0)
    gdA, gdB = pb.pact_lora_grads_nvfp4(G.dev_nvfp4(xq), G.dev_bf16(dY),
                                        pb.LoRA(G.dev_bf16(A), G.dev_bf16(B), 2.0))
    torch.cuda.synchronize()
    G.check_lora_grads(gdA, gdB, dA, dB, f"{M}x{N}x{K} r{r}")
