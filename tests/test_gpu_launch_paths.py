"""GPU parity of the GEMM launch variants that the layer workloads take at
large M, each asserted through the host-side plan diagnostics before it runs,
against the oracle on sampled rows within the GEMM tolerance
(|d| <= 2 ulp_bf16 + 1e-3 max_row|ref|, relative Frobenius <= 4e-3).
(simolm.com PACT blog, "Method": one NVFP4 GEMM for forward and input
gradient of every projection, FP32 accumulation, BF16 adapters.)

Variants covered here:
  * the 256 x 256 single-decode kernel with K split across workgroups and the
    LoRA-down fused into the same launch (Qwen-shaped down forward), and its
    split input gradient (Qwen-shaped gate/up input gradient);
  * the pipelined LoRA-down with two row groups per wavefront and 2, 3 or 4
    rank groups, in one or two passes over the ranks (grouped q|k|v and
    gate|up of the 3B-shaped layer at r = 32 and r = 16, single forward at
    r = 32), and the input gradient's transposed rank operand at M = 8192;
  * a LoRA scale that is not a power of two.
"""
import numpy as np
import pytest

from nvfp4_gemm_amd import pact as pb
from tests.test_gpu_grouped_gemm import _case as grouped_case
from tests.test_gpu_layout_gemm import _run_pair

pytestmark = pytest.mark.gpu


def _rows(M, n=24, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, M - 1], rng.integers(0, M, n)])).astype(np.int64)


def test_split_k_single_decode_fused_down_forward():
    """Qwen-shaped down projection forward: 4096 x 1536 over K = 8960, r = 16.
    Plan: kernel 0 (256 x 256 single decode) with K split 4 ways and the
    LoRA-down fused into the split-K launch."""
    M, N, K, r = 4096, 1536, 8960, 16
    assert pb.pact_debug_gemm_plan(M, N, K, r) == (0, 4, True)
    assert pb.pact_debug_lora_down_plan(M, N, K, r)[0] == 1
    _run_pair(M, N, K, r, seed=31, with_c=True, rows=_rows(M))


def test_split_k_single_decode_dgrad():
    """Qwen-shaped gate/up input gradient: output 4096 x 1536 contracted over
    N = 8960, r = 16.  Plan: kernel 0 with K split 2 ways; the LoRA-down runs
    after transposing the strided rank operand B."""
    M, N, K, r = 4096, 8960, 1536, 16
    assert pb.pact_debug_gemm_plan(M, K, N, r, dgrad=True)[:2] == (0, 2)
    assert pb.pact_debug_lora_down_plan(M, K, N, r, dgrad=True) == (3, [(1, 1, 8)])
    _run_pair(M, N, K, r, seed=37, with_c=True, rows=_rows(M, seed=1))


@pytest.mark.parametrize("rows,r,passes", [
    ([3072, 1024, 1024], 32, [(4, 2, 4), (2, 2, 8)]),   # 3B-shaped q|k|v, r = 32: 96 ranks, two passes
    ([8192, 8192], 32, [(4, 2, 4)]),                    # 3B-shaped gate|up, r = 32: 64 ranks
    ([3072, 1024, 1024], 16, [(3, 2, 8)]),              # 3B-shaped q|k|v, r = 16: 48 ranks
])
def test_grouped_fwd_pipelined_down_large_m(rows, r, passes):
    """Grouped forward at M = 8192, K = 3072 (the 3B-shaped layer and stack)
    on sampled rows; the LoRA-down runs the pipelined kernel with two row
    groups per wavefront in the asserted passes."""
    M, K = 8192, 3072
    ng = len(rows)
    assert pb.pact_debug_gemm_plan(M, sum(rows), K, ng * r)[1] == 1
    assert pb.pact_debug_lora_down_plan(M, sum(rows), K, r, ngroups=ng) == (2, passes)
    grouped_case(M, K, rows, r, seed=41 + r + ng, rows_sample=_rows(M, seed=2))


def test_single_fwd_pipelined_down_large_m():
    """Single forward and input gradient at M = 8192, 3072 x 3072, r = 32:
    the pipelined LoRA-down with two row groups and two rank groups per
    wavefront; the input gradient transposes B first."""
    M, N, K, r = 8192, 3072, 3072, 32
    assert pb.pact_debug_lora_down_plan(M, N, K, r) == (2, [(2, 2, 8)])
    assert pb.pact_debug_lora_down_plan(M, K, N, r, dgrad=True) == (3, [(2, 2, 8)])
    _run_pair(M, N, K, r, seed=43, with_c=True, rows=_rows(M, seed=3))


@pytest.mark.parametrize("M,N,K,r,s", [(300, 528, 1040, 16, 0.7), (1024, 2048, 8192, 16, 1.0 / 3.0),
                                       (4096, 1536, 8960, 16, 0.37)])
def test_non_power_of_two_lora_scale(M, N, K, r, s):
    """The GPU rounds T = bf16(s X A^T) with s inside, the oracle rounds
    bf16(X A^T) and scales the sum; for s not a power of two the two differ by
    one rounding of the rank-r term, which stays inside the GEMM tolerance."""
    rows = _rows(M, seed=4) if M > 1024 else None
    _run_pair(M, N, K, r, seed=47, with_c=False, rows=rows, s=s)


def test_column_split_plan_single():
    """8192 x 3072 over K = 8192 (3B-shaped down forward, gate/up input
    gradient): 384 tiles of 256 x 256 are 1.5 rounds of the CUs, so the plan
    runs columns [0, 2048) with the 256 x 256 kernel (exactly one round) and
    the rest with 128 x 256 tiles as a second launch; both directions on
    sampled rows."""
    M, N, K, r = 8192, 3072, 8192, 16
    assert pb.pact_debug_gemm_plan_columns(M, N, K, r) == (2048, 3)
    assert pb.pact_debug_gemm_plan_columns(M, N, K, r, dgrad=True) == (2048, 3)
    _run_pair(M, N, K, r, seed=53, with_c=True, rows=_rows(M, seed=5))
    # the transposed direction of the same pair: output [M][K] over N
    _run_pair(M, K, N, r, seed=59, with_c=True, rows=_rows(M, seed=6))


@pytest.mark.parametrize("M,K,rows,r,n1", [
    (4096, 1536, [8960, 8960], 16, 16384),          # Qwen-shaped gate|up: the split falls inside group 1
    (8192, 3072, [3072, 1024, 1024], 16, 4096),     # 3B-shaped q|k|v: the split falls on a group boundary
])
def test_column_split_plan_grouped(M, K, rows, r, n1):
    """Grouped forward whose plan splits the output columns across two
    launches: the second launch's group boundaries shift with its columns."""
    ng = len(rows)
    assert pb.pact_debug_gemm_plan_columns(M, sum(rows), K, ng * r)[0] == n1
    grouped_case(M, K, rows, r, seed=61 + ng, rows_sample=_rows(M, seed=7))
