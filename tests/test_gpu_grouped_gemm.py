"""GPU parity of the grouped forward GEMM (q, k, v or gate, up as one GEMM over
their concatenated weight rows with a block-diagonal BF16 LoRA term; simolm.com
PACT blog, "Method": the NVFP4 GEMM and LoRA term of each projection) against
the oracle's per-projection forward, within the GEMM tolerance
(|d| <= 2 ulp_bf16 + 1e-3 max_row|ref|, relative Frobenius <= 4e-3)."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_gemm_amd import pact as pb
from nvfp4_gemm_amd import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _case(M, K, rows, r, seed, rows_sample=None):
    rng = np.random.default_rng(seed)
    X = synth.student_t_bf16(rng, (M, K), 4.0, 0.5)
    xq = oracle.quantize_bf16(X)
    Ws = [synth.weight_bf16(rng, n, K) for n in rows]
    As = [synth.normal_bf16(rng, (r, K), 0.02) for _ in rows] if r else [None] * len(rows)
    Bs = [synth.normal_bf16(rng, (n, r), 0.01) for n in rows] if r else [None] * len(rows)
    s = 2.0
    refs = []
    for W, A, B in zip(Ws, As, Bs):
        f, _ = oracle.build_weight_layouts(W)
        refs.append(oracle.gemm_fwd(xq, X, f, A, B, s, rows=rows_sample))
    gx, gxq = G.dev_bf16(X), G.dev_nvfp4(xq)
    gW = pb.NVFP4Tensor.cat_rows([pb.pact_build_weight_layouts(G.dev_bf16(W))[0] for W in Ws])
    loras = [pb.LoRA(G.dev_bf16(A), G.dev_bf16(B), s) for A, B in zip(As, Bs)] if r else None
    Y = pb.pact_gemm_nvfp4_fwd_grouped(gxq, gW, rows, X=gx, loras=loras)
    torch.cuda.synchronize()
    Yh = G.host_bits(Y)
    if rows_sample is not None:
        Yh = Yh[rows_sample]
    c = 0
    for g, n in enumerate(rows):
        G.check_gemm_tolerance(np.ascontiguousarray(Yh[:, c:c + n]), refs[g], f"group {g} of {rows}")
        c += n
    return Y, gxq, gW, gx, loras


@pytest.mark.parametrize("M,K,rows,r", [
    (64, 256, [256, 64, 64], 16),        # q, k, v shaped
    (100, 512, [512, 128, 128], 8),       # ragged M
    (256, 512, [1024, 1024], 16),         # gate, up shaped
    (96, 256, [96, 32, 160, 64], 32),     # four groups, boundaries inside 256-column tiles
    (128, 1024, [512, 128, 128], 32),     # 96 ranks: LoRA-down in two passes
    (64, 256, [256, 64, 64], 0),          # frozen only
    (100, 4096, [128, 64, 64], 16),       # K split across workgroups
])
def test_grouped_fwd_parity(M, K, rows, r):
    _case(M, K, rows, r, seed=M + K + sum(rows) + r)


def test_grouped_fwd_layer_size_sampled_rows():
    """q, k, v of the Llama-1B-shaped layer (M = 1024, H = 2048, KV = 512, r =
    16) as bench.py runs them, on sampled rows."""
    S = synth.LAYERS["llama1b_layer"]
    rows = np.unique(np.random.default_rng(5).integers(0, S.tokens, 24)).astype(np.int64)
    _case(S.tokens, S.hidden, [S.hidden, S.kv, S.kv], S.rank, seed=9, rows_sample=rows)


def test_grouped_equals_separate_with_zero_B():
    """B = 0 in every group reproduces the frozen-only grouped output bit for
    bit (the LoRA term adds exact zeros)."""
    M, K, rows, r = 64, 256, [256, 64, 64], 16
    rng = np.random.default_rng(1)
    X = synth.student_t_bf16(rng, (M, K), 4.0, 0.5)
    Ws = [synth.weight_bf16(rng, n, K) for n in rows]
    gx, gxq = G.dev_bf16(X), pb.pact_quantize_nvfp4(G.dev_bf16(X))
    gW = pb.NVFP4Tensor.cat_rows([pb.pact_build_weight_layouts(G.dev_bf16(W))[0] for W in Ws])
    loras = [pb.LoRA(G.dev_bf16(synth.normal_bf16(rng, (r, K), 0.02)),
                     torch.zeros((n, r), dtype=torch.bfloat16, device="cuda"), 2.0) for n in rows]
    Y0 = pb.pact_gemm_nvfp4_fwd_grouped(gxq, gW, rows, X=gx, loras=None)
    Y1 = pb.pact_gemm_nvfp4_fwd_grouped(gxq, gW, rows, X=gx, loras=loras)
    torch.cuda.synchronize()
    assert torch.equal(Y0.float(), Y1.float())


def test_grouped_validation():
    M, K = 32, 256
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    xq = pb.pact_quantize_nvfp4(X)
    W = pb.NVFP4Tensor.empty(96, K)
    with pytest.raises(RuntimeError):
        pb.pact_gemm_nvfp4_fwd_grouped(xq, W, [64, 16, 16])   # groups must be multiples of 32
    with pytest.raises(RuntimeError):
        pb.pact_gemm_nvfp4_fwd_grouped(xq, W, [64, 64])       # rows do not add up


def test_grouped_fwd_strided_x_and_y():
    """X read through a leading dimension > K and Y written into a column range
    of a wider buffer; columns outside it are left untouched."""
    M, K, rows, r = 96, 256, [128, 64], 16
    rng = np.random.default_rng(4)
    Xh = synth.student_t_bf16(rng, (M, K), 4.0, 0.5)
    xq = oracle.quantize_bf16(Xh)
    Ws = [synth.weight_bf16(rng, n, K) for n in rows]
    As = [synth.normal_bf16(rng, (r, K), 0.02) for _ in rows]
    Bs = [synth.normal_bf16(rng, (n, r), 0.01) for n in rows]
    refs = [oracle.gemm_fwd(xq, Xh, oracle.build_weight_layouts(W)[0], A, B, 2.0) for W, A, B in zip(Ws, As, Bs)]
    Xw = torch.zeros((M, K + 64), dtype=torch.bfloat16, device="cuda")
    Xw[:, 64:] = G.dev_bf16(Xh)
    gW = pb.NVFP4Tensor.cat_rows([pb.pact_build_weight_layouts(G.dev_bf16(W))[0] for W in Ws])
    loras = [pb.LoRA(G.dev_bf16(A), G.dev_bf16(B), 2.0) for A, B in zip(As, Bs)]
    Yw = torch.full((M, sum(rows) + 64), 7.0, dtype=torch.bfloat16, device="cuda")
    pb.pact_gemm_nvfp4_fwd_grouped(G.dev_nvfp4(xq), gW, rows, X=Xw[:, 64:], loras=loras, Y=Yw[:, 32:32 + sum(rows)])
    torch.cuda.synchronize()
    Yh = G.host_bits(Yw)
    G.check_gemm_tolerance(np.ascontiguousarray(Yh[:, 32:32 + rows[0]]), refs[0], "group 0 strided")
    G.check_gemm_tolerance(np.ascontiguousarray(Yh[:, 32 + rows[0]:32 + sum(rows)]), refs[1], "group 1 strided")
    assert torch.all(Yw[:, :32] == 7.0) and torch.all(Yw[:, 32 + sum(rows):] == 7.0)
