"""GPU parity of the LoRA weight gradients on the NVFP4 stash (simolm.com PACT
blog, section "Method": activations kept for backward are NVFP4 copies, the
adapters stay BF16; kongchang.com PEFT explainer: the update B A x) against
the oracle: dB = dY^T T^, dA = T'^T X^.  The GPU sums over the tokens in FP32
(fixed order), the oracle in binary64.  The rank-r intermediates T^, T' are
FP32 sums (over K or N, up to 8192 terms) rounded to BF16, and the GPU's MFMA
summation order differs from the oracle's sequential one, so an entry may round
to the neighbouring BF16 value; the gradients inherit up to one BF16 ulp on
those terms, and such a term moves every entry of its rank together (row j of
dA, column j of dB).  Bound, in the GEMM outputs' form with "row" read as "the
entries of one rank": per element |d| <= 2 ulp_bf16(|ref|) + 1e-3 max_j|ref|,
and a relative Frobenius error <= 4e-3 (tests/_gpu.py check_lora_grads)."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_gemm_amd import pact as pb
from nvfp4_gemm_amd import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _case(M, N, K, r, seed, nu=4.0):
    rng = np.random.default_rng(seed)
    x = synth.to_bf16_bits(rng.standard_t(nu, (M, K)) * 0.5)
    xq = oracle.quantize_bf16(x)
    dY = synth.to_bf16_bits(rng.standard_normal((M, N)))
    A = synth.to_bf16_bits(0.02 * rng.standard_normal((r, K)))
    B = synth.to_bf16_bits(0.01 * rng.standard_normal((N, r)))
    return xq, dY, A, B


def _check(gdA, gdB, dA, dB, what):
    G.check_lora_grads(gdA, gdB, dA, dB, what)


@pytest.mark.parametrize("M,N,K,r", [(16, 16, 16, 1), (40, 48, 64, 8), (100, 528, 272, 16), (257, 1024, 512, 32),
                                     (64, 96, 128, 40), (1024, 2048, 2048, 16), (2048, 512, 3072, 64)])
def test_lora_grads_parity(M, N, K, r):
    xq, dY, A, B = _case(M, N, K, r, seed=M + N + K + r)
    dA, dB = oracle.lora_grads(xq, dY, A, B, 2.0)
    lora = pb.LoRA(G.dev_bf16(A), G.dev_bf16(B), 2.0)
    gxq, gdY = G.dev_nvfp4(xq), G.dev_bf16(dY)
    gdA, gdB = pb.pact_lora_grads_nvfp4(gxq, gdY, lora)
    gdA2, gdB2 = pb.pact_lora_grads_nvfp4(gxq, gdY, lora)
    torch.cuda.synchronize()
    _check(gdA, gdB, dA, dB, f"{M}x{N}x{K} r{r}")
    assert torch.equal(gdA, gdA2) and torch.equal(gdB, gdB2)  # deterministic


@pytest.mark.parametrize("shape,proj", [("llama1b_layer", "gate"), ("llama3b_layer", "down")])
def test_lora_grads_layer_sizes(shape, proj):
    """A projection of the layer workloads at full size, in the launch
    configuration bench.py uses."""
    S = synth.LAYERS[shape]
    N, K = S.projections()[proj]
    xq, dY, A, B = _case(S.tokens, N, K, S.rank, seed=3, nu=S.act_nu)
    dA, dB = oracle.lora_grads(xq, dY, A, B, S.lora_scale)
    gdA, gdB = pb.pact_lora_grads_nvfp4(G.dev_nvfp4(xq), G.dev_bf16(dY),
                                        pb.LoRA(G.dev_bf16(A), G.dev_bf16(B), S.lora_scale))
    torch.cuda.synchronize()
    _check(gdA, gdB, dA, dB, f"{shape} {proj}")


def test_lora_grads_no_tokens():
    q = pb.NVFP4Tensor.empty(1, 32)
    xq = pb.NVFP4Tensor(q.codes[:0], q.scales[:0], q.row_scale[:0])
    import ctypes
    L = pb.lib()
    A = torch.ones((4, 32), dtype=torch.bfloat16, device="cuda")
    B = torch.ones((16, 4), dtype=torch.bfloat16, device="cuda")
    dY = torch.ones((1, 16), dtype=torch.bfloat16, device="cuda")
    dA = torch.full((4, 32), 9.0, device="cuda")
    dB = torch.full((16, 4), 9.0, device="cuda")
    desc = pb.pact_nvfp4(q.codes.data_ptr(), q.scales.data_ptr(), q.row_scale.data_ptr(), 0, 32)
    lo = pb.pact_lora(A.data_ptr(), B.data_ptr(), 4, 2.0)
    assert L.pact_lora_grads_nvfp4(ctypes.byref(desc), ctypes.c_void_p(dY.data_ptr()), 16, 16, ctypes.byref(lo),
                                   None, ctypes.c_void_p(dA.data_ptr()), ctypes.c_void_p(dB.data_ptr()), None, 0,
                                   None) == 0
    torch.cuda.synchronize()
    assert torch.all(dA == 0) and torch.all(dB == 0)
    del xq


def test_lora_grads_strided_dy():
    """dY as a column slice of a wider buffer (leading dimension > N), as the
    layer bench passes the k and v gradients."""
    M, N, K, r = 300, 128, 256, 16
    xq, dY, A, B = _case(M, N, K, r, seed=77)
    dA, dB = oracle.lora_grads(xq, dY, A, B, 2.0)
    wide = torch.zeros((M, N + 96), dtype=torch.bfloat16, device="cuda")
    wide[:, 32:32 + N] = G.dev_bf16(dY)
    lora = pb.LoRA(G.dev_bf16(A), G.dev_bf16(B), 2.0)
    gdA, gdB = pb.pact_lora_grads_nvfp4(G.dev_nvfp4(xq), wide[:, 32:32 + N], lora)
    torch.cuda.synchronize()
    _check(gdA, gdB, dA, dB, "strided dY")


@pytest.mark.parametrize("M,N,K,r", [(300, 512, 256, 16), (1024, 2048, 8192, 16), (4096, 1536, 1536, 16)])
def test_lora_grads_with_dgrad_t(M, N, K, r):
    """T' = bf16(s dY B) taken from the workspace of the input-gradient GEMM
    of the same dY and adapter (its LoRA-down product) instead of computed
    again: the gradients meet the same bound against the oracle."""
    xq, dY, A, B = _case(M, N, K, r, seed=M + 5 * N + K)
    dA, dB = oracle.lora_grads(xq, dY, A, B, 2.0)
    lora = pb.LoRA(G.dev_bf16(A), G.dev_bf16(B), 2.0)
    gdY = G.dev_bf16(dY)
    W = synth.weight_bf16(np.random.default_rng(M), N, K)
    _, wb = pb.pact_build_weight_layouts(G.dev_bf16(W))
    ws = torch.empty((pb.pact_gemm_workspace(M, N, K, r),), dtype=torch.uint8, device="cuda")
    pb.pact_gemm_nvfp4_dgrad(pb.pact_quantize_nvfp4(gdY), wb, dY=gdY, lora=lora, ws=ws)
    gdA, gdB = pb.pact_lora_grads_nvfp4(G.dev_nvfp4(xq), gdY, lora, T_dy=ws)
    torch.cuda.synchronize()
    _check(gdA, gdB, dA, dB, f"{M}x{N}x{K} with the GEMM's T'")
