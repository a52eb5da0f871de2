"""The forward GEMM entry point that allocates nothing
(pact_gemm_nvfp4_fwd_noalloc: its workspace is a library-owned device array
per GPU) against the existing entry point pact_gemm_nvfp4_fwd with a caller
workspace, on consecutive calls whose sizes shrink: bit-identical where the
same launch plan fits the array, within the GEMM tolerance where the K-split
partials do not fit and the call runs in one pass over K; the oracle checks
sampled rows of every call.  (simolm.com PACT blog, "Method": the NVFP4
forward GEMM with FP32 accumulation and the BF16 LoRA term.)"""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_gemm_amd import pact as pb
from nvfp4_gemm_amd import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _case(M, N, K, r, seed, with_c):
    li = synth.single_linear_inputs(M=M, N=N, K=K, r=max(r, 1), seed=seed, act="t4", outliers=True)
    rng = np.random.default_rng(seed + 1)
    C = synth.normal_bf16(rng, (M, N), 0.5) if with_c else None
    return li, C


def test_noalloc_forward_matches_existing_entry_point():
    scratch = pb.pact_noalloc_scratch_bytes()
    assert scratch == 32 << 20
    # a large call whose split-K partials exceed the array (one pass over K),
    # then smaller ones whose whole workspace fits (the same plan: bit-identical)
    cases = [(4096, 1536, 8960, 16, True), (1024, 2048, 2048, 16, False), (300, 528, 1040, 8, True),
             (96, 160, 256, 0, False)]
    for i, (M, N, K, r, with_c) in enumerate(cases):
        print(f"noalloc case {i}: M={M} N={N} K={K} r={r} C={with_c}", flush=True)
        li, C = _case(M, N, K, r, seed=100 + i, with_c=with_c)
        lora = pb.LoRA(G.dev_bf16(li.A[:r]), G.dev_bf16(li.B[:, :r]), li.s) if r else None
        X = G.dev_bf16(li.X)
        gf, _ = pb.pact_build_weight_layouts(G.dev_bf16(li.W))
        gxq = pb.pact_quantize_nvfp4(X)
        gC = G.dev_bf16(C) if with_c else None
        ref = pb.pact_gemm_nvfp4_fwd(gxq, gf, X=X, lora=lora, C=gC)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        pb.pact_gemm_nvfp4_fwd_noalloc(gxq, gf, X=X, lora=lora, C=gC, Y=Y)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        same_plan = pb.pact_gemm_workspace(M, N, K, r) <= scratch
        if same_plan:
            assert torch.equal(Y, ref), f"case {i}: differs from pact_gemm_nvfp4_fwd"
        else:
            G.check_gemm_tolerance(G.host_bits(Y), G.host_bits(ref), f"case {i} vs pact_gemm_nvfp4_fwd")
        rows = np.unique(np.concatenate([[0, M - 1], np.arange(3, M, max(1, M // 20))]))
        want = oracle.gemm_fwd(oracle.quantize_bf16(li.X), li.X, oracle.build_weight_layouts(li.W)[0],
                               li.A[:r] if r else None, li.B[:, :r] if r else None, li.s, C, rows=rows)
        G.check_gemm_tolerance(G.host_bits(Y)[rows], want, f"case {i} vs oracle")
        # a repeat call gives the same bits (nothing left over from earlier calls matters)
        Y2 = torch.empty_like(Y)
        pb.pact_gemm_nvfp4_fwd_noalloc(gxq, gf, X=X, lora=lora, C=gC, Y=Y2)
        torch.cuda.synchronize()
        assert torch.equal(Y, Y2)
