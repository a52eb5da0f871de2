"""The data flow captured as a HIP graph (the way bench.py times a step)
reproduces the eager results bit for bit on every replay."""
import numpy as np
import pytest

from nvfp4_gemm_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    from nvfp4_gemm_amd import pact as pb
    from tests import _gpu as G

    M, N, K, r = 4096, 4096, 512, 16   # the forward GEMM takes the 256 x 256 kernel
    li = synth.single_linear_inputs(M=M, N=N, K=K, r=r, seed=21, act="t4", outliers=True)
    X, dY = G.dev_bf16(li.X), G.dev_bf16(li.dY)
    gamma = G.dev_bf16(synth.to_bf16_bits(1.0 + 0.1 * np.random.default_rng(5).standard_normal(K)))
    wf, wb = pb.pact_build_weight_layouts(G.dev_bf16(li.W))
    lora = pb.LoRA(G.dev_bf16(li.A), G.dev_bf16(li.B), li.s)
    E = lambda a, b: torch.empty((a, b), dtype=torch.bfloat16, device="cuda")
    n, nq, rstd = E(M, K), pb.NVFP4Tensor.empty(M, K), torch.empty(M, device="cuda")
    Y, h, hq = E(M, N), E(M, N), pb.NVFP4Tensor.empty(M, N)
    gq, uq = pb.NVFP4Tensor.empty(M, N), pb.NVFP4Tensor.empty(M, N)
    dyq, dX = pb.NVFP4Tensor.empty(M, N), E(M, K)
    ws = torch.empty((max(pb.pact_gemm_workspace(M, N, K, r), 16),), dtype=torch.uint8, device="cuda")

    def step():
        pb.pact_rmsnorm_quant_nvfp4(X, gamma, 1e-5, n, nq, rstd)
        pb.pact_gemm_nvfp4_fwd(nq, wf, X=n, lora=lora, Y=Y, ws=ws)
        pb.pact_silu_mul_quant_nvfp4(Y, Y, h, hq, gq, uq)
        pb.pact_quantize_nvfp4(dY, dyq)
        pb.pact_gemm_nvfp4_dgrad(dyq, wb, dY=dY, lora=lora, C=X, dX=dX, ws=ws)

    outs = [n, rstd, Y, h, dX] + [t for q in (nq, hq, gq, uq, dyq) for t in (q.codes, q.scales, q.row_scale)]
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in outs:
            t.zero_()                       # eager work between replays
        pb.pact_quantize_nvfp4(X, pb.NVFP4Tensor.empty(M, K))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, r0) in enumerate(zip(outs, ref)):
            assert torch.equal(t.view(torch.uint8), r0.view(torch.uint8)), f"replay {rep}: output {i} differs"
