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


def test_graph_replay_grouped_grads_adamw():
    """Grouped forward, LoRA weight gradients (side workgroups, split partials)
    and the AdamW step captured in one graph: every replay, with eager work in
    between, equals the eager run.  AdamW updates its state in place, so the
    state is reset to the same values before each replay and before the eager
    reference."""
    from nvfp4_gemm_amd import pact as pb
    from tests import _gpu as G

    M, H, KV, r = 512, 512, 128, 16
    rng = np.random.default_rng(8)
    X = G.dev_bf16(synth.student_t_bf16(rng, (M, H), 4.0, 0.5))
    Xq = pb.pact_quantize_nvfp4(X)
    rows = [H, KV, KV]
    Wf = pb.NVFP4Tensor.cat_rows([pb.pact_build_weight_layouts(G.dev_bf16(synth.weight_bf16(rng, n, H)))[0]
                                  for n in rows])
    n_par = sum(r * H + n * r for n in rows)
    wflat = torch.empty(n_par, dtype=torch.bfloat16, device="cuda")
    gflat = torch.zeros(n_par, dtype=torch.float32, device="cuda")
    loras, gviews, off = [], [], 0
    for n in rows:
        A = wflat[off:off + r * H].view(r, H)
        A.copy_(G.dev_bf16(synth.normal_bf16(rng, (r, H), 0.02)))
        gA = gflat[off:off + r * H].view(r, H)
        off += r * H
        B = wflat[off:off + n * r].view(n, r)
        B.copy_(G.dev_bf16(synth.normal_bf16(rng, (n, r), 0.01)))
        gB = gflat[off:off + n * r].view(n, r)
        off += n * r
        loras.append(pb.LoRA(A, B, 2.0))
        gviews.append((gA, gB))
    p0 = wflat.float()
    p, m, v = p0.clone(), torch.zeros_like(p0), torch.zeros_like(p0)
    w_out = torch.empty_like(wflat)
    Y = torch.empty((M, H + 2 * KV), dtype=torch.bfloat16, device="cuda")
    dY = G.dev_bf16(synth.normal_bf16(rng, (M, H + 2 * KV), 1.0))
    ws = torch.empty((pb.pact_gemm_workspace(M, H + 2 * KV, H, 3 * r),), dtype=torch.uint8, device="cuda")
    gws = torch.empty((max(pb.pact_lora_grads_workspace(M, n, H, r) for n in rows),), dtype=torch.uint8,
                      device="cuda")

    def step():
        pb.pact_gemm_nvfp4_fwd_grouped(Xq, Wf, rows, X=X, loras=loras, Y=Y, ws=ws)
        c = 0
        for g, n in enumerate(rows):
            pb.pact_lora_grads_nvfp4(Xq, dY[:, c:c + n], loras[g], dA=gviews[g][0], dB=gviews[g][1], ws=gws)
            c += n
        pb.pact_adamw_step(p, m, v, gflat, w_out, lr=1e-3, weight_decay=0.01, step=3)

    def reset():
        p.copy_(p0)
        m.zero_()
        v.zero_()

    outs = [Y, gflat, p, m, v, w_out]
    reset()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (Y, gflat, w_out):
            t.zero_()
        reset()
        pb.pact_quantize_nvfp4(X, pb.NVFP4Tensor.empty(M, H))     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, r0) in enumerate(zip(outs, ref)):
            assert torch.equal(t.view(torch.uint8), r0.view(torch.uint8)), f"replay {rep}: output {i} differs"
