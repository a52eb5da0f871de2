#!/usr/bin/env python3
"""Benchmark of libpact's hot path on one MI355X: one decoder layer's frozen
projections through the NVFP4 data flow, forward + input-gradient backward.

One step (every call goes through the C ABI):
  forward:  n1, n1q, rstd1 = rmsnorm_quant(x)
            q, k, v = fwd GEMMs on n1q (+ LoRA on n1)
            a := q (attention core is not part of the frozen path: identity
            stand-in), aq = Q(a), x2 = fwd_o(aq, a, C = x)
            n2, n2q, rstd2 = rmsnorm_quant(x2); g, u = fwd GEMMs on n2q
            h, hq, gq, uq = silu_mul_quant(g, u); x' = fwd_down(hq, h, C = x2)
  backward: dh = dgrad_down(Q(dx'), dx'); stand-in dg = du = dh
            dx2 = dgrad_up(Q(dh), dh, C = dgrad_gate(Q(dh), dh, C = dx'))
            da = dgrad_o(Q(dx2), dx2); stand-ins dq = da, dk = da[:, :KV],
            dv = da[:, KV:2KV]
            dx = dgrad_v(Q(dv), dv, C = dgrad_k(Q(dk), dk, C = dgrad_q(Q(dq), dq, C = dx2)))
Weights and both cached NVFP4 layouts are built once before timing.

Prints ONE JSON line.  `value` = frozen-projection GEMM FLOPs of the step
(2 M N K over the 7 forward and 7 input-gradient GEMMs) / wall time of the
whole step (every kernel included), in TFLOP/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 frozen-proj GEMM TFLOP/s (fwd+dgrad) + layer tokens/s, % of roofline"
PEAK_F16_MFMA_TFLOPS = 2500.0   # MI355X dense FP16/BF16 MFMA
PEAK_FP4_TFLOPS = 10100.0       # context only: scaled FP4 MFMA cannot apply per-16 E4M3 scales
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama1b_layer",
                    choices=["llama1b_layer", "qwen1.5b_layer", "llama3b_layer"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens in the oracle sample (0: pick for ~10-20 s of CPU work)")
    ap.add_argument("--seed", type=int, default=0)
    return ap.parse_args()


class Layer:
    """Device buffers and weights of one layer, plus the step schedule."""

    def __init__(self, shape, seed):
        import torch
        from nvfp4_gemm_amd import pact as pb
        from nvfp4_gemm_amd import synth
        self.pb, self.torch, self.S = pb, torch, shape
        li = synth.layer_inputs(shape, seed=seed)
        self.li = li
        dev = "cuda"
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).view(torch.bfloat16).to(dev)
        M, H, I, KV = shape.tokens, shape.hidden, shape.inter, shape.kv
        self.M, self.H, self.I, self.KV = M, H, I, KV
        self.x, self.g1, self.g2, self.dout = bf(li.x), bf(li.gamma1), bf(li.gamma2), bf(li.dout)
        self.names = list(shape.projections().keys())
        self.Wbf = {n: bf(li.W[n]) for n in self.names}
        self.lora = {n: pb.LoRA(bf(li.A[n]), bf(li.B[n]), shape.lora_scale) for n in self.names}
        E = lambda r, c: torch.empty((r, c), dtype=torch.bfloat16, device=dev)
        Q = pb.NVFP4Tensor.empty
        # forward activations
        self.n1, self.n1q, self.rstd1 = E(M, H), Q(M, H), torch.empty(M, device=dev)
        self.q, self.k, self.v = E(M, H), E(M, KV), E(M, KV)
        self.aq, self.x2 = Q(M, H), E(M, H)
        self.n2, self.n2q, self.rstd2 = E(M, H), Q(M, H), torch.empty(M, device=dev)
        self.gt, self.up = E(M, I), E(M, I)
        self.h, self.hq, self.gq, self.uq = E(M, I), Q(M, I), Q(M, I), Q(M, I)
        self.xo = E(M, H)
        # backward
        self.doq, self.dh, self.dhq = Q(M, H), E(M, I), Q(M, I)
        self.dx2, self.dx2q, self.da = E(M, H), Q(M, H), E(M, H)
        self.dqq, self.dkq, self.dvq, self.dx = Q(M, H), Q(M, KV), Q(M, KV), E(M, H)
        need = max(pb.pact_gemm_workspace(M, n, k, shape.rank) for n, k in shape.projections().values())
        self.ws = torch.empty((need,), dtype=torch.uint8, device=dev)
        self.Wf, self.Wb = {}, {}

    def build_layouts(self):
        pb = self.pb
        for n in self.names:
            self.Wf[n], self.Wb[n] = pb.pact_build_weight_layouts(self.Wbf[n])

    def calls(self):
        """The step as a list of (kind, flops, bytes, fn)."""
        pb, S = self.pb, self.S
        M, H, I, KV, r = self.M, self.H, self.I, self.KV, S.rank
        L, Wf, Wb, ws = self.lora, self.Wf, self.Wb, self.ws
        gemm_fl = lambda n, k: 2 * M * n * k
        lora_fl = lambda n, k: 2 * M * r * (n + k)
        nvb = lambda rows, cols: rows * cols * 9 // 16 + 4 * rows
        c = []
        c.append(("rmsnorm_quant", 0, M * H * 2 * 2 + nvb(M, H) + 4 * M,
                  lambda: pb.pact_rmsnorm_quant_nvfp4(self.x, self.g1, S.eps, self.n1, self.n1q, self.rstd1)))
        for nm, out in (("q", self.q), ("k", self.k), ("v", self.v)):
            n, k = S.projections()[nm]
            c.append(("gemm_fwd", gemm_fl(n, k), 0, (lambda nm=nm, out=out: pb.pact_gemm_nvfp4_fwd(
                self.n1q, Wf[nm], X=self.n1, lora=L[nm], Y=out, ws=ws)), lora_fl(n, k)))
        c.append(("quantize", 0, M * H * 2 + nvb(M, H), lambda: pb.pact_quantize_nvfp4(self.q, self.aq)))
        c.append(("gemm_fwd", gemm_fl(H, H), 0, lambda: pb.pact_gemm_nvfp4_fwd(
            self.aq, Wf["o"], X=self.q, lora=L["o"], C=self.x, Y=self.x2, ws=ws), lora_fl(H, H)))
        c.append(("rmsnorm_quant", 0, M * H * 2 * 2 + nvb(M, H) + 4 * M,
                  lambda: pb.pact_rmsnorm_quant_nvfp4(self.x2, self.g2, S.eps, self.n2, self.n2q, self.rstd2)))
        for nm, out in (("gate", self.gt), ("up", self.up)):
            c.append(("gemm_fwd", gemm_fl(I, H), 0, (lambda nm=nm, out=out: pb.pact_gemm_nvfp4_fwd(
                self.n2q, Wf[nm], X=self.n2, lora=L[nm], Y=out, ws=ws)), lora_fl(I, H)))
        c.append(("silu_mul_quant", 0, M * I * 2 * 3 + 3 * nvb(M, I),
                  lambda: pb.pact_silu_mul_quant_nvfp4(self.gt, self.up, self.h, self.hq, self.gq, self.uq)))
        c.append(("gemm_fwd", gemm_fl(H, I), 0, lambda: pb.pact_gemm_nvfp4_fwd(
            self.hq, Wf["down"], X=self.h, lora=L["down"], C=self.x2, Y=self.xo, ws=ws), lora_fl(H, I)))
        # backward (input gradients)
        c.append(("quantize", 0, M * H * 2 + nvb(M, H), lambda: pb.pact_quantize_nvfp4(self.dout, self.doq)))
        c.append(("gemm_dgrad", gemm_fl(H, I), 0, lambda: pb.pact_gemm_nvfp4_dgrad(
            self.doq, Wb["down"], dY=self.dout, lora=L["down"], dX=self.dh, ws=ws), lora_fl(H, I)))
        c.append(("quantize", 0, M * I * 2 + nvb(M, I), lambda: pb.pact_quantize_nvfp4(self.dh, self.dhq)))
        c.append(("gemm_dgrad", gemm_fl(I, H), 0, lambda: pb.pact_gemm_nvfp4_dgrad(
            self.dhq, Wb["gate"], dY=self.dh, lora=L["gate"], C=self.dout, dX=self.dx2, ws=ws), lora_fl(I, H)))
        c.append(("gemm_dgrad", gemm_fl(I, H), 0, lambda: pb.pact_gemm_nvfp4_dgrad(
            self.dhq, Wb["up"], dY=self.dh, lora=L["up"], C=self.dx2, dX=self.dx2, ws=ws), lora_fl(I, H)))
        c.append(("quantize", 0, M * H * 2 + nvb(M, H), lambda: pb.pact_quantize_nvfp4(self.dx2, self.dx2q)))
        c.append(("gemm_dgrad", gemm_fl(H, H), 0, lambda: pb.pact_gemm_nvfp4_dgrad(
            self.dx2q, Wb["o"], dY=self.dx2, lora=L["o"], dX=self.da, ws=ws), lora_fl(H, H)))
        dq, dk, dv = self.da, self.da[:, :KV], self.da[:, KV:2 * KV]
        c.append(("quantize", 0, M * H * 2 + nvb(M, H), lambda: pb.pact_quantize_nvfp4(dq, self.dqq)))
        c.append(("quantize", 0, M * KV * 2 + nvb(M, KV), lambda: pb.pact_quantize_nvfp4(dk, self.dkq)))
        c.append(("quantize", 0, M * KV * 2 + nvb(M, KV), lambda: pb.pact_quantize_nvfp4(dv, self.dvq)))
        c.append(("gemm_dgrad", gemm_fl(H, H), 0, lambda: pb.pact_gemm_nvfp4_dgrad(
            self.dqq, Wb["q"], dY=dq, lora=L["q"], C=self.dx2, dX=self.dx, ws=ws), lora_fl(H, H)))
        c.append(("gemm_dgrad", gemm_fl(KV, H), 0, lambda: pb.pact_gemm_nvfp4_dgrad(
            self.dkq, Wb["k"], dY=dk, lora=L["k"], C=self.dx, dX=self.dx, ws=ws), lora_fl(KV, H)))
        c.append(("gemm_dgrad", gemm_fl(KV, H), 0, lambda: pb.pact_gemm_nvfp4_dgrad(
            self.dvq, Wb["v"], dY=dv, lora=L["v"], C=self.dx, dX=self.dx, ws=ws), lora_fl(KV, H)))
        return [(t[0], t[1], t[2], t[3], t[4] if len(t) > 4 else 0) for t in c]

    def stash_bytes(self):
        M, H, I = self.M, self.H, self.I
        nv = lambda q: q.nbytes()
        pact = nv(self.n1q) + nv(self.aq) + nv(self.n2q) + nv(self.gq) + nv(self.uq) + nv(self.hq) + 8 * M
        bf16 = 2 * (5 * M * H + 3 * M * I) + 8 * M
        return pact, bf16


def cpu_baseline(S, li, sample_tokens):
    """The oracle, as it stands, on the first `sample_tokens` tokens of the same
    layer (every step of the data flow is per token, so this is the same
    computation on a smaller batch)."""
    import oracle
    names = list(S.projections().keys())
    rows = np.arange(sample_tokens)
    H, KV = S.hidden, S.kv
    t0 = time.perf_counter()
    Wf, Wb = {}, {}
    for n in names:
        Wf[n], Wb[n] = oracle.build_weight_layouts(li.W[n])
    t_layout = time.perf_counter() - t0
    x = li.x[rows]
    t0 = time.perf_counter()
    n1, n1q, _ = oracle.rmsnorm_quant(x, li.gamma1, S.eps)
    fw = lambda aq, X, nm, C=None: oracle.gemm_fwd(aq, X, Wf[nm], li.A[nm], li.B[nm], S.lora_scale, C)
    dg = lambda gq, dY, nm, C=None: oracle.gemm_dgrad(gq, dY, Wb[nm], li.A[nm], li.B[nm], S.lora_scale, C)
    q = fw(n1q, n1, "q")
    fw(n1q, n1, "k")
    fw(n1q, n1, "v")
    x2 = fw(oracle.quantize_bf16(q), q, "o", x)
    n2, n2q, _ = oracle.rmsnorm_quant(x2, li.gamma2, S.eps)
    g = fw(n2q, n2, "gate")
    u = fw(n2q, n2, "up")
    h, hq, _, _ = oracle.silu_mul_quant(g, u)
    fw(hq, h, "down", x2)
    dout = li.dout[rows]
    dh = dg(oracle.quantize_bf16(dout), dout, "down")
    dhq = oracle.quantize_bf16(dh)
    dx2 = dg(dhq, dh, "up", dg(dhq, dh, "gate", dout))
    da = dg(oracle.quantize_bf16(dx2), dx2, "o")
    dk, dv = np.ascontiguousarray(da[:, :KV]), np.ascontiguousarray(da[:, KV:2 * KV])
    dx = dg(oracle.quantize_bf16(da), da, "q", dx2)
    dx = dg(oracle.quantize_bf16(dk), dk, "k", dx)
    dg(oracle.quantize_bf16(dv), dv, "v", dx)
    t_step = time.perf_counter() - t0
    flops = 2 * sum(2 * sample_tokens * n * k for n, k in S.projections().values())
    return {"value": flops / t_step / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{sample_tokens} of {S.tokens} tokens through the full layer step "
                      f"(fwd + input-gradient, all 14 GEMMs, quantizers, norms); weight layouts "
                      f"built once outside the timed part ({t_layout:.1f} s)",
            "seconds": t_step, "tokens_per_s": sample_tokens / t_step}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the data flow is row-parallel and this build "
              "runs on a single MI355X (the sharding plan is described in DESIGN.md).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from nvfp4_gemm_amd import synth
    shape = synth.LAYERS[args.config]
    layer = Layer(shape, args.seed)
    st = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    e0, e1 = ev(), ev()
    e0.record(st)
    layer.build_layouts()
    e1.record(st)
    torch.cuda.synchronize()
    layout_ms = e0.elapsed_time(e1)
    calls = layer.calls()
    for _ in range(args.warmup):
        for c in calls:
            c[3]()
    torch.cuda.synchronize()
    # timed region: events around every call, on the stream the kernels run on
    evs = [[(ev(), ev()) for _ in calls] for _ in range(args.steps)]
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    t_start.record(st)
    for s in range(args.steps):
        for (a, b), c in zip(evs[s], calls):
            a.record(st)
            c[3]()
            b.record(st)
    t_end.record(st)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    per_kind = {}
    for s in range(args.steps):
        for (a, b), c in zip(evs[s], calls):
            k = per_kind.setdefault(c[0], {"ms": 0.0, "calls": 0, "flops": 0, "lora_flops": 0, "bytes": 0})
            k["ms"] += a.elapsed_time(b)
            k["calls"] += 1
            k["flops"] += c[1]
            k["lora_flops"] += c[4]
            k["bytes"] += c[2]
    frozen_flops = sum(c[1] for c in calls)
    value = frozen_flops / (ms_step * 1e-3) / 1e12
    gemm = {"ms": 0.0, "calls": 0, "flops": 0, "lora_flops": 0}
    for kind in ("gemm_fwd", "gemm_dgrad"):
        for f in gemm:
            gemm[f] += per_kind[kind][f]
    gemm_avg_ms = gemm["ms"] / gemm["calls"]
    gemm_flops_per_launch = (gemm["flops"] + gemm["lora_flops"]) / gemm["calls"]
    achieved = gemm_flops_per_launch / (gemm_avg_ms * 1e-3) / 1e12
    kinds = {}
    for kind, k in per_kind.items():
        d = {"avg_us": 1e3 * k["ms"] / k["calls"], "calls_per_step": k["calls"] // args.steps}
        if k["flops"]:
            d["frozen_tflops"] = k["flops"] / (k["ms"] * 1e-3) / 1e12
        if k["bytes"]:
            gbs = k["bytes"] / (k["ms"] * 1e-3) / 1e9
            d["GB/s"] = gbs
            d["hbm_frac"] = gbs / PEAK_HBM_GBS
        kinds[kind] = d
    pact_stash, bf16_stash = layer.stash_bytes()
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": shape.name, "tokens": shape.tokens, "hidden": shape.hidden,
                   "intermediate": shape.inter, "kv": shape.kv, "lora_rank": shape.rank,
                   "lora_scale": shape.lora_scale, "step": "layer forward + input-gradient backward, "
                   "7 frozen NVFP4 projections, fused RMSNorm/SiLU quantizers"},
        "tokens_per_s": shape.tokens / (ms_step * 1e-3),
        "frozen_gemm_tflops_kernel_time": gemm["flops"] / (gemm["ms"] * 1e-3) / 1e12,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_F16_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_F16_MFMA_TFLOPS, "traffic": None,
                     "kernel": "NVFP4 GEMM entry points (fwd + dgrad: LoRA-down + main GEMM kernels), "
                               "frozen + LoRA FLOPs per launch / mean launch time",
                     "fp4_peak_context": PEAK_FP4_TFLOPS},
        "kernels": kinds,
        "stash_bytes": {"pact_nvfp4": pact_stash, "bf16_lora": bf16_stash,
                        "ratio": bf16_stash / pact_stash},
        "layout_build_ms_7_projections": layout_ms,
        "peak_hbm_bytes": torch.cuda.max_memory_allocated(),
    }
    if not args.no_cpu_baseline:
        n = args.cpu_sample_tokens or min(shape.tokens, 256)
        out["cpu_baseline"] = cpu_baseline(shape, layer.li, n)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
