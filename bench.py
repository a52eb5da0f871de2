#!/usr/bin/env python3
"""Benchmark of libpact's hot path on one MI355X: the frozen projections of
LoRA decoder layers through the NVFP4 data flow, forward + input-gradient
backward (simolm.com PACT blog post, section "Method"; arXiv abstract of
"PACT: NVFP4 Data-Flow LoRA Fine-Tuning on Consumer GPUs").

One step of a layer (every call goes through the C ABI):
  forward:  n1, n1q, rstd1 = rmsnorm_quant(x)
            [q | k | v] = one grouped fwd GEMM on n1q over the concatenated
            weight rows (+ block-diagonal LoRA on n1)
            a := q (the attention core is not part of the frozen path: identity
            stand-in), aq = Q(a), x2 = fwd_o(aq, a, C = x)
            n2, n2q, rstd2 = rmsnorm_quant(x2); [g | u] = one grouped fwd GEMM on n2q
            h, hq, gq, uq = silu_mul_quant(g, u); x' = fwd_down(hq, h, C = x2)
  backward: dh = dgrad_down(Q(dx'), dx')
            dg, du, dgq, duq = silu_mul_bwd(dh, gq, uq)          (from the stash)
            dn2 = dgrad_up(duq, du, C = dgrad_gate(dgq, dg))
            dx2, dx2q = rmsnorm_bwd(dn2, n2q, gamma2, rstd2, C = dx')   (residual)
            da = dgrad_o(dx2q, dx2); attention backward stand-ins dq = da,
            dk = da[:, :KV], dv = da[:, KV:2KV]
            dn1 = dgrad_v(Q(dv), dv, C = dgrad_k(Q(dk), dk, C = dgrad_q(Q(dq), dq)))
            dx, Q(dx) = rmsnorm_bwd(dn1, n1q, gamma1, rstd1, C = dx2)
            (Q(dx) is the next layer's Q(dx'); Q(dx') is a separate call only
            for the last layer)
A stack runs the layers' forwards in order, keeping each layer's NVFP4 stash
(n1q, aq, n2q, gq, uq, hq, rstd1, rstd2), then the backwards in reverse order;
the backward consumes n1q, n2q, gq, uq and the rstd rows.
The single-linear workload is Q(X), fwd, Q(dY), dgrad.  Weights and both
cached NVFP4 layouts are built once before timing.

Prints ONE JSON line.  `value` = frozen-projection GEMM FLOPs of the step
(2 M N K over every forward and input-gradient GEMM) / wall time of the whole
step (every kernel included), in TFLOP/s.  The step is captured once as a HIP
graph and the timed region replays it (a training loop launches the same
step every iteration; the graph removes the per-call host overhead of the
Python binding).  A second timed region runs the step eagerly with events
around every call on its stream: the per-kernel durations and the roofline
figures come from it.

Other modes (used to calibrate and summarize rocprofv3 counter runs):
  --copy-calibration MIB   runs a plain device-to-device copy of MIB MiB
  --summarize-pmc DIR ...  turns rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
                           databases into the HBM-traffic summary text
  --library-gemm           times the vendor library's FP16 GEMM (hipBLASLt
                           through torch) on FP16 operands of the shapes of
                           one layer's frozen GEMMs, beside libpact's NVFP4
                           entry points on the same shapes: a practical
                           ceiling for the MFMA fraction
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import re
import os
import sqlite3
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 frozen-proj GEMM TFLOP/s (fwd+dgrad) + layer tokens/s, % of roofline"
PEAK_F16_MFMA_TFLOPS = 2500.0   # MI355X dense FP16/BF16 MFMA
PEAK_FP4_TFLOPS = 10100.0       # context only: scaled FP4 MFMA cannot apply per-16 E4M3 scales
PEAK_HBM_GBS = 8000.0
GEMM_SOURCE = os.path.join(ROOT, "nvfp4_gemm_amd", "csrc", "pact_gemm.hip")
CONFIGS = ["single_linear", "llama1b_layer", "qwen1.5b_layer", "llama3b_layer", "llama3b_stack28"]
# kernels of the GEMM entry points: LoRA-down, one main kernel, and (split K)
# the epilogue kernel; the main kernel's name marks one entry-point call
GEMM_KERNELS = ("gemm_kernel", "gemm8_kernel", "lora_down_kernel", "lora_down_pipe_kernel", "splitk_epi_kernel",
                "lora_transpose_kernel")
GEMM_MAIN_KERNELS = ("gemm_kernel", "gemm8_kernel")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama3b_stack28", choices=CONFIGS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens in the oracle sample (0: 1024, or 512 for the 3B-shaped layers)")
    ap.add_argument("--lora-grads", action="store_true",
                    help="add the LoRA weight gradients (dA, dB of every projection, from the NVFP4 stash) "
                         "to each layer's backward and one fused AdamW step over all adapters; timed as their "
                         "own kinds, never counted as frozen FLOPs (under graph replay the AdamW step number "
                         "is the captured one)")
    ap.add_argument("--ungrouped", action="store_true",
                    help="run q, k, v and gate, up as separate forward GEMMs (one call per projection)")
    ap.add_argument("--eager", action="store_true",
                    help="time the step without graph capture")
    ap.add_argument("--no-isolated", action="store_true",
                    help="skip the cache-flushed timing of the memory-bound kernels")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DB_DIR", "WRITE_DB_DIR", "COPY_FETCH_DIR",
                                                         "COPY_WRITE_DIR"))
    ap.add_argument("--summarize-row-pmc", nargs=5, metavar=("FETCH_DB_DIR", "WRITE_DB_DIR", "COPY_FETCH_DIR",
                                                             "COPY_WRITE_DIR", "KERNEL_STATS_CSV"),
                    help="row-kernel HBM traffic of the 3B-shaped stack (M = 8192) from counter runs, with the "
                         "durations of a kernel trace")
    ap.add_argument("--summarize-coverage", metavar="KERNEL_STATS_CSV",
                    help="kernel-variant coverage: every kernel compiled into libpact.so (from the compiler's "
                         "resource-usage remarks) against the launches in a kernel trace of the GPU test suite")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--pmc-out", default="")
    ap.add_argument("--pmc-command", default="")
    ap.add_argument("--library-gemm", action="store_true")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="stream each row kernel's read and write bytes with the streaming diagnostic and "
                         "compare the kernel's cold-cache rate with that ceiling (plus read-only, write-only "
                         "and copy at 1 GiB)")
    return ap.parse_args()


def nvb(rows, cols):
    """Bytes of an NVFP4 tensor: codes + E4M3 block scales + FP32 row scales."""
    return rows * cols * 9 // 16 + 4 * rows


class Stack:
    """Device buffers, weights and the step schedule of `layers` decoder layers."""

    def __init__(self, shape, seed, layers, lora_grads=False, grouped=True):
        import torch
        from nvfp4_gemm_amd import pact as pb
        from nvfp4_gemm_amd import synth
        self.pb, self.torch, self.S, self.L = pb, torch, shape, layers
        dev = "cuda"
        self.bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).view(
            torch.bfloat16).to(dev)
        M, H, I, KV = shape.tokens, shape.hidden, shape.inter, shape.kv
        self.M, self.H, self.I, self.KV = M, H, I, KV
        self.names = list(shape.projections().keys())
        E = lambda r, c: torch.empty((r, c), dtype=torch.bfloat16, device=dev)
        Q = pb.NVFP4Tensor.empty
        self.Wf, self.Wb, self.lora, self.g1, self.g2 = [], [], [], [], []
        self.layout_ms = 0.0
        st = torch.cuda.current_stream()
        self.lora_grads = lora_grads
        self.grouped = grouped
        if lora_grads:
            # every adapter of every layer lives in one flat buffer (BF16 copy for the GEMMs, FP32 master,
            # moments and gradients), so one AdamW launch updates them all
            r = shape.rank
            sizes = [r * k + n * r for _ in range(layers) for n, k in shape.projections().values()]
            self.n_params = sum(sizes)
            self.wflat = torch.empty(self.n_params, dtype=torch.bfloat16, device=dev)
            self.pflat = torch.empty(self.n_params, dtype=torch.float32, device=dev)
            self.mflat = torch.zeros(self.n_params, dtype=torch.float32, device=dev)
            self.vflat = torch.zeros(self.n_params, dtype=torch.float32, device=dev)
            self.gflat = torch.zeros(self.n_params, dtype=torch.float32, device=dev)
            self.gA, self.gB = [], []
            off = 0
        for l in range(layers):
            li = synth.layer_inputs(shape, seed=seed, layer=l)
            if l == 0:
                self.li0 = li
                self.x0, self.dout = self.bf(li.x), self.bf(li.dout)
            Wbf = {n: self.bf(li.W[n]) for n in self.names}
            self.g1.append(self.bf(li.gamma1))
            self.g2.append(self.bf(li.gamma2))
            if lora_grads:
                lo, gA, gB = {}, {}, {}
                for n in self.names:
                    nn, kk = shape.projections()[n]
                    r = shape.rank
                    assert off % 8 == 0 and (r * kk) % 8 == 0
                    A = self.wflat[off:off + r * kk].view(r, kk)
                    A.copy_(self.bf(li.A[n]))
                    gA[n] = self.gflat[off:off + r * kk].view(r, kk)
                    off += r * kk
                    B = self.wflat[off:off + nn * r].view(nn, r)
                    B.copy_(self.bf(li.B[n]))
                    gB[n] = self.gflat[off:off + nn * r].view(nn, r)
                    off += nn * r
                    lo[n] = pb.LoRA(A, B, shape.lora_scale)
                self.lora.append(lo)
                self.gA.append(gA)
                self.gB.append(gB)
            else:
                self.lora.append({n: pb.LoRA(self.bf(li.A[n]), self.bf(li.B[n]), shape.lora_scale)
                                  for n in self.names})
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            lay = {n: pb.pact_build_weight_layouts(Wbf[n]) for n in self.names}
            e1.record(st)
            torch.cuda.synchronize()
            self.layout_ms += e0.elapsed_time(e1)
            # forward layouts of projections that share an input, concatenated for the grouped GEMMs
            if grouped:
                self.Wf.append({"qkv": pb.NVFP4Tensor.cat_rows([lay[n][0] for n in ("q", "k", "v")]),
                                "gu": pb.NVFP4Tensor.cat_rows([lay[n][0] for n in ("gate", "up")]),
                                "o": lay["o"][0], "down": lay["down"][0]})
            else:
                self.Wf.append({n: lay[n][0] for n in self.names})
            self.Wb.append({n: lay[n][1] for n in self.names})
            del Wbf, lay
        # per-layer stash (kept from the forward to the backward)
        self.stash = [dict(n1q=Q(M, H), rstd1=torch.empty(M, device=dev), aq=Q(M, H), n2q=Q(M, H),
                           rstd2=torch.empty(M, device=dev), gq=Q(M, I), uq=Q(M, I), hq=Q(M, I))
                      for _ in range(layers)]
        # transient activations, shared by the layers
        self.xs = [self.x0, E(M, H), E(M, H)]    # layer input / output ping-pong (x0 is kept)
        self.n1, self.qkv = E(M, H), E(M, H + 2 * KV)
        self.q, self.k, self.v = self.qkv[:, :H], self.qkv[:, H:H + KV], self.qkv[:, H + KV:]
        self.x2, self.n2 = E(M, H), E(M, H)
        self.gu, self.h = E(M, 2 * I), E(M, I)
        self.gt, self.up = self.gu[:, :I], self.gu[:, I:]
        self.doq, self.dh = Q(M, H), E(M, I)
        self.dg, self.du, self.dgq, self.duq = E(M, I), E(M, I), Q(M, I), Q(M, I)
        self.dn = E(M, H)                        # gradient of a norm output (n2, then n1)
        self.dx2, self.dx2q, self.da = E(M, H), Q(M, H), E(M, H)
        self.dqq, self.dkq, self.dvq = Q(M, H), Q(M, KV), Q(M, KV)
        self.dxs = [self.dout, E(M, H), E(M, H)]
        rpad = (shape.rank + 15) // 16 * 16
        need = max([pb.pact_gemm_workspace(M, n, k, shape.rank) for n, k in shape.projections().values()]
                   + [pb.pact_gemm_workspace(M, H + 2 * KV, H, 3 * rpad), pb.pact_gemm_workspace(M, 2 * I, H, 2 * rpad)])
        self.ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
        if lora_grads:
            self.pflat.copy_(self.wflat.float())
            self.adam_step = 0
            r = shape.rank
            gneed = max(pb.pact_lora_grads_workspace(M, n, k, r) for n, k in shape.projections().values())
            self.gws = torch.empty((max(gneed, 16),), dtype=torch.uint8, device=dev)

    def calls(self):
        """The step as a list of (kind, frozen flops, bytes, fn, lora flops)."""
        pb, S = self.pb, self.S
        M, H, I, KV, r = self.M, self.H, self.I, self.KV, S.rank
        ws = self.ws
        gemm_fl = lambda n, k: 2 * M * n * k
        lora_fl = lambda n, k: 2 * M * r * (n + k)
        c = []

        def grads(nm, xq, dY, L, l):
            """dA, dB of projection nm of layer l (input xq from the stash, output gradient dY),
            right after the projection's input-gradient GEMM: its workspace still holds
            T' = bf16(s dY B), which the gradient call takes instead of computing it."""
            if not self.lora_grads:
                return
            n, k = S.projections()[nm]
            c.append(("lora_grads", 0, nvb(M, k) + 2 * M * n + 2 * r * (n + k) + 4 * r * (n + k),
                      lambda nm=nm, xq=xq, dY=dY, L=L, l=l: pb.pact_lora_grads_nvfp4(
                          xq, dY, L[nm], dA=self.gA[l][nm], dB=self.gB[l][nm], ws=self.gws, T_dy=ws),
                      4 * M * r * (n + k)))
        xin = lambda l: self.xs[0] if l == 0 else self.xs[1 + (l - 1) % 2]
        xout = lambda l: self.xs[1 + l % 2]
        for l in range(self.L):
            st, L, Wf = self.stash[l], self.lora[l], self.Wf[l]
            x, xo = xin(l), xout(l)
            c.append(("rmsnorm_quant", 0, M * H * 2 * 2 + nvb(M, H) + 4 * M,
                      lambda x=x, st=st, l=l: pb.pact_rmsnorm_quant_nvfp4(x, self.g1[l], S.eps, self.n1,
                                                                          st["n1q"], st["rstd1"]), 0))
            if self.grouped:  # q, k, v: one grouped GEMM over the concatenated weight rows (block-diagonal LoRA)
                c.append(("gemm_fwd", gemm_fl(H + 2 * KV, H), 0, (lambda st=st, L=L, Wf=Wf: pb.pact_gemm_nvfp4_fwd_grouped(
                    st["n1q"], Wf["qkv"], [H, KV, KV], X=self.n1, loras=[L["q"], L["k"], L["v"]], Y=self.qkv,
                    ws=ws)), lora_fl(H, H) + 2 * lora_fl(KV, H)))
            else:
                for nm, out in (("q", self.q), ("k", self.k), ("v", self.v)):
                    n, k = S.projections()[nm]
                    c.append(("gemm_fwd", gemm_fl(n, k), 0, (lambda nm=nm, out=out, st=st, L=L, Wf=Wf:
                              pb.pact_gemm_nvfp4_fwd(st["n1q"], Wf[nm], X=self.n1, lora=L[nm], Y=out, ws=ws)),
                              lora_fl(n, k)))
            c.append(("quantize", 0, M * H * 2 + nvb(M, H),
                      lambda st=st: pb.pact_quantize_nvfp4(self.q, st["aq"]), 0))
            c.append(("gemm_fwd", gemm_fl(H, H), 0, lambda x=x, st=st, L=L, Wf=Wf: pb.pact_gemm_nvfp4_fwd(
                st["aq"], Wf["o"], X=self.q, lora=L["o"], C=x, Y=self.x2, ws=ws), lora_fl(H, H)))
            c.append(("rmsnorm_quant", 0, M * H * 2 * 2 + nvb(M, H) + 4 * M,
                      lambda st=st, l=l: pb.pact_rmsnorm_quant_nvfp4(self.x2, self.g2[l], S.eps, self.n2,
                                                                     st["n2q"], st["rstd2"]), 0))
            if self.grouped:  # gate, up: one grouped GEMM
                c.append(("gemm_fwd", gemm_fl(2 * I, H), 0, (lambda st=st, L=L, Wf=Wf: pb.pact_gemm_nvfp4_fwd_grouped(
                    st["n2q"], Wf["gu"], [I, I], X=self.n2, loras=[L["gate"], L["up"]], Y=self.gu, ws=ws)),
                    2 * lora_fl(I, H)))
            else:
                for nm, out in (("gate", self.gt), ("up", self.up)):
                    c.append(("gemm_fwd", gemm_fl(I, H), 0, (lambda nm=nm, out=out, st=st, L=L, Wf=Wf:
                              pb.pact_gemm_nvfp4_fwd(st["n2q"], Wf[nm], X=self.n2, lora=L[nm], Y=out, ws=ws)),
                              lora_fl(I, H)))
            c.append(("silu_mul_quant", 0, M * I * 2 * 3 + 3 * nvb(M, I),
                      lambda st=st: pb.pact_silu_mul_quant_nvfp4(self.gt, self.up, self.h, st["hq"], st["gq"],
                                                                 st["uq"]), 0))
            c.append(("gemm_fwd", gemm_fl(H, I), 0, lambda xo=xo, st=st, L=L, Wf=Wf: pb.pact_gemm_nvfp4_fwd(
                st["hq"], Wf["down"], X=self.h, lora=L["down"], C=self.x2, Y=xo, ws=ws), lora_fl(H, I)))
        # backward (input gradients), last layer first
        for j, l in enumerate(reversed(range(self.L))):
            st, L, Wb = self.stash[l], self.lora[l], self.Wb[l]
            dout = self.dxs[0] if j == 0 else self.dxs[1 + (j - 1) % 2]
            dx = self.dxs[1 + j % 2]
            if j == 0:  # later layers get Q(dout) from the RMSNorm backward above them
                c.append(("quantize", 0, M * H * 2 + nvb(M, H),
                          lambda dout=dout: pb.pact_quantize_nvfp4(dout, self.doq), 0))
            c.append(("gemm_dgrad", gemm_fl(H, I), 0, lambda dout=dout, L=L, Wb=Wb: pb.pact_gemm_nvfp4_dgrad(
                self.doq, Wb["down"], dY=dout, lora=L["down"], dX=self.dh, ws=ws), lora_fl(H, I)))
            grads("down", st["hq"], dout, L, l)
            c.append(("silu_mul_bwd", 0, M * I * 2 + 2 * nvb(M, I) + 2 * M * I * 2 + 2 * nvb(M, I),
                      lambda st=st: pb.pact_silu_mul_bwd_quant_nvfp4(self.dh, st["gq"], st["uq"], self.dg, self.du,
                                                                     self.dgq, self.duq), 0))
            c.append(("gemm_dgrad", gemm_fl(I, H), 0, lambda L=L, Wb=Wb: pb.pact_gemm_nvfp4_dgrad(
                self.dgq, Wb["gate"], dY=self.dg, lora=L["gate"], dX=self.dn, ws=ws), lora_fl(I, H)))
            grads("gate", st["n2q"], self.dg, L, l)
            c.append(("gemm_dgrad", gemm_fl(I, H), 0, lambda L=L, Wb=Wb: pb.pact_gemm_nvfp4_dgrad(
                self.duq, Wb["up"], dY=self.du, lora=L["up"], C=self.dn, dX=self.dn, ws=ws), lora_fl(I, H)))
            grads("up", st["n2q"], self.du, L, l)
            c.append(("rmsnorm_bwd", 0, M * H * 2 + nvb(M, H) + 4 * M + M * H * 2 + M * H * 2 + nvb(M, H),
                      lambda st=st, l=l, dout=dout: pb.pact_rmsnorm_bwd_nvfp4(
                          self.dn, st["n2q"], self.g2[l], st["rstd2"], C=dout, dx=self.dx2, dxq=self.dx2q), 0))
            c.append(("gemm_dgrad", gemm_fl(H, H), 0, lambda L=L, Wb=Wb: pb.pact_gemm_nvfp4_dgrad(
                self.dx2q, Wb["o"], dY=self.dx2, lora=L["o"], dX=self.da, ws=ws), lora_fl(H, H)))
            grads("o", st["aq"], self.dx2, L, l)
            dq, dk, dv = self.da, self.da[:, :KV], self.da[:, KV:2 * KV]
            c.append(("quantize", 0, M * H * 2 + nvb(M, H), lambda dq=dq: pb.pact_quantize_nvfp4(dq, self.dqq), 0))
            c.append(("quantize", 0, M * KV * 2 + nvb(M, KV), lambda dk=dk: pb.pact_quantize_nvfp4(dk, self.dkq), 0))
            c.append(("quantize", 0, M * KV * 2 + nvb(M, KV), lambda dv=dv: pb.pact_quantize_nvfp4(dv, self.dvq), 0))
            c.append(("gemm_dgrad", gemm_fl(H, H), 0, lambda dq=dq, L=L, Wb=Wb: pb.pact_gemm_nvfp4_dgrad(
                self.dqq, Wb["q"], dY=dq, lora=L["q"], dX=self.dn, ws=ws), lora_fl(H, H)))
            grads("q", st["n1q"], dq, L, l)
            c.append(("gemm_dgrad", gemm_fl(KV, H), 0, lambda dk=dk, L=L, Wb=Wb: pb.pact_gemm_nvfp4_dgrad(
                self.dkq, Wb["k"], dY=dk, lora=L["k"], C=self.dn, dX=self.dn, ws=ws), lora_fl(KV, H)))
            grads("k", st["n1q"], dk, L, l)
            c.append(("gemm_dgrad", gemm_fl(KV, H), 0, lambda dv=dv, L=L, Wb=Wb: pb.pact_gemm_nvfp4_dgrad(
                self.dvq, Wb["v"], dY=dv, lora=L["v"], C=self.dn, dX=self.dn, ws=ws), lora_fl(KV, H)))
            grads("v", st["n1q"], dv, L, l)
            last = j == self.L - 1
            c.append(("rmsnorm_bwd", 0, M * H * 2 + nvb(M, H) + 4 * M + M * H * 2 + M * H * 2
                      + (0 if last else nvb(M, H)),
                      lambda st=st, l=l, dx=dx, last=last: pb.pact_rmsnorm_bwd_nvfp4(
                          self.dn, st["n1q"], self.g1[l], st["rstd1"], C=self.dx2, dx=dx,
                          dxq=None if last else self.doq, want_q=not last), 0))
        if self.lora_grads:
            def adam():
                self.adam_step += 1
                pb.pact_adamw_step(self.pflat, self.mflat, self.vflat, self.gflat, self.wflat, lr=1e-4,
                                   weight_decay=0.01, step=self.adam_step)
            c.append(("adamw", 0, 30 * self.n_params, adam, 0))
        return c

    def stash_bytes(self):
        """NVFP4 stash of the layers vs the BF16 stash the same frozen path keeps
        under BF16 LoRA ({x, n1, attn_out, x2, n2} [M,H] and {g, u, h} [M,I],
        plus the two FP32 rstd rows)."""
        M, H, I = self.M, self.H, self.I
        pact = sum(sum(v.nbytes() for k, v in st.items() if k.endswith("q")) + 8 * M for st in self.stash)
        bf16 = self.L * (2 * (5 * M * H + 3 * M * I) + 8 * M)
        return pact, bf16

    def config(self):
        S = self.S
        return {"workload": S.name, "layers": self.L, "tokens": S.tokens, "hidden": S.hidden,
                "intermediate": S.inter, "kv": S.kv, "lora_rank": S.rank, "lora_scale": S.lora_scale,
                "step": "forward + input-gradient backward of every layer, 7 frozen NVFP4 projections "
                        "per layer with BF16 LoRA, fused RMSNorm/SiLU quantizers"
                        + (", plus the LoRA weight gradients of every projection and one AdamW step over all "
                           "adapters" if self.lora_grads else ""),
                "lora_grads": self.lora_grads,
                "forward_gemms": "grouped q|k|v and gate|up" if self.grouped else "one per projection"}


class Linear:
    """The single NVFP4 LoRA linear: Q(X), fwd, Q(dY), dgrad."""

    def __init__(self, seed):
        import torch
        from nvfp4_gemm_amd import pact as pb
        from nvfp4_gemm_amd import synth
        p = synth.SINGLE_LINEAR
        self.pb, self.p = pb, p
        li = synth.single_linear_inputs(M=p["M"], N=p["N"], K=p["K"], r=p["r"], s=p["lora_scale"], seed=seed)
        self.li = li
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).view(torch.bfloat16).cuda()
        self.X, self.dY, W = bf(li.X), bf(li.dY), bf(li.W)
        self.lora = pb.LoRA(bf(li.A), bf(li.B), li.s)
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        self.Wf, self.Wb = pb.pact_build_weight_layouts(W)
        e1.record(st)
        torch.cuda.synchronize()
        self.layout_ms = e0.elapsed_time(e1)
        M, N, K = p["M"], p["N"], p["K"]
        self.xq, self.dyq = pb.NVFP4Tensor.empty(M, K), pb.NVFP4Tensor.empty(M, N)
        self.Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        self.dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        self.ws = torch.empty((max(pb.pact_gemm_workspace(M, N, K, p["r"]), 16),), dtype=torch.uint8,
                              device="cuda")
        self.M, self.N, self.K, self.L = M, N, K, 1

    def calls(self):
        pb, M, N, K, r = self.pb, self.M, self.N, self.K, self.p["r"]
        return [
            ("quantize", 0, M * K * 2 + nvb(M, K), lambda: pb.pact_quantize_nvfp4(self.X, self.xq), 0),
            ("gemm_fwd", 2 * M * N * K, 0, lambda: pb.pact_gemm_nvfp4_fwd(
                self.xq, self.Wf, X=self.X, lora=self.lora, Y=self.Y, ws=self.ws), 2 * M * r * (N + K)),
            ("quantize", 0, M * N * 2 + nvb(M, N), lambda: pb.pact_quantize_nvfp4(self.dY, self.dyq), 0),
            ("gemm_dgrad", 2 * M * N * K, 0, lambda: pb.pact_gemm_nvfp4_dgrad(
                self.dyq, self.Wb, dY=self.dY, lora=self.lora, dX=self.dX, ws=self.ws), 2 * M * r * (N + K)),
        ]

    def stash_bytes(self):
        return None

    def config(self):
        p = self.p
        return {"workload": p["name"], "tokens": p["M"], "N": p["N"], "K": p["K"], "lora_rank": p["r"],
                "lora_scale": p["lora_scale"], "step": "Q(X), forward GEMM, Q(dY), input-gradient GEMM"}


def cpu_baseline_layer(S, li, sample_tokens):
    """The oracle, as it stands, on the first `sample_tokens` tokens of one
    layer of the same workload (every step of the data flow is per token, so
    this is the same computation on a smaller batch)."""
    import oracle
    names = list(S.projections().keys())
    rows = np.arange(sample_tokens)
    KV = S.kv
    t0 = time.perf_counter()
    Wf, Wb = {}, {}
    for n in names:
        Wf[n], Wb[n] = oracle.build_weight_layouts(li.W[n])
    t_layout = time.perf_counter() - t0
    x = li.x[rows]
    dout = li.dout[rows]
    fw = lambda aq, X, nm, C=None: oracle.gemm_fwd(aq, X, Wf[nm], li.A[nm], li.B[nm], S.lora_scale, C)
    dg = lambda gq, dY, nm, C=None: oracle.gemm_dgrad(gq, dY, Wb[nm], li.A[nm], li.B[nm], S.lora_scale, C)

    def step():
        """The GPU step's schedule, call for call (grouped forwards are per projection here)."""
        n1, n1q, rstd1 = oracle.rmsnorm_quant(x, li.gamma1, S.eps)
        q = fw(n1q, n1, "q")
        fw(n1q, n1, "k")
        fw(n1q, n1, "v")
        x2 = fw(oracle.quantize_bf16(q), q, "o", x)
        n2, n2q, rstd2 = oracle.rmsnorm_quant(x2, li.gamma2, S.eps)
        g = fw(n2q, n2, "gate")
        u = fw(n2q, n2, "up")
        h, hq, gq, uq = oracle.silu_mul_quant(g, u)
        fw(hq, h, "down", x2)
        dh = dg(oracle.quantize_bf16(dout), dout, "down")
        dgr, du, dgq, duq = oracle.silu_mul_bwd_quant(dh, gq, uq)
        dn2 = dg(duq, du, "up", dg(dgq, dgr, "gate"))
        dx2, dx2q = oracle.rmsnorm_bwd(dn2, n2q, li.gamma2, rstd2, dout)
        da = dg(dx2q, dx2, "o")
        dk, dv = np.ascontiguousarray(da[:, :KV]), np.ascontiguousarray(da[:, KV:2 * KV])
        dn1 = dg(oracle.quantize_bf16(da), da, "q")
        dn1 = dg(oracle.quantize_bf16(dk), dk, "k", dn1)
        dn1 = dg(oracle.quantize_bf16(dv), dv, "v", dn1)
        oracle.rmsnorm_bwd(dn1, n1q, li.gamma1, rstd1, dx2)

    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        step()
        times.append(time.perf_counter() - t0)
    t_step = float(np.median(times))
    flops = 2 * sum(2 * sample_tokens * n * k for n, k in S.projections().values())
    return {"value": flops / t_step / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{sample_tokens} of {S.tokens} tokens through one full layer step, the GPU step's "
                      f"schedule (fwd + input-gradient: 14 GEMMs with LoRA, quantizers, norms, SiLU and "
                      f"RMSNorm backward), median of 3 runs; weight layouts built once outside the timed "
                      f"part ({t_layout:.1f} s)",
            "seconds": t_step, "tokens_per_s": sample_tokens / t_step}


def cpu_baseline_linear(lin):
    import oracle
    li, s = lin.li, lin.li.s
    wf, wb = oracle.build_weight_layouts(li.W)
    t0 = time.perf_counter()
    reps = 0
    while True:
        xq = oracle.quantize_bf16(li.X)
        oracle.gemm_fwd(xq, li.X, wf, li.A, li.B, s)
        dyq = oracle.quantize_bf16(li.dY)
        oracle.gemm_dgrad(dyq, li.dY, wb, li.A, li.B, s)
        reps += 1
        if time.perf_counter() - t0 > 5.0:
            break
    t_step = (time.perf_counter() - t0) / reps
    flops = 2 * 2 * lin.M * lin.N * lin.K
    return {"value": flops / t_step / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"the whole step, repeated {reps} times",
            "seconds": t_step * reps, "tokens_per_s": lin.M / t_step}


def isolated_timing(torch, calls, reps=10):
    """Cold-cache timing of the memory-bound kernels: for the largest call of
    each kind, each repetition first reads a 512 MiB buffer (twice the 256 MB
    Infinity Cache) with a reduction kernel, then times the call alone with
    events on its stream.  Reports the median.  The read pass evicts what the
    caches held, writing back what was dirty, before the timed region, so the
    call starts with its inputs in HBM only and with nothing of its own to
    write back.  (Overwriting the buffer instead would leave the cache full of
    dirty lines whose write-back the timed call would pay for.)"""
    flush = torch.zeros((512 << 20) // 4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    out = {}
    for kind in ("rmsnorm_quant", "quantize", "silu_mul_quant", "silu_mul_bwd", "rmsnorm_bwd", "adamw"):
        cs = [c for c in calls if c[0] == kind]
        if not cs:
            continue
        c = max(cs, key=lambda c: c[2])
        ts = []
        for _ in range(reps + 1):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            c[3]()
            b.record(st)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ms = float(np.median(ts[1:]))
        gbs = c[2] / (ms * 1e-3) / 1e9
        out[kind] = {"bytes": c[2], "median_us": ms * 1e3, "GB/s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}
    del flush
    return out


# Algorithmic (read, write) bytes per element of each row kernel's largest
# call (per-row scalars left out): the inputs it must read and the outputs it
# must write, as in the kernels' roofline table.
ROW_MIX = {"quantize": (2.0, 0.5625), "rmsnorm_quant": (2.0, 2.5625), "silu_mul_quant": (4.0, 3.6875),
           "silu_mul_bwd": (3.125, 5.125), "rmsnorm_bwd": (4.5625, 2.5625), "adamw": (16.0, 14.0)}


def hbm_ceiling(torch, calls, reps=10):
    """The HBM ceiling of each row kernel's read/write mix.  For the largest
    call of each kind, pact_debug_stream moves the same total bytes split in
    the kernel's read:write ratio, with the same cold-cache protocol as
    isolated_timing (a 512 MiB read pass before every timed repetition); the
    kernel's own cold-cache rate is then given as a fraction of that
    ceiling.  Plain read-only, write-only and copy streams of 1 GiB are
    reported beside them."""
    from nvfp4_gemm_amd import pact as pb
    kern = isolated_timing(torch, calls, reps)
    flush = torch.zeros((512 << 20) // 4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()

    def timed(rb, wb):
        src = torch.arange(max(rb, 16) // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty(max(wb, 16) // 4, dtype=torch.int32, device="cuda")
        ts = []
        for _ in range(reps + 1):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            pb.pact_debug_stream(src if rb else None, rb, dst, wb)
            b.record(st)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ms = float(np.median(ts[1:]))
        return {"read_bytes": rb, "write_bytes": wb, "median_us": ms * 1e3,
                "GB/s": (rb + wb) / (ms * 1e-3) / 1e9}

    out = {"streams_1GiB": {"read_only": timed(1 << 30, 0), "write_only": timed(0, 1 << 30),
                            "copy": timed(1 << 30, 1 << 30)}}
    for kind, k in kern.items():
        rd, wr = ROW_MIX[kind]
        rb = int(k["bytes"] * rd / (rd + wr)) // 16 * 16
        wb = (k["bytes"] - rb) // 16 * 16
        s = timed(rb, wb)
        out[kind] = {"kernel_bytes": k["bytes"], "kernel_us": k["median_us"], "kernel_GB/s": k["GB/s"],
                     "kernel_frac_of_8TBs": k["hbm_frac"], "stream_same_mix": s,
                     "kernel_frac_of_stream": k["GB/s"] / s["GB/s"]}
    del flush
    return out


def library_gemm(args):
    """One layer's frozen GEMMs (forward and input gradient, grouped as in the
    step) timed two ways on the same GPU: libpact's NVFP4 entry points (frozen
    GEMM plus the fused rank-r LoRA, from packed codes and scales) and the
    vendor library's FP16 GEMM on FP16 operands of the same shape (torch's
    F.linear with the weight as N x K rows, and a @ b with b as K x N; the
    faster of the two counts).  Both rates are frozen FLOPs 2 M N K over the
    mean time of 20 back-to-back calls."""
    import torch
    import torch.nn.functional as F
    from nvfp4_gemm_amd import synth
    if args.config == "single_linear":
        sys.exit("--library-gemm takes a layer configuration")
    shape = synth.LAYERS[args.config]
    M, H, I, KV = shape.tokens, shape.hidden, shape.inter, shape.kv
    # (entry point, N, K) in the order of the step's GEMM calls
    gemms = [("fwd qkv", H + 2 * KV, H), ("fwd o", H, H), ("fwd gate|up", 2 * I, H), ("fwd down", H, I),
             ("dgrad down", I, H), ("dgrad gate", H, I), ("dgrad up", H, I), ("dgrad o", H, H),
             ("dgrad q", H, H), ("dgrad k", H, KV), ("dgrad v", H, KV)]
    work = Stack(shape, args.seed, 1)
    ours = [c for c in work.calls() if c[0] in ("gemm_fwd", "gemm_dgrad")]
    assert len(ours) == len(gemms), len(ours)
    for c, (nm, n, k) in zip(ours, gemms):
        assert c[1] == 2 * M * n * k, (nm, c[1])
    for c in work.calls():      # the step once, so every input of the GEMM calls is set
        c[3]()
    st = torch.cuda.current_stream()

    def timed(fn, reps=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3   # us

    g = torch.Generator(device="cuda").manual_seed(args.seed)
    print(f"workload {work.config()['workload']}: one layer's frozen GEMMs, M = {M}")
    print(f"{'entry point':<12} {'N':>6} {'K':>6}  {'NVFP4 us':>9} {'TFLOP/s':>8}  {'lib FP16 us':>11} {'TFLOP/s':>8}"
          f"  {'ratio':>5}")
    tot = [0.0, 0.0, 0]
    for c, (nm, n, k) in zip(ours, gemms):
        us_ours = timed(c[3])
        x = torch.randn(M, k, dtype=torch.float16, device="cuda", generator=g)
        w = torch.randn(n, k, dtype=torch.float16, device="cuda", generator=g)
        wt = w.t().contiguous()
        us_lib = min(timed(lambda: F.linear(x, w)), timed(lambda: x @ wt))
        del x, w, wt
        fl = 2 * M * n * k
        tot[0] += us_ours
        tot[1] += us_lib
        tot[2] += fl
        print(f"{nm:<12} {n:>6} {k:>6}  {us_ours:>9.1f} {fl / us_ours / 1e6:>8.1f}  {us_lib:>11.1f} "
              f"{fl / us_lib / 1e6:>8.1f}  {us_lib / us_ours:>5.2f}", flush=True)
    r_ours, r_lib = tot[2] / tot[0] / 1e6, tot[2] / tot[1] / 1e6
    print(f"{'layer total':<26} {tot[0]:>9.1f} {r_ours:>8.1f}  {tot[1]:>11.1f} {r_lib:>8.1f}  {tot[1] / tot[0]:>5.2f}")
    print(f"fraction of the {PEAK_F16_MFMA_TFLOPS:.0f} TFLOP/s dense FP16 MFMA peak: NVFP4 entry points "
          f"{r_ours / PEAK_F16_MFMA_TFLOPS:.3f}, library FP16 GEMM {r_lib / PEAK_F16_MFMA_TFLOPS:.3f}")


def gemm_source_sha():
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_summary(workload):
    """HBM bytes per GEMM launch from the committed counter summary, when it
    was taken on the current GEMM source (else None)."""
    path = os.path.join(ROOT, "profiles", f"gemm_hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("gemm_source_sha256") != gemm_source_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_gemm_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib):
    """A plain device copy of known size, for calibrating the traffic counters."""
    import torch
    n = mib << 20
    src = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n}), flush=True)


def _pmc_rows(d, counter):
    dbs = glob.glob(os.path.join(d, "**", "*.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {d}")
    con = sqlite3.connect(dbs[0])
    return con.execute("select name, dispatch_id, counter_value from pmc_events where counter_name = ?",
                       (counter,)).fetchall()


def summarize_pmc(args):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch, summed over the device) of
    the GEMM kernels, scaled by what the same counters read for the copy."""
    fdir, wdir, cfdir, cwdir = args.summarize_pmc

    def gemm_totals(d, counter):
        """Traffic of the GEMM entry points' kernels and the number of entry
        points: main-kernel dispatches, less the second launches of
        column-split plans (a main kernel without K split whose preceding
        dispatch is a main kernel; every other entry point starts with its
        LoRA-down or, when that is fused, with a K-split main kernel)."""
        tot, names = 0.0, {}
        for name, did, v in _pmc_rows(d, counter):
            names[did] = name
            if any(m in name for m in GEMM_KERNELS):
                tot += v
        is_main = lambda n: any(m in n for m in GEMM_MAIN_KERNELS)
        second = re.compile(r"gemm_kernel<\d+, \d+, \d+, (true|false), false>")
        order = sorted(names)
        entries = 0
        for i, did in enumerate(order):
            n = names[did]
            if not is_main(n):
                continue
            if i > 0 and second.search(n) and is_main(names[order[i - 1]]):
                continue
            entries += 1
        return tot, entries

    def copy_kib(d, counter):
        vals = {}
        for name, did, v in _pmc_rows(d, counter):
            if "copy" in name.lower() or "elementwise" in name.lower():
                vals[did] = vals.get(did, 0.0) + v
        if not vals:
            raise SystemExit(f"no copy kernel dispatch in {d}")
        return max(vals.values())

    copy_bytes = args.copy_bytes
    cf, cw = copy_kib(cfdir, "FETCH_SIZE"), copy_kib(cwdir, "WRITE_SIZE")
    f_fetch, f_write = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    fetch, nf = gemm_totals(fdir, "FETCH_SIZE")
    write, nw = gemm_totals(wdir, "WRITE_SIZE")
    hbm = fetch * 1024.0 * f_fetch / nf + write * 1024.0 * f_write / nw
    lines = [
        "# HBM traffic of the NVFP4 GEMM entry points (LoRA-down, main and split-K epilogue kernels),",
        "# from rocprofv3 FETCH_SIZE and WRITE_SIZE counter runs, each scaled by the value",
        "# the same counter reads for a plain device copy of known size.",
        f"command: {args.pmc_command}",
        f"gemm_source_sha256: {gemm_source_sha()}",
        f"copy_bytes: {copy_bytes}",
        f"copy_fetch_kib: {cf:.1f}",
        f"copy_write_kib: {cw:.1f}",
        f"fetch_scale: {f_fetch:.4f}",
        f"write_scale: {f_write:.4f}",
        f"gemm_launches: {nf}",
        f"gemm_fetch_kib_total: {fetch:.1f}",
        f"gemm_write_kib_total: {write:.1f}",
        f"hbm_bytes_per_gemm_launch: {hbm:.1f}",
    ]
    text = "\n".join(lines) + "\n"
    if args.pmc_out:
        with open(args.pmc_out, "w") as f:
            f.write(text)
    print(text, end="")


# Row-kernel calls of the 3B-shaped layers (M = 8192, hidden 3072, intermediate
# 8192, kv 1024): kernel instantiation -> (call, rows, cols, algorithmic bytes
# per element, bytes per row), as in the kernels' roofline table.
ROW_CALLS_3B = {
    "row_kernel<1, 3, 1>": ("RMSNorm-quantize 8192x3072", 8192, 3072, 2.0 + 2.5625, 8),
    "row_kernel<1, 3, 0>": ("quantize 8192x3072", 8192, 3072, 2.5625, 4),
    "row_kernel<1, 1, 0>": ("quantize 8192x1024", 8192, 1024, 2.5625, 4),
    "row_kernel<4, 2, 2>": ("SiLU-multiply-quantize 8192x8192", 8192, 8192, 4.0 + 3.6875, 12),
    "bwd_kernel<8, 1, 3>": ("SiLU-multiply backward 8192x8192", 8192, 8192, 3.125 + 5.125, 16),
    "bwd_kernel<1, 3, 4>": ("RMSNorm backward 8192x3072 (+ residual)", 8192, 3072, 4.5625 + 2.5625, 12),
}


def summarize_row_pmc(args):
    """FETCH_SIZE / WRITE_SIZE per dispatch of each row kernel, scaled by the
    copy calibration, against its algorithmic bytes; durations from the
    kernel-trace statistics of the same workload."""
    fdir, wdir, cfdir, cwdir, stats = args.summarize_row_pmc

    def copy_kib(d, counter):
        vals = {}
        for name, did, v in _pmc_rows(d, counter):
            if "copy" in name.lower() or "elementwise" in name.lower():
                vals[did] = vals.get(did, 0.0) + v
        return max(vals.values())

    def per_kernel(d, counter):
        acc = {}
        for name, did, v in _pmc_rows(d, counter):
            for k in ROW_CALLS_3B:
                if k in name:
                    a = acc.setdefault(k, {})
                    a[did] = a.get(did, 0.0) + v
        return {k: (len(a), sum(a.values()) / len(a)) for k, a in acc.items()}

    import csv
    avg_us = {}
    with open(stats) as f:
        for r in csv.DictReader(f):
            for k in ROW_CALLS_3B:
                if k in r["Name"]:
                    avg_us[k] = float(r["AverageNs"]) / 1e3
    sf = args.copy_bytes / (copy_kib(cfdir, "FETCH_SIZE") * 1024.0)
    sw = args.copy_bytes / (copy_kib(cwdir, "WRITE_SIZE") * 1024.0)
    fe, wr = per_kernel(fdir, "FETCH_SIZE"), per_kernel(wdir, "WRITE_SIZE")
    lines = ["# HBM traffic of the row kernels (fused quantizers and nonlinear backward) in the 28-layer",
             "# llama3.2-3b-shaped stack (M=8192): rocprofv3 FETCH_SIZE and WRITE_SIZE per dispatch (KiB, summed",
             "# over the device), each scaled by the value the same counter reads for a plain device copy,",
             "# against the algorithmic bytes (every input byte read once, every output byte written once).",
             "# Durations: the same workload's kernel trace (eager and graph-replayed steps).  Both counters",
             "# count traffic between L2 and the fabric, which includes Infinity-Cache (MALL) hits.",
             f"command: {args.pmc_command}",
             f"fetch_scale: {sf:.4f}  write_scale: {sw:.4f}", "",
             f"{'kernel':<24} {'call':<42} {'disp':>5} {'alg MB':>8} {'read MB':>8} {'write MB':>9} "
             f"{'cnt/alg':>8} {'avg us':>7} {'alg TB/s':>9} {'of 8':>6}"]
    for k, (call, rows, cols, per_el, per_row) in ROW_CALLS_3B.items():
        if k not in fe or k not in wr:
            continue
        alg = rows * cols * per_el + rows * per_row
        rd, wt = fe[k][1] * 1024.0 * sf, wr[k][1] * 1024.0 * sw
        us = avg_us.get(k, float("nan"))
        tbs = alg / (us * 1e-6) / 1e12
        lines.append(f"{k:<24} {call:<42} {fe[k][0]:>5} {alg / 1e6:>8.1f} {rd / 1e6:>8.1f} {wt / 1e6:>9.1f} "
                     f"{(rd + wt) / alg:>8.2f} {us:>7.1f} {tbs:>9.2f} {tbs / 8.0:>6.3f}")
    text = "\n".join(lines) + "\n"
    if args.pmc_out:
        with open(args.pmc_out, "w") as f:
            f.write(text)
    print(text, end="")


def summarize_coverage(args):
    """Every kernel instantiation compiled into libpact.so, from hipcc's
    resource-usage remarks on each source (compiled again for this, same
    flags), against the number of launches of each in the kernel-trace
    statistics of one run of the GPU test suite."""
    import csv
    import subprocess
    from nvfp4_gemm_amd import build as B
    os.makedirs(B.BUILD, exist_ok=True)
    compiled = []
    for src in B.SOURCES:
        r = subprocess.run([B.HIPCC, *B.FLAGS, "-I", B.BUILD, "-c", os.path.join(B.CSRC, src), "-o", os.devnull,
                            "-Rpass-analysis=kernel-resource-usage"], capture_output=True, text=True)
        names = re.findall(r"Function Name: (\S+)", r.stderr)
        if r.returncode != 0:
            raise SystemExit(f"hipcc failed for {src}: {r.stderr[-400:]}")
        if not names:  # a source without kernels (the version and status strings)
            continue
        dem = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True).stdout.split("\n")
        compiled += [(src, d.strip()) for d in dem if d.strip()]
    tidy = lambda n: n.replace("pact::", "").replace("(anonymous namespace)::", "").strip().strip('"')
    launches = {}
    with open(args.summarize_coverage) as f:
        for r in csv.DictReader(f):
            launches[tidy(r["Name"])] = launches.get(tidy(r["Name"]), 0) + int(r["Calls"])
    lines = ["# Kernel-variant coverage of the GPU test suite: every kernel instantiation compiled into libpact.so",
             "# (from the compiler's resource-usage remarks, per source file) and how many times the kernel trace of",
             "# one run of the GPU test suite saw it launched.",
             f"command: {args.pmc_command}", "", f"{'source':<20} {'launches':>9}  kernel"]
    seen = 0
    for src, k in compiled:
        key = tidy(k)
        n = launches.get(key, 0)
        if n == 0:  # the trace prints 'void ' before templates; the demangler does not
            n = launches.get("void " + key, 0)
        seen += n > 0
        lines.append(f"{src:<20} {n:>9}  {key}")
    lines += ["", f"# {len(compiled)} compiled kernels, {seen} launched"]
    text = "\n".join(lines) + "\n"
    if args.pmc_out:
        with open(args.pmc_out, "w") as f:
            f.write(text)
    print(text, end="")


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_coverage:
        summarize_coverage(args)
        return
    if args.summarize_row_pmc:
        summarize_row_pmc(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only (--gpus 1): every step of the data flow is row-parallel, so "
              "tokens would shard across GPUs with no exchange in the forward and input-gradient passes, "
              "but runs on more than one GPU are not supported here.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.library_gemm:
        library_gemm(args)
        return
    import torch
    from nvfp4_gemm_amd import synth
    if args.config == "single_linear":
        work = Linear(args.seed)
    else:
        shape = synth.LAYERS[args.config]
        work = Stack(shape, args.seed, shape.layers, lora_grads=args.lora_grads, grouped=not args.ungrouped)
    st = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    calls = work.calls()
    if args.hbm_ceiling:
        for c in calls:  # one untimed pass: every output written once
            c[3]()
        torch.cuda.synchronize()
        print(json.dumps({"workload": work.config()["workload"], "hbm_ceiling": hbm_ceiling(torch, calls)}),
              flush=True)
        return
    torch.cuda.reset_peak_memory_stats()
    cpu_s = 0.0
    for _ in range(args.warmup):
        t0 = time.perf_counter()
        for c in calls:
            c[3]()
        cpu_s = max(cpu_s, time.perf_counter() - t0)
        torch.cuda.synchronize()
    # timed region: events around every call, on the stream the kernels run
    # on.  Each step starts behind a bounded GPU spin about twice as long as
    # the host takes to issue the step, so that the step's calls are queued
    # before the GPU reaches them and each event pair times device work only
    # (without it the small layers' per-call times would include the host's
    # launch latency).  The eager step time runs from the end of the spin.
    spin_cycles = int(min(max(2.0 * cpu_s, 1e-3), 0.2) * 2.4e9)
    evs = [[(ev(), ev()) for _ in calls] for _ in range(args.steps)]
    t_begin = [ev() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        torch.cuda._sleep(spin_cycles)
        t_begin[s].record(st)
        for (a, b), c in zip(evs[s], calls):
            a.record(st)
            c[3]()
            b.record(st)
    torch.cuda.synchronize()
    eager_ms_step = sum(t_begin[s].elapsed_time(evs[s][-1][1]) for s in range(args.steps)) / args.steps
    ms_step = eager_ms_step
    timing = "eager"
    if not args.eager:
        side = torch.cuda.Stream()
        side.wait_stream(st)
        with torch.cuda.stream(side):
            for c in calls:
                c[3]()
        st.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in calls:
                c[3]()
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = ev(), ev()
        g0.record(st)
        for _ in range(args.steps):
            graph.replay()
        g1.record(st)
        torch.cuda.synchronize()
        ms_step = g0.elapsed_time(g1) / args.steps
        timing = "hip_graph_replay"
        del graph
    peak_hbm = torch.cuda.max_memory_allocated()
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
        elif k["lora_flops"]:
            d["lora_tflops"] = k["lora_flops"] / (k["ms"] * 1e-3) / 1e12
        if k["bytes"]:
            # algorithmic bytes over in-step time: inputs written just before
            # can still be in the Infinity Cache, so this is not HBM bandwidth
            # (the cache-flushed figures are under kernels_isolated_cache_flushed)
            gbs = k["bytes"] / (k["ms"] * 1e-3) / 1e9
            d["alg_GB/s"] = gbs
            d["alg_frac_of_hbm_peak"] = gbs / PEAK_HBM_GBS
        kinds[kind] = d
    cfg = work.config()
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "step_timing": timing,
        "eager_ms_per_step": eager_ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": cfg,
        "tokens_per_s": work.M / (ms_step * 1e-3),
        "frozen_gemm_tflops_kernel_time": gemm["flops"] / (gemm["ms"] * 1e-3) / 1e12,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_F16_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_F16_MFMA_TFLOPS,
                     "traffic": traffic_summary(cfg["workload"]),
                     "kernel": "NVFP4 GEMM entry points (fwd + dgrad: LoRA-down + main GEMM kernels), "
                               "frozen + LoRA FLOPs per launch / mean launch time",
                     "traffic_unit": "HBM bytes per GEMM launch",
                     "fp4_peak_context": PEAK_FP4_TFLOPS},
        "kernels": kinds,
        "layout_build_ms": work.layout_ms,
        "peak_hbm_bytes": peak_hbm,
    }
    sb = work.stash_bytes()
    if sb:
        out["stash_bytes"] = {"pact_nvfp4": sb[0], "bf16_lora": sb[1], "ratio": sb[1] / sb[0]}
    if not args.no_isolated:
        out["kernels_isolated_cache_flushed"] = isolated_timing(torch, calls)
    if not args.no_cpu_baseline:
        if args.config == "single_linear":
            out["cpu_baseline"] = cpu_baseline_linear(work)
        else:
            # about 10-30 s of oracle work on the host: 1024 tokens of the
            # smaller layers, 512 of the 3B-shaped ones (403 MFLOP per token)
            per_token = 2 * sum(2 * n_ * k_ for n_, k_ in work.S.projections().values())
            n = args.cpu_sample_tokens or min(work.M, 1024 if per_token < 3e8 else 512)
            out["cpu_baseline"] = cpu_baseline_layer(work.S, work.li0, n)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
