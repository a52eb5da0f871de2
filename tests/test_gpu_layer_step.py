"""Teacher-forced parity of whole layer steps: the benchmark's own schedule
(bench.Stack.calls(): fused RMSNorm and SiLU-multiply quantizers, grouped and
single forward GEMMs with the BF16 LoRA term, input-gradient GEMMs, the
SiLU-multiply and RMSNorm backward from the NVFP4 stash, the LoRA weight
gradients and the AdamW step) runs call by call on the GPU, and after every
call the oracle recomputes that call from the GPU's own inputs, so errors
never compound.  Quantized outputs, BF16 norm/activation outputs and rstd must
be bit-exact (in full); GEMM outputs must meet the GEMM tolerance on sampled
rows (|d| <= 2 ulp_bf16 + 1e-3 max_row|ref|, relative Frobenius <= 4e-3).
(simolm.com PACT blog, "Method"; arXiv abstract of "PACT: NVFP4 Data-Flow
LoRA Fine-Tuning on Consumer GPUs".)

Workloads: the Llama-1B-shaped layer (M = 1024, with LoRA gradients and
AdamW), the Qwen-1.5B-shaped layer (M = 4096), the Llama-3B-shaped layer
(M = 8192, r = 32) and one layer of the 28-layer 3B-shaped stack (M = 8192,
r = 16, N(0, 1) input).
"""
import inspect

import numpy as np
import pytest
import torch

import bench
import oracle
from nvfp4_gemm_amd import pact as pb
from nvfp4_gemm_amd import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _nv(t: pb.NVFP4Tensor, r0=0, r1=None) -> oracle.NVFP4:
    h = G.host_nvfp4(t)
    return oracle.NVFP4(h.codes[r0:r1], h.scales[r0:r1], h.d[r0:r1])


def _h(t):
    return None if t is None else G.host_bits(t)


class Checker:
    """Stands in for the binding module inside bench.Stack: every entry point
    is called for real, then checked against the oracle on the inputs the GPU
    saw.  Attributes other than the wrapped entry points pass through."""

    WRAPPED = ("pact_quantize_nvfp4", "pact_rmsnorm_quant_nvfp4", "pact_silu_mul_quant_nvfp4",
               "pact_gemm_nvfp4_fwd", "pact_gemm_nvfp4_fwd_grouped", "pact_gemm_nvfp4_dgrad",
               "pact_silu_mul_bwd_quant_nvfp4", "pact_rmsnorm_bwd_nvfp4", "pact_lora_grads_nvfp4",
               "pact_adamw_step")

    def __init__(self, M, nsample=20, seed=0):
        rng = np.random.default_rng(seed)
        self.rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, nsample)])).astype(np.int64)
        self.counts = {}

    def __getattr__(self, name):
        fn = getattr(pb, name)
        if name not in self.WRAPPED:
            return fn
        check = getattr(self, "_" + name)
        sig = inspect.signature(fn)

        def wrapped(*args, **kwargs):
            ba = sig.bind(*args, **kwargs)
            ba.apply_defaults()
            torch.cuda.synchronize()
            pre = self._inputs(name, ba.arguments)
            out = fn(*args, **kwargs)
            torch.cuda.synchronize()
            check(ba.arguments, pre, out)
            self.counts[name] = self.counts.get(name, 0) + 1
            return out
        return wrapped

    # host copies of the inputs, taken before the call (outputs may alias inputs)
    def _inputs(self, name, a):
        if name == "pact_quantize_nvfp4":
            return {"x": _h(a["x"])}
        if name == "pact_rmsnorm_quant_nvfp4":
            return {"x": _h(a["x"]), "gamma": _h(a["gamma"])}
        if name == "pact_silu_mul_quant_nvfp4":
            return {"g": _h(a["g"]), "u": _h(a["u"])}
        if name in ("pact_gemm_nvfp4_fwd", "pact_gemm_nvfp4_dgrad"):
            aq, bq = (a["Xq"], a["W_fwd"]) if name.endswith("fwd") else (a["dYq"], a["W_bwd"])
            X = a["X"] if name.endswith("fwd") else a["dY"]
            L = a["lora"]
            return {"aq": _nv(aq), "bq": _nv(bq), "X": _h(X), "C": _h(a["C"]),
                    "A": _h(L.A) if L else None, "B": _h(L.B) if L else None, "s": L.scale if L else 1.0}
        if name == "pact_gemm_nvfp4_fwd_grouped":
            loras = a["loras"] or []
            return {"aq": _nv(a["Xq"]), "W": G.host_nvfp4(a["W_cat"]), "X": _h(a["X"]),
                    "AB": [(_h(L.A), _h(L.B), L.scale) for L in loras]}
        if name == "pact_silu_mul_bwd_quant_nvfp4":
            return {"dh": _h(a["dh"]), "gq": _nv(a["gq"]), "uq": _nv(a["uq"])}
        if name == "pact_rmsnorm_bwd_nvfp4":
            return {"dy": _h(a["dy"]), "yq": _nv(a["yq"]), "gamma": _h(a["gamma"]),
                    "rstd": a["rstd"].cpu().numpy(), "C": _h(a["C"])}
        if name == "pact_lora_grads_nvfp4":
            L = a["lora"]
            return {"xq": _nv(a["Xq"]), "dY": _h(a["dY"]), "A": _h(L.A), "B": _h(L.B), "s": L.scale}
        if name == "pact_adamw_step":
            return {k: a[k].cpu().numpy().copy() for k in ("p", "m", "v", "g")}
        raise AssertionError(name)

    def _pact_quantize_nvfp4(self, a, pre, out):
        G.assert_nvfp4_equal(out, oracle.quantize_bf16(pre["x"]), "quantize")

    def _pact_rmsnorm_quant_nvfp4(self, a, pre, out):
        y, yq, rstd = oracle.rmsnorm_quant(pre["x"], pre["gamma"], a["eps"])
        gy, gyq, grstd = out
        np.testing.assert_array_equal(G.host_bits(gy), y)
        G.assert_nvfp4_equal(gyq, yq, "rmsnorm yq")
        np.testing.assert_array_equal(grstd.cpu().numpy().view(np.uint32), rstd.view(np.uint32))

    def _pact_silu_mul_quant_nvfp4(self, a, pre, out):
        h, hq, gq, uq = oracle.silu_mul_quant(pre["g"], pre["u"])
        gh, ghq, ggq, guq = out
        np.testing.assert_array_equal(G.host_bits(gh), h)
        G.assert_nvfp4_equal(ghq, hq, "silu hq")
        G.assert_nvfp4_equal(ggq, gq, "silu gq")
        G.assert_nvfp4_equal(guq, uq, "silu uq")

    def _gemm(self, fn, pre, out, what):
        ref = fn(pre["aq"], pre["X"], pre["bq"], pre["A"], pre["B"], pre["s"], pre["C"], rows=self.rows)
        G.check_gemm_tolerance(G.host_bits(out)[self.rows], ref, what)

    def _pact_gemm_nvfp4_fwd(self, a, pre, out):
        self._gemm(oracle.gemm_fwd, pre, out, "fwd")

    def _pact_gemm_nvfp4_dgrad(self, a, pre, out):
        self._gemm(oracle.gemm_dgrad, pre, out, "dgrad")

    def _pact_gemm_nvfp4_fwd_grouped(self, a, pre, out):
        Y = G.host_bits(out)[self.rows]
        W = pre["W"]
        c = 0
        for g, n in enumerate(a["group_rows"]):
            wq = oracle.NVFP4(W.codes[c:c + n], W.scales[c:c + n], W.d[c:c + n])
            A, B, s = pre["AB"][g] if pre["AB"] else (None, None, 1.0)
            ref = oracle.gemm_fwd(pre["aq"], pre["X"], wq, A, B, s, rows=self.rows)
            G.check_gemm_tolerance(np.ascontiguousarray(Y[:, c:c + n]), ref, f"grouped fwd group {g}")
            c += n

    def _pact_silu_mul_bwd_quant_nvfp4(self, a, pre, out):
        dg, du, dgq, duq = oracle.silu_mul_bwd_quant(pre["dh"], pre["gq"], pre["uq"])
        gdg, gdu, gdgq, gduq = out
        np.testing.assert_array_equal(G.host_bits(gdg), dg)
        np.testing.assert_array_equal(G.host_bits(gdu), du)
        G.assert_nvfp4_equal(gdgq, dgq, "silu bwd dgq")
        G.assert_nvfp4_equal(gduq, duq, "silu bwd duq")

    def _pact_rmsnorm_bwd_nvfp4(self, a, pre, out):
        dx, dxq = oracle.rmsnorm_bwd(pre["dy"], pre["yq"], pre["gamma"], pre["rstd"], pre["C"])
        gdx, gdxq = out
        np.testing.assert_array_equal(G.host_bits(gdx), dx)
        if gdxq is not None:
            G.assert_nvfp4_equal(gdxq, dxq, "rmsnorm bwd dxq")

    def _pact_lora_grads_nvfp4(self, a, pre, out):
        dA, dB = oracle.lora_grads(pre["xq"], pre["dY"], pre["A"], pre["B"], pre["s"])
        G.check_lora_grads(out[0], out[1], dA, dB, "layer step")

    def _pact_adamw_step(self, a, pre, out):
        p, m, v, g = pre["p"], pre["m"], pre["v"], pre["g"]
        rp, rm, rv = oracle.adamw_step(p, m, v, g, lr=float(np.float32(a["lr"])),
                                       beta1=float(np.float32(a["beta1"])), beta2=float(np.float32(a["beta2"])),
                                       eps=float(np.float32(a["eps"])),
                                       weight_decay=float(np.float32(a["weight_decay"])), step=a["step"])
        gp, gm, gv = (a[k].cpu().numpy().astype(np.float64) for k in ("p", "m", "v"))
        assert np.max(np.abs(gm - rm)) <= 2.0 ** -20 * (np.max(np.abs(rm)) + 1e-30)
        assert np.max(np.abs(gv - rv)) <= 2.0 ** -20 * (np.max(np.abs(rv)) + 1e-30)
        assert np.max(np.abs(gp - rp)) <= 2.0 ** -18 * (np.max(np.abs(rp)) + 1e-3)
        if a["w"] is not None:
            w = G.host_bits(a["w"].view(1, -1))[0]
            np.testing.assert_array_equal(w, oracle.bf16_of_master(gp.astype(np.float32)))


@pytest.mark.parametrize("workload,layers_override,lora_grads", [
    ("llama1b_layer", None, True),
    ("qwen1.5b_layer", None, False),
    ("llama3b_layer", None, False),
    ("llama3b_stack28", 1, False),
])
def test_layer_step_teacher_forced(workload, layers_override, lora_grads):
    shape = synth.LAYERS[workload]
    layers = layers_override or shape.layers
    print(f"layer step {workload} layers={layers} lora_grads={lora_grads}", flush=True)
    st = bench.Stack(shape, 0, layers, lora_grads=lora_grads, grouped=True)
    # the cached layouts of layer 0, bit-exact against the oracle's
    li = st.li0
    for n in st.names:
        f, b = oracle.build_weight_layouts(li.W[n])
        G.assert_nvfp4_equal(st.Wb[0][n], b, f"W_bwd {n}")
    ck = Checker(shape.tokens)
    st.pb = ck
    calls = st.calls()
    for c in calls:
        c[3]()
    torch.cuda.synchronize()
    # every call of the step was checked
    expect = {"pact_rmsnorm_quant_nvfp4": 2, "pact_silu_mul_quant_nvfp4": 1,
              "pact_gemm_nvfp4_fwd": 2, "pact_gemm_nvfp4_fwd_grouped": 2, "pact_gemm_nvfp4_dgrad": 7,
              "pact_silu_mul_bwd_quant_nvfp4": 1, "pact_rmsnorm_bwd_nvfp4": 2}
    if lora_grads:
        expect.update({"pact_lora_grads_nvfp4": 7, "pact_adamw_step": 1})
    expect = {k: v * layers for k, v in expect.items()}
    expect["pact_quantize_nvfp4"] = 4 * layers + 1   # Q(a), Q(dq), Q(dk), Q(dv) per layer; Q(dout) once
    if lora_grads:
        expect["pact_adamw_step"] = 1
    assert ck.counts == expect, ck.counts
