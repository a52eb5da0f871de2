"""Seeded synthetic inputs for the NVFP4 frozen-projection data flow.

This module holds only input generation (numpy ``default_rng``), none of the
method's arithmetic, so that the CPU oracle and the HIP path are fed the very
same bytes.  BF16 tensors are returned as numpy ``uint16`` bit patterns.

Shapes follow the models the PACT pages evaluate (Llama-3.2-1B/3B and
Qwen2.5-1.5B, blog section "Results"); the value distributions are the
workload definitions this library is measured on (Student-t activations,
N(0, 0.02^2) weights with 0.1% outliers x20, BF16 LoRA adapters).  No dataset
item is reproduced: everything is drawn from the seeds below.

Recipe (one ``SeedSequence(seed).spawn`` child per tensor, in a fixed order):
samples are drawn in float64, rounded to float32 (round-to-nearest-even), then
to BF16 (round-to-nearest-even).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def to_bf16_bits(a) -> np.ndarray:
    """float array -> BF16 bit patterns (RNE via float32)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    kept = u >> 16
    dropped = u & 0xFFFF
    up = (dropped > 0x8000) | ((dropped == 0x8000) & ((kept & 1) == 1))
    return (kept + up.astype(np.uint64)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class LayerShape:
    """One decoder layer's frozen projections (N, K) and token count M."""
    name: str
    hidden: int
    inter: int
    kv: int
    tokens: int
    rank: int
    act_nu: float | None       # Student-t degrees of freedom (None: N(0,1))
    act_scale: float
    eps: float
    layers: int = 1
    lora_scale: float = 2.0

    def projections(self):
        H, I, KV = self.hidden, self.inter, self.kv
        return {"q": (H, H), "k": (KV, H), "v": (KV, H), "o": (H, H),
                "gate": (I, H), "up": (I, H), "down": (H, I)}

    def frozen_flops_fwd(self):
        return sum(2 * self.tokens * n * k for n, k in self.projections().values())


# The single LoRA linear and the four layer workloads.
SINGLE_LINEAR = dict(name="single_nvfp4_lora_linear_M256_N1024_K512_r8",
                     M=256, N=1024, K=512, r=8, lora_scale=2.0, seed=0)

LAYERS = {
    "llama1b_layer": LayerShape("llama3.2-1b-shaped_layer_M1024", 2048, 8192, 512, 1024, 16,
                                4.0, 0.5, 1e-5),
    "qwen1.5b_layer": LayerShape("qwen2.5-1.5b-shaped_layer_M4096", 1536, 8960, 256, 4096, 16,
                                 4.0, 0.5, 1e-6),
    "llama3b_layer": LayerShape("llama3.2-3b-shaped_layer_M8192", 3072, 8192, 1024, 8192, 32,
                                3.0, 0.5, 1e-5),
    "llama3b_stack28": LayerShape("llama3.2-3b-shaped_28layer_stack_M8192", 3072, 8192, 1024,
                                  8192, 16, None, 1.0, 1e-5, layers=28),
}


def _rngs(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def normal_bf16(rng, shape, std):
    return to_bf16_bits(rng.standard_normal(shape) * std)


def student_t_bf16(rng, shape, nu, scale):
    return to_bf16_bits(rng.standard_t(nu, size=shape) * scale)


def weight_bf16(rng, n, k, std=0.02, outlier_frac=0.001, outlier_mult=20.0):
    """N(0, std^2) with exactly round(frac*n*k) entries (without replacement) x mult."""
    w = rng.standard_normal((n, k)) * std
    n_out = int(round(outlier_frac * n * k))
    if n_out:
        idx = rng.choice(n * k, size=n_out, replace=False)
        w.reshape(-1)[idx] *= outlier_mult
    return to_bf16_bits(w)


@dataclass
class LinearInputs:
    X: np.ndarray
    W: np.ndarray
    A: np.ndarray
    B: np.ndarray
    dY: np.ndarray
    s: float


def single_linear_inputs(M=256, N=1024, K=512, r=8, s=2.0, seed=0, act="normal",
                         outliers=False) -> LinearInputs:
    """X [M,K] ~ N(0,1); W [N,K] ~ N(0,0.02^2); A [r,K] ~ N(0,0.02^2);
    B [N,r] ~ N(0,0.01^2); dY [M,N] ~ N(0,1).  act='t4' draws X from t(4)*0.5."""
    g = _rngs(seed, 5)
    if act == "normal":
        X = normal_bf16(g[0], (M, K), 1.0)
    else:
        X = student_t_bf16(g[0], (M, K), float(act[1:]), 0.5)
    W = weight_bf16(g[1], N, K, outlier_frac=0.001 if outliers else 0.0)
    A = normal_bf16(g[2], (r, K), 0.02)
    B = normal_bf16(g[3], (N, r), 0.01)
    dY = normal_bf16(g[4], (M, N), 1.0)
    return LinearInputs(X, W, A, B, dY, s)


@dataclass
class LayerInputs:
    shape: LayerShape
    x: np.ndarray                      # [M, H] layer input
    gamma1: np.ndarray                 # [H]
    gamma2: np.ndarray                 # [H]
    W: dict = field(default_factory=dict)      # name -> [N, K] bf16
    A: dict = field(default_factory=dict)      # name -> [r, K]
    B: dict = field(default_factory=dict)      # name -> [N, r]
    dout: np.ndarray | None = None     # [M, H] incoming gradient


def layer_inputs(shape: LayerShape, seed: int = 0, layer: int = 0, M: int | None = None,
                 with_weights: bool = True) -> LayerInputs:
    """Inputs of one decoder layer.  ``layer`` selects an independent weight set
    (stack workloads); ``M`` overrides the token count (smaller parity cases)."""
    M = shape.tokens if M is None else M
    H = shape.hidden
    names = list(shape.projections().keys())
    g = _rngs(seed * 1000 + layer, 4 + 3 * len(names))
    if shape.act_nu is None:
        x = normal_bf16(g[0], (M, H), shape.act_scale)
    else:
        x = student_t_bf16(g[0], (M, H), shape.act_nu, shape.act_scale)
    gamma1 = to_bf16_bits(1.0 + 0.1 * g[1].standard_normal(H))
    gamma2 = to_bf16_bits(1.0 + 0.1 * g[2].standard_normal(H))
    dout = normal_bf16(g[3], (M, H), 1.0)
    li = LayerInputs(shape, x, gamma1, gamma2, dout=dout)
    if with_weights:
        for i, nm in enumerate(names):
            n, k = shape.projections()[nm]
            li.W[nm] = weight_bf16(g[4 + 3 * i], n, k)
            li.A[nm] = normal_bf16(g[5 + 3 * i], (shape.rank, k), 0.02)
            li.B[nm] = normal_bf16(g[6 + 3 * i], (n, shape.rank), 0.01)
    return li


def calibration_bf16(rng, n, K, nu=4.0, scale=0.5, rank=32, mix=1.0):
    """Calibration activations [n, K] for the offline weight calibration:
    Student-t(nu) * scale noise plus a shared low-rank component (rank
    N(0, 1) factors with N(0, (scale mix)^2 / rank) loadings), so that the
    columns are correlated as a layer's inputs are."""
    Z = rng.standard_t(nu, size=(n, K)) * scale
    F = rng.standard_normal((n, rank))
    P = rng.standard_normal((rank, K)) * (scale * mix / np.sqrt(rank))
    return to_bf16_bits(Z + F @ P)
