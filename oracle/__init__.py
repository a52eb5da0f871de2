"""CPU oracle for the NVFP4 frozen-projection data flow of PACT.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product path
(``nvfp4_gemm_amd``) never imports it and shares no code with it.

The arithmetic lives in plain C (``pact_oracle.c``), compiled with gcc
``-O2 -ffp-contract=off -fopenmp`` (no fast-math); this module only builds that
library and marshals numpy arrays into it.  BF16 tensors are numpy ``uint16``
arrays of raw bit patterns.

Sources: the PACT blog post on simolm.com (sections "Method" and "FAQ"), the
arXiv abstract page of "PACT: NVFP4 Data-Flow LoRA Fine-Tuning on Consumer
GPUs", and the kongchang.com PEFT explainer (LoRA low-rank math).  Each C
function cites the passage it follows.

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pact_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no GPU involved)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
               "-shared", "-std=gnu11", "-Wall", _SRC, "-o", tmp, "-lquadmath", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.orc_e2m1_value.restype = ctypes.c_float
        L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_value.restype = ctypes.c_float
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_encode_mag.restype = ctypes.c_uint8
        L.orc_e2m1_encode_mag.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_quantize_rows_f32.argtypes = [P, I64, I64, I64, P, P, P]
        L.orc_quantize_rows_bf16.argtypes = [P, I64, I64, I64, P, P, P]
        L.orc_operand_values.argtypes = [P, P, I64, I64, P]
        L.orc_dequantize.argtypes = [P, P, P, I64, I64, P]
        L.orc_rmsnorm_quant.argtypes = [P, I64, P, ctypes.c_float, I64, I64, P, P, P, P, P]
        L.orc_sumsq_bf16.restype = ctypes.c_double
        L.orc_sumsq_bf16.argtypes = [P, I64]
        L.orc_sigmoid_mul_g.restype = ctypes.c_float
        L.orc_sigmoid_mul_g.argtypes = [ctypes.c_uint16]
        L.orc_sigmoid_check_table.restype = ctypes.c_int
        L.orc_silu_mul_quant.argtypes = [P, P, I64, I64, I64, P] + [P] * 9
        L.orc_build_weight_layouts.argtypes = [P, I64, I64] + [P] * 6 + [ctypes.c_int]
        gemm_args = [P, P, P, P, I64, I64, P, P, P, I64, P, P, ctypes.c_int32,
                     ctypes.c_float, P, P, I64, P]
        L.orc_gemm_fwd.argtypes = gemm_args
        L.orc_gemm_dgrad.argtypes = gemm_args
        L.orc_dsilu.restype = ctypes.c_float
        L.orc_dsilu.argtypes = [ctypes.c_uint16]
        L.orc_dsilu_check_table.restype = ctypes.c_int
        L.orc_silu_mul_bwd_quant.argtypes = [P, I64, I64, I64] + [P] * 6 + [P, P] + [P] * 6
        L.orc_dot_bf16_f32.restype = ctypes.c_double
        L.orc_dot_bf16_f32.argtypes = [P, P, I64]
        L.orc_rmsnorm_bwd.argtypes = [P, I64, P, P, P, P, P, P, I64, I64, I64, P, P, P, P]
        L.orc_lora_grads.argtypes = [P, P, P, I64, I64, P, I64, I64, P, P, ctypes.c_int32, ctypes.c_float, P, P]
        D = ctypes.c_double
        L.orc_adamw_step.argtypes = [P, P, P, P, I64, D, D, D, D, D, I64]
        L.orc_master_bf16.argtypes = [P, I64, P]
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_gptq_sweep.argtypes = [P, P, P, I64, I64, ctypes.c_int32, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


@dataclass
class NVFP4:
    """Canonical NVFP4 tensor: codes [rows, cols/2] (element 2j in the low
    nibble of byte j), E4M3 scale bytes [rows, cols/16], FP32 row scale [rows]."""
    codes: np.ndarray
    scales: np.ndarray
    d: np.ndarray

    @property
    def rows(self):
        return self.codes.shape[0]

    @property
    def cols(self):
        return self.codes.shape[1] * 2

    @staticmethod
    def empty(rows, cols):
        return NVFP4(np.zeros((rows, cols // 2), np.uint8),
                     np.zeros((rows, cols // 16), np.uint8),
                     np.zeros((rows,), np.float32))


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ---- element formats ------------------------------------------------------
def e2m1_value(code: int) -> float:
    return float(lib().orc_e2m1_value(code))


def e4m3_value(b: int) -> float:
    return float(lib().orc_e4m3_value(b))


def e2m1_encode_mag(r: float) -> int:
    return int(lib().orc_e2m1_encode_mag(r))


def e4m3_encode(t: float) -> int:
    return int(lib().orc_e4m3_encode(t))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x) -> int:
    return int(lib().orc_f32_to_bf16(float(np.float32(x))))


# ---- quantizer ------------------------------------------------------------
def quantize_bf16(x: np.ndarray) -> NVFP4:
    x = _c(x, np.uint16)
    rows, cols = x.shape
    if cols % 16:
        raise ValueError("row length must be a multiple of 16")
    out = NVFP4.empty(rows, cols)
    lib().orc_quantize_rows_bf16(_p(x), cols, rows, cols, _p(out.codes), _p(out.scales), _p(out.d))
    return out


def quantize_f32(x: np.ndarray) -> NVFP4:
    x = _c(x, np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle quantizer takes finite inputs only")
    rows, cols = x.shape
    out = NVFP4.empty(rows, cols)
    lib().orc_quantize_rows_f32(_p(x), cols, rows, cols, _p(out.codes), _p(out.scales), _p(out.d))
    return out


def operand_values(q: NVFP4) -> np.ndarray:
    b = np.zeros((q.rows, q.cols), np.float32)
    lib().orc_operand_values(_p(_c(q.codes, np.uint8)), _p(_c(q.scales, np.uint8)),
                             q.rows, q.cols, _p(b))
    return b


def dequantize(q: NVFP4) -> np.ndarray:
    out = np.zeros((q.rows, q.cols), np.float32)
    lib().orc_dequantize(_p(_c(q.codes, np.uint8)), _p(_c(q.scales, np.uint8)),
                         _p(_c(q.d, np.float32)), q.rows, q.cols, _p(out))
    return out


# ---- fused producers ------------------------------------------------------
def sumsq_bf16(x: np.ndarray) -> float:
    x = _c(x, np.uint16)
    return float(lib().orc_sumsq_bf16(_p(x), x.size))


def rmsnorm_quant(x: np.ndarray, gamma: np.ndarray, eps: float):
    """Returns (y bf16 bits [rows, cols], yq NVFP4, rstd f32 [rows])."""
    x = _c(x, np.uint16)
    gamma = _c(gamma, np.uint16)
    rows, cols = x.shape
    y = np.zeros((rows, cols), np.uint16)
    yq = NVFP4.empty(rows, cols)
    rstd = np.zeros((rows,), np.float32)
    lib().orc_rmsnorm_quant(_p(x), cols, _p(gamma), float(eps), rows, cols, _p(y),
                            _p(yq.codes), _p(yq.scales), _p(yq.d), _p(rstd))
    return y, yq, rstd


def sigmoid_table() -> np.ndarray:
    """sigma32(g) = g/(1+exp(-g)) correctly rounded to binary32, for all 65536
    BF16 bit patterns (NaN at non-finite patterns)."""
    L = lib()
    if L.orc_sigmoid_check_table() != 0:
        raise RuntimeError("oracle sigmoid table has inputs too close to a rounding boundary")
    return np.array([L.orc_sigmoid_mul_g(b) for b in range(65536)], np.float32)


def silu_mul_quant(g: np.ndarray, u: np.ndarray, want_stash: bool = True):
    """Returns (h bf16 bits, hq, gq, uq) with gq/uq None if not wanted."""
    g = _c(g, np.uint16)
    u = _c(u, np.uint16)
    rows, cols = g.shape
    assert u.shape == g.shape
    h = np.zeros((rows, cols), np.uint16)
    hq = NVFP4.empty(rows, cols)
    gq = NVFP4.empty(rows, cols) if want_stash else None
    uq = NVFP4.empty(rows, cols) if want_stash else None
    args = [_p(hq.codes), _p(hq.scales), _p(hq.d)]
    for q in (gq, uq):
        args += [_p(q.codes), _p(q.scales), _p(q.d)] if q is not None else [None] * 3
    lib().orc_silu_mul_quant(_p(g), _p(u), cols, rows, cols, _p(h), *args)
    return h, hq, gq, uq


def build_weight_layouts(W: np.ndarray | None = None, W_fwd: NVFP4 | None = None):
    """Returns (W_fwd NVFP4 [N,K], W_bwd NVFP4 [K,N])."""
    if W is not None:
        W = _c(W, np.uint16)
        N, K = W.shape
        if N % 16 or K % 16:
            raise ValueError("weight layouts need N and K multiples of 16")
        fwd = NVFP4.empty(N, K)
        use_given = 0
    else:
        N, K = W_fwd.rows, W_fwd.cols
        fwd = NVFP4(_c(W_fwd.codes, np.uint8).copy(), _c(W_fwd.scales, np.uint8).copy(),
                    _c(W_fwd.d, np.float32).copy())
        use_given = 1
    bwd = NVFP4.empty(K, N)
    lib().orc_build_weight_layouts(_p(W), N, K, _p(fwd.codes), _p(fwd.scales), _p(fwd.d),
                                   _p(bwd.codes), _p(bwd.scales), _p(bwd.d), use_given)
    return fwd, bwd


# ---- GEMMs ----------------------------------------------------------------
def _gemm(fn, aq: NVFP4, Xl, bq: NVFP4, A, B, s, C, rows):
    M, Kc = aq.rows, aq.cols
    Nout = bq.rows
    assert bq.cols == Kc
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = _c(rows, np.int64)
    r = 0 if A is None else int(A.shape[0])
    out = np.zeros((rows.size, Nout), np.uint16)
    Xl = None if Xl is None else _c(Xl, np.uint16)
    A = None if A is None else _c(A, np.uint16)
    B = None if B is None else _c(B, np.uint16)
    C = None if C is None else _c(C, np.uint16)
    if r > 0:
        assert Xl is not None and B is not None
    fn(_p(_c(aq.codes, np.uint8)), _p(_c(aq.scales, np.uint8)), _p(_c(aq.d, np.float32)),
       _p(Xl), M, Kc,
       _p(_c(bq.codes, np.uint8)), _p(_c(bq.scales, np.uint8)), _p(_c(bq.d, np.float32)), Nout,
       _p(A), _p(B), r, float(s), _p(C), _p(rows), rows.size, _p(out))
    return out


def gemm_fwd(xq: NVFP4, X, wq: NVFP4, A=None, B=None, s=1.0, C=None, rows=None):
    """Y = bf16(d_x d_w (Xq . Wq^T) + s (bf16(X A^T)) B^T (+ C)) for the listed rows.
    X [M,K] bf16 (LoRA input), A [r,K], B [N,r] bf16, C [M,N] bf16 or None."""
    return _gemm(lib().orc_gemm_fwd, xq, X, wq, A, B, s, C, rows)


def gemm_dgrad(dyq: NVFP4, dY, wbq: NVFP4, A=None, B=None, s=1.0, C=None, rows=None):
    """dX = bf16(d_dy d_wb (dYq . Wb^T) + s (bf16(dY B)) A (+ C)) for the listed rows.
    dY [M,N] bf16, W_bwd [K,N], A [r,K], B [N,r], C [M,K] or None."""
    return _gemm(lib().orc_gemm_dgrad, dyq, dY, wbq, A, B, s, C, rows)


# ---- nonlinear backward from the NVFP4 stash ------------------------------
def dsilu_table() -> np.ndarray:
    """d/dg (g sigma(g)) correctly rounded to binary32 for all 65536 BF16 bit
    patterns (NaN at non-finite patterns)."""
    L = lib()
    if L.orc_dsilu_check_table() != 0:
        raise RuntimeError("oracle dsilu table has inputs too close to a rounding boundary")
    return np.array([L.orc_dsilu(b) for b in range(65536)], np.float32)


def silu_mul_bwd_quant(dh: np.ndarray, gq: NVFP4, uq: NVFP4):
    """Returns (dg bf16 bits, du bf16 bits, dgq, duq) from dh and the gate/up stash."""
    dh = _c(dh, np.uint16)
    rows, cols = dh.shape
    assert (gq.rows, gq.cols) == (rows, cols) and (uq.rows, uq.cols) == (rows, cols)
    dg = np.zeros((rows, cols), np.uint16)
    du = np.zeros((rows, cols), np.uint16)
    dgq, duq = NVFP4.empty(rows, cols), NVFP4.empty(rows, cols)
    lib().orc_silu_mul_bwd_quant(
        _p(dh), cols, rows, cols,
        _p(_c(gq.codes, np.uint8)), _p(_c(gq.scales, np.uint8)), _p(_c(gq.d, np.float32)),
        _p(_c(uq.codes, np.uint8)), _p(_c(uq.scales, np.uint8)), _p(_c(uq.d, np.float32)),
        _p(dg), _p(du), _p(dgq.codes), _p(dgq.scales), _p(dgq.d), _p(duq.codes), _p(duq.scales),
        _p(duq.d))
    return dg, du, dgq, duq


def dot_bf16_f32(a: np.ndarray, b: np.ndarray) -> float:
    a = _c(a, np.uint16)
    b = _c(b, np.float32)
    assert a.size == b.size
    return float(lib().orc_dot_bf16_f32(_p(a), _p(b), a.size))


def rmsnorm_bwd(dy: np.ndarray, yq: NVFP4, gamma: np.ndarray, rstd: np.ndarray, C=None):
    """Returns (dx bf16 bits, dxq) from dy, the NVFP4 norm output, gamma and rstd."""
    dy = _c(dy, np.uint16)
    rows, cols = dy.shape
    assert (yq.rows, yq.cols) == (rows, cols)
    dx = np.zeros((rows, cols), np.uint16)
    dxq = NVFP4.empty(rows, cols)
    Cc = _c(C, np.uint16) if C is not None else None
    lib().orc_rmsnorm_bwd(_p(dy), cols, _p(_c(yq.codes, np.uint8)), _p(_c(yq.scales, np.uint8)),
                          _p(_c(yq.d, np.float32)), _p(_c(gamma, np.uint16)), _p(_c(rstd, np.float32)),
                          _p(Cc), cols, rows, cols, _p(dx), _p(dxq.codes), _p(dxq.scales), _p(dxq.d))
    return dx, dxq


# ---- LoRA weight gradients on the NVFP4 stash --------------------------------
def lora_grads(xq: NVFP4, dY: np.ndarray, A: np.ndarray, B: np.ndarray, s: float):
    """Returns (dA [r,K], dB [N,r]) in float64: dB = dY^T T^, dA = T'^T X^ with
    X^ = bf16(deq(xq)), T^ = s bf16(X^ A^T), T' = s bf16(dY B)."""
    dY = _c(dY, np.uint16)
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    M, N = dY.shape
    r, K = A.shape
    assert (xq.rows, xq.cols) == (M, K) and B.shape == (N, r)
    dA = np.zeros((r, K), np.float64)
    dB = np.zeros((N, r), np.float64)
    lib().orc_lora_grads(_p(_c(xq.codes, np.uint8)), _p(_c(xq.scales, np.uint8)), _p(_c(xq.d, np.float32)),
                         M, K, _p(dY), N, N, _p(A), _p(B), r, float(s), _p(dA), _p(dB))
    return dA, dB


# ---- optimizer --------------------------------------------------------------
def adamw_step(p, m, v, g, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float, step: int):
    """One AdamW step in binary64 on copies of (p, m, v); returns the new
    (p, m, v) as float64 arrays."""
    p = np.array(p, dtype=np.float64, copy=True).ravel()
    m = np.array(m, dtype=np.float64, copy=True).ravel()
    v = np.array(v, dtype=np.float64, copy=True).ravel()
    g = np.ascontiguousarray(np.asarray(g, dtype=np.float64).ravel())
    assert p.size == m.size == v.size == g.size
    lib().orc_adamw_step(_p(p), _p(m), _p(v), _p(g), p.size, float(lr), float(beta1), float(beta2), float(eps),
                         float(weight_decay), int(step))
    return p, m, v


def bf16_of_master(p) -> np.ndarray:
    """BF16 bits of the FP32 master copy of p: bf16(fl32(p))."""
    x = np.ascontiguousarray(np.asarray(p, dtype=np.float64))
    out = np.empty(x.shape, np.uint16)
    lib().orc_master_bf16(_p(x), x.size, _p(out))
    return out


# ---- NVFP4-adapted GPTQ (blog "Method", bullet 3; arXiv abstract) ---------
# Offline calibration of a frozen weight W [N, K] from calibration activations
# X [n, K]: the Hessian of the layer's output error is taken over the
# reconstructed NVFP4 activations X^ = deq(Q(X)) (the GEMM's actual input),
# H = (2/n) X^T X^; GPTQ (Frantar et al.) then quantizes W column by column,
# spreading each column's rounding error over the columns not yet quantized
# through the upper Cholesky factor of H^-1.  Linear algebra in binary64
# (numpy's matmul, Cholesky and inverse as library steps); the sweep is the
# C function orc_gptq_sweep.

def gptq_hessian(xq: NVFP4, scale: float | None = None) -> np.ndarray:
    """H = scale X^T X (binary64) over the dequantized NVFP4 rows X of xq;
    scale defaults to 2/n (n = rows of xq)."""
    X = dequantize(xq).astype(np.float64)
    if scale is None:
        scale = 2.0 / max(X.shape[0], 1)
    return scale * (X.T @ X)


def gptq_inverse_factor(H: np.ndarray, percdamp: float = 0.01):
    """GPTQ's preparation of H (copied): columns with zero diagonal are dead
    (their diagonal set to 1, their weights to 0); percdamp times the mean
    diagonal is added to the diagonal; then U, the upper Cholesky factor of
    H^-1 (H^-1 = U^T U), through H = L L^T, H^-1 = L^-T L^-1.
    Returns (U, dead mask)."""
    H = np.array(H, dtype=np.float64, copy=True)
    K = H.shape[0]
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    damp = percdamp * np.mean(np.diag(H))
    H[np.arange(K), np.arange(K)] += damp
    L = np.linalg.cholesky(H)
    Linv = np.linalg.inv(L)
    Hinv = Linv.T @ Linv
    U = np.linalg.cholesky(Hinv).T
    return np.ascontiguousarray(U), dead


def gptq_nvfp4(W: np.ndarray, H: np.ndarray, blocksize: int = 128, percdamp: float = 0.01) -> NVFP4:
    """NVFP4 forward layout of the BF16 weight W [N, K] calibrated by GPTQ
    with Hessian H [K, K]: row scales d of the plain quantizer (from W's row
    maxima), block scales and codes chosen column by column by the sweep."""
    W = _c(W, np.uint16)
    N, K = W.shape
    rtn = quantize_bf16(W)  # row scales d = fl32(max|w| / 2688)
    U, dead = gptq_inverse_factor(H, percdamp)
    Wd = bf16_to_f32(W).astype(np.float64)
    Wd[:, dead] = 0.0
    Wd = np.ascontiguousarray(Wd)
    out = NVFP4.empty(N, K)
    out.d[:] = rtn.d
    lib().orc_gptq_sweep(_p(U), _p(Wd), _p(_c(out.d, np.float32)), N, K, int(blocksize), _p(out.codes),
                         _p(out.scales))
    return out
