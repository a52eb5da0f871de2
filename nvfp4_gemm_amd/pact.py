"""Thin ctypes binding of libpact (include/pact.h).

Argument marshalling only: every step of the data flow runs in libpact's HIP
kernels.  PyTorch supplies device memory (tensors) and the stream.  If the
built library is missing the binding raises; there is no CPU fallback.

BF16 tensors are ``torch.bfloat16`` CUDA tensors (row-major, last stride 1);
NVFP4 tensors are :class:`NVFP4Tensor` (codes / scales / row_scale tensors).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpact.so")
_lib = None

P = ctypes.c_void_p
I64 = ctypes.c_int64


class pact_nvfp4(ctypes.Structure):
    _fields_ = [("codes", P), ("scales", P), ("row_scale", P), ("rows", I64), ("cols", I64)]


class pact_lora(ctypes.Structure):
    _fields_ = [("A", P), ("B", P), ("r", ctypes.c_int32), ("scale", ctypes.c_float)]


STATUS = {0: "PACT_OK", 1: "PACT_ERR_INVALID_ARG", 2: "PACT_ERR_UNSUPPORTED_SHAPE",
          3: "PACT_ERR_MISALIGNED", 4: "PACT_ERR_WORKSPACE", 5: "PACT_ERR_HIP"}

EXPORTS = ["pact_version", "pact_status_string", "pact_quantize_nvfp4",
           "pact_rmsnorm_quant_nvfp4", "pact_silu_mul_quant_nvfp4",
           "pact_build_weight_layouts_workspace", "pact_build_weight_layouts",
           "pact_gemm_workspace", "pact_gemm_nvfp4_fwd", "pact_gemm_nvfp4_dgrad",
           "pact_debug_sigmoid32", "pact_debug_gemm_plan", "pact_silu_mul_bwd_quant_nvfp4",
           "pact_rmsnorm_bwd_nvfp4", "pact_debug_dsilu32", "pact_lora_grads_workspace",
           "pact_lora_grads_nvfp4", "pact_adamw_step", "pact_gemm_nvfp4_fwd_grouped",
           "pact_debug_lora_down_plan", "pact_noalloc_scratch_bytes", "pact_gemm_nvfp4_fwd_noalloc",
           "pact_debug_gemm_plan_columns", "pact_gptq_hessian_nvfp4", "pact_gptq_workspace", "pact_gptq_nvfp4",
           "pact_debug_row_plan", "pact_debug_stream"]


class PactError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


def lib():
    """Load libpact.so (built in-tree by nvfp4_gemm_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libpact.so not built ({LIB_PATH}); run nvfp4_gemm_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        NV = ctypes.POINTER(pact_nvfp4)
        LO = ctypes.POINTER(pact_lora)
        st = ctypes.c_int
        L.pact_version.restype = ctypes.c_int
        L.pact_status_string.restype = ctypes.c_char_p
        L.pact_status_string.argtypes = [ctypes.c_int]
        L.pact_quantize_nvfp4.restype = st
        L.pact_quantize_nvfp4.argtypes = [P, I64, I64, I64, NV, P]
        L.pact_rmsnorm_quant_nvfp4.restype = st
        L.pact_rmsnorm_quant_nvfp4.argtypes = [P, I64, P, ctypes.c_float, I64, I64, P, I64, NV, P, P]
        L.pact_silu_mul_quant_nvfp4.restype = st
        L.pact_silu_mul_quant_nvfp4.argtypes = [P, I64, P, I64, I64, I64, P, I64, NV, NV, NV, P]
        L.pact_build_weight_layouts_workspace.restype = ctypes.c_size_t
        L.pact_build_weight_layouts_workspace.argtypes = [I64, I64]
        L.pact_build_weight_layouts.restype = st
        L.pact_build_weight_layouts.argtypes = [P, NV, I64, I64, NV, NV, P, ctypes.c_size_t, P]
        L.pact_gemm_workspace.restype = ctypes.c_size_t
        L.pact_gemm_workspace.argtypes = [I64, I64, I64, ctypes.c_int32]
        gemm_args = [NV, P, I64, NV, LO, P, P, I64, P, ctypes.c_size_t, P]
        L.pact_gemm_nvfp4_fwd.restype = st
        L.pact_gemm_nvfp4_fwd.argtypes = gemm_args
        L.pact_gemm_nvfp4_dgrad.restype = st
        L.pact_gemm_nvfp4_dgrad.argtypes = gemm_args
        L.pact_debug_sigmoid32.restype = st
        L.pact_debug_sigmoid32.argtypes = [P, P, I64, P]
        L.pact_silu_mul_bwd_quant_nvfp4.restype = st
        L.pact_silu_mul_bwd_quant_nvfp4.argtypes = [P, I64, NV, NV, I64, I64, P, P, I64, NV, NV, P]
        L.pact_rmsnorm_bwd_nvfp4.restype = st
        L.pact_rmsnorm_bwd_nvfp4.argtypes = [P, I64, NV, P, P, P, I64, I64, I64, P, I64, NV, P]
        L.pact_lora_grads_workspace.restype = ctypes.c_size_t
        L.pact_lora_grads_workspace.argtypes = [I64, I64, I64, ctypes.c_int32]
        L.pact_lora_grads_nvfp4.restype = st
        L.pact_lora_grads_nvfp4.argtypes = [NV, P, I64, I64, LO, P, P, P, P, ctypes.c_size_t, P]
        L.pact_gemm_nvfp4_fwd_grouped.restype = st
        L.pact_gemm_nvfp4_fwd_grouped.argtypes = [NV, P, I64, NV, ctypes.c_int32, ctypes.POINTER(I64),
                                                  LO, P, I64, P, ctypes.c_size_t, P]
        L.pact_adamw_step.restype = st
        L.pact_adamw_step.argtypes = [P, P, P, P, P, I64, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, I64, P]
        L.pact_debug_dsilu32.restype = st
        L.pact_debug_dsilu32.argtypes = [P, P, I64, P]
        L.pact_debug_stream.restype = st
        L.pact_debug_stream.argtypes = [P, I64, P, I64, P]
        L.pact_debug_gemm_plan.restype = st
        L.pact_debug_gemm_plan.argtypes = [I64, I64, I64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_int32)]
        D = ctypes.c_double
        L.pact_gptq_hessian_nvfp4.restype = st
        L.pact_gptq_hessian_nvfp4.argtypes = [NV, D, ctypes.c_int32, P, P]
        L.pact_gptq_workspace.restype = ctypes.c_size_t
        L.pact_gptq_workspace.argtypes = [I64, I64]
        L.pact_gptq_nvfp4.restype = st
        L.pact_gptq_nvfp4.argtypes = [P, I64, I64, I64, P, D, ctypes.c_int32, NV, P, ctypes.c_size_t, P]
        L.pact_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.pact_noalloc_scratch_bytes.argtypes = []
        L.pact_gemm_nvfp4_fwd_noalloc.restype = st
        L.pact_gemm_nvfp4_fwd_noalloc.argtypes = [NV, P, I64, NV, LO, P, P, I64, P]
        I32P = ctypes.POINTER(ctypes.c_int32)
        L.pact_debug_gemm_plan_columns.restype = st
        L.pact_debug_gemm_plan_columns.argtypes = [I64, I64, I64, ctypes.c_int32, ctypes.c_int32, I32P, I32P]
        L.pact_debug_row_plan.restype = st
        L.pact_debug_row_plan.argtypes = [ctypes.c_int32, I64, I32P, I32P]
        L.pact_debug_lora_down_plan.restype = st
        L.pact_debug_lora_down_plan.argtypes = [I64, I64, I64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                I32P, I32P, I32P, I32P, I32P]
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != 0:
        raise PactError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ld(t):
    assert t.dim() == 2 and t.stride(1) == 1, "row-major 2-D tensor expected"
    return t.stride(0)


@dataclass
class NVFP4Tensor:
    """codes uint8 [rows, cols/2], scales uint8 [rows, cols/16] (E4M3 bytes),
    row_scale float32 [rows]."""
    codes: torch.Tensor
    scales: torch.Tensor
    row_scale: torch.Tensor

    @property
    def rows(self):
        return self.codes.shape[0]

    @property
    def cols(self):
        return self.codes.shape[1] * 2

    @staticmethod
    def empty(rows: int, cols: int, device="cuda"):
        return NVFP4Tensor(torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
                           torch.empty((rows, cols // 16), dtype=torch.uint8, device=device),
                           torch.empty((rows,), dtype=torch.float32, device=device))

    def desc(self):
        return pact_nvfp4(self.codes.data_ptr(), self.scales.data_ptr(),
                          self.row_scale.data_ptr(), self.rows, self.cols)

    def nbytes(self):
        return self.codes.numel() + self.scales.numel() + 4 * self.row_scale.numel()

    @staticmethod
    def cat_rows(parts):
        """Row-wise concatenation (one copy), e.g. the forward layouts of the
        projections of a grouped GEMM."""
        return NVFP4Tensor(torch.cat([q.codes for q in parts]), torch.cat([q.scales for q in parts]),
                           torch.cat([q.row_scale for q in parts]))


def _desc_ref(q):
    return None if q is None else ctypes.byref(q.desc())


def pact_version() -> int:
    return int(lib().pact_version())


def pact_status_string(s: int) -> str:
    return lib().pact_status_string(s).decode()


def pact_quantize_nvfp4(x: torch.Tensor, out: NVFP4Tensor | None = None, stream=None):
    rows, cols = x.shape
    out = out if out is not None else NVFP4Tensor.empty(rows, cols, x.device)
    d = out.desc()
    _check(lib().pact_quantize_nvfp4(_ptr(x), _ld(x), rows, cols, ctypes.byref(d), _stream(stream)),
           "pact_quantize_nvfp4")
    return out


def pact_rmsnorm_quant_nvfp4(x, gamma, eps, y=None, yq=None, rstd=None, want_y=True,
                             want_rstd=True, stream=None):
    rows, cols = x.shape
    if y is None and want_y:
        y = torch.empty((rows, cols), dtype=torch.bfloat16, device=x.device)
    if yq is None:
        yq = NVFP4Tensor.empty(rows, cols, x.device)
    if rstd is None and want_rstd:
        rstd = torch.empty((rows,), dtype=torch.float32, device=x.device)
    d = yq.desc()
    _check(lib().pact_rmsnorm_quant_nvfp4(_ptr(x), _ld(x), _ptr(gamma), float(eps), rows, cols,
                                          _ptr(y), _ld(y) if y is not None else cols,
                                          ctypes.byref(d), _ptr(rstd), _stream(stream)),
           "pact_rmsnorm_quant_nvfp4")
    return y, yq, rstd


def pact_silu_mul_quant_nvfp4(g, u, h=None, hq=None, gq=None, uq=None, want_h=True,
                              want_stash=True, stream=None):
    rows, cols = g.shape
    if h is None and want_h:
        h = torch.empty((rows, cols), dtype=torch.bfloat16, device=g.device)
    if hq is None:
        hq = NVFP4Tensor.empty(rows, cols, g.device)
    if want_stash:
        gq = gq if gq is not None else NVFP4Tensor.empty(rows, cols, g.device)
        uq = uq if uq is not None else NVFP4Tensor.empty(rows, cols, g.device)
    dh, dg, du = hq.desc(), (gq.desc() if gq is not None else None), (uq.desc() if uq is not None else None)
    _check(lib().pact_silu_mul_quant_nvfp4(
        _ptr(g), _ld(g), _ptr(u), _ld(u), rows, cols, _ptr(h), _ld(h) if h is not None else cols,
        ctypes.byref(dh), ctypes.byref(dg) if dg is not None else None,
        ctypes.byref(du) if du is not None else None, _stream(stream)), "pact_silu_mul_quant_nvfp4")
    return h, hq, gq, uq


def pact_build_weight_layouts_workspace(N: int, K: int) -> int:
    return int(lib().pact_build_weight_layouts_workspace(N, K))


def pact_build_weight_layouts(W=None, W_fwd_in: NVFP4Tensor | None = None, N=None, K=None,
                              W_fwd=None, W_bwd=None, ws=None, stream=None):
    if W is not None:
        N, K = W.shape
        dev = W.device
    else:
        N, K = W_fwd_in.rows, W_fwd_in.cols
        dev = W_fwd_in.codes.device
    W_fwd = W_fwd if W_fwd is not None else NVFP4Tensor.empty(N, K, dev)
    W_bwd = W_bwd if W_bwd is not None else NVFP4Tensor.empty(K, N, dev)
    need = pact_build_weight_layouts_workspace(N, K)
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    df, db = W_fwd.desc(), W_bwd.desc()
    din = W_fwd_in.desc() if W_fwd_in is not None else None
    _check(lib().pact_build_weight_layouts(_ptr(W), ctypes.byref(din) if din is not None else None,
                                           N, K, ctypes.byref(df), ctypes.byref(db), _ptr(ws),
                                           ws.numel(), _stream(stream)),
           "pact_build_weight_layouts")
    return W_fwd, W_bwd


def pact_gemm_workspace(M: int, N: int, K: int, r: int) -> int:
    return int(lib().pact_gemm_workspace(M, N, K, r))


@dataclass
class LoRA:
    """BF16 adapters of one projection W [N, K]: A [r, K], B [N, r], scale."""
    A: torch.Tensor
    B: torch.Tensor
    scale: float

    @property
    def r(self):
        return self.A.shape[0]

    def desc(self):
        return pact_lora(self.A.data_ptr(), self.B.data_ptr(), self.r, float(self.scale))


def _gemm(fn, name, aq, Xl, bq, lora, C, out, ws, stream):
    M, Nout = aq.rows, bq.rows
    if out is None:
        out = torch.empty((M, Nout), dtype=torch.bfloat16, device=aq.codes.device)
    r = lora.r if lora is not None else 0
    if ws is None:
        need = pact_gemm_workspace(M, Nout, aq.cols, r)
        if need > 0:
            ws = torch.empty((need,), dtype=torch.uint8, device=aq.codes.device)
    da, db = aq.desc(), bq.desc()
    dl = lora.desc() if lora is not None else None
    _check(fn(ctypes.byref(da), _ptr(Xl), _ld(Xl) if Xl is not None else 0, ctypes.byref(db),
              ctypes.byref(dl) if dl is not None else None, _ptr(C), _ptr(out), _ld(out), _ptr(ws),
              ws.numel() if ws is not None else 0, _stream(stream)), name)
    return out


def pact_gemm_nvfp4_fwd(Xq: NVFP4Tensor, W_fwd: NVFP4Tensor, X=None, lora: LoRA | None = None,
                        C=None, Y=None, ws=None, stream=None):
    """Y = bf16(d_x d_w Xq.W_fwd^T + s bf16(X A^T) B^T (+ C))."""
    return _gemm(lib().pact_gemm_nvfp4_fwd, "pact_gemm_nvfp4_fwd", Xq, X, W_fwd, lora, C, Y, ws,
                 stream)


def pact_gptq_hessian_nvfp4(Xq: NVFP4Tensor, H=None, scale: float | None = None, accumulate: bool = False,
                            stream=None):
    """H [K][K] float64 = scale X^T X (+ H when accumulate) over the
    dequantized NVFP4 rows of Xq; scale defaults to 2 / rows."""
    K = Xq.cols
    if H is None:
        H = torch.empty((K, K), dtype=torch.float64, device=Xq.codes.device)
    if scale is None:
        scale = 2.0 / max(Xq.rows, 1)
    d = Xq.desc()
    _check(lib().pact_gptq_hessian_nvfp4(ctypes.byref(d), float(scale), 1 if accumulate else 0, _ptr(H),
                                         _stream(stream)), "pact_gptq_hessian_nvfp4")
    return H


def pact_gptq_workspace(N: int, K: int) -> int:
    return int(lib().pact_gptq_workspace(N, K))


def pact_gptq_nvfp4(W, H, percdamp: float = 0.01, blocksize: int = 128, W_fwd: NVFP4Tensor | None = None,
                    ws=None, stream=None) -> NVFP4Tensor:
    """GPTQ-calibrated forward NVFP4 layout of the BF16 weight W [N][K] with
    Hessian H [K][K] (float64; overwritten as scratch)."""
    N, K = W.shape
    W_fwd = W_fwd if W_fwd is not None else NVFP4Tensor.empty(N, K, W.device)
    if ws is None:
        ws = torch.empty((max(pact_gptq_workspace(N, K), 16),), dtype=torch.uint8, device=W.device)
    d = W_fwd.desc()
    _check(lib().pact_gptq_nvfp4(_ptr(W), _ld(W), N, K, _ptr(H), float(percdamp), int(blocksize), ctypes.byref(d),
                                 _ptr(ws), ws.numel(), _stream(stream)), "pact_gptq_nvfp4")
    return W_fwd


def pact_noalloc_scratch_bytes() -> int:
    return int(lib().pact_noalloc_scratch_bytes())


def pact_gemm_nvfp4_fwd_noalloc(Xq: NVFP4Tensor, W_fwd: NVFP4Tensor, X=None, lora: LoRA | None = None,
                                C=None, Y=None, stream=None):
    """pact_gemm_nvfp4_fwd with the library's own per-GPU workspace (the call
    allocates nothing; Y must be given for that)."""
    M, N = Xq.rows, W_fwd.rows
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=Xq.codes.device)
    da, db = Xq.desc(), W_fwd.desc()
    dl = lora.desc() if lora is not None else None
    _check(lib().pact_gemm_nvfp4_fwd_noalloc(ctypes.byref(da), _ptr(X), _ld(X) if X is not None else 0,
                                             ctypes.byref(db), ctypes.byref(dl) if dl is not None else None,
                                             _ptr(C), _ptr(Y), _ld(Y), _stream(stream)),
           "pact_gemm_nvfp4_fwd_noalloc")
    return Y


def pact_gemm_nvfp4_fwd_grouped(Xq: NVFP4Tensor, W_cat: NVFP4Tensor, group_rows, X=None, loras=None, Y=None,
                                ws=None, stream=None):
    """The projections of W_cat (rows group_rows[0], group_rows[1], ...) as one
    GEMM with a block-diagonal LoRA term: Y [M][sum group_rows]."""
    M, Nout = Xq.rows, W_cat.rows
    ng = len(group_rows)
    if Y is None:
        Y = torch.empty((M, Nout), dtype=torch.bfloat16, device=Xq.codes.device)
    r = loras[0].r if loras else 0
    if ws is None:
        need = pact_gemm_workspace(M, Nout, Xq.cols, ng * ((r + 15) // 16 * 16) if r else 0)
        if need > 0:
            ws = torch.empty((need,), dtype=torch.uint8, device=Xq.codes.device)
    rows = (ctypes.c_int64 * ng)(*[int(n) for n in group_rows])
    lo = (pact_lora * ng)(*[l.desc() for l in loras]) if loras else None
    dx, dw = Xq.desc(), W_cat.desc()
    _check(lib().pact_gemm_nvfp4_fwd_grouped(ctypes.byref(dx), _ptr(X), _ld(X) if X is not None else 0,
                                             ctypes.byref(dw), ng, rows, lo, _ptr(Y), _ld(Y), _ptr(ws),
                                             ws.numel() if ws is not None else 0, _stream(stream)),
           "pact_gemm_nvfp4_fwd_grouped")
    return Y


def pact_gemm_nvfp4_dgrad(dYq: NVFP4Tensor, W_bwd: NVFP4Tensor, dY=None, lora: LoRA | None = None,
                          C=None, dX=None, ws=None, stream=None):
    """dX = bf16(d_dy d_wb dYq.W_bwd^T + s bf16(dY B) A (+ C))."""
    return _gemm(lib().pact_gemm_nvfp4_dgrad, "pact_gemm_nvfp4_dgrad", dYq, dY, W_bwd, lora, C, dX,
                 ws, stream)


def pact_silu_mul_bwd_quant_nvfp4(dh, gq: NVFP4Tensor, uq: NVFP4Tensor, dg=None, du=None, dgq=None,
                                  duq=None, want_bf16=True, stream=None):
    """dg = bf16((dh u') dsilu32(g')), du = bf16(dh sigma32(g')) from the NVFP4
    gate/up stash (g', u' its BF16 values); dgq = Q(dg), duq = Q(du)."""
    rows, cols = dh.shape
    if want_bf16:
        dg = dg if dg is not None else torch.empty((rows, cols), dtype=torch.bfloat16, device=dh.device)
        du = du if du is not None else torch.empty((rows, cols), dtype=torch.bfloat16, device=dh.device)
    dgq = dgq if dgq is not None else NVFP4Tensor.empty(rows, cols, dh.device)
    duq = duq if duq is not None else NVFP4Tensor.empty(rows, cols, dh.device)
    if dg is not None and du is not None:
        assert _ld(dg) == _ld(du), "dg and du share one leading dimension"
    ld_out = _ld(dg) if dg is not None else (_ld(du) if du is not None else cols)
    a, b, c, d = gq.desc(), uq.desc(), dgq.desc(), duq.desc()
    _check(lib().pact_silu_mul_bwd_quant_nvfp4(
        _ptr(dh), _ld(dh), ctypes.byref(a), ctypes.byref(b), rows, cols, _ptr(dg), _ptr(du), ld_out,
        ctypes.byref(c), ctypes.byref(d), _stream(stream)), "pact_silu_mul_bwd_quant_nvfp4")
    return dg, du, dgq, duq


def pact_rmsnorm_bwd_nvfp4(dy, yq: NVFP4Tensor, gamma, rstd, C=None, dx=None, dxq=None, want_dx=True,
                           want_q=True, stream=None):
    """dx = bf16((dy gamma - x^ c) rstd (+ C)), x^ = deq(yq)/gamma, c = mean(dy deq(yq));
    dxq = Q(dx)."""
    rows, cols = dy.shape
    if want_dx and dx is None:
        dx = torch.empty((rows, cols), dtype=torch.bfloat16, device=dy.device)
    if want_q and dxq is None:
        dxq = NVFP4Tensor.empty(rows, cols, dy.device)
    a = yq.desc()
    q = dxq.desc() if dxq is not None else None
    _check(lib().pact_rmsnorm_bwd_nvfp4(
        _ptr(dy), _ld(dy), ctypes.byref(a), _ptr(gamma), _ptr(rstd), _ptr(C), _ld(C) if C is not None else cols,
        rows, cols, _ptr(dx), _ld(dx) if dx is not None else cols, ctypes.byref(q) if q is not None else None,
        _stream(stream)), "pact_rmsnorm_bwd_nvfp4")
    return dx, dxq


def pact_lora_grads_workspace(M: int, N: int, K: int, r: int) -> int:
    return int(lib().pact_lora_grads_workspace(M, N, K, r))


def pact_lora_grads_nvfp4(Xq: NVFP4Tensor, dY, lora: LoRA, dA=None, dB=None, ws=None, stream=None, T_dy=None):
    """dB = dY^T bf16(s X^ A^T) [N, r] and dA = bf16(s dY B)^T X^ [r, K], FP32,
    with X^ the BF16 values of the stashed NVFP4 input.  T_dy: bf16(s dY B)
    already computed ([M][round_up(r, 16)] BF16 at its start, e.g. the
    workspace of the input-gradient GEMM of the same dY and lora), or None."""
    M, N = dY.shape
    K, r = Xq.cols, lora.r
    if dA is None:
        dA = torch.empty((r, K), dtype=torch.float32, device=dY.device)
    if dB is None:
        dB = torch.empty((N, r), dtype=torch.float32, device=dY.device)
    if ws is None:
        ws = torch.empty((max(pact_lora_grads_workspace(M, N, K, r), 16),), dtype=torch.uint8, device=dY.device)
    dx, dl = Xq.desc(), lora.desc()
    if T_dy is not None:
        assert T_dy.device == dY.device and T_dy.numel() * T_dy.element_size() >= M * ((r + 15) // 16 * 16) * 2
    _check(lib().pact_lora_grads_nvfp4(ctypes.byref(dx), _ptr(dY), _ld(dY), N, ctypes.byref(dl), _ptr(T_dy),
                                       _ptr(dA), _ptr(dB), _ptr(ws), ws.numel(), _stream(stream)),
           "pact_lora_grads_nvfp4")
    return dA, dB


def pact_adamw_step(p, m, v, g, w=None, *, lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                    weight_decay: float = 0.0, step: int, stream=None):
    """In-place AdamW step over flat FP32 tensors p, m, v with gradient g;
    writes bf16(p) into w when given."""
    n = p.numel()
    assert m.numel() == n and v.numel() == n and g.numel() == n and (w is None or w.numel() == n)
    _check(lib().pact_adamw_step(_ptr(p), _ptr(m), _ptr(v), _ptr(g), _ptr(w) if w is not None else None, n,
                                 float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), int(step),
                                 _stream(stream)), "pact_adamw_step")


def pact_debug_dsilu32(g_bits: torch.Tensor, stream=None) -> torch.Tensor:
    out = torch.empty(g_bits.shape, dtype=torch.float32, device=g_bits.device)
    _check(lib().pact_debug_dsilu32(_ptr(g_bits), _ptr(out), g_bits.numel(), _stream(stream)),
           "pact_debug_dsilu32")
    return out


def pact_debug_stream(src, read_bytes: int, dst: torch.Tensor, write_bytes: int, stream=None) -> None:
    """Streams read_bytes of src and write_bytes of dst (the HBM-ceiling
    diagnostic; src may be None when read_bytes is 0)."""
    _check(lib().pact_debug_stream(_ptr(src) if src is not None else None, int(read_bytes), _ptr(dst),
                                   int(write_bytes), _stream(stream)), "pact_debug_stream")


def pact_debug_sigmoid32(g_bits: torch.Tensor, stream=None) -> torch.Tensor:
    out = torch.empty(g_bits.shape, dtype=torch.float32, device=g_bits.device)
    _check(lib().pact_debug_sigmoid32(_ptr(g_bits), _ptr(out), g_bits.numel(), _stream(stream)),
           "pact_debug_sigmoid32")
    return out


def pact_debug_gemm_plan(M: int, N: int, K: int, r: int = 0, dgrad: bool = False) -> tuple[int, int, bool]:
    """(kernel, ks, fused) of the GEMM launch plan for output [M][N] over K
    with LoRA rank r, as the forward (dgrad False) or input-gradient entry
    point chooses it; fused: the LoRA-down runs inside the split-K launch."""
    k, ks, f = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().pact_debug_gemm_plan(M, N, K, r, 1 if dgrad else 0, ctypes.byref(k), ctypes.byref(ks),
                                      ctypes.byref(f)), "pact_debug_gemm_plan")
    return k.value, ks.value, bool(f.value)


def pact_debug_gemm_plan_columns(M: int, N: int, K: int, r: int = 0, dgrad: bool = False) -> tuple[int, int]:
    """(n1, kernel2) of the launch plan's column split: output columns
    [0, n1) in the first launch, [n1, N) with kernel kernel2; n1 == 0: none."""
    n1, k2 = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().pact_debug_gemm_plan_columns(M, N, K, r, 1 if dgrad else 0, ctypes.byref(n1), ctypes.byref(k2)),
           "pact_debug_gemm_plan_columns")
    return n1.value, k2.value


ROW_OPS = {"quantize": 0, "rmsnorm_quant": 1, "silu_mul_quant": 2, "silu_mul_bwd": 3, "rmsnorm_bwd": 4}


def pact_debug_row_plan(op: str, cols: int) -> tuple[int, int]:
    """(wavefronts per row, 16-element blocks per lane) of the row kernel of
    op (a ROW_OPS key) for rows of cols elements."""
    w, b = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().pact_debug_row_plan(ROW_OPS[op], cols, ctypes.byref(w), ctypes.byref(b)), "pact_debug_row_plan")
    return w.value, b.value


LORA_DOWN_ROUTES = {1: "fused into the split-K launch", 2: "pipelined", 3: "transpose, then pipelined",
                    4: "strided gather"}


def pact_debug_lora_down_plan(M: int, N: int, K: int, r: int, ngroups: int = 1,
                              dgrad: bool = False) -> tuple[int, list[tuple[int, int, int]]]:
    """(route, passes) of the LoRA-down product of the GEMM call with output
    [M][N] over K, rank r per projection and ngroups projections (host only):
    route as in LORA_DOWN_ROUTES; passes = [(rank groups, row groups per
    wavefront, wavefronts per workgroup), ...], empty when fused."""
    route, npass = ctypes.c_int32(), ctypes.c_int32()
    rg, rpw, nw = (ctypes.c_int32 * 4)(), (ctypes.c_int32 * 4)(), (ctypes.c_int32 * 4)()
    _check(lib().pact_debug_lora_down_plan(M, N, K, r, ngroups, 1 if dgrad else 0, ctypes.byref(route),
                                           ctypes.byref(npass), rg, rpw, nw), "pact_debug_lora_down_plan")
    return route.value, [(rg[i], rpw[i], nw[i]) for i in range(npass.value)]
