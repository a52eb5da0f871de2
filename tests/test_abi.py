"""The C ABI (include/pact.h): libpact.so loads, exports every declared entry
point, and rejects bad arguments with the documented status before touching
the device -- all checked on the host, without a GPU."""
import ctypes
import os
import re

import pytest

from nvfp4_gemm_amd import pact as pb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pact.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pact_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pb.LIB_PATH):
        from nvfp4_gemm_amd import build
        build.build()
    return pb.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert sorted(pb.EXPORTS) == names


def test_version_and_status_strings(L):
    assert pb.pact_version() == 1
    for code, name in pb.STATUS.items():
        assert pb.pact_status_string(code) == name


def _nv(codes=0x1000, scales=0x2000, d=0x3000, rows=4, cols=32):
    return pb.pact_nvfp4(codes, scales, d, rows, cols)


FAKE = 0x7f0000001000  # never dereferenced: validation fails before any device access


def test_quantize_validation(L):
    q = _nv(rows=4, cols=32)
    s = None
    assert L.pact_quantize_nvfp4(None, 32, 4, 32, ctypes.byref(q), s) == 1
    assert L.pact_quantize_nvfp4(FAKE, 32, 4, 24, ctypes.byref(_nv(cols=24)), s) == 2
    assert L.pact_quantize_nvfp4(FAKE, 32, -1, 32, ctypes.byref(q), s) == 1
    assert L.pact_quantize_nvfp4(FAKE + 2, 32, 4, 32, ctypes.byref(q), s) == 3
    assert L.pact_quantize_nvfp4(FAKE, 36, 4, 32, ctypes.byref(q), s) == 3   # ld % 8
    assert L.pact_quantize_nvfp4(FAKE, 16, 4, 32, ctypes.byref(q), s) == 1   # ld < cols
    assert L.pact_quantize_nvfp4(FAKE, 32, 4, 32, None, s) == 1
    assert L.pact_quantize_nvfp4(FAKE, 32, 4, 32, ctypes.byref(_nv(rows=5)), s) == 1
    assert L.pact_quantize_nvfp4(FAKE, 32, 4, 32, ctypes.byref(_nv(codes=0x1001)), s) == 3
    big = 32768 + 16
    assert L.pact_quantize_nvfp4(FAKE, big, 1, big, ctypes.byref(_nv(rows=1, cols=big)), s) == 2


def test_rmsnorm_silu_validation(L):
    q = _nv(rows=4, cols=32)
    assert L.pact_rmsnorm_quant_nvfp4(FAKE, 32, None, 1e-5, 4, 32, None, 32, ctypes.byref(q), None, None) == 1
    assert L.pact_rmsnorm_quant_nvfp4(FAKE, 32, FAKE, -1.0, 4, 32, None, 32, ctypes.byref(q), None, None) == 1
    assert L.pact_rmsnorm_quant_nvfp4(FAKE, 32, FAKE, 1e-5, 4, 32, None, 32, None, None, None) == 1
    assert L.pact_rmsnorm_quant_nvfp4(FAKE, 32, FAKE, 1e-5, 4, 32, None, 32, ctypes.byref(q), FAKE + 4, None) == 3
    assert L.pact_silu_mul_quant_nvfp4(FAKE, 32, None, 32, 4, 32, None, 32, ctypes.byref(q), None, None, None) == 1
    assert L.pact_silu_mul_quant_nvfp4(FAKE, 32, FAKE, 32, 4, 40, None, 40, ctypes.byref(_nv(cols=40)), None, None, None) == 2
    assert L.pact_silu_mul_quant_nvfp4(FAKE, 32, FAKE, 32, 4, 32, None, 32, ctypes.byref(q),
                                       ctypes.byref(_nv(rows=3)), None, None) == 1


def test_layout_validation(L):
    N, K = 32, 64
    f, b = _nv(rows=N, cols=K), _nv(rows=K, cols=N)
    need = L.pact_build_weight_layouts_workspace(N, K)
    assert need >= 4 * K
    args = (N, K, ctypes.byref(f), ctypes.byref(b))
    assert L.pact_build_weight_layouts(None, None, *args, FAKE, need, None) == 1         # neither W nor W_fwd_in
    assert L.pact_build_weight_layouts(FAKE, ctypes.byref(f), *args, FAKE, need, None) == 1  # both
    assert L.pact_build_weight_layouts(FAKE, None, *args, None, 0, None) == 4
    assert L.pact_build_weight_layouts(FAKE, None, *args, FAKE, need - 1, None) == 4
    assert L.pact_build_weight_layouts(FAKE, None, 24, K, ctypes.byref(_nv(rows=24, cols=K)),
                                       ctypes.byref(_nv(rows=K, cols=24)), FAKE, need, None) == 2
    assert L.pact_build_weight_layouts(FAKE, None, N, K, ctypes.byref(f), ctypes.byref(_nv(rows=N, cols=K)),
                                       FAKE, need, None) == 1  # backward layout must be [K][N]


def test_gemm_validation(L):
    M, N, K = 8, 32, 64
    xq, wq = _nv(rows=M, cols=K), _nv(rows=N, cols=K)
    assert L.pact_gemm_workspace(M, N, K, 0) == 0
    need = L.pact_gemm_workspace(M, N, K, 16)
    assert need >= 2 * 16 * M  # T = bf16(s X A^T), [M][r] BF16
    fwd = L.pact_gemm_nvfp4_fwd
    assert fwd(None, None, 0, ctypes.byref(wq), None, None, FAKE, N, None, 0, None) == 1
    assert fwd(ctypes.byref(xq), None, 0, ctypes.byref(_nv(rows=N, cols=48)), None, None, FAKE, N, None, 0, None) == 1
    assert fwd(ctypes.byref(_nv(rows=M, cols=40)), None, 0, ctypes.byref(_nv(rows=N, cols=40)), None, None,
               FAKE, N, None, 0, None) == 2
    assert fwd(ctypes.byref(xq), None, 0, ctypes.byref(wq), None, None, FAKE + 8, N, None, 0, None) == 3
    assert fwd(ctypes.byref(xq), None, 0, ctypes.byref(wq), None, None, FAKE, N - 8, None, 0, None) == 1
    lo = pb.pact_lora(FAKE, FAKE, 16, 2.0)
    assert fwd(ctypes.byref(xq), None, K, ctypes.byref(wq), ctypes.byref(lo), None, FAKE, N, FAKE, need, None) == 1
    assert fwd(ctypes.byref(xq), FAKE, K, ctypes.byref(wq), ctypes.byref(lo), None, FAKE, N, None, 0, None) == 4
    t_min = (2 * 16 * M + 255) // 256 * 256  # the LoRA-down product alone; the rest of `need` is optional
    assert fwd(ctypes.byref(xq), FAKE, K, ctypes.byref(wq), ctypes.byref(lo), None, FAKE, N, FAKE, t_min - 1, None) == 4
    bad_rank = pb.pact_lora(FAKE, FAKE, -1, 2.0)
    assert fwd(ctypes.byref(xq), FAKE, K, ctypes.byref(wq), ctypes.byref(bad_rank), None, FAKE, N, FAKE, need, None) == 1
    nullA = pb.pact_lora(None, FAKE, 16, 2.0)
    assert fwd(ctypes.byref(xq), FAKE, K, ctypes.byref(wq), ctypes.byref(nullA), None, FAKE, N, FAKE, need, None) == 1
    dg = L.pact_gemm_nvfp4_dgrad
    dyq, wb = _nv(rows=M, cols=N), _nv(rows=K, cols=N)
    assert dg(ctypes.byref(dyq), None, 0, ctypes.byref(_nv(rows=K, cols=K)), None, None, FAKE, K, None, 0, None) == 1
    assert dg(ctypes.byref(dyq), FAKE, N, ctypes.byref(wb), ctypes.byref(lo), None, FAKE, K, None, 0, None) == 4


def test_gemm_plan_host_logic(L):
    """The launch plan (host logic, no GPU work): large outputs run in one
    pass; a small output with long K splits K, and the workspace query then
    covers the FP32 partials of either direction."""
    k, ks, fu = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    assert L.pact_debug_gemm_plan(-1, 8, 8, 0, 0, ctypes.byref(k), ctypes.byref(ks), None) == 1
    assert L.pact_debug_gemm_plan(8, 8, 8, 0, 0, None, ctypes.byref(ks), None) == 1
    assert L.pact_debug_gemm_plan(8, 8, 8, 300, 0, ctypes.byref(k), ctypes.byref(ks), None) == 1
    assert L.pact_debug_gemm_plan(8192, 8192, 3072, 0, 0, ctypes.byref(k), ctypes.byref(ks), None) == 0
    assert ks.value == 1
    assert L.pact_debug_gemm_plan(1024, 512, 2048, 0, 0, ctypes.byref(k), ctypes.byref(ks), ctypes.byref(fu)) == 0
    assert ks.value > 1 and 0 <= k.value <= 4 and fu.value == 0
    split = ks.value
    parts = split * (1024 // 32) * (512 // 32) * 4096
    assert L.pact_gemm_workspace(1024, 512, 2048, 0) >= parts
    assert L.pact_gemm_workspace(1024, 512, 2048, 16) >= parts + 2 * 16 * 1024
    assert L.pact_gemm_workspace(1024, 2048, 512, 16) >= parts + 2 * 16 * 1024  # the input-gradient direction
    assert L.pact_debug_gemm_plan(100, 200, 520, 0, 0, ctypes.byref(k), ctypes.byref(ks), None) == 0
    assert ks.value == 1  # K % 64 != 0: no split


def test_gemm_plan_lora_down_placement(L):
    """The LoRA-down of a split-K GEMM runs inside the split launch only where
    its workgroups do not hold back the GEMM's: a few short rows fit beside the
    GEMM workgroups; at 4096 tokens over 8960 columns (three row groups per
    down workgroup) the input gradient's strided down runs as a launch of its
    own, and a fused forward down needs a split deep enough (ks > 2) that the
    GEMM's second round absorbs it."""
    k, ks, fu = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    assert L.pact_debug_gemm_plan(1024, 512, 2048, 16, 0, ctypes.byref(k), ctypes.byref(ks), ctypes.byref(fu)) == 0
    assert ks.value > 1 and fu.value == 1
    assert L.pact_debug_gemm_plan(4096, 1536, 8960, 16, 1, ctypes.byref(k), ctypes.byref(ks), ctypes.byref(fu)) == 0
    assert fu.value == 0
    assert L.pact_debug_gemm_plan(4096, 1536, 8960, 16, 0, ctypes.byref(k), ctypes.byref(ks), ctypes.byref(fu)) == 0
    assert fu.value == 0 or ks.value > 2


def test_gemm_plan_column_split_host_logic(L):
    """A column split puts whole rounds of 256 x 256 tiles in the first launch
    (n1 a multiple of 256 with (M / 256) (n1 / 256) a multiple of the CU
    count) and appears only where one launch would leave a partly filled
    round; invalid arguments are rejected."""
    i32 = ctypes.c_int32
    n1, k2 = i32(), i32()
    assert L.pact_debug_gemm_plan_columns(-1, 8, 8, 0, 0, ctypes.byref(n1), ctypes.byref(k2)) == 1
    assert L.pact_debug_gemm_plan_columns(8, 8, 8, 0, 0, None, ctypes.byref(k2)) == 1
    assert L.pact_debug_gemm_plan_columns(8192, 3072, 8192, 16, 0, ctypes.byref(n1), ctypes.byref(k2)) == 0
    assert n1.value == 2048 and 2 <= k2.value <= 4 and (8192 // 256) * (n1.value // 256) % 256 == 0
    for M, N, K in [(8192, 8192, 3072), (8192, 16384, 3072), (1024, 2048, 2048), (256, 1024, 512)]:
        assert L.pact_debug_gemm_plan_columns(M, N, K, 16, 0, ctypes.byref(n1), ctypes.byref(k2)) == 0
        assert n1.value == 0  # whole rounds already, or fewer tiles than CUs


def test_lora_down_plan_host_logic(L):
    """The LoRA-down diagnostic agrees with the GEMM plan (route 1 exactly
    when the plan fuses it into the split-K launch), takes one pass per 64
    padded ranks, and rejects invalid arguments without touching a device."""
    i32 = ctypes.c_int32
    route, npass = i32(), i32()
    rg, rpw, nw = (i32 * 4)(), (i32 * 4)(), (i32 * 4)()
    call = lambda *a: L.pact_debug_lora_down_plan(*a, ctypes.byref(route), ctypes.byref(npass), rg, rpw, nw)
    assert call(-1, 8, 8, 16, 1, 0) == 1
    assert call(8, 8, 8, 0, 1, 0) == 1
    assert call(8, 8, 8, 16, 0, 0) == 1
    assert call(8, 8, 8, 16, 5, 0) == 1                 # more groups than a grouped GEMM takes
    assert call(8, 8, 8, 16, 2, 1) == 1                 # the input gradient has one projection
    assert call(8, 8, 8, 96, 3, 0) == 1                 # 288 padded ranks
    assert L.pact_debug_lora_down_plan(8, 8, 8, 16, 1, 0, None, ctypes.byref(npass), rg, rpw, nw) == 1
    k, ks, fu = i32(), i32(), i32()
    for M, N, K, r, g, dg in [(1024, 2048, 8192, 16, 1, 0), (4096, 1536, 8960, 16, 1, 0), (1024, 512, 2048, 16, 1, 1),
                              (8192, 5120, 3072, 32, 3, 0), (8192, 3072, 8192, 32, 1, 1), (256, 1024, 512, 8, 1, 0)]:
        assert call(M, N, K, r, g, dg) == 0
        assert L.pact_debug_gemm_plan(M, N, K, r * g if g > 1 else r, dg, ctypes.byref(k), ctypes.byref(ks),
                                      ctypes.byref(fu)) == 0
        assert (route.value == 1) == (fu.value == 1 and ks.value > 1)
        if route.value != 1:
            rpad = g * ((r + 15) // 16 * 16)
            assert npass.value == (rpad + 63) // 64
            assert sum(rg[i] for i in range(npass.value)) * 16 == rpad
            assert all(rpw[i] == (2 if M >= 4096 and rg[i] >= 2 and route.value != 4 else 1)
                       for i in range(npass.value))
            assert route.value == (3 if dg and M >= 4096 else (4 if dg else 2))


def test_noalloc_gemm_rejects_oversized_lora_product(L):
    """The no-allocation forward GEMM refuses, before any device work, a
    LoRA-down product larger than its fixed per-GPU array (600000 rows x 32
    ranks of BF16 = 38.4 MB > 32 MiB), and null operands."""
    assert L.pact_noalloc_scratch_bytes() == 32 << 20
    x = pb.pact_nvfp4(16, 16, 16, 600000, 256)
    w = pb.pact_nvfp4(16, 16, 16, 64, 256)
    lo = pb.pact_lora(16, 16, 32, 2.0)
    assert L.pact_gemm_nvfp4_fwd_noalloc(ctypes.byref(x), 16, 256, ctypes.byref(w), ctypes.byref(lo), None, 16, 64,
                                         None) == 4  # PACT_ERR_WORKSPACE
    assert L.pact_gemm_nvfp4_fwd_noalloc(None, 16, 256, ctypes.byref(w), None, None, 16, 64, None) == 1


def test_gptq_validation(L):
    """The GPTQ entry points reject bad arguments before any device work."""
    D = ctypes.c_double
    x = pb.pact_nvfp4(16, 16, 16, 32, 256)
    assert L.pact_gptq_hessian_nvfp4(None, D(1.0), 0, 16, None) == 1
    assert L.pact_gptq_hessian_nvfp4(ctypes.byref(x), D(1.0), 0, None, None) == 1
    x_bad = pb.pact_nvfp4(16, 16, 16, 32, 40)
    assert L.pact_gptq_hessian_nvfp4(ctypes.byref(x_bad), D(1.0), 0, 16, None) == 2
    assert L.pact_gptq_hessian_nvfp4(ctypes.byref(x), D(1.0), 0, 8, None) == 3  # H misaligned
    N, K = 32, 256
    need = L.pact_gptq_workspace(N, K)
    assert need >= 8 * (2 * K * K + N * K)
    w = pb.pact_nvfp4(16, 16, 16, N, K)
    call = lambda K_=K, bs=128, ws_bytes=need, damp=0.01, Wp=16, wd=w: L.pact_gptq_nvfp4(
        Wp, K_, N, K_, 16, D(damp), bs, ctypes.byref(wd), 16, ws_bytes, None)
    assert call(bs=8) == 1 and call(bs=256) == 1 and call(damp=-1.0) == 1
    assert call(bs=40) == 2                                  # not a multiple of 16
    w2 = pb.pact_nvfp4(16, 16, 16, N, 272)
    assert call(K_=272, wd=w2, ws_bytes=L.pact_gptq_workspace(N, 272)) == 2   # K % 64 != 0
    assert call(ws_bytes=need - 1) == 4
    assert call(Wp=None) == 1


def test_backward_validation(L):
    """Argument checks of the backward entry points (host only, nothing is
    launched on an error)."""
    rows, cols = 4, 32
    q = _nv(rows=rows, cols=cols)
    bad = _nv(rows=rows, cols=cols + 16)
    silu = L.pact_silu_mul_bwd_quant_nvfp4
    ok = (FAKE, cols, ctypes.byref(q), ctypes.byref(q), rows, cols, FAKE, FAKE, cols,
          ctypes.byref(q), ctypes.byref(q), None)
    assert silu(FAKE, cols, ctypes.byref(q), ctypes.byref(q), rows, 24, FAKE, FAKE, cols,
                ctypes.byref(q), ctypes.byref(q), None) == 2                   # cols % 16
    assert silu(FAKE, cols, ctypes.byref(bad), ctypes.byref(q), *ok[4:]) == 1  # gq shape
    assert silu(*ok[:9], None, ctypes.byref(q), None) == 1                    # dgq required
    assert silu(FAKE + 8, *ok[1:]) == 3                                       # misaligned dh
    rms = L.pact_rmsnorm_bwd_nvfp4
    args = [FAKE, cols, ctypes.byref(q), FAKE, FAKE, None, cols, rows, cols, FAKE, cols, ctypes.byref(q), None]
    a = list(args); a[9] = None; a[11] = None
    assert rms(*a) == 1                                                       # no output
    a = list(args); a[4] = None
    assert rms(*a) == 1                                                       # rstd required
    a = list(args); a[4] = FAKE + 4
    assert rms(*a) == 3                                                       # misaligned rstd
    a = list(args); a[2] = ctypes.byref(bad)
    assert rms(*a) == 1                                                       # yq shape
    assert L.pact_debug_dsilu32(None, FAKE, 4, None) == 1


def test_lora_grads_validation(L):
    """Argument checks of the LoRA-gradient entry point (host only)."""
    M, N, K, r = 8, 32, 64, 4
    q = _nv(rows=M, cols=K)
    lo = pb.pact_lora(FAKE, FAKE, r, 2.0)
    f = L.pact_lora_grads_nvfp4
    need = L.pact_lora_grads_workspace(M, N, K, r)
    assert need >= 2 * M * 16 * 2                                             # holds T^ and T'
    assert L.pact_lora_grads_workspace(M, N, K, 0) == 0
    assert f(ctypes.byref(q), FAKE, N, N, None, None, FAKE, FAKE, FAKE, need, None) == 1        # no adapter
    big = pb.pact_lora(FAKE, FAKE, 65, 2.0)
    assert f(ctypes.byref(q), FAKE, N, N, ctypes.byref(big), None, FAKE, FAKE, FAKE, need, None) == 2  # r > 64
    assert f(ctypes.byref(q), FAKE, N, 24, ctypes.byref(lo), None, FAKE, FAKE, FAKE, need, None) == 2  # N % 16
    assert f(ctypes.byref(q), FAKE, N, N, ctypes.byref(lo), None, FAKE + 4, FAKE, FAKE, need, None) == 3  # dA
    assert f(ctypes.byref(q), FAKE, N, N, ctypes.byref(lo), FAKE + 4, FAKE, FAKE, FAKE, need, None) == 3  # T'
    assert f(ctypes.byref(q), FAKE, N, N, ctypes.byref(lo), None, FAKE, FAKE, FAKE, need - 1, None) == 4  # workspace
    assert f(ctypes.byref(q), FAKE, N - 8, N, ctypes.byref(lo), None, FAKE, FAKE, FAKE, need, None) == 1  # ld < N


def test_adamw_validation(L):
    """Argument checks of the AdamW entry point (host only)."""
    f = L.pact_adamw_step
    hp = (1e-3, 0.9, 0.999, 1e-8, 0.1)
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, *hp, 1, None) == 0          # nothing to do
    assert f(None, None, None, None, None, 0, *hp, 1, None) == 0
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, *hp, 1, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 16, *hp, 0, None) == 1         # step counts from 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 1e-3, 1.0, 0.999, 1e-8, 0.1, 1, None) == 1   # beta1 = 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 16, -1e-3, 0.9, 0.999, 1e-8, 0.1, 1, None) == 1  # lr < 0
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 16, float("nan"), 0.9, 0.999, 1e-8, 0.1, 1, None) == 1
    assert f(FAKE, None, FAKE, FAKE, FAKE, 16, *hp, 1, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE + 4, FAKE, 16, *hp, 1, None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE + 8, 16, *hp, 1, None) == 3


def test_row_plan_host_logic(L):
    """The row kernels' launch shapes: the nine widths of the GPU variant test
    select every compiled (wavefronts per row, blocks per lane) of each row
    kernel, a shape covers the row (64 lanes x wavefronts x blocks >= blocks of
    the row), and invalid arguments are rejected like the entry points do."""
    from tests.test_gpu_variant_coverage import WIDTHS
    i32 = ctypes.c_int32
    w, b = i32(), i32()
    fwd = {(1, 1), (1, 2), (1, 3), (4, 1), (4, 2), (4, 3), (8, 2), (8, 3), (8, 4)}
    bwd = {(1, 1), (1, 2), (1, 3), (4, 1), (8, 1), (8, 2), (8, 3), (8, 4)}
    compiled = {0: fwd, 1: fwd, 2: fwd - {(4, 3)}, 3: bwd, 4: bwd}
    for op, shapes in compiled.items():
        seen = set()
        for cols in WIDTHS + [16, 48, 4096, 8960, 9232, 32768]:
            assert L.pact_debug_row_plan(op, cols, ctypes.byref(w), ctypes.byref(b)) == 0
            assert (w.value, b.value) in shapes
            assert 64 * w.value * b.value >= cols // 16
            if cols in WIDTHS:
                seen.add((w.value, b.value))
        assert seen == shapes, (op, shapes - seen)
    assert L.pact_debug_row_plan(5, 1024, ctypes.byref(w), ctypes.byref(b)) == 1
    assert L.pact_debug_row_plan(0, 0, ctypes.byref(w), ctypes.byref(b)) == 1
    assert L.pact_debug_row_plan(0, 1024, None, ctypes.byref(b)) == 1
    assert L.pact_debug_row_plan(0, 40, ctypes.byref(w), ctypes.byref(b)) == 2
    assert L.pact_debug_row_plan(0, 32784, ctypes.byref(w), ctypes.byref(b)) == 2


def test_stream_diagnostic_validation(L):
    """The HBM-ceiling diagnostic rejects bad arguments before any device work."""
    f = L.pact_debug_stream
    assert f(FAKE, -16, FAKE, 16, None) == 1
    assert f(FAKE, 16, FAKE, -16, None) == 1
    assert f(FAKE, 16, None, 16, None) == 1
    assert f(None, 16, FAKE, 16, None) == 1
    assert f(FAKE, 8, FAKE, 16, None) == 3
    assert f(FAKE, 16, FAKE, 24, None) == 3
    assert f(FAKE + 4, 16, FAKE, 16, None) == 3
    assert f(FAKE, 16, FAKE + 8, 16, None) == 3
    assert f(None, 0, FAKE, 0, None) == 0  # nothing to move: no launch
