"""GPU parity of the row quantizer and the fused RMSNorm / SiLU*mul producers
against the oracle: bit-exact codes, scale bytes, row scales, rstd and BF16
outputs (simolm.com PACT blog, "Method": quantization fused into RMSNorm and
SiLU-multiply)."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_gemm_amd import pact as pb
from nvfp4_gemm_amd import synth
from tests import _exact as ex
from tests import _gpu as G
from tests.test_oracle_quant import representable_row

pytestmark = pytest.mark.gpu


def _edge_rows(cols, rng):
    rows = [np.zeros(cols), -np.zeros(cols), np.full(cols, 0.15625), np.full(cols, -3.0)]
    r = rng.standard_normal(cols) * 0.01
    r[rng.integers(cols)] = 1e4                    # one huge outlier
    rows.append(r)
    rows.append(rng.standard_normal(cols) * 1e-38)  # subnormal-range values and scales
    rows.append(rng.standard_normal(cols) * np.exp2(rng.integers(-60, 60, cols)))
    t = np.zeros(cols)
    t[::7] = -1e-30
    rows.append(t)
    return synth.to_bf16_bits(np.stack(rows))


def _tie_rows(cols, rng):
    """Rows with closed-form codes (representable_row): row scale 2^k, every
    element an E2M1 value times its block's E4M3 scale, and with ties=True
    elements placed exactly on the E2M1 rounding midpoints 0.25 ... 5 (times
    the block scale), which round to the even code."""
    xs, codes, scales, ks = [], [], [], []
    for k in (-24, -3, 0, 7):
        for ties in (False, True, True):
            x, c, sc = representable_row(rng, cols // 16, k, ties)
            xs.append(x), codes.append(c), scales.append(sc), ks.append(k)
    return np.stack(xs), np.stack(codes), np.stack(scales), np.array(ks)


def _saturating_rows(cols, rng, n=6):
    """Rows whose blocks span 20 binades below the row maximum: many block
    scales fall in E4M3's subnormal range (or round down), so the block's
    largest elements lie above 6 times the block scale and saturate to 6."""
    nb = cols // 16
    x = rng.standard_normal((n, cols))
    x *= np.repeat(np.exp2(-rng.uniform(0, 20, (n, nb))), 16, axis=1)
    return synth.to_bf16_bits(x)


def _count_saturated(xb, q):
    """Elements with |x| > 6 S_b (S_b = decoded block scale times row scale)."""
    sc = np.array([oracle.e4m3_value(i) for i in range(256)], np.float64)
    S = sc[q.scales].repeat(16, axis=1) * q.d.astype(np.float64)[:, None]
    xf = np.abs(synth.bf16_bits_to_f32(xb).astype(np.float64))
    return int(np.sum((S > 0) & (xf > 6 * S)))


@pytest.mark.parametrize("cols", [16, 512, 3072, 8960])
def test_quantize_ties_and_saturation(cols):
    """E2M1 ties to even and saturation at 6 through the GPU's converter:
    closed-form codes on tie-crafted representable rows, the oracle's codes on
    rows that saturate (the test checks that they do)."""
    rng = np.random.default_rng(cols + 11)
    X, C, S, ks = _tie_rows(cols, rng)
    xb = synth.to_bf16_bits(X)
    assert np.array_equal(synth.bf16_bits_to_f32(xb).astype(np.float64), X)  # exact in BF16
    sat = _saturating_rows(cols, rng)
    allx = np.concatenate([xb, sat])
    want = oracle.quantize_bf16(allx)
    assert _count_saturated(sat, oracle.quantize_bf16(sat)) > 0
    got = pb.pact_quantize_nvfp4(G.dev_bf16(allx))
    torch.cuda.synchronize()
    G.assert_nvfp4_equal(got, want, f"ties/saturation {cols}")
    gh = G.host_nvfp4(got)
    n = X.shape[0]
    np.testing.assert_array_equal(ex.unpack_codes(gh.codes[:n]), C)
    np.testing.assert_array_equal(gh.scales[:n], S)
    np.testing.assert_array_equal(gh.d[:n], np.exp2(ks).astype(np.float32))


@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (5, 512), (7, 1024), (33, 3072),
                                       (9, 8960), (5, 9232), (4, 16384), (2, 32768)])
def test_quantize_parity(rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    x = np.concatenate([synth.student_t_bf16(rng, (rows, cols), 3.0, 0.5), _edge_rows(cols, rng)])
    want = oracle.quantize_bf16(x)
    got = pb.pact_quantize_nvfp4(G.dev_bf16(x))
    torch.cuda.synchronize()
    G.assert_nvfp4_equal(got, want, f"quantize {x.shape}")


def test_quantize_strided_and_deterministic():
    rng = np.random.default_rng(1)
    full = synth.student_t_bf16(rng, (37, 1040), 4.0, 0.5)
    xd = G.dev_bf16(full)[:, :1024]  # leading dimension 1040 > cols
    want = oracle.quantize_bf16(full[:, :1024])
    a = pb.pact_quantize_nvfp4(xd)
    b = pb.pact_quantize_nvfp4(xd)
    torch.cuda.synchronize()
    G.assert_nvfp4_equal(a, want, "strided")
    G.assert_nvfp4_equal(b, G.host_nvfp4(a), "repeat")


@pytest.mark.parametrize("rows,cols,eps", [(5, 512, 1e-5), (17, 2048, 1e-5), (8, 1536, 1e-6),
                                           (9, 3072, 1e-5), (3, 8960, 1e-6), (4, 9232, 1e-5), (66, 64, 1e-5)])
def test_rmsnorm_parity(rows, cols, eps):
    rng = np.random.default_rng(cols + rows)
    x = np.concatenate([synth.student_t_bf16(rng, (rows, cols), 3.0, 0.5), _edge_rows(cols, rng)[2:]])
    gamma = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(cols))
    y, yq, rstd = oracle.rmsnorm_quant(x, gamma, eps)
    gy, gyq, grstd = pb.pact_rmsnorm_quant_nvfp4(G.dev_bf16(x), G.dev_bf16(gamma), eps)
    _, gyq2, _ = pb.pact_rmsnorm_quant_nvfp4(G.dev_bf16(x), G.dev_bf16(gamma), eps, want_y=False,
                                            want_rstd=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(grstd.cpu().numpy().view(np.uint32), rstd.view(np.uint32))
    np.testing.assert_array_equal(G.host_bits(gy), y)
    G.assert_nvfp4_equal(gyq, yq, "rmsnorm yq")
    G.assert_nvfp4_equal(gyq2, yq, "rmsnorm yq (no y)")


@pytest.mark.parametrize("rows,cols", [(6, 256), (9, 8192), (5, 8960), (4, 9232), (3, 1536), (70, 16)])
def test_silu_parity(rows, cols):
    rng = np.random.default_rng(rows + 3 * cols)
    ties = synth.to_bf16_bits(_tie_rows(cols, rng)[0][:4])
    sat = _saturating_rows(cols, rng, n=4)
    g = np.concatenate([synth.student_t_bf16(rng, (rows, cols), 4.0, 0.5), _edge_rows(cols, rng), ties, sat])
    u = np.concatenate([synth.student_t_bf16(rng, (rows, cols), 4.0, 0.5), _edge_rows(cols, rng)[::-1], sat,
                        ties])
    h, hq, gq, uq = oracle.silu_mul_quant(g, u)
    gh, ghq, ggq, guq = pb.pact_silu_mul_quant_nvfp4(G.dev_bf16(g), G.dev_bf16(u))
    _, ghq2, n1, n2 = pb.pact_silu_mul_quant_nvfp4(G.dev_bf16(g), G.dev_bf16(u), want_h=False,
                                                    want_stash=False)
    torch.cuda.synchronize()
    assert n1 is None and n2 is None
    np.testing.assert_array_equal(G.host_bits(gh), h)
    G.assert_nvfp4_equal(ghq, hq, "hq")
    G.assert_nvfp4_equal(ggq, gq, "gq")
    G.assert_nvfp4_equal(guq, uq, "uq")
    G.assert_nvfp4_equal(ghq2, hq, "hq (no stash)")


def test_sigmoid32_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    want = oracle.sigmoid_table()
    got = pb.pact_debug_sigmoid32(torch.from_numpy(bits.view(np.int16).copy()).cuda()).cpu().numpy()
    bad = np.flatnonzero(finite & (got.view(np.uint32) != want.view(np.uint32)))
    assert bad.size == 0, [(hex(int(b)), float(got[b]), float(want[b])) for b in bad[:8]]


@pytest.mark.parametrize("shape", ["llama1b_layer", "llama3b_layer"])
def test_full_layer_shapes(shape):
    """Bit-exact at the layer workloads' full sizes: RMSNorm over [M, H], SiLU
    over [M, I], and the incoming-gradient quantizer over [M, I]."""
    S = synth.LAYERS[shape]
    M, H, I = S.tokens, S.hidden, S.inter
    rng = np.random.default_rng(5)
    x = synth.student_t_bf16(rng, (M, H), S.act_nu, S.act_scale)
    gamma = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(H))
    y, yq, rstd = oracle.rmsnorm_quant(x, gamma, S.eps)
    gy, gyq, grstd = pb.pact_rmsnorm_quant_nvfp4(G.dev_bf16(x), G.dev_bf16(gamma), S.eps)
    g = synth.student_t_bf16(rng, (M, I), S.act_nu, S.act_scale)
    u = synth.student_t_bf16(rng, (M, I), S.act_nu, S.act_scale)
    h, hq, gq, uq = oracle.silu_mul_quant(g, u)
    gh, ghq, ggq, guq = pb.pact_silu_mul_quant_nvfp4(G.dev_bf16(g), G.dev_bf16(u))
    dq = pb.pact_quantize_nvfp4(G.dev_bf16(g))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(G.host_bits(gy), y)
    np.testing.assert_array_equal(grstd.cpu().numpy().view(np.uint32), rstd.view(np.uint32))
    G.assert_nvfp4_equal(gyq, yq, "yq")
    np.testing.assert_array_equal(G.host_bits(gh), h)
    G.assert_nvfp4_equal(ghq, hq, "hq")
    G.assert_nvfp4_equal(ggq, gq, "gq")
    G.assert_nvfp4_equal(guq, uq, "uq")
    G.assert_nvfp4_equal(dq, gq, "quantize")
