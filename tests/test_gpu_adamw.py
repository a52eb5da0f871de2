"""GPU parity of the fused AdamW step (hotdry.top Unsloth post, section on
paged optimizers: two moments per trainable parameter in 32-bit state; AdamW
with decoupled weight decay) against the oracle's binary64 step.

The GPU computes in binary32 (a fixed operation order, coefficients rounded
once from binary64), the oracle in binary64; each step is teacher-forced (the
oracle starts from the GPU's state).  Bounds from one rounding per operation
(unit roundoff u = 2^-24), with slack:
  |m - m_ref| <= 2^-21 (|b1 m| + |(1-b1) g|)     (no cancellation blow-up: absolute)
  |v - v_ref| <= 2^-21 (b2 v + (1-b2) g^2)       (both terms non-negative)
  |p - p_ref| <= 2^-20 (|p| + |upd|) + lr/(1-b1^t) 2^-20 (|b1 m| + |(1-b1) g|) / den
with upd = the reference update and den = sqrt(v_ref/(1-b2^t)) + eps.  The
BF16 copy must be exactly bf16 of the GPU's FP32 master, and within one BF16
ulp of bf16 of the reference."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_gemm_amd import pact as pb

pytestmark = pytest.mark.gpu

f32 = lambda x: float(np.float32(x))


def _check_step(p0, m0, v0, g, got, hp, t):
    p, m, v, w = got
    rp, rm, rv = oracle.adamw_step(p0, m0, v0, g, step=t, **hp)
    b1, b2, lr, eps = hp["beta1"], hp["beta2"], hp["lr"], hp["eps"]
    am = np.abs(b1 * m0) + np.abs((1 - b1) * g)
    assert np.all(np.abs(m - rm) <= 2.0 ** -21 * am), "m"
    assert np.all(np.abs(v - rv) <= 2.0 ** -21 * (b2 * v0 + (1 - b2) * g * g)), "v"
    bc1, bc2 = 1 - b1 ** t, 1 - b2 ** t
    den = np.sqrt(rv / bc2) + eps
    upd = lr * (rm / bc1) / den
    tol = 2.0 ** -20 * (np.abs(p0) + np.abs(upd)) + lr / bc1 * 2.0 ** -20 * am / den
    assert np.all(np.abs(p - rp) <= tol), f"p: worst {np.max(np.abs(p - rp) - tol):.3e}"
    if w is not None:
        np.testing.assert_array_equal(w, oracle.bf16_of_master(p))
        dw = np.abs(w.astype(np.int64) - oracle.bf16_of_master(rp).astype(np.int64))
        assert np.all(dw <= 1)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("n", [1, 3, 4, 1000, 4099, (1 << 20) + 5])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_adamw_parity(n, wd):
    rng = np.random.default_rng(n + int(wd * 10))
    hp = dict(lr=f32(1e-3), beta1=f32(0.9), beta2=f32(0.999), eps=f32(1e-8), weight_decay=f32(wd))
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    dp, dm, dv = _dev(p), _dev(m), _dev(v)
    dw = torch.empty(n, dtype=torch.int16, device="cuda")
    for t, scale in enumerate((1.0, 1e-6, 1e3, 0.0), start=1):
        g = (rng.standard_normal(n) * scale).astype(np.float32)
        if n > 8:
            g[::7] = 0.0
        p0, m0, v0 = (x.cpu().numpy().astype(np.float64) for x in (dp, dm, dv))
        pb.pact_adamw_step(dp, dm, dv, _dev(g), dw, step=t, **hp)
        torch.cuda.synchronize()
        got = (dp.cpu().numpy().astype(np.float64), dm.cpu().numpy().astype(np.float64),
               dv.cpu().numpy().astype(np.float64), dw.cpu().numpy().view(np.uint16))
        _check_step(p0, m0, v0, g.astype(np.float64), got, hp, t)


def test_adamw_without_bf16_copy_and_large_step():
    """w = NULL updates the FP32 state only; a late step (bias corrections ~1)."""
    rng = np.random.default_rng(11)
    n = 777
    hp = dict(lr=f32(3e-2), beta1=f32(0.5), beta2=f32(0.9), eps=f32(1e-6), weight_decay=f32(0.01))
    p = rng.standard_normal(n).astype(np.float32)
    m = (rng.standard_normal(n) * 0.1).astype(np.float32)
    v = (rng.random(n) * 0.01).astype(np.float32)
    g = rng.standard_normal(n).astype(np.float32)
    dp, dm, dv = _dev(p), _dev(m), _dev(v)
    pb.pact_adamw_step(dp, dm, dv, _dev(g), None, step=1000, **hp)
    torch.cuda.synchronize()
    got = tuple(x.cpu().numpy().astype(np.float64) for x in (dp, dm, dv)) + (None,)
    _check_step(p.astype(np.float64), m.astype(np.float64), v.astype(np.float64), g.astype(np.float64), got, hp,
                1000)


def test_adamw_empty():
    z = torch.empty(0, dtype=torch.float32, device="cuda")
    pb.pact_adamw_step(z, z, z, z, None, lr=1e-3, step=1)
    torch.cuda.synchronize()
