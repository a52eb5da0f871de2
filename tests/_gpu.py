"""Helpers for GPU parity tests: move seeded host inputs (numpy BF16 bit
patterns) to the device and bring results back for comparison with the
oracle.  Conversion only; no arithmetic of the method."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from nvfp4_gemm_amd import pact as pb


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_nvfp4(q: oracle.NVFP4) -> pb.NVFP4Tensor:
    return pb.NVFP4Tensor(torch.from_numpy(np.ascontiguousarray(q.codes)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(q.scales)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(q.d)).cuda())


def host_nvfp4(t: pb.NVFP4Tensor) -> oracle.NVFP4:
    return oracle.NVFP4(t.codes.cpu().numpy(), t.scales.cpu().numpy(), t.row_scale.cpu().numpy())


def assert_nvfp4_equal(got, want: oracle.NVFP4, what=""):
    g = host_nvfp4(got) if isinstance(got, pb.NVFP4Tensor) else got
    for name in ("codes", "scales"):
        a, b = getattr(g, name), getattr(want, name)
        if not np.array_equal(a, b):
            idx = np.argwhere(a != b)
            raise AssertionError(f"{what} {name}: {len(idx)} mismatches, first at {idx[:5].tolist()}: "
                                 f"got {a[tuple(idx[0])]} want {b[tuple(idx[0])]}")
    # row scales compared as bit patterns
    if not np.array_equal(g.d.view(np.uint32), want.d.view(np.uint32)):
        idx = np.argwhere(g.d.view(np.uint32) != want.d.view(np.uint32))
        raise AssertionError(f"{what} row scale mismatches at {idx[:5].ravel().tolist()}")


def bf16_vals(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    v = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(v)) - 7)


def check_gemm_tolerance(got_bits: np.ndarray, ref_bits: np.ndarray, what=""):
    """Per element |d| <= 2 ulp_bf16(|ref|) + 1e-3 max_row|ref|, and the
    relative Frobenius error <= 4e-3."""
    g, r = bf16_vals(got_bits), bf16_vals(ref_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    rowmax = np.max(np.abs(r), axis=1, keepdims=True) if r.size else r
    bound = 2 * ulp_bf16(r) + 1e-3 * rowmax
    err = np.abs(g - r)
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance, first {i.tolist()} "
                             f"got {g[tuple(i)]} ref {r[tuple(i)]} bound {bound[tuple(i)]}")
    nr = np.linalg.norm(r)
    if nr > 0:
        rel = np.linalg.norm(g - r) / nr
        assert rel <= 4e-3, f"{what}: relative Frobenius error {rel}"
    return float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0



def check_lora_grads(gdA, gdB, dA, dB, what=""):
    """GPU LoRA gradients (FP32) against the oracle's (float64).  Both share
    the rank index j: dA [r,K] row j and dB [N,r] column j are the products of
    one rank intermediate (T'[:, j], T^[:, j]) with the tokens, so an entry of
    T^ or T' that rounds to the neighbouring BF16 value on one side moves that
    whole row or column together.  Bound, in the GEMM's form with "row" read
    as "the entries of one rank": per element |d| <= 2 ulp_bf16(|ref|) +
    1e-3 max_j|ref|, and a relative Frobenius error <= 4e-3."""
    for got, ref, axis, name in ((gdA, dA, 1, "dA"), (gdB, dB, 0, "dB")):
        g = got.cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
        rank_max = np.max(np.abs(ref), axis=axis, keepdims=True) if ref.size else ref
        bound = 2 * ulp_bf16(ref) + 1e-3 * rank_max
        err = np.abs(g - ref)
        bad = err > bound
        if bad.any():
            i = tuple(np.argwhere(bad)[0])
            raise AssertionError(f"{what} {name}: {bad.sum()} elements out of tolerance, first {i}: got {g[i]} "
                                 f"ref {ref[i]} bound {bound[i]}")
        nr = np.linalg.norm(ref)
        assert np.linalg.norm(g - ref) <= 4e-3 * nr + 1e-30, f"{what} {name}: relative Frobenius error"
