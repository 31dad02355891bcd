"""Shared helpers of the GPU parity tests: input staging and the tolerances.

Tolerances (per output tensor):
  * routing indices, counts, offsets, permutation, Xp: bit-exact;
  * gate weights (fp32): |w - w_ref| <= 1e-5 * |w_ref| per element;
  * bf16 outputs (Act, Y, out): relative L2 <= 5e-3 and
    max|out - ref| <= 2e-2 * max|ref| over the whole tensor;
  * fp32 outputs: relative L2 <= 1e-5 and max|out - ref| <= 1e-4 * max|ref|
    (fp32 accumulation over d, n <= 256 terms gives about 1e-6).
"""
from __future__ import annotations

import numpy as np
import torch

import synth


def to_np(t: torch.Tensor) -> np.ndarray:
    return synth.to_numpy(t)


def as_f64(a) -> np.ndarray:
    """numpy float64 view of a tensor/array; bf16 bit patterns are widened exactly."""
    if isinstance(a, torch.Tensor):
        return a.detach().float().cpu().numpy().astype(np.float64)
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def check_close(out, ref, dtype: str, what: str = "output"):
    o = as_f64(out)
    r = as_f64(ref)
    assert o.shape == r.shape, (what, o.shape, r.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite values"
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(o - r) / nr if nr > 0 else np.linalg.norm(o)
    mx = np.max(np.abs(r)) if r.size else 0.0
    err = np.max(np.abs(o - r)) if r.size else 0.0
    if dtype == "bf16":
        assert rel <= 5e-3, f"{what}: relative L2 {rel:.3e} > 5e-3"
        assert err <= 2e-2 * mx + 1e-30, f"{what}: max abs err {err:.3e} > 2e-2 * {mx:.3e}"
    else:
        assert rel <= 1e-5, f"{what}: relative L2 {rel:.3e} > 1e-5"
        assert err <= 1e-4 * mx + 1e-30, f"{what}: max abs err {err:.3e} > 1e-4 * {mx:.3e}"
    return rel, err


def check_weights(w, w_ref):
    g = as_f64(w)
    r = as_f64(w_ref)
    bad = np.abs(g - r) > 1e-5 * np.abs(r)
    assert not bad.any(), f"{int(bad.sum())} gate weights off by more than 1e-5 relative, e.g. " \
                          f"{g[bad][:4]} vs {r[bad][:4]}"


def check_equal(out, ref, what: str):
    o = to_np(out) if isinstance(out, torch.Tensor) else np.asarray(out)
    r = np.asarray(ref)
    assert o.shape == r.shape, (what, o.shape, r.shape)
    if not np.array_equal(o, r):
        bad = np.argwhere(o.reshape(r.shape) != r)
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {bad[:4].tolist()}: "
                             f"{o[tuple(bad[0])]} vs {r[tuple(bad[0])]}")


def cuda(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().to("cuda")


def from_np(a: np.ndarray, dtype: torch.dtype | None = None) -> torch.Tensor:
    """Host tensor from numpy; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t if dtype is None else t.to(dtype)
