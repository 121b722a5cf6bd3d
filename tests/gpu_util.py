"""Helpers for the GPU parity tests: host <-> device transfer of the seeded
inputs and the tolerance checks.  Imports torch lazily."""

from __future__ import annotations

import numpy as np

# Tolerances: float32 paths within 1e-5 max-abs; bfloat16 outputs within
# |d| <= 1.5e-2 + 1e-2 * |ref| element-wise; base-2 LSE within 1e-3 absolute.
F32_ATOL = 1e-5
BF16_ATOL, BF16_RTOL = 1.5e-2, 1e-2
LSE_ATOL = 1e-3


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm device")
    import paged_kv_cache_plan_amd as pkv
    pkv.lib()          # the native library must load; there is no other path
    return torch


def to_dev(x: np.ndarray, dtype: str):
    import torch
    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    if x.dtype == np.int32 or dtype == "i32":
        return torch.from_numpy(x.astype(np.int32)).cuda()
    return torch.from_numpy(x.astype(np.float32)).cuda()


def to_host(t, dtype: str) -> np.ndarray:
    """Device tensor -> numpy in storage form (uint16 bit patterns for bf16)."""
    import torch
    if dtype == "bf16":
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def empty_like_out(shape, dtype: str, fill=float("nan")):
    import torch
    t = torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    t.fill_(fill)
    return t


def check_close(got, ref, dtype: str, what: str, mask=None):
    """Assert element-wise agreement; returns a small report dict."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    assert np.isfinite(ref).all(), f"{what}: reference has non-finite values"
    assert np.isfinite(got).all(), f"{what}: {np.count_nonzero(~np.isfinite(got))} non-finite outputs"
    err = np.abs(got - ref)
    if dtype == "f32":
        bad = err > F32_ATOL
    else:
        bad = err > BF16_ATOL + BF16_RTOL * np.abs(ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    rep = {"max_abs": float(err.max()) if err.size else 0.0, "rel_rms": float(err.max() / rms) if rms else 0.0,
           "n": int(ref.size)}
    assert not bad.any(), f"{what}: {np.count_nonzero(bad)} of {bad.size} outside tolerance, {rep}"
    return rep


def check_lse(got, ref, what: str, atol=LSE_ATOL, mask=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    same_inf = np.isneginf(got) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(got - ref))
    assert np.all(np.isfinite(err)), f"{what}: non-finite LSE mismatch"
    assert err.max(initial=0.0) <= atol, f"{what}: LSE max err {err.max()}"
    return float(err.max(initial=0.0))
