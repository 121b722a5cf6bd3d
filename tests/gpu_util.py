"""Helpers for the GPU parity tests: host <-> device transfer of the seeded
inputs and the tolerance checks.  Imports torch lazily."""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Tolerances: float32 paths within 1e-5 max-abs; bfloat16 outputs within
# |d| <= 1.5e-2 + 1e-2 * |ref| element-wise; base-2 LSE within 1e-3 absolute.
F32_ATOL = 1e-5
BF16_ATOL, BF16_RTOL = 1.5e-2, 1e-2
LSE_ATOL = 1e-3

# Regression guard, tighter than the pass bar above and asserted beside it on
# the bf16 workloads.  The GPU forms every score from exact bf16 products
# accumulated in fp32 and sums the weights in fp32, so its base-2 LSE differs
# from the float64 oracle by ~1e-6 (measured at most 2.2e-6 over the full
# decode, prefill and MLA batches).  Its two coarse roundings (the weights to
# bf16 before the value product, the output to bf16) each add a relative
# error of at most 2^-9 per element; in rows dominated by a few keys the
# weight rounding does not average out, and the relative L2 error per
# (row, head) reaches 3.7e-3 on the prefill batch.  Removing (or duplicating)
# one key of median weight out of K moves the LSE by about 0.6 / (K ln 2),
# >= 1e-4 for K <= 8192 (the LSE bound catches it); a wrong value row of a
# key of about average weight moves the output by about sqrt(2 / (e K)) relative L2,
# >= 1e-2 for K <= 8192 (the output bound catches it).  tests/test_guard.py
# plants such a key in the oracle and checks that the bounds reject it at
# the full decode and prefill sizes.
GUARD_O_REL_L2 = 6e-3
GUARD_LSE = 5e-5


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


def guard_stats(got, ref, lse_got, lse_ref):
    """Per (row, head): relative L2 error of the output and absolute LSE
    error, on [rows, heads, dim] / [rows, heads] arrays.  Entries the caller
    did not compute (NaN in ref) are NaN; empty rows (ref LSE -inf) are 0
    when got is empty too, else inf."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    lg = np.asarray(lse_got, dtype=np.float64)
    lr = np.asarray(lse_ref, dtype=np.float64)
    num = np.sqrt(np.sum((got - ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(ref ** 2, axis=-1))
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(den > 0, num / den, num)
        lerr = np.abs(lg - lr)
    empty = np.isneginf(lr)
    lerr = np.where(empty, np.where(np.isneginf(lg), 0.0, np.inf), lerr)
    rel = np.where(empty, np.where(np.isneginf(lg), 0.0, np.inf), rel)
    return rel, lerr


def check_guard(got, ref, lse_got, lse_ref, what: str, o_rel_l2: float = GUARD_O_REL_L2,
                lse_atol: float = GUARD_LSE):
    """Regression guard on [rows, heads, dim] outputs and [rows, heads] LSEs:
    every computed (row, head) must have ||got - ref||_2 <= o_rel_l2 *
    ||ref||_2 and |lse_got - lse_ref| <= lse_atol (an empty reference row
    must be empty).  Returns the largest of each statistic."""
    rel, lerr = guard_stats(got, ref, lse_got, lse_ref)
    live = ~np.isnan(np.asarray(lse_ref, dtype=np.float64))
    rel, lerr = rel[live], lerr[live]
    rep = {"o_rel_l2_max": float(rel.max(initial=0.0)), "lse_max": float(lerr.max(initial=0.0)),
           "pairs": int(live.sum())}
    assert not np.isnan(rel).any() and rel.max(initial=0.0) <= o_rel_l2, \
        f"{what}: guard: {np.count_nonzero(~(rel <= o_rel_l2))} (row, head) outputs past {o_rel_l2} relative L2, {rep}"
    assert not np.isnan(lerr).any() and lerr.max(initial=0.0) <= lse_atol, \
        f"{what}: guard: {np.count_nonzero(~(lerr <= lse_atol))} LSEs past {lse_atol}, {rep}"
    return rep


def oracle_in_threads(fn, head_groups, workers=None):
    """Run ``fn(heads=group)`` (an oracle call that fills only the listed
    heads, NaN elsewhere) for every group in parallel threads (numpy releases
    the GIL in its kernels; BLAS runs one thread per call) and combine the
    results.  Returns (o, lse) as the oracle call does."""
    from threadpoolctl import threadpool_limits
    workers = workers or min(16, os.cpu_count() or 1, len(head_groups))
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(lambda g: fn(heads=list(g)), head_groups))
    o, lse = parts[0]
    o, lse = o.copy(), lse.copy()
    for po, pl in parts[1:]:
        o = np.where(np.isnan(po), o, po)
        lse = np.where(np.isnan(pl), lse, pl)
    return o, lse
