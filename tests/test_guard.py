"""The regression guard of the GPU parity tests (``gpu_util.check_guard``)
against mistakes planted in the oracle, on the CPU.

The benchmark spec tolerances (1.5e-2 + 1e-2 |ref| on bf16 outputs, 1e-3 on the
LSE) are loose enough at the full decode and prefill sizes that one key
missing from a row's softmax would pass them: with K keys a key of average
weight moves the LSE by about 1 / (K ln 2) (6.7e-4 at the decode batch's mean
K of 2160).  The guard is asserted next to them in the GPU tests.  Here:

* one key removed from a row's visible set -- the oracle run with a custom
  mask that hides the row's key of median weight -- fails the guard for every
  request of the full decode batch and for sampled rows of the longest
  request of the full prefill batch;
* the exact output rounded to bf16 (the kernels' last rounding) passes it.
"""

import numpy as np
import pytest

import workloads as wl
from oracle import attention as oat
from tests import gpu_util as gu


def _bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (via float32, ties to even), as float64."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _quantile_key(q_row, keys, visible, sm_scale, frac):
    """Index of the visible key whose softmax weight has rank frac among the
    row's visible keys (0.5: the median weight)."""
    s = sm_scale * (keys[visible] @ q_row)
    idx = np.flatnonzero(visible)
    return int(idx[np.argsort(s)[int(frac * len(idx))]])


def _median_key(q_row, keys, visible, sm_scale):
    return _quantile_key(q_row, keys, visible, sm_scale, 0.5)


def test_guard_rejects_one_dropped_key_at_decode_size():
    b = wl.make("decode")
    kw = dict(qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr), kv_indices=list(b.kv_indices),
              kv_last_page_len=list(b.kv_last_page_len), page_size=b.page_size, layout=b.layout,
              num_kv_heads=b.num_kv_heads, sm_scale=b.sm_scale, q_dtype="bf16", kv_dtype="bf16")
    ro, rl = oat.paged_attention(b.q, b.k_cache, b.v_cache, **kw)
    # The kernels' final rounding alone stays inside the guard.
    rep = gu.check_guard(_bf16_round(ro), ro, rl, rl, "decode bf16-rounded")
    assert rep["pairs"] == b.batch_size * b.num_qo_heads
    # Drop, in every request, the key of median weight for head 0.
    segs = []
    for r in range(b.batch_size):
        k_len = b.kv_lens[r]
        keys = oat.upcast(oat.gather_request(b.k_cache, b.layout, b.kv_indptr, b.kv_indices, b.page_size, r,
                                             k_len), "bf16")[:, 0]
        j = _median_key(oat.upcast(b.q[r, 0], "bf16"), keys, np.ones(k_len, bool), b.sm_scale)
        m = np.ones(k_len, bool)
        m[j] = False
        segs.append(m)
    do, dl = oat.paged_attention(b.q, b.k_cache, b.v_cache, custom_mask=np.concatenate(segs),
                                 causal=False, **kw)
    rel, lerr = gu.guard_stats(do, ro, dl, rl)
    assert np.all(lerr[:, 0] > gu.GUARD_LSE), lerr[:, 0].min()
    assert np.all(lerr[:, 0] > 3 * gu.GUARD_LSE)          # with margin
    # For head 0, whose median key went missing, the benchmark spec bars alone
    # accept the planted error in most requests (all but short histories).
    passes = [abs(dl[r, 0] - rl[r, 0]) <= gu.LSE_ATOL and
              np.all(np.abs(do[r, 0] - ro[r, 0]) <= gu.BF16_ATOL + gu.BF16_RTOL * np.abs(ro[r, 0]))
              for r in range(b.batch_size)]
    assert sum(passes) >= b.batch_size // 2, sum(passes)


def test_guard_rejects_one_wrong_value_row_at_decode_size():
    """The output bound: in every request of the full decode batch, the value
    row of a key of about average weight for head 0 (rank 0.7 of the row's
    weights: with these scores the mean weight lies above the median)
    replaced by another key's row
    -- a wrong value gather that leaves the scores and the LSE exact -- moves
    head 0's output past the guard."""
    b = wl.make("decode")
    kw = dict(qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr), kv_indices=list(b.kv_indices),
              kv_last_page_len=list(b.kv_last_page_len), page_size=b.page_size, layout=b.layout,
              num_kv_heads=b.num_kv_heads, sm_scale=b.sm_scale, q_dtype="bf16", kv_dtype="bf16", heads=[0])
    ro, rl = oat.paged_attention(b.q, b.k_cache, b.v_cache, **kw)
    v_bad = b.v_cache.copy()
    for r in range(b.batch_size):
        k_len = b.kv_lens[r]
        keys = oat.upcast(oat.gather_request(b.k_cache, b.layout, b.kv_indptr, b.kv_indices, b.page_size, r,
                                             k_len), "bf16")[:, 0]
        j = _quantile_key(oat.upcast(b.q[r, 0], "bf16"), keys, np.ones(k_len, bool), b.sm_scale, 0.7)
        src = (j + k_len // 2) % k_len                 # another key of the same request
        pages = b.kv_indices[b.kv_indptr[r]:b.kv_indptr[r + 1]]
        v_bad[pages[j // b.page_size], j % b.page_size, 0] = b.v_cache[pages[src // b.page_size],
                                                                      src % b.page_size, 0]
    do, dl = oat.paged_attention(b.q, b.k_cache, v_bad, **kw)
    rel, lerr = gu.guard_stats(do, ro, dl, rl)
    assert np.all(lerr[:, 0] == 0.0)                   # the scores did not move
    assert np.all(rel[:, 0] > gu.GUARD_O_REL_L2), np.sort(rel[:, 0])[:4]


def test_guard_rejects_one_dropped_key_at_prefill_size():
    b = wl.make("prefill")
    r = int(np.argmax(b.kv_lens))                      # the longest history (7520 keys)
    q_len, k_len = b.qo_lens[r], b.kv_lens[r]
    heads = [0, 17]
    kw = dict(qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr), kv_indices=list(b.kv_indices),
              kv_last_page_len=list(b.kv_last_page_len), page_size=b.page_size, layout=b.layout,
              num_kv_heads=b.num_kv_heads, sm_scale=b.sm_scale, q_dtype="bf16", kv_dtype="bf16",
              requests=[r], heads=heads)
    ro, rl = oat.paged_attention(b.q, b.k_cache, b.v_cache, causal=True, **kw)
    r0, r1 = int(b.qo_indptr[r]), int(b.qo_indptr[r + 1])
    gu.check_guard(_bf16_round(ro[r0:r1][:, heads]), ro[r0:r1][:, heads], rl[r0:r1][:, heads],
                   rl[r0:r1][:, heads], "prefill bf16-rounded")
    # Causal mask of every request; in request r, rows i in `rows` lose their
    # median-weight key for head 0.
    segs = []
    rows = [0, 1, q_len // 3, q_len // 2, q_len - 2, q_len - 1]
    for c in range(b.batch_size):
        ql, kl = b.qo_lens[c], b.kv_lens[c]
        m = np.arange(kl)[None, :] <= kl - ql + np.arange(ql)[:, None]
        if c == r:
            keys = oat.upcast(oat.gather_request(b.k_cache, b.layout, b.kv_indptr, b.kv_indices, b.page_size, r,
                                                 k_len), "bf16")[:, 0]
            for i in rows:
                m[i, _median_key(oat.upcast(b.q[r0 + i, 0], "bf16"), keys, m[i], b.sm_scale)] = False
        segs.append(m.reshape(-1))
    do, dl = oat.paged_attention(b.q, b.k_cache, b.v_cache, causal=False,
                                 custom_mask=np.concatenate(segs), **kw)
    rel, lerr = gu.guard_stats(do[r0:r1][:, heads], ro[r0:r1][:, heads], dl[r0:r1][:, heads], rl[r0:r1][:, heads])
    assert np.all(lerr[rows, 0] > gu.GUARD_LSE), lerr[rows, 0]
    others = np.setdiff1d(np.arange(q_len), rows)
    assert np.all(lerr[others] == 0.0)                 # only the planted rows moved
    assert np.all(np.abs(dl[r0:r1][rows, 0] - rl[r0:r1][rows, 0]) <= gu.LSE_ATOL)


def test_guard_flags_empty_row_mismatch_and_bad_outputs():
    ref = np.ones((2, 1, 4))
    lse = np.array([[1.0], [-np.inf]])
    gu.check_guard(ref, ref, lse, lse, "identical")
    got = ref.copy()
    got[0, 0, 0] += 0.02                               # relative L2 0.01
    with pytest.raises(AssertionError, match="relative L2"):
        gu.check_guard(got, ref, lse, lse, "bad")
    bad_lse = np.array([[1.0], [0.0]])                 # an empty row reported as non-empty
    with pytest.raises(AssertionError, match="past"):
        gu.check_guard(ref, ref, bad_lse, lse, "empty")
    with pytest.raises(AssertionError, match="LSEs past"):
        gu.check_guard(ref, ref, lse + np.array([[1e-4], [0.0]]), lse, "lse")
