"""Pins for oracle.cascade.

The cascade's result has a plain definition: each request attends to the
concatenation of its nodes' keys, level by level ("FlashInfer 中的 KV-Cache
布局", multi-level cascade layout; the merge of disjoint key sets is exact,
"Deep Dive - FlashInfer", "Core mechanism: schedule work around state").
These tests compute that definition independently -- keys gathered one token
at a time through ``metadata.token_address`` into one flat sequence per
request, then torch's float64 scaled-dot-product attention with an explicit
bottom-right mask -- and compare.  They also check the invariance under
moving a shared page into the leaves, the one-level case, and the
validation reasons.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as at
from oracle import cascade as cc
from oracle import metadata as md

LN2 = math.log(2.0)


def _node_of(indptr, row):
    for n in range(len(indptr) - 1):
        if indptr[n] <= row < indptr[n + 1]:
            return n
    raise AssertionError(row)


def _flat_keys(b, levels, cache, layout, page_size, lvl_lens):
    """Keys [K, H, D] of the request owning ``rows``: the nodes on its path, in level order."""
    toks = []
    for li, lv in enumerate(levels):
        n = _node_of(list(lv["qo_indptr"]), b)
        for j in range(lvl_lens[li][n]):
            page, slot = md.token_address(list(lv["kv_indptr"]), list(lv["kv_indices"]), page_size, n, j)
            toks.append(cache[page, slot] if layout == "NHD" else cache[page, :, slot])
    return np.stack(toks)


def _flattened_reference(batch, causal):
    """Per request: torch SDPA (float64) over its concatenated keys; lse via logsumexp."""
    levels = batch.extra["levels"]
    P = batch.page_size
    lens = [[int(k) for k in md.kv_lens(list(lv["kv_indptr"]), list(lv["kv_indices"]),
                                        list(lv["kv_last_page_len"]), P)] for lv in levels]
    g = batch.num_qo_heads // batch.num_kv_heads
    q_all = at.upcast(batch.q, batch.dtype)
    o = np.zeros(q_all.shape)
    lse = np.zeros(q_all.shape[:2])
    for b in range(batch.batch_size):
        r0, r1 = int(batch.qo_indptr[b]), int(batch.qo_indptr[b + 1])
        if r1 == r0:
            continue
        k = at.upcast(_flat_keys(r0, levels, batch.k_cache, batch.layout, P, lens), batch.dtype)
        v = at.upcast(_flat_keys(r0, levels, batch.v_cache, batch.layout, P, lens), batch.dtype)
        n_q, n_k = r1 - r0, k.shape[0]
        i = torch.arange(n_q)[:, None]
        j = torch.arange(n_k)[None, :]
        mask = (j <= n_k - n_q + i) if causal else torch.ones(n_q, n_k, dtype=torch.bool)
        qt = torch.from_numpy(q_all[r0:r1]).transpose(0, 1)                      # [H, n_q, D]
        kt = torch.from_numpy(np.repeat(k, g, axis=1)).transpose(0, 1).contiguous()
        vt = torch.from_numpy(np.repeat(v, g, axis=1)).transpose(0, 1).contiguous()
        out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                               scale=batch.sm_scale)
        s = batch.sm_scale * (qt @ kt.transpose(1, 2))
        s = s.masked_fill(~mask, -math.inf)
        o[r0:r1] = out.transpose(0, 1).numpy()
        lse[r0:r1] = (torch.logsumexp(s, dim=-1) / LN2).transpose(0, 1).numpy()
    return o, lse


def _run(batch, causal, levels=None):
    return cc.cascade_attention(batch.q, batch.k_cache, batch.v_cache,
                                levels=batch.extra["levels"] if levels is None else levels,
                                page_size=batch.page_size, layout=batch.layout,
                                num_kv_heads=batch.num_kv_heads, causal=causal, sm_scale=batch.sm_scale,
                                q_dtype=batch.dtype, kv_dtype=batch.dtype)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("causal", [True, False])
def test_cascade_equals_attention_over_concatenated_keys(layout, causal):
    batch = workloads.make("cascade_small", layout=layout, causal=causal)
    o, lse = _run(batch, causal)
    ref_o, ref_lse = _flattened_reference(batch, causal)
    assert np.max(np.abs(o - ref_o)) < 1e-10
    assert np.max(np.abs(lse - ref_lse)) < 1e-10


def test_shared_node_with_more_rows_than_keys():
    # Level 1 nodes hold 1..2 keys while their subtrees hold up to 12 query
    # rows: every row still sees every shared key.
    batch = workloads.make("cascade_small", seed=7, level_kv=[(9, 9), (1, 2), (1, 6)], qo_range=(2, 4))
    levels = batch.extra["levels"]
    assert any(levels[1]["qo_indptr"][n + 1] - levels[1]["qo_indptr"][n] > levels[1]["kv_lens"][n]
               for n in range(len(levels[1]["kv_lens"])))
    o, lse = _run(batch, True)
    ref_o, ref_lse = _flattened_reference(batch, True)
    assert np.max(np.abs(o - ref_o)) < 1e-10
    assert np.max(np.abs(lse - ref_lse)) < 1e-10


def test_bf16_storage_tree():
    batch = workloads.make("cascade_small", seed=11, dtype="bf16", tree=[[5], [2, 3], [1] * 5],
                           level_kv=[(30, 40), (3, 17), (1, 9)])
    o, lse = _run(batch, True)
    ref_o, ref_lse = _flattened_reference(batch, True)
    assert np.max(np.abs(o - ref_o)) < 1e-10
    assert np.max(np.abs(lse - ref_lse)) < 1e-10


def test_one_level_cascade_is_paged_attention():
    batch = workloads.make("cascade_small")
    leaf = batch.extra["levels"][-1]
    o, lse = _run(batch, True, levels=[leaf])
    ref_o, ref_lse = at.paged_attention(batch.q, batch.k_cache, batch.v_cache, qo_indptr=leaf["qo_indptr"],
                                        kv_indptr=leaf["kv_indptr"], kv_indices=leaf["kv_indices"],
                                        kv_last_page_len=leaf["kv_last_page_len"], page_size=batch.page_size,
                                        layout=batch.layout, num_kv_heads=batch.num_kv_heads, causal=True,
                                        sm_scale=batch.sm_scale)
    assert np.array_equal(o, ref_o) and np.array_equal(lse, ref_lse)


def test_moving_a_shared_page_into_the_leaves():
    # Root node: its first page moves into a new level of its own; the
    # result must not change (the merge is exact up to rounding).
    batch = workloads.make("cascade_small", level_kv=[(36, 36), (5, 20), (1, 12)])
    levels = batch.extra["levels"]
    root = levels[0]
    P = batch.page_size
    assert root["kv_indptr"][1] >= 2 and root["kv_last_page_len"][0] == P
    first = {"qo_indptr": root["qo_indptr"], "kv_indptr": np.array([0, 1], np.int32),
             "kv_indices": root["kv_indices"][:1], "kv_last_page_len": np.array([P], np.int32)}
    rest = {"qo_indptr": root["qo_indptr"], "kv_indptr": np.array([0, root["kv_indptr"][1] - 1], np.int32),
            "kv_indices": root["kv_indices"][1:], "kv_last_page_len": root["kv_last_page_len"]}
    o1, lse1 = _run(batch, True)
    o2, lse2 = _run(batch, True, levels=[first, rest] + levels[1:])
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(lse1 - lse2)) < 1e-12


def _validate(levels, **kw):
    return cc.validate_levels(levels, page_size=4, max_num_pages=64, **kw)


def _lv(qo, kv_pages, last):
    indptr = [0]
    for n in kv_pages:
        indptr.append(indptr[-1] + n)
    return {"qo_indptr": qo, "kv_indptr": indptr, "kv_indices": list(range(indptr[-1])),
            "kv_last_page_len": last}


def test_validation_accepts_tree_and_returns_lengths():
    levels = [_lv([0, 5], [3], [2]), _lv([0, 2, 5], [1, 2], [4, 1]), _lv([0, 1, 2, 4, 5], [1, 1, 1, 1], [1, 2, 2, 3])]
    assert _validate(levels) == [[10], [4, 5], [1, 2, 2, 3]]


def test_validation_reasons():
    with pytest.raises(md.MetadataError) as e:
        _validate([])
    assert e.value.reason == "cascade_rows"
    # Row counts differ between levels.
    with pytest.raises(md.MetadataError) as e:
        _validate([_lv([0, 4], [3], [2]), _lv([0, 1, 2, 4, 5], [1, 1, 1, 1], [1, 2, 2, 3])])
    assert e.value.reason == "cascade_rows"
    # Boundary 3 of level 0 is not a boundary of level 1.
    with pytest.raises(md.MetadataError) as e:
        _validate([_lv([0, 3, 5], [1, 1], [4, 4]), _lv([0, 2, 5], [1, 2], [4, 4])])
    assert e.value.reason == "cascade_nesting"
    # The last level keeps qo_len <= kv_len ...
    with pytest.raises(md.MetadataError) as e:
        _validate([_lv([0, 5], [3], [2]), _lv([0, 2, 5], [1, 1], [1, 2])])
    assert e.value.reason == "qo_exceeds_kv"
    # ... a shared level does not need it.
    assert _validate([_lv([0, 5], [1], [1]), _lv([0, 2, 5], [1, 1], [2, 3])]) == [[1], [2, 3]]
    # Page-table rules hold per level.
    with pytest.raises(md.MetadataError) as e:
        _validate([_lv([0, 5], [3], [5]), _lv([0, 5], [2], [4])])
    assert e.value.reason == "last_page_len"
