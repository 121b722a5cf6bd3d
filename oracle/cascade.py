"""Oracle part 4: multi-level cascade attention over one paged cache.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

"FlashInfer 中的 KV-Cache 布局", multi-level cascade inference data layout:
queries and outputs stay one ragged tensor and every level's keys live in
one shared paged cache; each level views them through its own qo_indptr
(the cumulative count of query tokens in each subtree) and its own page table
(kv_page_indptr, kv_page_indices, kv_last_page_len, with the meaning of the
page-table section).  Each level yields an attention state per query row and
head; the states of a row merge into its output because the merge of
disjoint key sets is exact ("Deep Dive - FlashInfer", "Core mechanism:
schedule work around state": output plus log-sum-exp is the composable unit
across workers, devices and shared prefixes).

Readings (the layout page leaves these open):
* every level covers all query rows (its qo_indptr ends at the row count)
  and the levels nest: each node's rows are a union of whole nodes of the
  next level, so the nodes form a tree whose last level has one leaf per
  request;
* the keys of a shared (non-last) level precede every query token of its
  subtree, so each row of the node sees all of them; the bottom-right causal
  rule ("Causality uses logical positions, not page numbers") applies only
  at the last level, where a node is one request;
* the page-table rules of ``metadata.validate`` hold per level, except that
  a shared node may hold fewer keys than its subtree has query rows.

This module computes each level with ``attention.paged_attention`` and folds
the per-level states with ``merge.merge_states`` in level order.
"""

from __future__ import annotations

import numpy as np

from . import attention as att
from . import merge as mg
from . import metadata as md


def validate_levels(levels, *, page_size: int, max_num_pages: int, num_qo_heads: int = 1,
                    num_kv_heads: int = 1) -> list[list[int]]:
    """Check a cascade's per-level metadata; return each level's node kv_len.

    ``levels``: list of dicts with qo_indptr, kv_indptr, kv_indices,
    kv_last_page_len (one entry per node).  Checked in this order:
    1. at least one level (reason "cascade_rows");
    2. per level, the page-table rules of ``metadata.validate`` (qo_len <=
       kv_len only at the last level);
    3. every level's qo_indptr ends at the same row count ("cascade_rows");
    4. every node boundary of a level is a node boundary of the next level
       ("cascade_nesting").
    """
    if not levels:
        raise md.MetadataError("cascade_rows", "a cascade needs at least one level")
    lens = []
    last_level = len(levels) - 1
    for li, lv in enumerate(levels):
        kw = dict(qo_indptr=lv["qo_indptr"], kv_indptr=lv["kv_indptr"], kv_indices=lv["kv_indices"],
                  kv_last_page_len=lv["kv_last_page_len"], page_size=page_size, max_num_pages=max_num_pages,
                  num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads)
        if li == last_level:
            lens.append(md.validate(**kw))
        else:
            # Shared levels: the same rules without qo_len <= kv_len.  Checked
            # by validating a copy whose every node has a single query row.
            n = len(lv["kv_last_page_len"])
            lens.append(md.validate(**{**kw, "qo_indptr": list(range(n + 1))}))
            md._check_indptr("qo_indptr", lv["qo_indptr"], n)
    rows = [int(lv["qo_indptr"][len(lv["kv_last_page_len"])]) for lv in levels]
    if any(r != rows[0] for r in rows):
        raise md.MetadataError("cascade_rows", f"levels cover {rows} query rows")
    for li in range(last_level):
        upper = set(int(x) for x in levels[li]["qo_indptr"])
        lower = set(int(x) for x in levels[li + 1]["qo_indptr"])
        if not upper <= lower:
            raise md.MetadataError("cascade_nesting",
                                   f"level {li} has node boundaries {sorted(upper - lower)} "
                                   f"that level {li + 1} does not")
    return lens


def level_states(q, k_cache, v_cache, *, levels, page_size: int, layout: str, num_kv_heads: int,
                 causal: bool = True, sm_scale: float | None = None, q_dtype: str = "f32",
                 kv_dtype: str = "f32"):
    """Per-level attention states: (o [L, nnz, Hq, Dv], lse [L, nnz, Hq]) in float64.

    Level l is plain paged attention of the ragged queries against that
    level's page table, with nodes in place of requests; only the last level
    is causal.
    """
    outs, lses = [], []
    for li, lv in enumerate(levels):
        o, lse = att.paged_attention(
            q, k_cache, v_cache, qo_indptr=lv["qo_indptr"], kv_indptr=lv["kv_indptr"],
            kv_indices=lv["kv_indices"], kv_last_page_len=lv["kv_last_page_len"], page_size=page_size,
            layout=layout, num_kv_heads=num_kv_heads, causal=causal and li == len(levels) - 1,
            sm_scale=sm_scale, q_dtype=q_dtype, kv_dtype=kv_dtype)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


def cascade_attention(q, k_cache, v_cache, *, levels, page_size: int, layout: str, num_kv_heads: int,
                      causal: bool = True, sm_scale: float | None = None, q_dtype: str = "f32",
                      kv_dtype: str = "f32"):
    """Cascade attention: every row's per-level states merged in level order.

    Returns (o [nnz, Hq, Dv], lse [nnz, Hq]) in float64, lse in base 2.
    """
    o, lse = level_states(q, k_cache, v_cache, levels=levels, page_size=page_size, layout=layout,
                          num_kv_heads=num_kv_heads, causal=causal, sm_scale=sm_scale, q_dtype=q_dtype,
                          kv_dtype=kv_dtype)
    # merge_states folds axis 1: [rows, levels, heads, dim].
    return mg.merge_states(np.transpose(o, (1, 0, 2, 3)), np.transpose(lse, (1, 0, 2)))
