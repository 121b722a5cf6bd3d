"""Pins for oracle.planner.  The split policy is our reading (the pages give
trade-offs, not an algorithm), so it is pinned by a hand-worked example and by
the partition invariants the merge needs: page-aligned, disjoint chunks that
cover every key a tile may see exactly once (Deep Dive - FlashInfer, 'A worked
split-KV example': overlapping chunks double-count keys)."""

import math

import numpy as np
import pytest

from oracle import planner as pl


def test_hand_worked_decode_split():
    """Two decode requests of 600 and 100 tokens, page 16 (38 and 7 pages).
    Unforced with one CU and target 1: chunk = max(16, 45) = 45 pages, nothing
    splits.  Forced to 16-page chunks: request 0 splits into keys [0,256),
    [256,512), [512,600) with partial rows 0, 1, 2; request 1 stays direct.
    Emission is by descending key count: 256, 256, 100, 88."""
    args = dict(mode="decode", qo_indptr=None, kv_indptr=[0, 38, 45], kv_last_page_len=[8, 4],
                page_size=16, heads_y=1, rows=1, causal=True, num_cus=1, target_per_cu=1, tail_split=1)
    p = pl.plan(**args)
    assert p["chunk_pages"] == 45 and not p["split"] and p["merges"] == []
    assert p["items"] == [[0, 1, 0, 600, 599, 0, -1, 0], [1, 1, 0, 100, 99, 38, -1, 1]]
    p = pl.plan(**args, fixed_split_pages=16)
    assert p["split"] and p["num_partial_rows"] == 3
    assert p["merges"] == [[0, 1, 0, 3]]
    assert p["items"] == [[0, 1, 0, 256, 599, 0, 0, 0], [0, 1, 256, 512, 599, 0, 1, 0],
                          [1, 1, 0, 100, 99, 38, -1, 1], [0, 1, 512, 600, 599, 0, 2, 0]]


def test_hand_worked_tail_split():
    """The same two requests with 16-page chunks and tail split 2.  Request 0's
    final chunk [512,600) spans 6 pages and becomes 3-page pieces [512,560)
    and [560,600); request 1's only chunk [0,100) spans 7 pages and becomes
    4-page pieces [0,64) and [64,100), so it now merges too.  Partial rows:
    request 0 slots 0..3, request 1 slots 4, 5.  Emission by descending key count:
    256, 256, 64, 48, 40, 36."""
    p = pl.plan(mode="decode", qo_indptr=None, kv_indptr=[0, 38, 45], kv_last_page_len=[8, 4], page_size=16,
                heads_y=1, rows=1, causal=True, num_cus=1, fixed_split_pages=16, tail_split=2)
    assert p["merges"] == [[0, 1, 0, 4], [1, 1, 4, 2]] and p["num_partial_rows"] == 6
    assert p["items"] == [[0, 1, 0, 256, 599, 0, 0, 0], [0, 1, 256, 512, 599, 0, 1, 0],
                          [1, 1, 0, 64, 99, 38, 4, 1], [0, 1, 512, 560, 599, 0, 2, 0],
                          [0, 1, 560, 600, 599, 0, 3, 0], [1, 1, 64, 100, 99, 38, 5, 1]]
    # a one-page final chunk is left whole
    p = pl.plan(mode="decode", qo_indptr=None, kv_indptr=[0, 17], kv_last_page_len=[5], page_size=16,
                heads_y=1, rows=1, causal=True, num_cus=1, fixed_split_pages=16, tail_split=2)
    assert [(i[2], i[3]) for i in p["items"]] == [(0, 256), (256, 261)]


def test_default_tail_split_needs_few_units_per_cu():
    """The default decode tail split applies while the kept chunks times
    heads_y are at most 5 per CU.  The two requests above keep 3 + 1 = 4
    chunks: with one head slice on one CU (4 <= 5) the default is the split
    plan above; with two head slices (8 > 5) it is off, so request 0 keeps its
    three chunks [0,256), [256,512), [512,600) (slots 0..2) and request 1 its
    one [0,100), written directly; on two CUs (8 <= 10) it is on again.  An
    explicit tail_split is used as given, and prefill never splits by
    default."""
    kw = dict(mode="decode", qo_indptr=None, kv_indptr=[0, 38, 45], kv_last_page_len=[8, 4], page_size=16,
              rows=1, causal=True, fixed_split_pages=16)
    split = pl.plan(heads_y=1, num_cus=1, tail_split=2, **kw)
    assert pl.plan(heads_y=1, num_cus=1, **kw) == split
    off = pl.plan(heads_y=2, num_cus=1, **kw)
    assert off["merges"] == [[0, 1, 0, 3]] and off["num_partial_rows"] == 3
    assert off["items"] == [[0, 1, 0, 256, 599, 0, 0, 0], [0, 1, 256, 512, 599, 0, 1, 0],
                            [1, 1, 0, 100, 99, 38, -1, 1], [0, 1, 512, 600, 599, 0, 2, 0]]
    assert pl.plan(heads_y=2, num_cus=1, tail_split=2, **kw)["items"] == split["items"]
    assert pl.plan(heads_y=2, num_cus=2, **kw)["items"] == split["items"]
    assert pl.plan(heads_y=2, num_cus=1, tail_split=1, **kw) == off
    pre = dict(kw, mode="prefill", qo_indptr=[0, 1, 2])
    assert pl.plan(heads_y=1, num_cus=1, **pre) == pl.plan(heads_y=1, num_cus=1, tail_split=1, **pre)


def test_order_follows_key_count_not_rows():
    """One prefill request, 6 new rows after a 26-token prefix (K = 32), page
    4, tiles of 4 rows, one chunk.  Tile 0 (4 rows) sees keys < 30, tile 1
    (2 rows) sees keys < 32: tile 1 has more keys, so it is emitted first even
    though it has fewer rows (a tile's kernel time follows its keys)."""
    p = pl.plan(mode="prefill", qo_indptr=[0, 6], kv_indptr=[0, 8], kv_last_page_len=[4],
                page_size=4, heads_y=1, rows=4, causal=True, num_cus=1, fixed_split_pages=8)
    # tile 1: diag = K - q + 4 = 30, kv_end = K; tile 0: diag 26, kv_end = 26 + 4
    assert p["items"] == [[4, 2, 0, 32, 30, 0, -1, 0], [0, 4, 0, 30, 26, 0, -1, 0]]


def test_hand_worked_causal_pruning():
    """One prefill request, 6 new rows after a 26-token prefix (K = 32), page 4,
    tiles of 4 rows, 2-page (8-key) chunks.  Tile 0 (rows 0..3, diag 26) sees
    keys < 30: chunks [0,8) [8,16) [16,24) [24,30).  Tile 1 (rows 4,5, diag 30)
    sees keys < 32: chunks up to [24,32)."""
    p = pl.plan(mode="prefill", qo_indptr=[0, 6], kv_indptr=[0, 8], kv_last_page_len=[4],
                page_size=4, heads_y=1, rows=4, causal=True, num_cus=1, fixed_split_pages=2)
    t0 = sorted(i for i in p["items"] if i[0] == 0)
    t1 = sorted(i for i in p["items"] if i[0] == 4)
    assert [(i[2], i[3]) for i in t0] == [(0, 8), (8, 16), (16, 24), (24, 30)]
    assert [(i[2], i[3]) for i in t1] == [(0, 8), (8, 16), (16, 24), (24, 32)]
    assert all(i[4] == 26 and i[1] == 4 for i in t0) and all(i[4] == 30 and i[1] == 2 for i in t1)
    assert p["merges"] == [[0, 4, 0, 4], [4, 2, 16, 4]]
    assert p["num_partial_rows"] == 24


def _random_case(rng, mode):
    b = int(rng.integers(1, 9))
    page = int(rng.choice([1, 3, 4, 16]))
    if mode == "prefill":
        q = [int(x) for x in rng.integers(0, 40, size=b)]
        k = [qi + int(rng.integers(0, 90)) for qi in q]
        k = [max(1, x) for x in k]
        qo = list(np.cumsum([0] + q))
    else:
        k = [int(x) for x in rng.integers(1, 700, size=b)]
        qo = None
    n = [math.ceil(x / page) for x in k]
    last = [x - (m - 1) * page for x, m in zip(k, n)]
    return dict(qo_indptr=qo, kv_indptr=list(np.cumsum([0] + n)), kv_last_page_len=last, page_size=page,
                k=k)


@pytest.mark.parametrize("mode", ["decode", "prefill", "mla"])
def test_partition_invariants(mode):
    rng = np.random.default_rng(21)
    for trial in range(60):
        c = _random_case(rng, mode)
        rows = int(rng.choice([1, 2, 4, 32])) if mode == "prefill" else 1
        causal = bool(rng.integers(2)) if mode == "prefill" else True
        fixed = int(rng.choice([0, 0, 1, 2, 7]))
        tail = int(rng.choice([0, 1, 2, 3]))
        p = pl.plan(mode=mode, qo_indptr=c["qo_indptr"], kv_indptr=c["kv_indptr"],
                    kv_last_page_len=c["kv_last_page_len"], page_size=c["page_size"],
                    heads_y=int(rng.integers(1, 9)), rows=rows, causal=causal,
                    num_cus=int(rng.integers(1, 300)), fixed_split_pages=fixed, tail_split=tail)
        chunk_tok = p["chunk_pages"] * c["page_size"]
        qo = c["qo_indptr"] or list(range(len(c["k"]) + 1))
        by_tile = {}
        for it in p["items"]:
            q_row0, n_rows, lo, hi, diag, page_base, slot, b = it
            # page-aligned pieces, each inside one chunk
            assert lo % c["page_size"] == 0 and 0 <= lo < hi and lo // chunk_tok == (hi - 1) // chunk_tok
            assert page_base == c["kv_indptr"][b] and qo[b] <= q_row0 < qo[b + 1]
            assert q_row0 + n_rows <= qo[b + 1] and n_rows >= 1
            by_tile.setdefault((b, q_row0), []).append(it)
        # every query row is covered by exactly one tile
        covered = sorted(r for (b, r0), its in by_tile.items() for r in range(r0, r0 + its[0][1]))
        assert covered == list(range(qo[-1]))
        for (b, r0), its in by_tile.items():
            k_len, q_len = c["k"][b], qo[b + 1] - qo[b]
            l0 = r0 - qo[b]
            diag = (k_len - q_len + l0) if causal else k_len
            limit = min(k_len, diag + its[0][1])
            spans = sorted((i[2], i[3]) for i in its)
            # chunks tile [0, limit) exactly once
            assert spans[0][0] == 0 and spans[-1][1] == limit
            assert all(a[1] == b_[0] for a, b_ in zip(spans, spans[1:]))
            assert all(i[4] == diag for i in its)
            if len(its) == 1:
                assert its[0][6] == -1
            else:
                m = [x for x in p["merges"] if x[0] == r0]
                assert len(m) == 1 and m[0][1] == its[0][1] and m[0][3] == len(its)
                slots = sorted(i[6] for i in its)
                assert slots == [m[0][2] + c_ * its[0][1] for c_ in range(len(its))]
        total = sum(m[1] * m[3] for m in p["merges"])
        assert total == p["num_partial_rows"]
        costs = [i[3] - i[2] for i in p["items"]]
        assert costs == sorted(costs, reverse=True)
        if fixed == 1:
            assert all(i[3] - i[2] <= c["page_size"] for i in p["items"])


def test_rows_per_tile_rule():
    assert pl.rows_per_tile("decode", 4, "bf16") == 1
    assert pl.rows_per_tile("prefill", 4, "f32") == 1
    assert pl.rows_per_tile("prefill", 4, "bf16") == 64
    assert pl.rows_per_tile("prefill", 1, "bf16") == 256
    assert pl.rows_per_tile("prefill", 256, "bf16") == 1
    assert pl.rows_per_tile("prefill", 512, "bf16") == 1
    assert pl.rows_per_tile("prefill", 4, "fp8") == 64
    assert pl.rows_per_tile("decode", 4, "fp8") == 1
    assert pl.rows_per_tile("prefill", 4, "fp8", masked=True) == 64
    assert pl.rows_per_tile("prefill", 1, "fp8", masked=True) == 1
    assert pl.rows_per_tile("prefill", 4, "bf16", masked=True) == 64
    assert pl.rows_per_tile("prefill", 1, "bf16", masked=True) == 1
    # Head dims other than 128 run one row per item (no MFMA tile instantiation).
    assert pl.rows_per_tile("prefill", 4, "bf16", head_dim=64) == 1
    assert pl.rows_per_tile("prefill", 2, "fp8", head_dim=256) == 1
    assert pl.rows_per_tile("prefill", 4, "bf16", head_dim=128) == 64


def test_empty_batch_and_empty_requests():
    p = pl.plan(mode="prefill", qo_indptr=[0], kv_indptr=[0], kv_last_page_len=[], page_size=4,
                heads_y=2, rows=4, causal=True, num_cus=8)
    assert p["items"] == [] and p["merges"] == []
    p = pl.plan(mode="prefill", qo_indptr=[0, 0, 2], kv_indptr=[0, 1, 2], kv_last_page_len=[3, 4],
                page_size=4, heads_y=1, rows=4, causal=True, num_cus=8)
    assert [i[7] for i in p["items"]] == [1]


def test_hand_worked_cascade():
    """Two levels over 3 query rows, page 4, group 1, float32 (one row per tile).
    Level 0: one node (rows 0..2) with 10 keys (3 pages); prefill mode (3 rows),
    not causal, 8-key chunks: [0,8) and [8,10) for each of the 3 row tiles.
    Level 1: nodes of 1 row each (decode mode) with 5, 2 and 4 keys (2, 1, 1
    pages), one chunk each.  Level 0's partial rows come first (tile r gets
    slots 2r, 2r+1), then level 1's (6, 7, 8).  Level 1's page_base is shifted
    by level 0's 3 page ids."""
    levels = [{"qo_indptr": [0, 3], "kv_indptr": [0, 3], "kv_last_page_len": [2]},
              {"qo_indptr": [0, 1, 2, 3], "kv_indptr": [0, 2, 3, 4], "kv_last_page_len": [1, 2, 4]}]
    p = pl.plan_cascade(levels=levels, page_size=4, group=1, kv_dtype="f32", heads_y=1, causal=True,
                        num_cus=1, fixed_split_pages=2, tail_split=1)
    assert [lv["mode"] for lv in p["levels"]] == ["prefill", "decode"]
    assert [lv["num_items"] for lv in p["levels"]] == [6, 3]
    assert p["items"][:6] == [[0, 1, 0, 8, 10, 0, 0, 0], [1, 1, 0, 8, 10, 0, 2, 0], [2, 1, 0, 8, 10, 0, 4, 0],
                              [0, 1, 8, 10, 10, 0, 1, 0], [1, 1, 8, 10, 10, 0, 3, 0], [2, 1, 8, 10, 10, 0, 5, 0]]
    assert p["items"][6:] == [[0, 1, 0, 5, 4, 3, 6, 0], [2, 1, 0, 4, 3, 6, 8, 2], [1, 1, 0, 2, 1, 5, 7, 1]]
    assert p["row_ptr"] == [0, 3, 6, 9]
    assert p["slots"] == [0, 1, 6, 2, 3, 7, 4, 5, 8]
    assert p["num_partial_rows"] == 9


def test_cascade_plan_invariants():
    """Random trees: every partial row belongs to exactly one query row; each
    row lists one state per chunk of the tile holding it at every level; the
    level's items cover its nodes' keys as in a plain plan."""
    rng = np.random.default_rng(5)
    for trial in range(40):
        n_req = int(rng.integers(1, 10))
        qo_lens = [int(x) for x in rng.integers(0 if trial % 3 else 1, 5, size=n_req)]
        if trial % 3 == 0:
            qo_lens = [1] * n_req
        rows = list(np.cumsum([0] + qo_lens))
        # level 0: one root; level 1: random groups; level 2: leaves
        cuts = sorted(set([0, n_req] + [int(x) for x in rng.integers(0, n_req + 1, size=2)]))
        page = int(rng.choice([1, 4, 16]))
        levels = []
        for bounds in ([0, n_req], cuts, list(range(n_req + 1))):
            nodes = len(bounds) - 1
            k = [int(rng.integers(1, 90)) for _ in range(nodes)]
            if bounds == list(range(n_req + 1)):
                k = [max(x, q) for x, q in zip(k, qo_lens)]
            n = [math.ceil(x / page) for x in k]
            levels.append({"qo_indptr": [rows[b] for b in bounds], "kv_indptr": list(np.cumsum([0] + n)),
                           "kv_last_page_len": [x - (m - 1) * page for x, m in zip(k, n)], "k": k})
        group = int(rng.choice([1, 4, 8]))
        dtype = str(rng.choice(["f32", "bf16"]))
        causal = bool(rng.integers(2))
        p = pl.plan_cascade(levels=levels, page_size=page, group=group, kv_dtype=dtype, heads_y=2,
                            causal=causal, num_cus=int(rng.integers(1, 300)),
                            fixed_split_pages=int(rng.choice([0, 1, 3])), tail_split=int(rng.choice([0, 1, 2])))
        total = rows[-1]
        assert p["total_rows"] == total and len(p["row_ptr"]) == total + 1
        assert sorted(p["slots"]) == list(range(p["num_partial_rows"]))
        off = 0
        page_base = 0
        slot_base = 0
        for li, (lv, info) in enumerate(zip(levels, p["levels"])):
            its = p["items"][off:off + info["num_items"]]
            off += info["num_items"]
            qo = lv["qo_indptr"]
            one_row = all(qo[n + 1] - qo[n] == 1 for n in range(len(qo) - 1))
            assert info["mode"] == ("decode" if one_row else "prefill")
            # the same items as a plain plan of the level, shifted
            ref = pl.plan(mode=info["mode"], qo_indptr=None if one_row else qo, kv_indptr=lv["kv_indptr"],
                          kv_last_page_len=lv["kv_last_page_len"], page_size=page, heads_y=2,
                          rows=info["rows_per_tile"], causal=causal and li == 2,
                          num_cus=1, fixed_split_pages=info["chunk_pages"], all_partial=True,
                          tail_split=1 if info["mode"] == "prefill" else 0)
            if p["levels"][li]["chunk_pages"] == ref["chunk_pages"]:
                for it in its:
                    assert it[5] - page_base == lv["kv_indptr"][it[7]] and it[6] >= slot_base
            page_base += lv["kv_indptr"][-1]
            slot_base += info["num_partial_rows"]
            # every row gets exactly the chunks of its level-l tile
            for r in range(total):
                mine = [it for it in its if it[0] <= r < it[0] + it[1]]
                assert mine, (li, r)
                lst = p["slots"][p["row_ptr"][r]:p["row_ptr"][r + 1]]
                got = sorted(it[6] + (r - it[0]) for it in mine)
                assert all(s in lst for s in got)
        assert off == len(p["items"])
        for r in range(total):
            assert p["row_ptr"][r + 1] - p["row_ptr"][r] >= 3


def test_masked_prefill_tile_rows():
    assert pl.rows_per_tile("prefill", 4, "bf16", masked=True) == 64
    assert pl.rows_per_tile("prefill", 4, "bf16", masked=False) == 64
    assert pl.rows_per_tile("prefill", 1, "bf16", masked=True) == 1
    assert pl.rows_per_tile("prefill", 1, "bf16", masked=False) == 256
    assert pl.rows_per_tile("prefill", 4, "f32", masked=True) == 1


def test_hand_worked_ragged_plan():
    """Two requests: 3 rows over 40 keys, 2 rows over 17 keys; virtual pages
    of 16 keys (3 and 2 pages); one-row tiles, not causal, 2-page chunks:
    request 0 chunks [0,32) [32,40), request 1 [0,17).  page_base is the
    request index."""
    p = pl.plan_ragged(qo_indptr=[0, 3, 5], kv_indptr=[0, 40, 57], heads_y=1, rows=1, causal=False, num_cus=1,
                       fixed_split_pages=2, tail_split=1)
    assert p["chunk_pages"] == 2
    req0 = sorted((i[0], i[2], i[3]) for i in p["items"] if i[7] == 0)
    assert req0 == [(r, lo, hi) for r in range(3) for lo, hi in ((0, 32), (32, 40))]
    req1 = sorted((i[0], i[2], i[3], i[6]) for i in p["items"] if i[7] == 1)
    assert req1 == [(3, 0, 17, -1), (4, 0, 17, -1)]
    assert all(i[5] == i[7] for i in p["items"])
    # a request without keys (and rows) makes no items
    p = pl.plan_ragged(qo_indptr=[0, 0, 2], kv_indptr=[0, 0, 5], heads_y=1, rows=1, causal=True, num_cus=1)
    assert [i[7] for i in p["items"]] == [1, 1]
