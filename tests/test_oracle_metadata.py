"""Pins for oracle.metadata: values the pages print, plus derived closed forms.

Each test names the passage it pins.  Derived values (not printed on the
pages) are worked out by hand in the test's docstring from the printed ones.
"""

import numpy as np
import pytest

from oracle import metadata as md
from tests.conftest import load_golden


def test_worked_example_metadata():
    """Deep Dive - FlashInfer, 'Why inference attention becomes irregular'."""
    g = load_golden("worked_example.json")
    p = g["page_size"]
    assert md.indptr_from_lengths(g["qo_lens"]) == g["qo_indptr"]
    assert md.indptr_from_lengths([len(x) for x in g["pages"]]) == g["kv_indptr"]
    assert [x for pages in g["pages"] for x in pages] == g["kv_indices"]
    lens = [md.kv_len(pages, tail, p) for pages, tail in zip(g["pages"], g["kv_last_page_len"])]
    assert lens == g["kv_len"]
    assert md.kv_lens(g["kv_indptr"], g["kv_indices"], g["kv_last_page_len"], p) == g["kv_len"]
    # every reported KV length counts the new tokens: prefix + new = kv_len
    assert [a + b for a, b in zip(g["prefix_lens"], g["qo_lens"])] == g["kv_len"]
    assert md.validate(qo_indptr=g["qo_indptr"], kv_indptr=g["kv_indptr"], kv_indices=g["kv_indices"],
                       kv_last_page_len=g["kv_last_page_len"], page_size=p,
                       max_num_pages=16) == g["kv_len"]


@pytest.mark.parametrize("case", range(4))
def test_worked_example_rejections(case):
    """The four rejected page lists of the same section's check."""
    g = load_golden("worked_example.json")
    pages, tail = g["rejected_page_lists"][case]
    with pytest.raises(md.MetadataError) as e:
        md.kv_len(pages, tail, g["page_size"])
    assert e.value.reason in ("empty_page_list", "last_page_len", "page_index")


def test_addresses_and_mask():
    """Deep Dive - FlashInfer, 'Causality uses logical positions, not page numbers'."""
    g = load_golden("addresses_mask.json")
    ids, p, ql, kl = g["page_ids"], g["page_size"], g["q_len"], g["kv_len"]
    indptr = [0, len(ids)]
    addr = [md.token_address(indptr, ids, p, 0, j) for j in range(kl)]
    assert list(addr[5]) == g["token5"]
    assert list(addr[-1]) == g["last_token"]
    assert ([pg for pg, _ in addr] != sorted(pg for pg, _ in addr)) == g["page_order_is_unsorted"]
    rows = ["".join("1" if md.visible(i, j, ql, kl) else "." for j in range(kl)) for i in range(ql)]
    assert rows == g["printed_mask"]
    assert [md.visible_count(i, ql, kl) for i in range(ql)] == g["row_counts"]


def test_visible_pairs_worked_batch():
    """Derived from the bottom-right rule on the worked batch: R0 (Q=3, K=6)
    rows see 4, 5, 6 keys; R1 (Q=1, K=2) sees 2; R2 sees 6..9 (printed).
    Total 15 + 2 + 30 = 47 visible (row, key) pairs per head."""
    counts = {0: (3, 6), 1: (1, 2), 2: (4, 9)}
    per_row = {b: [md.visible_count(i, q, k) for i in range(q)] for b, (q, k) in counts.items()}
    assert per_row == {0: [4, 5, 6], 1: [2], 2: [6, 7, 8, 9]}
    assert sum(sum(v) for v in per_row.values()) == 47


def test_decode_row_sees_everything():
    """A single query row (decode) sees all K keys under the same rule."""
    for k in (1, 2, 17, 300):
        assert md.visible_count(0, 1, k) == k


def test_append_slots_worked_example():
    """Derived: the new tokens of each request are its last q_b positions
    (kv_len counts them), addressed as (pages[pos // 4], pos % 4).
    R0: positions 3,4,5 -> (7,3),(2,0),(2,1); R1: position 1 -> (11,1);
    R2: positions 5..8 -> (14,1),(14,2),(14,3),(6,0).  R2's first target is
    the printed (14, 1)."""
    g = load_golden("worked_example.json")
    targets = md.append_targets(g["qo_indptr"], g["kv_indptr"], g["kv_indices"],
                                g["kv_last_page_len"], g["page_size"])
    assert targets == [(7, 3), (2, 0), (2, 1), (11, 1), (14, 1), (14, 2), (14, 3), (6, 0)]
    assert list(targets[4]) == load_golden("addresses_mask.json")["token5"]


def test_append_rejects_collisions_and_overflow():
    with pytest.raises(md.MetadataError) as e:
        # two requests sharing page 5 and both appending into its last slot
        md.append_targets([0, 1, 2], [0, 1, 2], [5, 5], [4, 4], 4)
    assert e.value.reason == "append_collision"
    with pytest.raises(md.MetadataError) as e:
        md.append_targets([0, 3], [0, 1], [5], [2], 4)
    assert e.value.reason == "qo_exceeds_kv"


def test_token_table_to_page_table():
    """GPU attention backends: FlashInfer and FlashAttention, 'What it prints'
    and the first exercise's answer: the same two requests as page-size-1
    CSR metadata and as a page-size-4 page-number table."""
    g = load_golden("token_to_page.json")
    one = md.token_table_to_page_table(g["token_rows"], g["seq_lens"], 1)
    assert one["kv_indptr"] == g["page_size_1"]["kv_indptr"]
    assert one["kv_indices"] == g["page_size_1"]["kv_indices"]
    assert one["kv_last_page_len"] == g["page_size_1"]["kv_last_page_len"]
    four = md.token_table_to_page_table(g["token_rows"], g["seq_lens"], 4)
    assert four["page_table"] == g["page_size_4"]["page_table"]
    # derived: 5 tokens on pages of 4 leave a tail of 1, 6 tokens a tail of 2
    assert four["kv_last_page_len"] == [1, 2]
    assert md.kv_lens(four["kv_indptr"], four["kv_indices"], four["kv_last_page_len"], 4) == \
        g["page_size_4"]["cache_seqlens"]
    qo = [s - c for s, c in zip(g["seq_lens"], g["cached_lens"])]
    assert md.indptr_from_lengths(qo) == g["page_size_1"]["qo_indptr"] == g["page_size_4"]["cu_seqlens_q"]


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("single", [True, False])
def test_element_offset_matches_numpy_strides(layout, single):
    """The NHD/HND shapes of "FlashInfer 中的 KV-Cache 布局" ('页表布局'),
    checked against numpy's own row-major index computation."""
    pages, p, h, d = 5, 4, 3, 8
    inner = (p, h, d) if layout == "NHD" else (h, p, d)
    shape = (pages, 2) + inner if single else (pages,) + inner
    rng = np.random.default_rng(0)
    for _ in range(200):
        page, slot, head, dim, kv = (int(rng.integers(n)) for n in (pages, p, h, d, 2))
        idx_inner = (slot, head, dim) if layout == "NHD" else (head, slot, dim)
        idx = (page, kv) + idx_inner if single else (page,) + idx_inner
        want = int(np.ravel_multi_index(idx, shape))
        got = md.element_offset(layout, page=page, slot=slot, head=head, dim=dim, page_size=p,
                                num_heads=h, head_dim=d, kv=kv if single else None)
        assert got == want


BASE = dict(qo_indptr=[0, 3, 4, 8], kv_indptr=[0, 2, 3, 6], kv_indices=[7, 2, 11, 3, 14, 6],
            kv_last_page_len=[2, 2, 1], page_size=4, max_num_pages=16)


@pytest.mark.parametrize("change,reason", [
    (dict(kv_indptr=[1, 2, 3, 6]), "indptr_start"),
    (dict(qo_indptr=[0, 3, 2, 8]), "indptr_order"),
    (dict(kv_indptr=[0, 2, 3]), "indptr_length"),
    (dict(kv_indptr=[0, 2, 2, 6], kv_indices=[7, 2, 3, 14, 6, 1]), "empty_page_list"),
    (dict(kv_last_page_len=[2, 0, 1]), "last_page_len"),
    (dict(kv_last_page_len=[2, 5, 1]), "last_page_len"),
    (dict(kv_indices=[7, 2, 11, 3, 16, 6]), "page_index"),
    (dict(kv_indices=[7, 2, 11, 3, -1, 6]), "page_index"),
    (dict(kv_indptr=[0, 2, 3, 7]), "indices_length"),
    (dict(qo_indptr=[0, 3, 6, 10]), "qo_exceeds_kv"),
    (dict(page_size=0), "page_size"),
])
def test_validate_rules(change, reason):
    args = dict(BASE)
    args.update(change)
    with pytest.raises(md.MetadataError) as e:
        md.validate(**args)
    assert e.value.reason == reason


def test_validate_heads_and_decode():
    with pytest.raises(md.MetadataError) as e:
        md.validate(**BASE, num_qo_heads=6, num_kv_heads=4)
    assert e.value.reason == "head_group"
    with pytest.raises(md.MetadataError) as e:
        md.validate(**BASE, decode=True)
    assert e.value.reason == "decode_qo_len"
    args = dict(BASE, qo_indptr=None)
    assert md.validate(**args, decode=True) == [6, 2, 9]
    # an empty request (qo_len 0) is allowed: it contributes no rows
    assert md.validate(**dict(BASE, qo_indptr=[0, 3, 3, 7])) == [6, 2, 9]
    # an empty batch is valid
    assert md.validate(qo_indptr=[0], kv_indptr=[0], kv_indices=[], kv_last_page_len=[],
                       page_size=4, max_num_pages=1) == []
