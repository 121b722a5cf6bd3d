"""The seeded input generator builds valid batches of the stated shapes."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import metadata as md


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 7
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]     # ties to even both ways
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.to_bf16_bits(x), want)


@pytest.mark.parametrize("name,kw", [
    ("worked", dict(literal_pages=True)),
    ("worked", {}),
    ("decode", dict(scale=0.05)),
    ("skewed", dict(scale=0.02)),
    ("prefill", dict(scale=0.02)),
    ("mla", dict(scale=0.05)),
])
def test_batches_are_valid(name, kw):
    b = wl.make(name, poison=True, **kw)
    lens = md.validate(qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                       kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                       page_size=b.page_size, max_num_pages=b.max_num_pages,
                       num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
                       decode=(b.mode != "prefill"))
    assert lens == b.kv_lens
    assert all(x.dtype == np.int32 for x in (b.qo_indptr, b.kv_indptr, b.kv_indices, b.kv_last_page_len))
    # pages are unique across requests (a shuffled pool)
    assert len(set(b.kv_indices.tolist())) == len(b.kv_indices)


def test_worked_literal_pages_and_sizes():
    b = wl.make("worked", literal_pages=True)
    assert b.kv_indices.tolist() == [7, 2, 11, 3, 14, 6]
    assert b.kv_indptr.tolist() == [0, 2, 3, 6] and b.kv_last_page_len.tolist() == [2, 2, 1]
    assert b.q.shape == (8, 4, 64) and b.k_cache.shape == (16, 4, 2, 64)
    assert b.k_new.shape == (8, 2, 64)


def test_full_size_shapes_and_ranges():
    d = wl.make("decode")
    assert d.batch_size == 64 and d.max_num_pages == 20000 and d.k_cache.shape == (20000, 16, 8, 128)
    assert min(d.kv_lens) >= 512 and max(d.kv_lens) <= 4096
    s = wl.make("skewed")
    assert s.kv_lens[0] == 32768 and all(256 <= x <= 1024 for x in s.kv_lens[1:])
    assert s.max_num_pages == sum(s.kv_lens) and set(s.kv_last_page_len.tolist()) == {1}


def test_poison_marks_only_unowned_slots():
    b = wl.make("worked", literal_pages=True, poison=True)
    # history slots (before the append) are finite, everything else NaN
    hist = {(7, 0), (7, 1), (7, 2), (11, 0), (3, 0), (3, 1), (3, 2), (3, 3), (14, 0)}
    for page in range(16):
        for slot in range(4):
            finite = np.isfinite(b.k_cache[page, slot]).all()
            assert finite == ((page, slot) in hist)


@pytest.mark.parametrize("name,kw", [("worked", {}), ("decode", {"scale": 0.1}), ("skewed", {"scale": 0.05}),
                                     ("prefill", {"scale": 0.1}), ("mla", {"scale": 0.1}),
                                     ("cascade", {"scale": 0.05}), ("cascade_small", {})])
def test_metadata_only_batches_match(name, kw):
    """payload=False stops after the metadata draws, which come first: the
    metadata equals that of the full batch and no tensor is drawn."""
    full = wl.make(name, **kw)
    meta = wl.make(name, payload=False, **kw)
    for f in ("qo_indptr", "kv_indptr", "kv_indices", "kv_last_page_len"):
        assert np.array_equal(getattr(full, f), getattr(meta, f)), f
    assert full.kv_lens == meta.kv_lens and full.qo_lens == meta.qo_lens and full.max_num_pages == meta.max_num_pages
    assert meta.q is None and meta.k_cache is None
    if "levels" in full.extra:
        for a, b in zip(full.extra["levels"], meta.extra["levels"]):
            assert all(np.array_equal(np.asarray(a[k]), np.asarray(b[k])) for k in a)
