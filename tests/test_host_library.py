"""CPU tests of the native host library (no kernel launches): the C ABI
loads and exports everything include/pkv.h declares, the validator agrees with
the oracle rule by rule, and the native planner matches the oracle's planner
specification bit for bit."""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import workloads as wl
from oracle import metadata as md
from oracle import planner as pl

pkv = pytest.importorskip("paged_kv_cache_plan_amd")
from paged_kv_cache_plan_amd import _abi  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pkv.LIB_PATH)
    declared = _declared_functions()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(lib, name), name
    # and the binding declares exactly those
    assert sorted(_abi.SIGNATURES) == declared


def test_version_string():
    assert "gfx950" in pkv.version()


BASE = dict(qo_indptr=[0, 3, 4, 8], kv_indptr=[0, 2, 3, 6], kv_indices=[7, 2, 11, 3, 14, 6],
            kv_last_page_len=[2, 2, 1], page_size=4, max_num_pages=16)

CASES = [
    dict(kv_indptr=[1, 2, 3, 6]),
    dict(qo_indptr=[0, 3, 2, 8]),
    dict(kv_indptr=[0, 2, 2, 6], kv_indices=[7, 2, 3, 14, 6, 1]),
    dict(kv_last_page_len=[2, 0, 1]),
    dict(kv_last_page_len=[2, 5, 1]),
    dict(kv_indices=[7, 2, 11, 3, 16, 6]),
    dict(kv_indices=[7, 2, 11, 3, -1, 6]),
    dict(kv_indptr=[0, 2, 3, 7]),
    dict(qo_indptr=[0, 3, 6, 10]),
    dict(page_size=0),
    dict(num_qo_heads=6, num_kv_heads=4),
    dict(decode=True),
    dict(qo_indptr=[0, 3, 3, 7]),
    dict(),
]


@pytest.mark.parametrize("change", CASES)
def test_validator_matches_oracle(change):
    args = dict(BASE)
    args.update(change)
    try:
        want = md.validate(**args)
        want_reason = None
    except md.MetadataError as e:
        want_reason = e.reason
    if want_reason is None:
        got = pkv.validate(**args)
        assert list(got) == want
    else:
        with pytest.raises(pkv.PkvError) as e:
            pkv.validate(**args)
        assert e.value.status == _abi.ERR_METADATA
        assert e.value.reason == _abi.META_REASONS[want_reason]


def test_validator_rejects_int64_metadata():
    with pytest.raises(TypeError):
        pkv.validate(**dict(BASE, kv_indptr=np.array([0, 2, 3, 6], dtype=np.int64)))


def test_append_validation():
    pkv.validate_append(append_indptr=[0, 3, 4, 8], kv_indptr=[0, 2, 3, 6], kv_indices=[7, 2, 11, 3, 14, 6],
                        kv_last_page_len=[2, 2, 1], page_size=4, max_num_pages=16)
    with pytest.raises(pkv.PkvError) as e:
        pkv.validate_append(append_indptr=[0, 1, 2], kv_indptr=[0, 1, 2], kv_indices=[5, 5],
                            kv_last_page_len=[4, 4], page_size=4, max_num_pages=8)
    assert e.value.reason == _abi.META_REASONS["append_collision"]
    with pytest.raises(pkv.PkvError) as e:
        pkv.validate_append(append_indptr=[0, 3], kv_indptr=[0, 1], kv_indices=[5], kv_last_page_len=[2],
                            page_size=4, max_num_pages=8)
    assert e.value.reason == _abi.META_REASONS["qo_exceeds_kv"]


def _compare_plans(mode, qo_indptr, kv_indptr, kv_indices, last, page_size, hq, hkv, dtype, causal, num_cus,
                   fixed=0, target=0, mla_groups=0, tail=0):
    params = pkv.plan_params(mode=mode, batch_size=len(last), num_qo_heads=hq, num_kv_heads=hkv,
                             head_dim_qk=576 if mode == "mla" else 128, head_dim_vo=512 if mode == "mla" else 128,
                             page_size=page_size, causal=causal, dtype=dtype, num_cus=num_cus,
                             fixed_split_pages=fixed, target_per_cu=target, mla_head_groups=mla_groups,
                             tail_split=tail)
    info, items, merges = pkv.plan_compute(params, qo_indptr=qo_indptr if mode == "prefill" else None,
                                           kv_indptr=kv_indptr, kv_indices=kv_indices, kv_last_page_len=last)
    rows = pl.rows_per_tile(mode, hq // hkv, dtype)
    assert info["rows_per_tile"] == rows
    spec = pl.plan(mode=mode, qo_indptr=list(qo_indptr) if mode == "prefill" else None,
                   kv_indptr=list(kv_indptr), kv_last_page_len=list(last), page_size=page_size,
                   heads_y=info["heads_y"], rows=rows, causal=causal, num_cus=num_cus, fixed_split_pages=fixed,
                   target_per_cu=target, tail_split=tail)
    assert items.tolist() == spec["items"]
    assert merges.tolist() == spec["merges"]
    assert info["num_partial_rows"] == spec["num_partial_rows"]
    assert info["chunk_pages"] == spec["chunk_pages"]
    assert bool(info["split"]) == spec["split"]
    return info


@pytest.mark.parametrize("name,kw", [
    ("worked", dict(literal_pages=True)),
    ("decode", {}),
    ("decode", dict(batch=2048, kv_range=(1, 96), seed=4104)),   # past the default tail split's reach
    ("skewed", {}),
    ("prefill", {}),
    ("mla", {}),
])
def test_planner_matches_spec_on_workloads(name, kw):
    b = wl.make(name, payload=False, **kw, **({} if name == "worked" else {"scale": 1.0}))
    mode = b.mode
    hkv = b.num_kv_heads
    for num_cus in (256, 80):
        info = _compare_plans(mode, b.qo_indptr, b.kv_indptr, b.kv_indices, b.kv_last_page_len, b.page_size,
                              b.num_qo_heads, hkv, b.dtype, b.causal, num_cus)
        assert info["num_items"] > 0
    if name == "skewed":
        assert info["split"] == 1


def test_planner_matches_spec_randomised():
    rng = np.random.default_rng(33)
    for trial in range(150):
        mode = ["decode", "prefill", "mla"][trial % 3]
        b = int(rng.integers(1, 12))
        page = int(rng.choice([1, 4, 16, 64]))
        if mode == "prefill":
            q = [int(x) for x in rng.integers(0, 300, size=b)]
            k = [max(1, qi + int(rng.integers(0, 3000))) for qi in q]
        else:
            q = [1] * b
            k = [int(x) for x in rng.integers(1, 20000, size=b)]
        n = [math.ceil(x / page) for x in k]
        kv_indptr = np.array([0] + list(np.cumsum(n)), dtype=np.int32)
        last = np.array([x - (m - 1) * page for x, m in zip(k, n)], dtype=np.int32)
        qo = np.array([0] + list(np.cumsum(q)), dtype=np.int32)
        hq, hkv = (128, 1) if mode == "mla" else [(32, 8), (8, 8), (16, 2), (64, 8)][trial % 4]
        dtype = "bf16" if (mode == "mla" or trial % 5) else "f32"
        _compare_plans(mode, qo, kv_indptr, None, last, page, hq, hkv, dtype, bool(trial % 2),
                       int(rng.integers(1, 400)), fixed=int(rng.choice([0, 0, 0, 1, 3, 50])),
                       target=int(rng.choice([0, 1, 2, 8])), tail=int(rng.choice([0, 1, 2, 3])))


def test_fingerprint_tracks_metadata():
    params = pkv.plan_params(mode="decode", batch_size=3, num_qo_heads=4, num_kv_heads=2, head_dim_qk=128,
                             page_size=4, num_cus=8)
    base = dict(qo_indptr=None, kv_indptr=[0, 2, 3, 6], kv_indices=[7, 2, 11, 3, 14, 6], kv_last_page_len=[2, 2, 1])
    f0 = pkv.plan_compute(params, **base)[0]["fingerprint"]
    assert pkv.plan_compute(params, **base)[0]["fingerprint"] == f0
    moved = dict(base, kv_indices=[7, 2, 11, 3, 14, 5])
    assert pkv.plan_compute(params, **moved)[0]["fingerprint"] != f0
    grown = dict(base, kv_last_page_len=[2, 2, 2])
    assert pkv.plan_compute(params, **grown)[0]["fingerprint"] != f0


def test_plan_rejects_bad_inputs():
    params = pkv.plan_params(mode="prefill", batch_size=3, num_qo_heads=4, num_kv_heads=2, head_dim_qk=64,
                             page_size=4, num_cus=8, dtype="f32", max_num_pages=16)
    with pytest.raises(pkv.PkvError) as e:
        pkv.plan_compute(params, qo_indptr=[0, 3, 4, 8], kv_indptr=[0, 2, 3, 6], kv_indices=[7, 2, 11, 3, 99, 6],
                         kv_last_page_len=[2, 2, 1])
    assert e.value.status == _abi.ERR_METADATA and e.value.reason == _abi.META_REASONS["page_index"]
    with pytest.raises(pkv.PkvError) as e:
        pkv.plan_compute(params, qo_indptr=None, kv_indptr=[0, 2, 3, 6], kv_indices=None, kv_last_page_len=[2, 2, 1])
    assert e.value.status == _abi.ERR_INVALID_ARG
    mla = pkv.plan_params(mode="mla", batch_size=1, num_qo_heads=100, num_kv_heads=1, head_dim_qk=576,
                          head_dim_vo=512, page_size=64, num_cus=8)
    with pytest.raises(pkv.PkvError) as e:
        pkv.plan_compute(mla, qo_indptr=None, kv_indptr=[0, 1], kv_indices=None, kv_last_page_len=[5])
    assert e.value.status == _abi.ERR_UNSUPPORTED


# ---------------------------------------------------------------- cascade --

from oracle import cascade as oc  # noqa: E402


def _cascade_params(hq, hkv, page, dtype, causal, num_cus, fixed=0, target=0, tail=0, max_pages=0):
    return pkv.plan_params(mode="prefill", batch_size=0, num_qo_heads=hq, num_kv_heads=hkv, head_dim_qk=128,
                           page_size=page, causal=causal, dtype=dtype, num_cus=num_cus, fixed_split_pages=fixed,
                           target_per_cu=target, tail_split=tail, max_num_pages=max_pages)


def _compare_cascade(levels, page, hq, hkv, dtype, causal, num_cus, fixed=0, target=0, tail=0):
    params = _cascade_params(hq, hkv, page, dtype, causal, num_cus, fixed, target, tail)
    info, lvl, items, row_ptr, slots = pkv.cascade_plan_compute(params, levels)
    spec = pl.plan_cascade(levels=levels, page_size=page, group=hq // hkv, kv_dtype=dtype, heads_y=hkv,
                           causal=causal, num_cus=num_cus, fixed_split_pages=fixed, target_per_cu=target,
                           tail_split=tail)
    assert items.tolist() == spec["items"]
    assert row_ptr.tolist() == spec["row_ptr"]
    assert slots.tolist() == spec["slots"]
    assert info["num_partial_rows"] == spec["num_partial_rows"] == info["num_merge_slots"]
    assert info["total_rows"] == spec["total_rows"]
    assert [x["num_items"] for x in lvl] == [x["num_items"] for x in spec["levels"]]
    assert [x["mode"] for x in lvl] == [{"decode": 0, "prefill": 1}[x["mode"]] for x in spec["levels"]]
    assert [x["chunk_pages"] for x in lvl] == [x["chunk_pages"] for x in spec["levels"]]
    return info


@pytest.mark.parametrize("name", ["cascade", "cascade_small"])
def test_cascade_planner_matches_spec_on_workloads(name):
    b = wl.make(name, payload=False)
    for num_cus in (256, 80):
        info = _compare_cascade(b.extra["levels"], b.page_size, b.num_qo_heads, b.num_kv_heads, b.dtype,
                                b.causal, num_cus)
        assert info["num_items"] > 0


def test_cascade_planner_matches_spec_randomised():
    rng = np.random.default_rng(44)
    for trial in range(60):
        n_req = int(rng.integers(1, 12))
        qo_lens = [1] * n_req if trial % 2 else [int(x) for x in rng.integers(0, 40, size=n_req)]
        rows = list(np.cumsum([0] + qo_lens))
        page = int(rng.choice([1, 4, 16]))
        depth = int(rng.integers(1, 4))
        bounds = [[0, n_req]]
        for _ in range(depth - 2):
            bounds.append(sorted(set(bounds[-1] + [int(x) for x in rng.integers(0, n_req + 1, size=2)])))
        if depth > 1:
            bounds.append(list(range(n_req + 1)))
        else:
            bounds = [list(range(n_req + 1))]
        levels = []
        for li, bd in enumerate(bounds):
            k = [int(rng.integers(1, 3000)) for _ in range(len(bd) - 1)]
            if li == len(bounds) - 1:
                k = [max(x, q) for x, q in zip(k, qo_lens)]
            n = [math.ceil(x / page) for x in k]
            levels.append({"qo_indptr": np.array([rows[i] for i in bd], np.int32),
                           "kv_indptr": np.array([0] + list(np.cumsum(n)), np.int32),
                           "kv_last_page_len": np.array([x - (m - 1) * page for x, m in zip(k, n)], np.int32)})
        hq, hkv = [(32, 8), (8, 8), (16, 2)][trial % 3]
        _compare_cascade(levels, page, hq, hkv, "bf16" if trial % 4 else "f32", bool(trial % 3),
                         int(rng.integers(1, 400)), fixed=int(rng.choice([0, 0, 1, 3])),
                         target=int(rng.choice([0, 1, 4])), tail=int(rng.choice([0, 1, 2])))


def _lv(qo, kv_pages, last, indices=None):
    indptr = [0]
    for n in kv_pages:
        indptr.append(indptr[-1] + n)
    return {"qo_indptr": qo, "kv_indptr": indptr,
            "kv_indices": list(range(indptr[-1])) if indices is None else indices, "kv_last_page_len": last}


CASCADE_CASES = [
    [],
    [_lv([0, 5], [3], [2]), _lv([0, 2, 5], [1, 2], [4, 1]), _lv([0, 1, 2, 4, 5], [1, 1, 1, 1], [1, 2, 2, 3])],
    [_lv([0, 4], [3], [2]), _lv([0, 1, 2, 4, 5], [1, 1, 1, 1], [1, 2, 2, 3])],
    [_lv([0, 3, 5], [1, 1], [4, 4]), _lv([0, 2, 5], [1, 2], [4, 4])],
    [_lv([0, 5], [3], [2]), _lv([0, 2, 5], [1, 1], [1, 2])],
    [_lv([0, 5], [1], [1]), _lv([0, 2, 5], [1, 1], [2, 3])],
    [_lv([0, 5], [3], [5]), _lv([0, 5], [2], [4])],
    [_lv([0, 5], [3], [2], indices=[0, 1, 99]), _lv([0, 5], [2], [4])],
    [_lv([1, 5], [3], [2]), _lv([0, 5], [2], [4])],
    [_lv([0, 5], [0], [2]), _lv([0, 5], [2], [4])],
]


@pytest.mark.parametrize("levels", CASCADE_CASES)
def test_cascade_validation_matches_oracle(levels):
    try:
        want = oc.validate_levels(levels, page_size=4, max_num_pages=64)
        want_reason = None
    except md.MetadataError as e:
        want_reason = e.reason
    params = _cascade_params(1, 1, 4, "f32", True, 8, max_pages=64)
    if want_reason is None:
        info = pkv.cascade_plan_compute(params, levels)[0]
        assert info["num_levels"] == len(levels) and want
    else:
        with pytest.raises(pkv.PkvError) as e:
            pkv.cascade_plan_compute(params, levels)
        assert e.value.status == _abi.ERR_METADATA
        assert e.value.reason == _abi.META_REASONS[want_reason]


# --------------------------------------------------- fixed-capacity plans --

@pytest.mark.parametrize("mode", ["decode", "prefill", "mla"])
def test_graph_capacities_bound_every_plan(mode):
    """The derived capacities of a fixed-capacity plan hold every plan the
    planner spec makes for batches within them (random lengths, fixed split
    sizes, targets and tail splits)."""
    rng = np.random.default_rng({"decode": 1, "prefill": 2, "mla": 3}[mode])
    for trial in range(40):
        B = int(rng.integers(1, 24))
        page = int(rng.choice([1, 4, 16, 64]))
        max_pages = int(rng.integers(B, 40 * B + 1))
        max_rows = int(rng.integers(B, 300 * B)) if mode == "prefill" else B
        hq, hkv = (128, 1) if mode == "mla" else [(32, 8), (8, 2), (16, 16)][trial % 3]
        dtype = "bf16" if (mode == "mla" or trial % 4) else "f32"
        fixed = int(rng.choice([0, 0, 1, 5]))
        target, tail = int(rng.choice([0, 1, 3])), int(rng.choice([0, 1, 2, 3]))
        num_cus = int(rng.integers(1, 300))
        params = pkv.plan_params(mode=mode, batch_size=B, num_qo_heads=hq, num_kv_heads=hkv,
                                 head_dim_qk=576 if mode == "mla" else 128, head_dim_vo=512 if mode == "mla" else 128,
                                 page_size=page, dtype=dtype, num_cus=num_cus, fixed_split_pages=fixed,
                                 target_per_cu=target, tail_split=tail)
        caps, ws, st = pkv.graph_plan_size(params, pkv.graph_caps(max_total_rows=max_rows, max_total_pages=max_pages))
        assert ws >= st > 0
        for _ in range(5):
            # a batch at (or near) the capacities
            n = np.maximum(1, rng.multinomial(max_pages - B, np.ones(B) / B) + 1) if rng.random() < 0.7 else \
                rng.integers(1, max(2, max_pages // B) + 1, size=B)
            n = [int(x) for x in n]
            if sum(n) > max_pages:
                continue
            last = [int(rng.integers(1, page + 1)) for _ in range(B)]
            k = [page * (m - 1) + t for m, t in zip(n, last)]
            if mode == "prefill":
                q = [int(x) for x in rng.multinomial(max_rows, np.ones(B) / B)]
                q = [min(a, b) for a, b in zip(q, k)]
                qo = list(np.cumsum([0] + q))
            else:
                qo = None
            spec = pl.plan(mode=mode, qo_indptr=qo, kv_indptr=list(np.cumsum([0] + n)), kv_last_page_len=last,
                           page_size=page, heads_y=hkv if mode != "mla" else 1, rows=pl.rows_per_tile(mode, hq // hkv,
                                                                                                      dtype),
                           causal=bool(trial % 2), num_cus=num_cus, fixed_split_pages=fixed, target_per_cu=target,
                           tail_split=tail)
            assert len(spec["items"]) <= caps["max_items"], (trial, len(spec["items"]), caps)
            assert len(spec["merges"]) <= caps["max_merges"]
            assert spec["num_partial_rows"] <= caps["max_partial_rows"]


# --------------------------------------------------- ragged KV, custom masks --

from oracle import mask as omask  # noqa: E402


def test_ragged_planner_matches_spec_randomised():
    rng = np.random.default_rng(55)
    for trial in range(80):
        B = int(rng.integers(1, 10))
        kv = [int(x) for x in rng.integers(0, 3000, size=B)]
        q = [int(rng.integers(0, k + 1)) if k else 0 for k in kv]
        hq, hkv = [(32, 8), (8, 8), (16, 2)][trial % 3]
        dtype = "bf16" if trial % 4 else "f32"
        masked = trial % 5 == 0
        causal = bool(trial % 2) and not masked
        fixed, tail = int(rng.choice([0, 0, 1, 3])), int(rng.choice([0, 1, 2]))
        num_cus = int(rng.integers(1, 300))
        params = pkv.plan_params(mode="prefill", batch_size=B, num_qo_heads=hq, num_kv_heads=hkv, head_dim_qk=128,
                                 page_size=16, causal=causal, dtype=dtype, num_cus=num_cus, fixed_split_pages=fixed,
                                 tail_split=tail, ragged=True, custom_mask=masked)
        qo = np.array([0] + list(np.cumsum(q)), np.int32)
        kvp = np.array([0] + list(np.cumsum(kv)), np.int32)
        info, items, merges = pkv.plan_compute(params, qo_indptr=qo, kv_indptr=kvp, kv_indices=None,
                                               kv_last_page_len=None)
        rows = pl.rows_per_tile("prefill", hq // hkv, dtype, masked=masked)
        spec = pl.plan_ragged(qo_indptr=list(qo), kv_indptr=list(kvp), heads_y=hkv, rows=rows, causal=causal,
                              num_cus=num_cus, fixed_split_pages=fixed, tail_split=tail)
        assert items.tolist() == spec["items"] and merges.tolist() == spec["merges"]
        assert info["rows_per_tile"] == rows
        assert info["mask_bits"] == (omask.mask_indptr(q, kv)[-1] if masked else 0)


@pytest.mark.parametrize("qo,kv", [
    ([0, 3, 5], [0, 40, 57]),
    ([1, 3, 5], [0, 40, 57]),
    ([0, 3, 2], [0, 40, 57]),
    ([0, 3, 5], [0, 40, 39]),
    ([0, 3, 50], [0, 40, 57]),
    ([0, 0, 0], [0, 0, 9]),
])
def test_ragged_validation_matches_oracle(qo, kv):
    try:
        omask.validate_ragged(qo_indptr=qo, kv_indptr=kv, num_qo_heads=4, num_kv_heads=2)
        want = None
    except md.MetadataError as e:
        want = e.reason
    params = pkv.plan_params(mode="prefill", batch_size=2, num_qo_heads=4, num_kv_heads=2, head_dim_qk=64,
                             page_size=16, causal=False, dtype="f32", num_cus=4, ragged=True)
    kw = dict(qo_indptr=np.array(qo, np.int32), kv_indptr=np.array(kv, np.int32), kv_indices=None,
              kv_last_page_len=None)
    if want is None:
        pkv.plan_compute(params, **kw)
    else:
        with pytest.raises(pkv.PkvError) as e:
            pkv.plan_compute(params, **kw)
        assert e.value.reason == _abi.META_REASONS[want]


def test_mask_and_ragged_parameter_rules():
    base = dict(batch_size=1, num_qo_heads=4, num_kv_heads=2, head_dim_qk=64, page_size=4, dtype="f32", num_cus=4)
    meta = dict(qo_indptr=np.array([0, 2], np.int32), kv_indptr=np.array([0, 1], np.int32),
                kv_indices=np.array([0], np.int32), kv_last_page_len=np.array([3], np.int32))
    with pytest.raises(pkv.PkvError) as e:       # a custom mask replaces the causal rule
        pkv.plan_compute(pkv.plan_params(mode="prefill", causal=True, custom_mask=True, **base), **meta)
    assert e.value.status == _abi.ERR_INVALID_ARG
    for mode in ("decode", "mla"):
        with pytest.raises(pkv.PkvError) as e:
            pkv.plan_compute(pkv.plan_params(mode=mode, causal=False, ragged=True, **base),
                             **dict(meta, qo_indptr=None))
        assert e.value.status == _abi.ERR_UNSUPPORTED
    info = pkv.plan_compute(pkv.plan_params(mode="prefill", causal=False, custom_mask=True, **base), **meta)[0]
    assert info["mask_bits"] == 2 * 3 and info["rows_per_tile"] == 1   # float32: the row kernel


def test_timing_events_are_armed_in_pairs():
    """pkv_time_next_attention takes both events or neither (no GPU needed:
    arming only stores the handles for the next launch)."""
    lib = pkv.lib()
    assert lib.pkv_time_next_attention(None, None) == _abi.OK
    assert lib.pkv_time_next_attention(ctypes.c_void_p(16), None) == _abi.ERR_INVALID_ARG
    assert lib.pkv_time_next_attention(None, ctypes.c_void_p(16)) == _abi.ERR_INVALID_ARG
    with pytest.raises(ValueError):
        pkv.time_next_attention(object(), None)
    pkv.time_next_attention()          # disarm: both NULL


def test_binding_rejects_bad_host_and_device_arguments():
    """Argument checks of the Python binding that run before any C call: host
    metadata must be int32 (never silently cast), device arguments must be
    device tensors of the right dtype, and metadata lengths must match the
    batch size the plan was made for."""
    import torch
    from paged_kv_cache_plan_amd import _check_batch, _dev, _dtype_code, _host_i32
    assert _host_i32(None, "x") == (None, None)
    arr, ptr = _host_i32([0, 3, 4], "x")
    assert arr.dtype == np.int32 and list(arr) == [0, 3, 4] and ptr is not None
    for bad in (np.array([0, 1], np.int64), torch.tensor([0, 1], dtype=torch.int64), [0.5, 1.0]):
        with pytest.raises(TypeError):
            _host_i32(bad if not isinstance(bad, list) else np.asarray(bad), "x")
    with pytest.raises(TypeError):
        _dev(torch.zeros(4), "q")                       # a host tensor where a device one is needed
    with pytest.raises(TypeError):
        _dev(np.zeros(4), "q")
    assert _dtype_code(torch.zeros(1, dtype=torch.bfloat16)) == _abi.BF16
    assert _dtype_code(torch.zeros(1, dtype=torch.uint8)) == _abi.FP8_E4M3
    with pytest.raises(TypeError):
        _dtype_code(torch.zeros(1, dtype=torch.float16))
    p = pkv.plan_params(mode="prefill", batch_size=2, num_qo_heads=4, num_kv_heads=2, head_dim_qk=64,
                        page_size=4, dtype="f32")
    _check_batch(p, [0, 1, 2], [0, 1, 2], [1, 1])
    for qo, kvp, last in (([0, 1], [0, 1, 2], [1, 1]), ([0, 1, 2], [0, 1], [1, 1]), ([0, 1, 2], [0, 1, 2], [1]),
                          ([0, 1, 2], None, [1, 1]), ([0, 1, 2], [0, 1, 2], None)):
        with pytest.raises(ValueError):
            _check_batch(p, qo, kvp, last)
    r = pkv.plan_params(mode="prefill", batch_size=2, num_qo_heads=4, num_kv_heads=2, head_dim_qk=64,
                        page_size=4, dtype="f32", ragged=True)
    _check_batch(r, [0, 1, 2], [0, 3, 5], None)          # ragged plans take no tail lengths


def _p32(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


# A 256-byte aligned address that is never dereferenced: every call below
# fails its size check before it touches device memory or the device.
FAKE_DEVICE_PTR = ctypes.c_void_p(1 << 20)


def test_plan_create_rejects_small_workspace_and_staging():
    """pkv_plan_create refuses a workspace or pinned staging buffer smaller
    than the plan needs (PKV_ERR_WORKSPACE) before any upload, and a missing
    workspace when the plan needs one."""
    lib = pkv.lib()
    params = pkv.plan_params(mode="decode", batch_size=3, num_qo_heads=4, num_kv_heads=2, head_dim_qk=64,
                             page_size=4, dtype="f32", num_cus=4, fixed_split_pages=1, max_num_pages=16)
    kvp, idx = np.array([0, 2, 3, 6], np.int32), np.array([7, 2, 11, 3, 14, 6], np.int32)
    last = np.array([2, 2, 1], np.int32)
    info = pkv.plan_compute(params, qo_indptr=None, kv_indptr=kvp, kv_indices=idx, kv_last_page_len=last)[0]
    ws, st = info["workspace_bytes"], info["staging_bytes"]
    assert ws > st > 0 and info["num_partial_rows"] > 0
    staging = np.zeros(st + 256, np.uint8)
    handle = ctypes.c_void_p()

    def create(ws_ptr, ws_bytes, st_ptr, st_bytes):
        return lib.pkv_plan_create(ctypes.byref(params), None, _p32(kvp), _p32(idx), len(idx), _p32(last), ws_ptr,
                                   ws_bytes, st_ptr, st_bytes, None, ctypes.byref(handle))

    stp = ctypes.c_void_p(staging.ctypes.data)
    assert create(FAKE_DEVICE_PTR, ws - 1, stp, st) == _abi.ERR_WORKSPACE
    assert b"workspace" in lib.pkv_last_error()
    assert create(None, ws, stp, st) == _abi.ERR_WORKSPACE
    assert create(FAKE_DEVICE_PTR, ws, stp, st - 1) == _abi.ERR_WORKSPACE
    assert b"staging" in lib.pkv_last_error()
    assert create(ctypes.c_void_p((1 << 20) + 16), ws, stp, st) == _abi.ERR_INVALID_ARG   # not 256-aligned
    assert not handle.value


def test_graph_and_cascade_plans_reject_small_workspace():
    lib = pkv.lib()
    params = pkv.plan_params(mode="decode", batch_size=2, num_qo_heads=4, num_kv_heads=2, head_dim_qk=64,
                             page_size=4, dtype="f32", num_cus=4, max_num_pages=16)
    caps = pkv.graph_caps(max_total_pages=8)
    _, ws, st = pkv.graph_plan_size(params, caps)
    staging = np.zeros(st, np.uint8)
    handle = ctypes.c_void_p()
    assert lib.pkv_graph_plan_create(ctypes.byref(params), ctypes.byref(caps), FAKE_DEVICE_PTR, ws - 1,
                                     ctypes.c_void_p(staging.ctypes.data), st, None,
                                     ctypes.byref(handle)) == _abi.ERR_WORKSPACE
    assert lib.pkv_graph_plan_create(ctypes.byref(params), ctypes.byref(caps), FAKE_DEVICE_PTR, ws,
                                     ctypes.c_void_p(staging.ctypes.data), st - 1, None,
                                     ctypes.byref(handle)) == _abi.ERR_WORKSPACE
    levels = [dict(qo_indptr=[0, 2], kv_indptr=[0, 2], kv_indices=[1, 2], kv_last_page_len=[4]),
              dict(qo_indptr=[0, 1, 2], kv_indptr=[0, 1, 2], kv_indices=[3, 4], kv_last_page_len=[2, 3])]
    cparams = pkv.plan_params(mode="prefill", batch_size=0, num_qo_heads=4, num_kv_heads=2, head_dim_qk=64,
                              page_size=4, dtype="f32", num_cus=4, max_num_pages=16)
    info = pkv.cascade_plan_compute(cparams, levels)[0]
    arr, keep = pkv._cascade_levels(levels)
    cst = np.zeros(info["staging_bytes"], np.uint8)
    chandle = ctypes.c_void_p()
    assert lib.pkv_cascade_plan_create(ctypes.byref(cparams), 2, arr, FAKE_DEVICE_PTR, info["workspace_bytes"] - 1,
                                       ctypes.c_void_p(cst.ctypes.data), cst.size, None,
                                       ctypes.byref(chandle)) == _abi.ERR_WORKSPACE
    assert not handle.value and not chandle.value


def test_mla_plans_that_run_need_the_pool_size():
    """An MLA run bounds page ids by the plan's max_num_pages (pkv_run_mla
    takes no cache descriptor), so creating an MLA plan without it is refused;
    host-only planning (pkv_plan_compute) does not need it."""
    lib = pkv.lib()
    params = pkv.plan_params(mode="mla", batch_size=1, num_qo_heads=128, num_kv_heads=1, head_dim_qk=576,
                             head_dim_vo=512, page_size=64, dtype="bf16", num_cus=4)
    kvp, last, idx = np.array([0, 2], np.int32), np.array([10], np.int32), np.array([5, 9], np.int32)
    info = pkv.plan_compute(params, qo_indptr=None, kv_indptr=kvp, kv_indices=idx, kv_last_page_len=last)[0]
    staging = np.zeros(max(256, info["staging_bytes"]), np.uint8)
    handle = ctypes.c_void_p()
    st = lib.pkv_plan_create(ctypes.byref(params), None, _p32(kvp), _p32(idx), len(idx), _p32(last),
                             FAKE_DEVICE_PTR, 1 << 30, ctypes.c_void_p(staging.ctypes.data), staging.size, None,
                             ctypes.byref(handle))
    assert st == _abi.ERR_INVALID_ARG and b"max_num_pages" in lib.pkv_last_error()
    caps = pkv.graph_caps(max_total_pages=4)
    gst = lib.pkv_graph_plan_create(ctypes.byref(params), ctypes.byref(caps), FAKE_DEVICE_PTR, 1 << 30,
                                    ctypes.c_void_p(staging.ctypes.data), staging.size, None, ctypes.byref(handle))
    assert gst == _abi.ERR_INVALID_ARG and not handle.value


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prefill_at_head_dim_64_plans_one_row_tiles(dtype):
    """bf16 / fp8 prefill at a head dim the MFMA tile kernel is not built for
    runs on the row kernel, which streams an item's keys once per row: the
    planner gives it one-row tiles, as the oracle's planner spec does."""
    rng = np.random.default_rng(11)
    kv_lens = [int(x) for x in rng.integers(40, 300, size=5)]
    qo_lens = [int(rng.integers(1, k + 1)) for k in kv_lens]
    page = 16
    pages = [(k + page - 1) // page for k in kv_lens]
    kvp = np.array(md.indptr_from_lengths(pages), np.int32)
    last = np.array([k - page * (n - 1) for k, n in zip(kv_lens, pages)], np.int32)
    qo = np.array(md.indptr_from_lengths(qo_lens), np.int32)
    params = pkv.plan_params(mode="prefill", batch_size=5, num_qo_heads=8, num_kv_heads=2, head_dim_qk=64,
                             page_size=page, dtype="bf16", kv_dtype=dtype, num_cus=16)
    info, items, merges = pkv.plan_compute(params, qo_indptr=qo, kv_indptr=kvp, kv_indices=None,
                                           kv_last_page_len=last)
    rows = pl.rows_per_tile("prefill", 4, dtype, head_dim=64)
    assert rows == 1 and info["rows_per_tile"] == 1
    spec = pl.plan(mode="prefill", qo_indptr=list(qo), kv_indptr=list(kvp), kv_last_page_len=list(last),
                   page_size=page, heads_y=2, rows=rows, causal=True, num_cus=16)
    assert items.tolist() == spec["items"] and merges.tolist() == spec["merges"]
    assert info["num_items"] >= sum(qo_lens)


def test_noalloc_run_rejects_batches_beyond_its_array():
    """pkv_run_noalloc refuses, with the size it needed, a batch whose work
    list and partial states exceed PKV_NOALLOC_SCRATCH_BYTES (before any
    device call), and the plan kinds it does not run."""
    lib = pkv.lib()
    batch, pages = 512, 8
    params = pkv.plan_params(mode="decode", batch_size=batch, num_qo_heads=64, num_kv_heads=8, head_dim_qk=128,
                             page_size=16, dtype="bf16", num_cus=256, fixed_split_pages=1, max_num_pages=batch * pages)
    kvp = np.arange(0, batch * pages + 1, pages, dtype=np.int32)
    last = np.full(batch, 16, np.int32)
    info = pkv.plan_compute(params, qo_indptr=None, kv_indptr=kvp, kv_indices=None, kv_last_page_len=last)[0]
    assert info["workspace_bytes"] > pkv.NOALLOC_SCRATCH_BYTES
    assert "#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)" in open(os.path.join(ROOT, "include", "pkv.h")).read()
    assert pkv.NOALLOC_SCRATCH_BYTES == 32 << 20
    desc = _abi.CacheDesc()
    st = lib.pkv_run_noalloc(ctypes.byref(params), None, _p32(kvp), None, 0, _p32(last), FAKE_DEVICE_PTR, 64 * 128,
                             128, ctypes.byref(desc), FAKE_DEVICE_PTR, FAKE_DEVICE_PTR, 64 * 128, 128, None,
                             ctypes.c_float(0.0), None)
    assert st == _abi.ERR_WORKSPACE
    assert str(info["workspace_bytes"]).encode() in lib.pkv_last_error()
    mla = pkv.plan_params(mode="mla", batch_size=1, num_qo_heads=128, num_kv_heads=1, head_dim_qk=576,
                          head_dim_vo=512, page_size=64, dtype="bf16", num_cus=4, max_num_pages=4)
    st = lib.pkv_run_noalloc(ctypes.byref(mla), None, _p32(np.array([0, 1], np.int32)), None, 0,
                             _p32(np.array([3], np.int32)), FAKE_DEVICE_PTR, 0, 0, ctypes.byref(desc),
                             FAKE_DEVICE_PTR, FAKE_DEVICE_PTR, 0, 0, None, ctypes.c_float(0.0), None)
    assert st == _abi.ERR_INVALID_ARG


def test_row_waves_choice_and_checks():
    """Decode plans pick one-wave row workgroups when their items average at
    most 384 keys and number at least 24 per CU (times the kv heads), else 4
    waves; an explicit row_waves is used as given.  Other values, one-wave
    plans outside decode and one-wave fixed-capacity plans are refused."""
    def info(b, **kw):
        params = pkv.plan_params(mode=b.mode, batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                                 num_kv_heads=b.num_kv_heads, head_dim_qk=b.head_dim, page_size=b.page_size,
                                 causal=b.causal, dtype=b.dtype, **kw)
        return pkv.plan_compute(params, qo_indptr=b.qo_indptr if b.mode == "prefill" else None,
                                kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                                kv_last_page_len=b.kv_last_page_len)[0]
    short = wl.make("decode", payload=False, batch=2048, kv_range=(1, 96), seed=4104)   # 2048 items of ~47 keys
    assert info(short, num_cus=256)["row_waves"] == 1          # 64 (item, head) units per CU
    assert info(short, num_cus=512)["row_waves"] == 1          # 32 per CU
    assert info(short, num_cus=1024)["row_waves"] == 4         # 16 per CU
    assert info(short, num_cus=256, row_waves=4)["row_waves"] == 4
    dec = wl.make("decode", payload=False)                      # 188 items of ~734 keys
    assert info(dec, num_cus=256)["row_waves"] == 4
    assert info(dec, num_cus=256, row_waves=1)["row_waves"] == 1
    assert info(wl.make("skewed", payload=False), num_cus=256)["row_waves"] == 4
    assert info(wl.make("prefill", payload=False, scale=0.1), num_cus=256)["row_waves"] == 4
    with pytest.raises(pkv.PkvError) as e:
        info(dec, num_cus=256, row_waves=2)
    assert e.value.status == _abi.ERR_INVALID_ARG
    with pytest.raises(pkv.PkvError) as e:
        info(wl.make("prefill", payload=False, scale=0.1), num_cus=256, row_waves=1)
    assert e.value.status == _abi.ERR_UNSUPPORTED
    params = pkv.plan_params(mode="decode", batch_size=2, num_qo_heads=4, num_kv_heads=2, head_dim_qk=64,
                             page_size=4, dtype="f32", num_cus=4, max_num_pages=16, row_waves=1)
    caps = pkv.graph_caps(max_total_pages=8)
    _, ws, st = pkv.graph_plan_size(params, caps)
    staging = np.zeros(st, np.uint8)
    handle = ctypes.c_void_p()
    assert pkv.lib().pkv_graph_plan_create(ctypes.byref(params), ctypes.byref(caps), FAKE_DEVICE_PTR, ws,
                                           ctypes.c_void_p(staging.ctypes.data), st, None,
                                           ctypes.byref(handle)) == _abi.ERR_UNSUPPORTED
    assert not handle.value
