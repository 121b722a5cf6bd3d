"""Seeded synthetic inputs for paged KV-cache attention.

This module only draws inputs: request lengths, page permutations and
N(0, 1) payloads, packed as CSR page-table metadata and caches.  It holds none
of the attention arithmetic and is the one module that both the CPU oracle
(tests, bench baseline) and the HIP path (tests, bench) import.

Draw order per workload (one ``numpy.random.default_rng(seed)``): lengths,
page permutation, Q, K pool, V pool, new K, new V.  A pool draws values only
for the pages some request owns, in ascending page id, 2048 pages at a time.  bfloat16 payloads are
drawn as float32 N(0, 1) and rounded to nearest-even bfloat16 here, so the GPU
and the oracle see the same bits.  With ``poison=True`` every pool slot that
no request owns (unused pages, page tails past last_page_len, and the slots
an append is about to fill) holds NaN, so any read of them shows.

Workloads (sizes follow the pages' worked example and the serving mixes
described there):
  worked    3 requests, qo 3/1/4, kv 6/2/9, page 4, pool 16, heads 4/2, dim
            64, float32, NHD, causal, sm_scale 1/8.  ``literal_pages=True``
            uses the pages' own page ids 7,2 | 11 | 3,14,6.
  decode    64 requests, qo 1, kv U[512, 4096], page 16, pool 20000 pages,
            heads 32/8, dim 128, bfloat16, NHD.
  skewed    16 requests, qo 1, one kv 32768 and 15 kv U[256, 1024], page 1,
            pool = exactly the tokens used, heads 32/8, dim 128, bfloat16, NHD.
  prefill   8 requests, qo U[512, 2048], prefix U[0, 8192], kv = prefix + qo,
            page 16, HND, heads 32/8, dim 128, bfloat16, causal; new K/V are
            appended before attention.
  mla       32 requests, qo 1, kv U[1024, 8192], page 64, latent cache
            [pages, 64, 512 + 64] bfloat16, 128 heads, sm_scale 1/sqrt(576).
  cascade   shared-prefix decode over a 3-level tree: 64 requests; level 0
            one node (all requests) with a 16384-token prefix; level 1 eight
            nodes of 8 requests, U[1024, 4096] tokens each; level 2 one leaf
            per request, U[128, 1024] tokens ending with its query row; page
            16, heads 32/8, dim 128, bfloat16, NHD.  Shared nodes hold whole
            pages (lengths rounded up to the page size), so the batch also has
            a flat one-level page table (``flat_levels``).  Each level has its own
            page table over one shared pool ("FlashInfer 中的 KV-Cache 布局",
            multi-level cascade layout).  ``cascade_small`` is the same tree
            shape at 8 requests (nodes 3/2/3), page 4, heads 4/2, dim 64,
            float32, qo U[1, 4] per leaf, causal.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)        # E4M3: exponent and mantissa all ones

WORKLOADS = ("worked", "decode", "skewed", "prefill", "mla", "cascade", "cascade_small")
SEEDS = {"worked": 1000, "decode": 1001, "skewed": 1002, "prefill": 1003, "mla": 1004, "cascade": 1005,
         "cascade_small": 1006}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def to_fp8_codes(x: np.ndarray) -> np.ndarray:
    """Round float32 to E4M3 (nearest, ties to even, saturating at 448, as
    torch's float8_e4m3fn conversion does); return the 8-bit codes."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _payload(rng, shape, dtype: str):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "fp8":
        return to_fp8_codes(x)
    return to_bf16_bits(x) if dtype == "bf16" else x


def _storage(dtype: str):
    return {"bf16": np.uint16, "fp8": np.uint8}.get(dtype, np.float32)


def _pool(rng, shape, dtype: str, owned_pages):
    """A page pool whose owned pages (in ascending page id) get fresh N(0, 1)
    draws; pages nobody owns stay zero (or NaN once poisoned)."""
    pool = np.zeros(shape, dtype=_storage(dtype))
    pages = np.unique(np.asarray(owned_pages, dtype=np.int64))
    step = 2048
    for i in range(0, len(pages), step):
        sel = pages[i:i + step]
        pool[sel] = _payload(rng, (len(sel),) + tuple(shape[1:]), dtype)
    return pool


@dataclass
class Batch:
    """One synthetic batch.  Arrays are numpy; metadata is int32."""
    name: str
    mode: str                      # "decode" | "prefill" | "mla"
    dtype: str                     # "f32" | "bf16": queries and outputs (and K/V unless kv_dtype says)
    layout: str                    # "NHD" | "HND" (ignored for mla)
    page_size: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    causal: bool
    sm_scale: float
    qo_lens: list
    kv_lens: list
    qo_indptr: np.ndarray
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    kv_last_page_len: np.ndarray
    max_num_pages: int
    q: np.ndarray = None           # [nnz, Hq, D]             (mla: q_ckv [B, H, 512])
    k_cache: np.ndarray = None     # tuple form, layout-shaped (mla: unified [pages, P, 576])
    v_cache: np.ndarray = None
    q_kpe: np.ndarray = None       # mla only: [B, H, 64]
    k_new: np.ndarray = None       # [nnz, Hkv, D] appended tokens (prefill/worked)
    v_new: np.ndarray = None
    append_indptr: np.ndarray = None
    extra: dict = field(default_factory=dict)
    kv_dtype: str = None           # K/V storage when it differs from dtype ("fp8": E4M3 codes)

    def __post_init__(self):
        if self.kv_dtype is None:
            self.kv_dtype = self.dtype

    @property
    def batch_size(self) -> int:
        return len(self.qo_lens)

    @property
    def nnz(self) -> int:
        return int(self.qo_indptr[-1])


def _csr(kv_lens, page_size, pages_for_request):
    n_pages = [max(1, math.ceil(k / page_size)) for k in kv_lens]
    kv_indptr = np.zeros(len(kv_lens) + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(n_pages)
    kv_indices = np.concatenate([np.asarray(pages_for_request(b, n), dtype=np.int32)
                                 for b, n in enumerate(n_pages)]) if kv_lens else np.zeros(0, np.int32)
    last = np.asarray([k - (n - 1) * page_size for k, n in zip(kv_lens, n_pages)], dtype=np.int32)
    return n_pages, kv_indptr, kv_indices.astype(np.int32), last


def _cache_shape(layout, pages, page_size, heads, dim):
    return (pages, page_size, heads, dim) if layout == "NHD" else (pages, heads, page_size, dim)


def _poison(cache, layout, used_slots, dtype):
    """Replace every (page, slot) not in ``used_slots`` by NaN."""
    pages, page_size = cache.shape[0], (cache.shape[1] if layout == "NHD" else cache.shape[2])
    keep = np.zeros((pages, page_size), dtype=bool)
    if len(used_slots):
        keep[used_slots[:, 0], used_slots[:, 1]] = True
    nan = {"bf16": BF16_NAN, "fp8": FP8_NAN}.get(dtype, np.float32(np.nan))
    if layout == "NHD":
        cache[~keep] = nan
    else:
        cache.transpose(0, 2, 1, 3)[~keep] = nan


def _slots(kv_indptr, kv_indices, page_size, b, lo, hi):
    j = np.arange(lo, hi)
    pages = kv_indices[kv_indptr[b]:kv_indptr[b + 1]]
    return np.stack([pages[j // page_size], j % page_size], axis=1) if len(j) else np.zeros((0, 2), np.int64)


def _gqa_batch(name, rng, *, mode, qo_lens, kv_lens, page_size, pool, pages_for_request, hq, hkv,
               dim, dtype, layout, causal, sm_scale, with_append, poison, kv_dtype=None, payload=True):
    kv_dtype = dtype if kv_dtype is None else kv_dtype
    n_pages, kv_indptr, kv_indices, last = _csr(kv_lens, page_size, pages_for_request)
    qo_indptr = np.zeros(len(qo_lens) + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_lens)
    nnz = int(qo_indptr[-1])
    if not payload:
        return Batch(name=name, mode=mode, dtype=dtype, kv_dtype=kv_dtype, layout=layout, page_size=page_size,
                     num_qo_heads=hq, num_kv_heads=hkv, head_dim=dim, causal=causal, sm_scale=sm_scale,
                     qo_lens=list(qo_lens), kv_lens=list(kv_lens), qo_indptr=qo_indptr,
                     kv_indptr=kv_indptr, kv_indices=kv_indices, kv_last_page_len=last, max_num_pages=pool,
                     append_indptr=qo_indptr.copy() if with_append else None)
    q = _payload(rng, (nnz, hq, dim), dtype)
    shape = _cache_shape(layout, pool, page_size, hkv, dim)
    k_cache = _pool(rng, shape, kv_dtype, kv_indices)
    v_cache = _pool(rng, shape, kv_dtype, kv_indices)
    k_new = v_new = append_indptr = None
    if with_append:
        k_new = _payload(rng, (nnz, hkv, dim), kv_dtype)
        v_new = _payload(rng, (nnz, hkv, dim), kv_dtype)
        append_indptr = qo_indptr.copy()
    if poison:
        # Slots holding cached history keep their values; everything else
        # (free pages, tails, and slots the append will fill) becomes NaN.
        hist = [_slots(kv_indptr, kv_indices, page_size, b, 0,
                       kv_lens[b] - (qo_lens[b] if with_append else 0)) for b in range(len(kv_lens))]
        used = np.concatenate(hist) if hist else np.zeros((0, 2), np.int64)
        _poison(k_cache, layout, used, kv_dtype)
        _poison(v_cache, layout, used, kv_dtype)
    return Batch(name=name, mode=mode, dtype=dtype, kv_dtype=kv_dtype, layout=layout, page_size=page_size,
                 num_qo_heads=hq, num_kv_heads=hkv, head_dim=dim, causal=causal, sm_scale=sm_scale,
                 qo_lens=list(qo_lens), kv_lens=list(kv_lens), qo_indptr=qo_indptr,
                 kv_indptr=kv_indptr, kv_indices=kv_indices, kv_last_page_len=last,
                 max_num_pages=pool, q=q, k_cache=k_cache, v_cache=v_cache, k_new=k_new,
                 v_new=v_new, append_indptr=append_indptr)


def make(name: str, *, seed: int | None = None, poison: bool = False, literal_pages: bool = False,
         scale: float = 1.0, payload: bool = True, **overrides) -> Batch:
    """Build workload ``name`` (one of WORKLOADS).

    ``scale`` < 1 shrinks lengths/batch for quick CPU tests while keeping the
    workload's structure; ``overrides`` replace individual knobs (e.g.
    ``layout="HND"``, ``page_size=1``, ``batch=4``).  ``payload=False``
    stops after the metadata draws (which come first, so the metadata is the
    same) and leaves every tensor None: for planner and validator checks.
    """
    rng = np.random.default_rng(SEEDS[name] if seed is None else seed)
    o = dict(overrides)
    if name == "worked":
        qo_lens, kv_lens = o.get("qo_lens", [3, 1, 4]), o.get("kv_lens", [6, 2, 9])
        page_size, pool = o.get("page_size", 4), o.get("pool", 16)
        perm = rng.permutation(pool)
        if literal_pages:
            fixed = {0: [7, 2], 1: [11], 2: [3, 14, 6]}
            pages_for = lambda b, n: fixed[b]
        else:
            starts = np.cumsum([0] + [math.ceil(k / page_size) for k in kv_lens])
            pages_for = lambda b, n: perm[starts[b]:starts[b] + n]
        return _gqa_batch("worked", rng, mode="prefill", qo_lens=qo_lens, kv_lens=kv_lens,
                          page_size=page_size, pool=pool, pages_for_request=pages_for,
                          hq=o.get("hq", 4), hkv=o.get("hkv", 2), dim=o.get("dim", 64),
                          dtype=o.get("dtype", "f32"), layout=o.get("layout", "NHD"), causal=True,
                          sm_scale=o.get("sm_scale", 1.0 / 8.0), with_append=True, poison=poison,
                          payload=payload)
    if name in ("decode", "skewed"):
        if name == "decode":
            batch = o.get("batch", max(1, int(round(64 * scale))))
            lo, hi = o.get("kv_range", (max(1, int(512 * scale)), max(1, int(4096 * scale))))
            kv_lens = [int(x) for x in rng.integers(lo, hi, size=batch, endpoint=True)]
            page_size = o.get("page_size", 16)
            pool = o.get("pool", max(int(20000 * scale), sum(math.ceil(k / page_size) for k in kv_lens)))
            layout = o.get("layout", "NHD")
        else:
            batch = o.get("batch", 16)
            long_len = o.get("long_len", max(1, int(32768 * scale)))
            lo, hi = o.get("kv_range", (max(1, int(256 * scale)), max(1, int(1024 * scale))))
            kv_lens = [long_len] + [int(x) for x in rng.integers(lo, hi, size=batch - 1, endpoint=True)]
            page_size = o.get("page_size", 1)
            pool = o.get("pool", sum(math.ceil(k / page_size) for k in kv_lens))
            layout = o.get("layout", "NHD")
        perm = rng.permutation(pool)
        starts = np.cumsum([0] + [math.ceil(k / page_size) for k in kv_lens])
        return _gqa_batch(name, rng, mode="decode", qo_lens=[1] * batch, kv_lens=kv_lens,
                          page_size=page_size, pool=pool,
                          pages_for_request=lambda b, n: perm[starts[b]:starts[b] + n],
                          hq=o.get("hq", 32), hkv=o.get("hkv", 8), dim=o.get("dim", 128),
                          dtype=o.get("dtype", "bf16"), layout=layout, causal=True,
                          sm_scale=o.get("sm_scale", 1.0 / math.sqrt(o.get("dim", 128))),
                          with_append=o.get("with_append", False), poison=poison, kv_dtype=o.get("kv_dtype"),
                          payload=payload)
    if name == "prefill":
        batch = o.get("batch", 8)
        qlo, qhi = o.get("qo_range", (max(1, int(512 * scale)), max(1, int(2048 * scale))))
        plo, phi = o.get("prefix_range", (0, int(8192 * scale)))
        qo_lens = [int(x) for x in rng.integers(qlo, qhi, size=batch, endpoint=True)]
        prefix = [int(x) for x in rng.integers(plo, phi, size=batch, endpoint=True)]
        kv_lens = [p + q for p, q in zip(prefix, qo_lens)]
        page_size = o.get("page_size", 16)
        need = sum(math.ceil(k / page_size) for k in kv_lens)
        pool = o.get("pool", need + need // 4 + 1)
        perm = rng.permutation(pool)
        starts = np.cumsum([0] + [math.ceil(k / page_size) for k in kv_lens])
        dim = o.get("dim", 128)
        return _gqa_batch("prefill", rng, mode="prefill", qo_lens=qo_lens, kv_lens=kv_lens,
                          page_size=page_size, pool=pool,
                          pages_for_request=lambda b, n: perm[starts[b]:starts[b] + n],
                          hq=o.get("hq", 32), hkv=o.get("hkv", 8), dim=dim,
                          dtype=o.get("dtype", "bf16"), layout=o.get("layout", "HND"),
                          causal=o.get("causal", True), sm_scale=o.get("sm_scale", 1.0 / math.sqrt(dim)),
                          with_append=True, poison=poison, kv_dtype=o.get("kv_dtype"), payload=payload)
    if name == "mla":
        batch = o.get("batch", max(1, int(round(32 * scale))))
        lo, hi = o.get("kv_range", (max(1, int(1024 * scale)), max(1, int(8192 * scale))))
        kv_lens = [int(x) for x in rng.integers(lo, hi, size=batch, endpoint=True)]
        page_size = o.get("page_size", 64)
        need = sum(math.ceil(k / page_size) for k in kv_lens)
        pool = o.get("pool", need + need // 4 + 1)
        perm = rng.permutation(pool)
        starts = np.cumsum([0] + [math.ceil(k / page_size) for k in kv_lens])
        n_pages, kv_indptr, kv_indices, last = _csr(
            kv_lens, page_size, lambda b, n: perm[starts[b]:starts[b] + n])
        heads = o.get("heads", 128)
        d_ckv, d_kpe = 512, 64
        qo_indptr = np.arange(batch + 1, dtype=np.int32)
        if not payload:
            return Batch(name="mla", mode="mla", dtype="bf16", layout="NHD", page_size=page_size,
                         num_qo_heads=heads, num_kv_heads=1, head_dim=d_ckv + d_kpe, causal=False,
                         sm_scale=o.get("sm_scale", 1.0 / math.sqrt(d_ckv + d_kpe)), qo_lens=[1] * batch,
                         kv_lens=kv_lens, qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices,
                         kv_last_page_len=last, max_num_pages=pool)
        q_ckv = _payload(rng, (batch, heads, d_ckv), "bf16")
        q_kpe = _payload(rng, (batch, heads, d_kpe), "bf16")
        cache = _pool(rng, (pool, page_size, d_ckv + d_kpe), "bf16", kv_indices)
        if poison:
            used = np.concatenate([_slots(kv_indptr, kv_indices, page_size, b, 0, kv_lens[b])
                                   for b in range(batch)])
            keep = np.zeros((pool, page_size), dtype=bool)
            keep[used[:, 0], used[:, 1]] = True
            cache[~keep] = BF16_NAN
        qo_indptr = np.arange(batch + 1, dtype=np.int32)
        return Batch(name="mla", mode="mla", dtype="bf16", layout="NHD", page_size=page_size,
                     num_qo_heads=heads, num_kv_heads=1, head_dim=d_ckv + d_kpe, causal=False,
                     sm_scale=o.get("sm_scale", 1.0 / math.sqrt(d_ckv + d_kpe)),
                     qo_lens=[1] * batch, kv_lens=kv_lens, qo_indptr=qo_indptr,
                     kv_indptr=kv_indptr, kv_indices=kv_indices, kv_last_page_len=last,
                     max_num_pages=pool, q=q_ckv, q_kpe=q_kpe, k_cache=cache, v_cache=None)
    if name in ("cascade", "cascade_small"):
        return _cascade(name, rng, o, scale, poison, payload)
    raise KeyError(name)


def _cascade(name, rng, o, scale, poison, payload=True):
    """A request tree as levels of nodes over one page pool.

    ``tree`` lists, per level, how many consecutive requests each node holds
    (the last level must be all ones: one leaf per request).  ``level_kv``
    gives each level's (lo, hi) token range per node; a leaf's range is
    raised to at least its qo_len, since the leaf holds the request's new
    tokens.  Every node owns its own pages (shared nodes once, not once per
    request).  Q rows are ragged over requests, like a prefill batch.
    """
    small = name == "cascade_small"
    if small:
        tree = o.get("tree", [[8], [3, 2, 3], [1] * 8])
        level_kv = o.get("level_kv", [(37, 37), (5, 20), (1, 12)])
        qo_range = o.get("qo_range", (1, 4))
        defaults = dict(page_size=4, hq=4, hkv=2, dim=64, dtype="f32", layout="NHD")
    else:
        tree = o.get("tree", [[1 * 64], [8] * 8, [1] * 64])
        level_kv = o.get("level_kv", [(int(16384 * scale),) * 2, (int(1024 * scale), int(4096 * scale)),
                                      (int(128 * scale), int(1024 * scale))])
        qo_range = o.get("qo_range", (1, 1))
        defaults = dict(page_size=16, hq=32, hkv=8, dim=128, dtype="bf16", layout="NHD")
    cfg = {k: o.get(k, v) for k, v in defaults.items()}
    page_size, hq, hkv, dim, dtype, layout = (cfg[k] for k in ("page_size", "hq", "hkv", "dim", "dtype", "layout"))
    batch = sum(tree[0])
    for lv in tree:
        if sum(lv) != batch:
            raise ValueError("every level must cover every request")
    if any(n != 1 for n in tree[-1]):
        raise ValueError("the last level holds one leaf per request")
    # Lengths: qo per request, then kv per node, level by level.
    qo_lens = [int(x) for x in rng.integers(qo_range[0], qo_range[1], size=batch, endpoint=True)]
    node_kv = []
    for li, lv in enumerate(tree):
        lo, hi = level_kv[li]
        lens = [int(x) for x in rng.integers(max(1, lo), max(1, hi), size=len(lv), endpoint=True)]
        if li == len(tree) - 1:
            lens = [max(k, q) for k, q in zip(lens, qo_lens)]
        elif o.get("shared_full_pages", not small):
            lens = [-(-k // page_size) * page_size for k in lens]
        node_kv.append(lens)
    n_pages = [[math.ceil(k / page_size) for k in lens] for lens in node_kv]
    need = sum(sum(x) for x in n_pages)
    pool = o.get("pool", need + need // 8 + 1)
    perm = rng.permutation(pool)
    levels = []
    start = 0
    for li, lv in enumerate(tree):
        rows = np.zeros(len(lv) + 1, dtype=np.int32)
        req = np.cumsum([0] + list(lv))
        rows[1:] = [sum(qo_lens[req[i]:req[i + 1]]) for i in range(len(lv))]
        rows = np.cumsum(rows).astype(np.int32)
        starts = start + np.cumsum([0] + n_pages[li])
        _, kv_indptr, kv_indices, last = _csr(node_kv[li], page_size,
                                              lambda b, n, s=starts: perm[s[b]:s[b] + n])
        start = int(starts[-1])
        levels.append({"qo_indptr": rows, "kv_indptr": kv_indptr, "kv_indices": kv_indices,
                       "kv_last_page_len": last, "kv_lens": node_kv[li], "num_requests": list(lv)})
    qo_indptr = np.zeros(batch + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_lens)
    nnz = int(qo_indptr[-1])
    leaf = levels[-1]
    if not payload:
        return Batch(name=name, mode="cascade", dtype=dtype, layout=layout, page_size=page_size,
                     num_qo_heads=hq, num_kv_heads=hkv, head_dim=dim, causal=o.get("causal", True),
                     sm_scale=o.get("sm_scale", 1.0 / math.sqrt(dim)), qo_lens=qo_lens,
                     kv_lens=list(leaf["kv_lens"]), qo_indptr=qo_indptr, kv_indptr=leaf["kv_indptr"],
                     kv_indices=leaf["kv_indices"], kv_last_page_len=leaf["kv_last_page_len"],
                     max_num_pages=pool, append_indptr=qo_indptr.copy(), extra={"levels": levels})
    q = _payload(rng, (nnz, hq, dim), dtype)
    shape = _cache_shape(layout, pool, page_size, hkv, dim)
    all_pages = np.concatenate([lv["kv_indices"] for lv in levels])
    k_cache = _pool(rng, shape, dtype, all_pages)
    v_cache = _pool(rng, shape, dtype, all_pages)
    leaf = levels[-1]
    k_new = _payload(rng, (nnz, hkv, dim), dtype)
    v_new = _payload(rng, (nnz, hkv, dim), dtype)
    if poison:
        used = []
        for li, lv in enumerate(levels):
            for b in range(len(lv["kv_lens"])):
                hi = lv["kv_lens"][b] - (qo_lens[b] if li == len(levels) - 1 else 0)
                used.append(_slots(lv["kv_indptr"], lv["kv_indices"], page_size, b, 0, hi))
        used = np.concatenate(used)
        _poison(k_cache, layout, used, dtype)
        _poison(v_cache, layout, used, dtype)
    return Batch(name=name, mode="cascade", dtype=dtype, layout=layout, page_size=page_size,
                 num_qo_heads=hq, num_kv_heads=hkv, head_dim=dim, causal=o.get("causal", True),
                 sm_scale=o.get("sm_scale", 1.0 / math.sqrt(dim)), qo_lens=qo_lens,
                 kv_lens=list(leaf["kv_lens"]), qo_indptr=qo_indptr, kv_indptr=leaf["kv_indptr"],
                 kv_indices=leaf["kv_indices"], kv_last_page_len=leaf["kv_last_page_len"],
                 max_num_pages=pool, q=q, k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new,
                 append_indptr=qo_indptr.copy(), extra={"levels": levels})


def flat_levels(b: Batch) -> dict:
    """One-level page table of a cascade batch whose shared nodes hold whole
    pages: request r's pages are those of its nodes, level by level."""
    levels = b.extra["levels"]
    P = b.page_size
    for lv in levels[:-1]:
        if any(k % P for k in lv["kv_lens"]):
            raise ValueError("a shared node ends inside a page")
    indptr, indices, lens = [0], [], []
    for r in range(b.batch_size):
        row = int(b.qo_indptr[r])
        total = 0
        for lv in levels:
            qo = lv["qo_indptr"]
            n = int(np.searchsorted(qo, row, side="right")) - 1
            while qo[n + 1] == qo[n]:      # skip empty nodes that share the boundary
                n += 1
            indices.extend(int(x) for x in lv["kv_indices"][lv["kv_indptr"][n]:lv["kv_indptr"][n + 1]])
            total += lv["kv_lens"][n]
        indptr.append(len(indices))
        lens.append(total)
    return {"kv_indptr": np.asarray(indptr, np.int32), "kv_indices": np.asarray(indices, np.int32),
            "kv_last_page_len": levels[-1]["kv_last_page_len"].copy(), "kv_lens": lens}
