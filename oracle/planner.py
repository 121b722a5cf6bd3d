"""Oracle part 3: the work-partition specification of plan().

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

The pages say what a plan holds -- offsets, the request-to-tile assignment,
temporary-buffer sizes and whether to split KV work (Deep Dive - FlashInfer,
"Plan then run: inspector-executor for GPU kernels") -- and what a split
policy trades off: small chunks cost merge work and metadata traffic, large
chunks cost tail latency ("Load balancing and split-KV decisions").  They
give no algorithm.  This module is our reading, written out as plain
integer steps; the native planner implements the same steps independently
and the two must agree bit for bit.  Splits are disjoint, page-aligned and
cover every visible key exactly once, which the partition invariants in the
tests check by enumeration.

Modes: "decode" (one query row per request), "prefill" (ragged rows,
optionally causal) and "mla" (one row per request, heads split into groups).

Work item fields (eight int32 each, in this order):
  q_row0    first global query row of the tile (qo_indptr[b] + first local row)
  num_rows  rows in the tile
  kv_start  first key of the chunk
  kv_end    one past the last key the tile may see inside the chunk
  diag      row r of the tile sees key j iff j <= diag + r (causal limit)
  page_base kv_indptr[b]
  out_slot  -1: write o/lse directly; else first partial row of this chunk
  batch     request index b
Merge item fields (four int32): q_row0, num_rows, slot0, num_chunks; the
partial rows of chunk c are slot0 + c * num_rows + r.
"""

from __future__ import annotations

DECODE, PREFILL, MLA = "decode", "prefill", "mla"

MIN_SPLIT_TOKENS = 256          # a chunk holds at least this many tokens
MAX_CHUNK_PAGES = 1024          # and at most this many pages (a kernel stages a chunk's page ids on chip)
DEFAULT_TARGET_PER_CU = {DECODE: 3, PREFILL: 4, MLA: 1}
DEFAULT_TAIL_SPLIT = {DECODE: 2, PREFILL: 1, MLA: 1}
TAIL_SPLIT_MAX_PER_CU = 5       # the default tail split applies up to this many (item, head) units per CU
CASCADE_TARGET_PER_CU = 1       # cascade levels run one launch each: one item per CU by default
MFMA_TILE_ROWS = 256            # prefill tile height counted in (row, head) pairs
MFMA_HEAD_DIM = 128             # the head dim whose prefill runs 256-pair tiles


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


RAGGED_PAGE = 16                # ragged keys are chunked as if in pages of this many tokens


def rows_per_tile(mode: str, group: int, kv_dtype: str, masked: bool = False, head_dim: int = 128) -> int:
    """Query rows per work item: for prefill over a bfloat16 or fp8 cache at
    head_dim 128 as many rows as fit a 256-high tile of (row, head) pairs;
    1 otherwise (decode, MLA, float32 prefill, other head dims, and
    custom-masked prefill with one query head per kv head)."""
    if mode != PREFILL or kv_dtype not in ("bf16", "fp8"):
        return 1
    if head_dim != MFMA_HEAD_DIM:
        return 1
    if masked and group < 2:
        return 1
    return max(1, MFMA_TILE_ROWS // group)


def plan(*, mode: str, qo_indptr, kv_indptr, kv_last_page_len, page_size: int, heads_y: int,
         rows: int, causal: bool, num_cus: int, fixed_split_pages: int = 0,
         target_per_cu: int = 0, tail_split: int = 0, all_partial: bool = False) -> dict:
    """Partition a batch into work items and merge items.

    Steps (all integer):
    1. tiles_b = ceil(q_b / rows) query tiles per request (none if q_b = 0).
       ``heads_y`` is the number of head slices each item is replicated over
       (kv heads, or MLA head groups).
    2. Page work W = sum_b tiles_b * n_b * heads_y; target T = target_per_cu *
       num_cus items.
    3. Chunk size C (pages) = fixed_split_pages if given, else
       max(ceil(256 / P), ceil(W / T)); either way at most 1024.  MLA (whose
       kernel holds one workgroup per CU) then grows C to the smallest size
       whose item count times heads_y is at most T (or 1024), so that the
       per-request rounding does not spill a second, nearly empty round.
    4. Chunk c of request b covers keys [c*C*P, min((c+1)*C*P, K_b)).
    5. For tile t (local rows l0 .. l0+rows-1) the causal limit is
       diag = K_b - q_b + l0 (non-causal: diag = K_b); a chunk whose first key
       exceeds diag + rows - 1 is dropped, and kv_end is clipped to
       diag + rows.
    5b. Tail split S: if S > 1, the tile's last kept chunk, when it spans
       more than one page, is replaced by pieces of ceil(pages / S) pages
       from its first key on (the last piece ends where the chunk ended).
       The longest-first order of step 7 then finishes on small items.  An
       explicit tail_split is used as given.  The default is 1 (off) except
       for decode, where it is 2 when the kept chunks of step 5 times heads_y
       number at most TAIL_SPLIT_MAX_PER_CU * num_cus; past that the batch
       already ends on small items, and the extra items and merges only cost.
    6. A tile with one kept chunk writes directly (unless ``all_partial``,
       used by cascades, where every tile's rows must be merged later);
       otherwise its chunks get consecutive partial rows and one merge item.
       Partial rows are handed out tile by tile in (b, t) order.
    7. Items are emitted by descending key count kv_end - kv_start (a tile's
       kernel time follows its keys, not its rows), ties broken by ascending
       (b, t, c).
    """
    batch = len(kv_last_page_len)
    if qo_indptr is None:
        qo_indptr = list(range(batch + 1))
    if mode != PREFILL:
        causal = True        # a single decode row sees every key; diag = K - 1
    if target_per_cu <= 0:
        target_per_cu = DEFAULT_TARGET_PER_CU[mode]
    n_pages = [kv_indptr[b + 1] - kv_indptr[b] for b in range(batch)]
    k_lens = [page_size * (n_pages[b] - 1) + kv_last_page_len[b] for b in range(batch)]
    q_lens = [qo_indptr[b + 1] - qo_indptr[b] for b in range(batch)]
    tiles = [_cdiv(q, rows) for q in q_lens]

    work = sum(tiles[b] * n_pages[b] * heads_y for b in range(batch))
    target = target_per_cu * num_cus
    if fixed_split_pages > 0:
        chunk = fixed_split_pages
    else:
        chunk = max(_cdiv(MIN_SPLIT_TOKENS, page_size), _cdiv(work, target))
    chunk = min(chunk, MAX_CHUNK_PAGES)
    if mode == MLA and fixed_split_pages <= 0:
        def units(c):
            return sum(tiles[b] * _cdiv(n_pages[b], c) for b in range(batch)) * heads_y
        lo, hi = chunk, MAX_CHUNK_PAGES
        if units(hi) <= target:
            while lo < hi:                      # smallest c in [lo, hi] with units(c) <= target
                mid = (lo + hi) // 2
                if units(mid) <= target:
                    hi = mid
                else:
                    lo = mid + 1
            chunk = lo
        else:
            chunk = MAX_CHUNK_PAGES
    chunk_tokens = chunk * page_size

    def kept_chunks(b, t):
        """Steps 4-5: the (kv_start, kv_end) chunks that tile t of request b sees."""
        diag = (k_lens[b] - q_lens[b] + t * rows) if causal else k_lens[b]
        limit = min(k_lens[b], diag + min(rows, q_lens[b] - t * rows))   # keys < limit are seen by some row
        kept = []
        for c in range(_cdiv(n_pages[b], chunk)):
            lo = c * chunk_tokens
            if lo >= limit:
                continue
            kept.append((lo, min(lo + chunk_tokens, k_lens[b], limit)))
        return kept

    if tail_split <= 0:
        tail_split = DEFAULT_TAIL_SPLIT[mode]
        units = heads_y * sum(len(kept_chunks(b, t)) for b in range(batch) for t in range(tiles[b]))
        if units > TAIL_SPLIT_MAX_PER_CU * num_cus:
            tail_split = 1

    raw = []          # (key count, b, t, c_kept, fields) before slot assignment
    merges = []
    slot = 0
    split_any = False
    for b in range(batch):
        k_len = k_lens[b]
        for t in range(tiles[b]):
            l0 = t * rows
            n_rows = min(rows, q_lens[b] - l0)
            diag = (k_len - q_lens[b] + l0) if causal else k_len
            kept = kept_chunks(b, t)
            if tail_split > 1 and kept:
                lo, hi = kept[-1]
                pages = _cdiv(hi - lo, page_size)
                if pages > 1:
                    step = _cdiv(pages, tail_split) * page_size
                    kept[-1:] = [(s, min(hi, s + step)) for s in range(lo, hi, step)]
            q_row0 = qo_indptr[b] + l0
            if len(kept) == 1 and not all_partial:
                lo, hi = kept[0]
                raw.append((hi - lo, b, t, 0,
                            [q_row0, n_rows, lo, hi, diag, kv_indptr[b], -1, b]))
                continue
            split_any = True
            merges.append([q_row0, n_rows, slot, len(kept)])
            for ci, (lo, hi) in enumerate(kept):
                raw.append((hi - lo, b, t, ci,
                            [q_row0, n_rows, lo, hi, diag, kv_indptr[b], slot + ci * n_rows, b]))
            slot += len(kept) * n_rows
    raw.sort(key=lambda e: (-e[0], e[1], e[2], e[3]))
    return {
        "items": [e[4] for e in raw],
        "merges": merges,
        "num_partial_rows": slot,
        "chunk_pages": chunk,
        "split": split_any,
        "rows_per_tile": rows,
        "target": target,
    }


def plan_cascade(*, levels, page_size: int, group: int, kv_dtype: str, heads_y: int, causal: bool,
                 num_cus: int, fixed_split_pages: int = 0, target_per_cu: int = 0,
                 tail_split: int = 0, head_dim: int = 128) -> dict:
    """Work list of a multi-level cascade ("FlashInfer 中的 KV-Cache 布局",
    multi-level cascade layout: each level has its own qo_indptr and page
    table over the shared queries and cache).

    ``levels``: list of dicts with qo_indptr, kv_indptr, kv_last_page_len.
    Steps (our reading; the pages give the layout, not a schedule):
    1. Level l is planned as "decode" when every node has exactly one query
       row, else as "prefill"; rows per tile follow ``rows_per_tile``; only
       the last level is causal.
    2. Each level is planned by ``plan`` with ``all_partial``: every tile's
       states go to partial rows, numbered on from the previous level's.
       Unless ``target_per_cu`` is given, every level targets one item per
       CU (a level is one launch of its own; larger chunks also mean fewer
       partial states to merge).
    3. A level's page_base is offset by the page ids of all earlier levels
       (kv_indptr[-1] of each): the device array holds the levels' page
       lists back to back, level 0 first.
    4. Merge list, one entry per query row in row order: the partial rows of
       that row's states, level by level, chunk by chunk (row_ptr has
       rows + 1 entries, slots lists the partial rows).
    Items of a level keep ``plan``'s order; levels run in level order.
    """
    out_levels = []
    items = []
    slot_base = 0
    page_base = 0
    total_rows = int(levels[0]["qo_indptr"][-1])
    per_row = [[] for _ in range(total_rows)]
    for li, lv in enumerate(levels):
        qo = [int(x) for x in lv["qo_indptr"]]
        nodes = len(qo) - 1
        mode = DECODE if nodes > 0 and all(qo[n + 1] - qo[n] == 1 for n in range(nodes)) else PREFILL
        rows = rows_per_tile(mode, group, kv_dtype, head_dim=head_dim)
        p = plan(mode=mode, qo_indptr=None if mode == DECODE else qo, kv_indptr=[int(x) for x in lv["kv_indptr"]],
                 kv_last_page_len=[int(x) for x in lv["kv_last_page_len"]], page_size=page_size, heads_y=heads_y,
                 rows=rows, causal=causal and li == len(levels) - 1, num_cus=num_cus,
                 fixed_split_pages=fixed_split_pages,
                 target_per_cu=target_per_cu if target_per_cu > 0 else CASCADE_TARGET_PER_CU, tail_split=tail_split,
                 all_partial=True)
        for it in p["items"]:
            it = list(it)
            it[5] += page_base
            it[6] += slot_base
            items.append(it)
        for q_row0, n_rows, slot0, n_chunks in p["merges"]:
            for r in range(n_rows):
                per_row[q_row0 + r].extend(slot_base + slot0 + c * n_rows + r for c in range(n_chunks))
        out_levels.append({"mode": mode, "rows_per_tile": rows, "num_items": len(p["items"]),
                           "chunk_pages": p["chunk_pages"], "num_partial_rows": p["num_partial_rows"]})
        slot_base += p["num_partial_rows"]
        page_base += int(lv["kv_indptr"][-1])
    row_ptr = [0]
    slots = []
    for lst in per_row:
        slots.extend(lst)
        row_ptr.append(len(slots))
    return {"levels": out_levels, "items": items, "row_ptr": row_ptr, "slots": slots,
            "num_partial_rows": slot_base, "total_rows": total_rows}


def plan_ragged(*, qo_indptr, kv_indptr, heads_y: int, rows: int, causal: bool, num_cus: int,
                fixed_split_pages: int = 0, target_per_cu: int = 0, tail_split: int = 0) -> dict:
    """Work list over ragged keys ("FlashInfer 中的 KV-Cache 布局", "Ragged
    Tensor": request b's keys are data[kv_indptr[b]:kv_indptr[b+1]]).

    The keys are chunked as if they sat in pages of RAGGED_PAGE tokens (a
    request of K keys has ceil(K / RAGGED_PAGE) such pages, the last holding
    the rest), planned by ``plan`` in prefill mode, and every item's
    page_base is then the request index b: the device reads request b's first
    key position from entry b of kv_indptr and addresses keys as one
    contiguous run from there.  A request with no keys has no rows (qo_len <=
    kv_len), hence no tiles.
    """
    batch = len(kv_indptr) - 1
    lens = [kv_indptr[b + 1] - kv_indptr[b] for b in range(batch)]
    pages = [_cdiv(k, RAGGED_PAGE) for k in lens]
    v_indptr = [0]
    for n in pages:
        v_indptr.append(v_indptr[-1] + n)
    last = [k - RAGGED_PAGE * (n - 1) if n else 0 for k, n in zip(lens, pages)]
    p = plan(mode=PREFILL, qo_indptr=qo_indptr, kv_indptr=v_indptr, kv_last_page_len=last,
             page_size=RAGGED_PAGE, heads_y=heads_y, rows=rows, causal=causal, num_cus=num_cus,
             fixed_split_pages=fixed_split_pages, target_per_cu=target_per_cu, tail_split=tail_split)
    for it in p["items"]:
        it[5] = it[7]
    return p
