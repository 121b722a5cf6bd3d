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
MFMA_TILE_ROWS = 256            # prefill tile height counted in (row, head) pairs


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def rows_per_tile(mode: str, group: int, kv_dtype: str) -> int:
    """Query rows per work item: 1 for decode, MLA and float32 prefill; for
    bfloat16 prefill as many rows as fit a 256-high tile of (row, head) pairs."""
    if mode != PREFILL or kv_dtype == "f32":
        return 1
    return max(1, MFMA_TILE_ROWS // group)


def plan(*, mode: str, qo_indptr, kv_indptr, kv_last_page_len, page_size: int, heads_y: int,
         rows: int, causal: bool, num_cus: int, fixed_split_pages: int = 0,
         target_per_cu: int = 0, tail_split: int = 0) -> dict:
    """Partition a batch into work items and merge items.

    Steps (all integer):
    1. tiles_b = ceil(q_b / rows) query tiles per request (none if q_b = 0).
       ``heads_y`` is the number of head slices each item is replicated over
       (kv heads, or MLA head groups).
    2. Page work W = sum_b tiles_b * n_b * heads_y; target T = target_per_cu *
       num_cus items.
    3. Chunk size C (pages) = fixed_split_pages if given, else
       max(ceil(256 / P), ceil(W / T)); either way at most 1024.
    4. Chunk c of request b covers keys [c*C*P, min((c+1)*C*P, K_b)).
    5. For tile t (local rows l0 .. l0+rows-1) the causal limit is
       diag = K_b - q_b + l0 (non-causal: diag = K_b); a chunk whose first key
       exceeds diag + rows - 1 is dropped, and kv_end is clipped to
       diag + rows.
    5b. Tail split S (default 2 for decode, else 1 = off): if S > 1, the
       tile's last kept chunk, when it spans more than one page, is replaced
       by pieces of ceil(pages / S) pages from its first key on (the last
       piece ends where the chunk ended).  The longest-first order of step 7
       then finishes on small items.
    6. A tile with one kept chunk writes directly; otherwise its chunks get
       consecutive partial rows and one merge item.  Partial rows are handed
       out tile by tile in (b, t) order.
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
    if tail_split <= 0:
        tail_split = DEFAULT_TAIL_SPLIT[mode]
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
    chunk_tokens = chunk * page_size

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
            limit = min(k_len, diag + n_rows)          # keys < limit are seen by some row
            kept = []
            for c in range(_cdiv(n_pages[b], chunk)):
                lo = c * chunk_tokens
                hi = min(lo + chunk_tokens, k_len)
                if lo >= limit:
                    continue
                kept.append((lo, min(hi, limit)))
            if tail_split > 1 and kept:
                lo, hi = kept[-1]
                pages = _cdiv(hi - lo, page_size)
                if pages > 1:
                    step = _cdiv(pages, tail_split) * page_size
                    kept[-1:] = [(s, min(hi, s + step)) for s in range(lo, hi, step)]
            q_row0 = qo_indptr[b] + l0
            if len(kept) == 1:
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
