"""Oracle part 1: paged-KV metadata, in plain Python integers.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): only tests, the smoke
check and the bench's CPU baseline use this module.

Everything here is integer bookkeeping: the CSR page table, the length
contract, logical-to-physical addresses, the bottom-right causal mask, the
slot map of an append, and the conversion between a token-location table
and a page-number table.  No numpy, so each line can be read against the
pages directly.
"""

from __future__ import annotations

NHD = "NHD"
HND = "HND"


class MetadataError(ValueError):
    """A metadata rule was broken.  ``reason`` names the rule (see REASONS)."""

    def __init__(self, reason: str, message: str):
        super().__init__(f"{reason}: {message}")
        self.reason = reason


# Names of the validation rules.  The rules marked "completion" are not
# stated on the pages; they are the plainest reading that the rest supports.
REASONS = (
    "batch_size",        # B >= 0
    "page_size",         # page_size >= 1
    "indptr_length",     # an indptr has B+1 entries
    "indptr_start",      # indptr[0] == 0       (KV-Cache layouts, "Ragged Tensor")
    "indptr_order",      # indptr non-decreasing
    "empty_page_list",   # every request owns >= 1 page (Deep Dive, length check)
    "last_page_len",     # 1 <= last_page_len <= page_size (KV-Cache layouts, page table note)
    "page_index",        # 0 <= kv_indices[i] < max_num_pages (pool bound)
    "indices_length",    # kv_indptr[B] <= len(kv_indices)
    "qo_exceeds_kv",     # completion: qo_len <= kv_len (kv_len counts the new tokens)
    "head_group",        # completion: num_qo_heads % num_kv_heads == 0, both >= 1
    "decode_qo_len",     # completion: decode mode has exactly one query row per request
    "append_collision",  # completion: two appended tokens may not share a slot
    "cascade_rows",      # completion: every cascade level covers the same query rows
    "cascade_nesting",   # completion: cascade levels nest (each node is a union of next-level nodes)
    "mask_length",       # the flattened custom mask holds sum(qo_len * kv_len) entries (KV-Cache layouts, mask layout)
)


def kv_len(page_ids, last_page_len: int, page_size: int) -> int:
    """KV length of one request from its page list and tail length.

    Deep Dive - FlashInfer, section "Why inference attention becomes
    irregular": the length is page_size * (pages - 1) + last_page_len with a
    tail of 1..page_size slots; the same rule is stated under the page-table
    layout of "FlashInfer 中的 KV-Cache 布局".  Empty page lists, negative
    page IDs and out-of-range tails are rejected, as that section's check does.
    """
    if not page_ids:
        raise MetadataError("empty_page_list", "a request needs at least one page")
    for p in page_ids:
        if type(p) is not int or p < 0:
            raise MetadataError("page_index", f"page id {p!r} is not a nonnegative int")
    if type(last_page_len) is not int or not (1 <= last_page_len <= page_size):
        raise MetadataError("last_page_len", f"tail {last_page_len!r} outside 1..{page_size}")
    return page_size * (len(page_ids) - 1) + last_page_len


def indptr_from_lengths(lengths) -> list[int]:
    """Exclusive prefix sum with a leading zero.

    "FlashInfer 中的 KV-Cache 布局", section "Ragged Tensor": an indptr has
    num_requests + 1 entries, starts at 0, and entry i+1 minus entry i is the
    length of request i.
    """
    out = [0]
    for n in lengths:
        out.append(out[-1] + n)
    return out


def kv_lens(kv_indptr, kv_indices, kv_last_page_len, page_size: int) -> list[int]:
    """Per-request KV lengths of a CSR page table (applies ``kv_len`` per row;
    numpy integers are converted to Python ints first).

    "FlashInfer 中的 KV-Cache 布局", section "页表布局" (page-table layout):
    request i's pages are kv_indices[kv_indptr[i]:kv_indptr[i+1]].
    """
    b = len(kv_indptr) - 1
    ip = [int(x) for x in kv_indptr]
    return [kv_len([int(p) for p in kv_indices[ip[i]:ip[i + 1]]], int(kv_last_page_len[i]), page_size)
            for i in range(b)]


def _check_indptr(name: str, indptr, batch: int):
    if len(indptr) != batch + 1:
        raise MetadataError("indptr_length", f"{name} has {len(indptr)} entries, expected {batch + 1}")
    if batch >= 0 and indptr[0] != 0:
        raise MetadataError("indptr_start", f"{name}[0] = {indptr[0]}, expected 0")
    for i in range(batch):
        if indptr[i + 1] < indptr[i]:
            raise MetadataError("indptr_order", f"{name} decreases at {i}")


def validate(*, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size: int,
             max_num_pages: int, num_qo_heads: int = 1, num_kv_heads: int = 1,
             decode: bool = False) -> list[int]:
    """Check a batch's metadata; return per-request kv_len or raise MetadataError.

    The rules, in the order they are checked (the first broken one is
    reported):

    1. B >= 0 and page_size >= 1.
    2. Each indptr has B+1 entries, starts at 0 and never decreases
       ("FlashInfer 中的 KV-Cache 布局", "Ragged Tensor" and "页表布局").
       ``qo_indptr`` may be None in decode mode (one row per request, as the
       decode wrapper in Deep Dive - FlashInfer, "Plan then run", takes none).
    3. kv_indptr[B] <= len(kv_indices).
    4. Per request: at least one page, every page id in [0, max_num_pages),
       tail in 1..page_size (Deep Dive - FlashInfer, the length contract
       and its rejection cases).
    5. Completions (not stated on the pages): qo_len <= kv_len, because the
       reported kv_len already includes the new tokens (Deep Dive - FlashInfer,
       "Why inference attention becomes irregular"); heads group evenly;
       decode mode has qo_len == 1.
    """
    batch = len(kv_last_page_len)
    if batch < 0:
        raise MetadataError("batch_size", "negative batch")
    if type(page_size) is not int or page_size < 1:
        raise MetadataError("page_size", f"page_size {page_size!r} < 1")
    if num_qo_heads < 1 or num_kv_heads < 1 or num_qo_heads % num_kv_heads != 0:
        raise MetadataError("head_group", f"{num_qo_heads} qo heads do not group over {num_kv_heads} kv heads")
    if qo_indptr is not None:
        _check_indptr("qo_indptr", qo_indptr, batch)
    _check_indptr("kv_indptr", kv_indptr, batch)
    if kv_indptr[batch] > len(kv_indices):
        raise MetadataError("indices_length", f"kv_indptr[B] = {kv_indptr[batch]} > {len(kv_indices)} indices")
    lens = []
    for b in range(batch):
        pages = list(kv_indices[kv_indptr[b]:kv_indptr[b + 1]])
        if not pages:
            raise MetadataError("empty_page_list", f"request {b} owns no page")
        for p in pages:
            if not (0 <= p < max_num_pages):
                raise MetadataError("page_index", f"request {b}: page {p} outside [0, {max_num_pages})")
        tail = kv_last_page_len[b]
        if not (1 <= tail <= page_size):
            raise MetadataError("last_page_len", f"request {b}: tail {tail} outside 1..{page_size}")
        lens.append(page_size * (len(pages) - 1) + tail)
    for b in range(batch):
        q = 1 if qo_indptr is None else qo_indptr[b + 1] - qo_indptr[b]
        if decode and q != 1:
            raise MetadataError("decode_qo_len", f"request {b}: decode needs qo_len 1, got {q}")
        if q > lens[b]:
            raise MetadataError("qo_exceeds_kv", f"request {b}: qo_len {q} > kv_len {lens[b]}")
    return lens


def token_address(kv_indptr, kv_indices, page_size: int, b: int, j: int) -> tuple[int, int]:
    """(physical page, slot) of logical token j of request b.

    Deep Dive - FlashInfer, "Causality uses logical positions, not page
    numbers": token j lives in the (j // page_size)-th page of the request's
    list, at slot j % page_size; the list keeps logical order, never sorted.
    """
    return kv_indices[kv_indptr[b] + j // page_size], j % page_size


def element_offset(layout: str, *, page: int, slot: int, head: int, dim: int, page_size: int,
                   num_heads: int, head_dim: int, kv: int | None = None) -> int:
    """Element offset of one K or V scalar in a paged cache.

    "FlashInfer 中的 KV-Cache 布局", section "页表布局": the single-tensor
    cache is [pages, 2, ...] with index 0 = K and 1 = V; the tuple form is a
    pair of [pages, ...] tensors.  The last three dims are
    (page_size, heads, head_dim) for NHD and (heads, page_size, head_dim) for
    HND ("布局：NHD/HND").  ``kv=None`` selects the tuple form.
    """
    if layout == NHD:
        inner = (slot * num_heads + head) * head_dim + dim
    elif layout == HND:
        inner = (head * page_size + slot) * head_dim + dim
    else:
        raise ValueError(layout)
    per_page = page_size * num_heads * head_dim
    if kv is None:
        return page * per_page + inner
    return (page * 2 + kv) * per_page + inner


def visible(i: int, j: int, q_len: int, kv_len_: int) -> bool:
    """Bottom-right causal mask: local query row i may see key j iff j <= K - Q + i.

    Deep Dive - FlashInfer, "Causality uses logical positions, not page
    numbers".  A decode row (Q = 1) therefore sees all K keys.
    """
    return 0 <= j < kv_len_ and j <= kv_len_ - q_len + i


def visible_count(i: int, q_len: int, kv_len_: int) -> int:
    """Number of keys row i sees (counted from the mask, one key at a time)."""
    return sum(1 for j in range(kv_len_) if visible(i, j, q_len, kv_len_))


def append_targets(append_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size: int):
    """(page, slot) that each appended token is written to, in token order.

    The metadata passed to an append already counts the new tokens (Deep
    Dive - FlashInfer, "Why inference attention becomes irregular"), so the
    n_b new tokens of request b are its last n_b logical positions
    K_b - n_b + t, addressed as in ``token_address``.  The pages are
    allocated by the caller beforehand ("FlashInfer 中的 KV-Cache 布局",
    section on the MLA page layout, FlashInfer API note on append).
    Raises ``MetadataError('qo_exceeds_kv')`` if a request appends more
    tokens than it holds and ``'append_collision'`` if two tokens would share
    one slot (a write race on the device).
    """
    batch = len(kv_last_page_len)
    lens = kv_lens(kv_indptr, kv_indices, kv_last_page_len, page_size)
    out = []
    seen = {}
    for b in range(batch):
        n = append_indptr[b + 1] - append_indptr[b]
        if n > lens[b]:
            raise MetadataError("qo_exceeds_kv", f"request {b}: appends {n} > kv_len {lens[b]}")
        for t in range(n):
            where = token_address(kv_indptr, kv_indices, page_size, b, lens[b] - n + t)
            if where in seen:
                raise MetadataError("append_collision", f"slot {where} written twice")
            seen[where] = (b, t)
            out.append(where)
    return out


def token_table_to_page_table(token_rows, seq_lens, page_size: int) -> dict:
    """Convert per-token slot tables to page-level CSR metadata.

    "GPU attention backends: FlashInfer and FlashAttention", sections
    "FlashAttention: a page-number table" and the first exercise's answer:
    with a token-location table, every page_size-th location starts a page
    and dividing it by page_size gives the page number; kv_indptr accumulates
    ceil(len / page_size); the tail is len - (pages - 1) * page_size.  With
    page_size 1 the token table row is itself kv_indices and every tail is 1.
    """
    kv_indptr = [0]
    kv_indices = []
    last = []
    table = []
    for row, n in zip(token_rows, seq_lens):
        starts = list(row[0:n:page_size])
        pages = [loc // page_size for loc in starts]
        table.append(pages)
        kv_indices.extend(pages)
        kv_indptr.append(kv_indptr[-1] + len(pages))
        last.append(n - (len(pages) - 1) * page_size)
    return {"kv_indptr": kv_indptr, "kv_indices": kv_indices, "kv_last_page_len": last,
            "page_table": table}
