"""Oracle part 2: paged attention in numpy float64.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

For every request and every query head: gather that request's keys and values
through explicit (page, slot) index arrays, upcast them exactly to float64,
score them against the query rows, mask with the bottom-right causal rule,
and take a stable softmax.  Each output row comes with its base-2
log-sum-exp.  No tiling, no online softmax, no fusion: one dense matmul per
(request, head).
"""

from __future__ import annotations

import math

import numpy as np

from . import metadata as md

LN2 = math.log(2.0)


def fp8_e4m3_value(code: int) -> float:
    """Value of one 8-bit E4M3 code (the OCP 8-bit floating-point format:
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    holds the subnormals m/8 * 2^-6; the one all-ones pattern per sign is NaN
    and there is no infinity, so the largest finite value is 448)."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_FP8_TABLE = np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)


def upcast(x, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values.

    ``dtype`` is "f32" (a float32 array), "bf16" (the raw 16-bit patterns of
    bfloat16 numbers in a uint16 array; a bfloat16 is the upper half of a
    float32, so shifting the pattern up by 16 bits is exact) or "fp8" (uint8
    E4M3 codes, see ``fp8_e4m3_value``; every code is exact in float64).
    """
    x = np.asarray(x)
    if dtype == "f32":
        return x.astype(np.float64)
    if dtype == "bf16":
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "fp8":
        return _FP8_TABLE[x.astype(np.uint8)]
    raise ValueError(dtype)


def attend_rows(q_rows, k, v, mask, sm_scale: float):
    """Softmax attention of n query rows over K keys with a visibility mask.

    q_rows [n, Dqk], k [K, Dqk], v [K, Dv], mask [n, K] (True = visible).
    Returns o [n, Dv] and the base-2 statistic lse [n] =
    log2(sum over visible keys of exp(sm_scale * q.k)).  A row that sees no key
    is the empty state (zero vector, -inf) of Deep Dive - FlashInfer,
    "A worked split-KV example".
    """
    n = q_rows.shape[0]
    dv = v.shape[1]
    s = sm_scale * (q_rows @ k.T)
    s = np.where(mask, s, -np.inf)
    o = np.zeros((n, dv))
    lse = np.full(n, -np.inf)
    live = mask.any(axis=1)
    if live.any():
        sl = s[live]
        m = sl.max(axis=1, keepdims=True)
        e = np.exp(sl - m)
        z = e.sum(axis=1, keepdims=True)
        o[live] = (e @ v) / z
        lse[live] = (m[:, 0] + np.log(z[:, 0])) / LN2
    return o, lse


def gather_request(cache, layout: str, kv_indptr, kv_indices, page_size: int, b: int, n_tokens: int):
    """Rows [n_tokens, H, D] of request b, gathered through the page table.

    Token j comes from (kv_indices[kv_indptr[b] + j // P], j % P): Deep Dive -
    FlashInfer, "Causality uses logical positions, not page numbers".  The
    cache is one tensor of the tuple form of "FlashInfer 中的 KV-Cache 布局"
    ("页表布局"): NHD [pages, P, H, D] or HND [pages, H, P, D].
    """
    j = np.arange(n_tokens)
    pages = np.asarray(kv_indices[kv_indptr[b]:kv_indptr[b + 1]], dtype=np.int64)
    page_of = pages[j // page_size]
    slot_of = j % page_size
    if layout == md.NHD:
        return cache[page_of, slot_of]
    if layout == md.HND:
        return cache[page_of, :, slot_of]
    raise ValueError(layout)


def paged_attention(q, k_cache, v_cache, *, qo_indptr, kv_indptr, kv_indices, kv_last_page_len,
                    page_size: int, layout: str, num_kv_heads: int, causal: bool = True,
                    sm_scale: float | None = None, q_dtype: str = "f32", kv_dtype: str = "f32",
                    requests=None, heads=None, key_range=None, custom_mask=None, k_scale: float = 1.0,
                    v_scale: float = 1.0):
    """Batched attention of ragged queries against a paged KV cache.

    q [nnz, Hq, Dqk]; k_cache/v_cache in the tuple form (see
    ``gather_request``).  Query rows of request b are
    qo_indptr[b]:qo_indptr[b+1] ("FlashInfer 中的 KV-Cache 布局", "Ragged
    Tensor"); its KV length follows the length contract (``metadata.kv_len``).
    Query head h reads kv head h // (Hq / Hkv), the repeat-interleave grouping
    of the dense reference in Deep Dive - FlashInfer, "Plan then run".
    With ``causal`` row i sees key j iff j <= K - Q + i (bottom-right
    alignment, "Causality uses logical positions, not page numbers");
    otherwise it sees every key.  sm_scale defaults to 1/sqrt(Dqk), the scale
    of the ordinary logits in "Core mechanism: schedule work around state".

    ``custom_mask``: a flattened boolean 2-D ragged mask ("FlashInfer 中的
    KV-Cache 布局", "掩码布局"): request b's q_b x K_b block, query-major,
    starts at the sum of q x K over the earlier requests; True keeps a key.
    It takes the place of the causal rule.

    ``k_scale`` / ``v_scale`` multiply every stored key / value (the
    dequantisation of a low-precision cache, one factor per tensor).

    ``requests`` / ``heads`` restrict the work to a sample (other outputs stay
    NaN).  ``key_range`` = (lo, hi) restricts every request to keys
    lo <= j < hi on top of the mask (used to form split-KV partial states).
    Returns (o [nnz, Hq, Dv], lse [nnz, Hq]) in float64, lse in base 2.
    """
    q = np.asarray(q)
    nnz, hq, dqk = q.shape
    hkv = num_kv_heads
    if hq % hkv:
        raise md.MetadataError("head_group", f"{hq} % {hkv}")
    group = hq // hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(dqk)
    dv = v_cache.shape[-1]
    lens = md.kv_lens(kv_indptr, kv_indices, kv_last_page_len, page_size)
    batch = len(lens)
    o = np.full((nnz, hq, dv), np.nan)
    lse = np.full((nnz, hq), np.nan)
    reqs = range(batch) if requests is None else requests
    head_list = range(hq) if heads is None else heads
    mask_off = [0]
    for b in range(batch):
        mask_off.append(mask_off[-1] + (qo_indptr[b + 1] - qo_indptr[b]) * lens[b])
    if custom_mask is not None and len(custom_mask) != mask_off[-1]:
        raise md.MetadataError("mask_length", f"mask has {len(custom_mask)} entries, the batch needs {mask_off[-1]}")
    for b in reqs:
        r0, r1 = qo_indptr[b], qo_indptr[b + 1]
        n_q = r1 - r0
        if n_q == 0:
            continue
        k_len = lens[b]
        kb = upcast(gather_request(k_cache, layout, kv_indptr, kv_indices, page_size, b, k_len), kv_dtype) * k_scale
        vb = upcast(gather_request(v_cache, layout, kv_indptr, kv_indices, page_size, b, k_len), kv_dtype) * v_scale
        i = np.arange(n_q)[:, None]
        j = np.arange(k_len)[None, :]
        if custom_mask is not None:
            mask = np.asarray(custom_mask[mask_off[b]:mask_off[b + 1]], dtype=bool).reshape(n_q, k_len)
        else:
            mask = (j <= k_len - n_q + i) if causal else np.ones((n_q, k_len), dtype=bool)
        if key_range is not None:
            mask = mask & (j >= key_range[0]) & (j < key_range[1])
        qb = upcast(q[r0:r1], q_dtype)
        for h in head_list:
            kvh = h // group
            o[r0:r1, h], lse[r0:r1, h] = attend_rows(qb[:, h], kb[:, kvh], vb[:, kvh], mask, sm_scale)
    return o, lse


def mla_decode(q_ckv, q_kpe, ckv_cache, kpe_cache, *, kv_indptr, kv_indices, kv_last_page_len,
               page_size: int, sm_scale: float, dtype: str = "bf16", requests=None, heads=None,
               key_range=None):
    """Multi-head latent attention decode over a paged latent cache.

    "FlashInfer 中的 KV-Cache 布局", section "多头潜在注意力页布局" (MLA page
    layout): the cache has no head dimension; each token stores a compressed
    key/value row ckv (512) and a positional key part kpe (64), usable as
    zero-copy slices of one [pages, P, 576] tensor.  Every query head scores a
    token as sm_scale * (q_ckv . ckv + q_kpe . kpe) and the output is the
    softmax-weighted sum of the ckv rows (512 wide).  One query row per
    request sees all of its keys.

    q_ckv [B, H, 512], q_kpe [B, H, 64]; ckv_cache [pages, P, 512] and
    kpe_cache [pages, P, 64] (views of one array are fine).  Returns float64
    o [B, H, 512] and base-2 lse [B, H].
    """
    q_ckv = np.asarray(q_ckv)
    q_kpe = np.asarray(q_kpe)
    batch, h_all, d_ckv = q_ckv.shape
    lens = md.kv_lens(kv_indptr, kv_indices, kv_last_page_len, page_size)
    o = np.full((batch, h_all, d_ckv), np.nan)
    lse = np.full((batch, h_all), np.nan)
    reqs = range(batch) if requests is None else requests
    head_list = list(range(h_all)) if heads is None else list(heads)
    for b in reqs:
        k_len = lens[b]
        j = np.arange(k_len)
        pages = np.asarray(kv_indices[kv_indptr[b]:kv_indptr[b + 1]], dtype=np.int64)
        page_of, slot_of = pages[j // page_size], j % page_size
        ckv = upcast(ckv_cache[page_of, slot_of], dtype)
        kpe = upcast(kpe_cache[page_of, slot_of], dtype)
        keys = np.concatenate([ckv, kpe], axis=1)
        mask = np.ones((len(head_list), k_len), dtype=bool)
        if key_range is not None:
            mask &= (j >= key_range[0])[None, :] & (j < key_range[1])[None, :]
        qrows = np.concatenate([upcast(q_ckv[b, head_list], dtype), upcast(q_kpe[b, head_list], dtype)], axis=1)
        ob, lb = attend_rows(qrows, keys, ckv, mask, sm_scale)
        o[b, head_list] = ob
        lse[b, head_list] = lb
    return o, lse
