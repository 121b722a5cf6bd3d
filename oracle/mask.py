"""Oracle part 5: ragged KV and the 2-D ragged custom mask.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

"FlashInfer 中的 KV-Cache 布局":
* "Ragged Tensor": the keys (values) of all requests are packed without
  padding into one data tensor; request i owns data[indptr[i]:indptr[i+1]],
  indptr has num_requests + 1 entries and starts at 0.
* "掩码布局（2D Ragged Tensor）": request i's mask is a qo_len[i] x
  kv_len[i] boolean matrix, flattened query-major (query index first, key
  index last); the flattened masks of all requests are concatenated into one
  1-D array whose request offsets are mask_indptr[0] = 0,
  mask_indptr[i+1] = mask_indptr[i] + qo_len[i] * kv_len[i].  The flattened
  array may be packed 8 elements per byte in little-endian bit order
  (element e is bit e % 8 of byte e // 8).

Readings: a True entry keeps the key, a False entry removes it from the
softmax (its score becomes -inf before the softmax), and a custom mask takes
the place of the causal rule.  A row whose mask removes every key is the
empty state (zero vector, -inf).
"""

from __future__ import annotations

import math

import numpy as np

from . import attention as att
from . import metadata as md


def mask_indptr(qo_lens, kv_lens) -> list[int]:
    """Start offset of every request's flattened mask (plus the total)."""
    out = [0]
    for q, k in zip(qo_lens, kv_lens):
        out.append(out[-1] + q * k)
    return out


def packbits_little(bits) -> bytes:
    """Pack 0/1 values, 8 per byte, element e at bit e % 8 of byte e // 8."""
    bits = [1 if b else 0 for b in bits]
    out = bytearray((len(bits) + 7) // 8)
    for e, b in enumerate(bits):
        if b:
            out[e // 8] |= 1 << (e % 8)
    return bytes(out)


def unpackbits_little(packed, n: int) -> list[int]:
    """Inverse of ``packbits_little`` for the first n elements."""
    return [(packed[e // 8] >> (e % 8)) & 1 for e in range(n)]


def request_mask(mask_flat, indptr, b: int, q_len: int, kv_len: int) -> np.ndarray:
    """Request b's [q_len, kv_len] boolean mask from the flattened array."""
    seg = np.asarray(mask_flat[indptr[b]:indptr[b + 1]], dtype=bool)
    if seg.size != q_len * kv_len:
        raise md.MetadataError("mask_length", f"request {b}: mask segment of {seg.size} != {q_len} x {kv_len}")
    return seg.reshape(q_len, kv_len)


def check_mask_length(mask_flat, qo_lens, kv_lens):
    total = mask_indptr(qo_lens, kv_lens)[-1]
    if len(mask_flat) != total:
        raise md.MetadataError("mask_length", f"mask has {len(mask_flat)} entries, the batch needs {total}")


def validate_ragged(*, qo_indptr, kv_indptr, num_qo_heads: int = 1, num_kv_heads: int = 1) -> list[int]:
    """Check ragged metadata; return per-request kv_len.  Rules in order:
    heads group evenly; each indptr starts at 0 and never decreases ("Ragged
    Tensor"); qo_indptr and kv_indptr cover the same requests; qo_len <=
    kv_len (completion, as for the paged cache: kv_len counts the new
    tokens).  A request may hold no keys (then no rows)."""
    if num_qo_heads < 1 or num_kv_heads < 1 or num_qo_heads % num_kv_heads:
        raise md.MetadataError("head_group", f"{num_qo_heads} qo heads do not group over {num_kv_heads} kv heads")
    batch = len(kv_indptr) - 1
    if batch < 0 or len(qo_indptr) != batch + 1:
        raise md.MetadataError("batch_size", "qo_indptr and kv_indptr differ in length")
    md._check_indptr("qo_indptr", qo_indptr, batch)
    md._check_indptr("kv_indptr", kv_indptr, batch)
    lens = [kv_indptr[b + 1] - kv_indptr[b] for b in range(batch)]
    for b in range(batch):
        q = qo_indptr[b + 1] - qo_indptr[b]
        if q > lens[b]:
            raise md.MetadataError("qo_exceeds_kv", f"request {b}: qo_len {q} > kv_len {lens[b]}")
    return lens


def ragged_attention(q, k_data, v_data, *, qo_indptr, kv_indptr, num_kv_heads: int, causal: bool = True,
                     custom_mask=None, sm_scale: float | None = None, q_dtype: str = "f32",
                     kv_dtype: str = "f32"):
    """Batched attention of ragged queries against ragged keys and values.

    q [nnz_q, Hq, D]; k_data / v_data [nnz_kv, Hkv, D] (NHD, the layout the
    ragged section gives).  Request b's keys are k_data[kv_indptr[b]:
    kv_indptr[b+1]].  Visibility: the custom mask when one is given (a
    flattened bool array as described above), else the bottom-right causal
    rule when ``causal``, else every key.  GQA and the base-2 LSE as in
    ``attention.paged_attention``.
    """
    q = np.asarray(q)
    nnz, hq, dqk = q.shape
    group = hq // num_kv_heads
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(dqk)
    batch = len(qo_indptr) - 1
    qo_lens = [qo_indptr[b + 1] - qo_indptr[b] for b in range(batch)]
    kv_lens = [kv_indptr[b + 1] - kv_indptr[b] for b in range(batch)]
    if custom_mask is not None:
        check_mask_length(custom_mask, qo_lens, kv_lens)
        m_indptr = mask_indptr(qo_lens, kv_lens)
    dv = v_data.shape[-1]
    o = np.full((nnz, hq, dv), np.nan)
    lse = np.full((nnz, hq), np.nan)
    for b in range(batch):
        r0, r1 = qo_indptr[b], qo_indptr[b + 1]
        n_q, k_len = r1 - r0, kv_lens[b]
        if n_q == 0:
            continue
        kb = att.upcast(k_data[kv_indptr[b]:kv_indptr[b + 1]], kv_dtype)
        vb = att.upcast(v_data[kv_indptr[b]:kv_indptr[b + 1]], kv_dtype)
        if custom_mask is not None:
            mask = request_mask(custom_mask, m_indptr, b, n_q, k_len)
        else:
            i = np.arange(n_q)[:, None]
            j = np.arange(k_len)[None, :]
            mask = (j <= k_len - n_q + i) if causal else np.ones((n_q, k_len), dtype=bool)
        qb = att.upcast(q[r0:r1], q_dtype)
        for h in range(hq):
            o[r0:r1, h], lse[r0:r1, h] = att.attend_rows(qb[:, h], kb[:, h // group], vb[:, h // group], mask,
                                                         sm_scale)
    return o, lse
