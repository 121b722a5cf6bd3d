"""Pins for oracle.mask and the custom-mask path of oracle.attention.

* The bit packing against numpy's packbits with little-endian bit order (the
  routine the layout page names) and a hand-worked example.
* Mask offsets: cumsum of qo_len * kv_len, worked by hand.
* Ragged attention against paged attention over page size 1 with identity
  page ids (the ragged tensor is that page table), and against torch's
  float64 scaled-dot-product attention with the same boolean mask.
* A custom mask equal to the causal rule (or all True) gives the causal (or
  the non-causal) result; a row whose mask is all False is the empty state.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as at
from oracle import mask as mk
from oracle import metadata as md

LN2 = math.log(2.0)


def test_packbits_hand_example_and_numpy():
    bits = [1, 0, 0, 0, 0, 0, 0, 0, 0, 1, 1]
    assert mk.packbits_little(bits) == bytes([0x01, 0x06])
    rng = np.random.default_rng(1)
    for n in (0, 1, 7, 8, 9, 63, 64, 1000):
        b = rng.integers(0, 2, size=n).astype(bool)
        assert mk.packbits_little(b) == np.packbits(b, bitorder="little").tobytes()
        assert mk.unpackbits_little(mk.packbits_little(b), n) == [int(x) for x in b]


def test_mask_indptr_hand_example():
    # qo 3/1/4, kv 6/2/9 (the pages' three-request batch): 18, 2, 36
    assert mk.mask_indptr([3, 1, 4], [6, 2, 9]) == [0, 18, 20, 56]


def _ragged_case(rng, qo_lens, kv_lens, hq=4, hkv=2, d=16):
    qo = md.indptr_from_lengths(qo_lens)
    kv = md.indptr_from_lengths(kv_lens)
    q = rng.standard_normal((qo[-1], hq, d))
    k = rng.standard_normal((kv[-1], hkv, d))
    v = rng.standard_normal((kv[-1], hkv, d))
    return qo, kv, q, k, v


def _random_mask(rng, qo_lens, kv_lens, p=0.6, keep_rows=True):
    segs = []
    for q, k in zip(qo_lens, kv_lens):
        m = rng.random((q, k)) < p
        if keep_rows and k:
            m[np.arange(q), rng.integers(0, k, size=q)] = True
        segs.append(m.reshape(-1))
    return np.concatenate(segs) if segs else np.zeros(0, bool)


@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_equals_paged_with_page_size_one(masked, causal):
    rng = np.random.default_rng(2)
    qo_lens, kv_lens = [3, 0, 5, 2], [7, 4, 5, 9]
    qo, kv, q, k, v = _ragged_case(rng, qo_lens, kv_lens)
    mask = _random_mask(rng, qo_lens, kv_lens) if masked else None
    o, lse = mk.ragged_attention(q, k, v, qo_indptr=qo, kv_indptr=kv, num_kv_heads=2, causal=causal,
                                 custom_mask=mask)
    # page size 1, page ids = token ids: [pages, 1, H, D]
    po, pl_ = at.paged_attention(q, k[:, None], v[:, None], qo_indptr=qo, kv_indptr=kv,
                                 kv_indices=list(range(kv[-1])), kv_last_page_len=[1] * len(kv_lens), page_size=1,
                                 layout="NHD", num_kv_heads=2, causal=causal, custom_mask=mask)
    assert np.array_equal(np.isnan(o), np.isnan(po))
    live = ~np.isnan(o)
    assert np.max(np.abs(o[live] - po[live])) < 1e-12
    assert np.max(np.abs(lse[~np.isnan(lse)] - pl_[~np.isnan(pl_)])) < 1e-12


def test_custom_mask_against_torch_sdpa():
    rng = np.random.default_rng(3)
    qo_lens, kv_lens = [4, 6, 1], [9, 6, 13]
    qo, kv, q, k, v = _ragged_case(rng, qo_lens, kv_lens, hq=6, hkv=3, d=8)
    mask = _random_mask(rng, qo_lens, kv_lens, p=0.4)
    o, lse = mk.ragged_attention(q, k, v, qo_indptr=qo, kv_indptr=kv, num_kv_heads=3, custom_mask=mask,
                                 sm_scale=0.3)
    off = mk.mask_indptr(qo_lens, kv_lens)
    for b in range(3):
        r0, r1 = qo[b], qo[b + 1]
        m = torch.from_numpy(mask[off[b]:off[b + 1]].reshape(qo_lens[b], kv_lens[b]))
        qt = torch.from_numpy(q[r0:r1]).transpose(0, 1)
        kt = torch.from_numpy(np.repeat(k[kv[b]:kv[b + 1]], 2, axis=1)).transpose(0, 1).contiguous()
        vt = torch.from_numpy(np.repeat(v[kv[b]:kv[b + 1]], 2, axis=1)).transpose(0, 1).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=0.3)
        s = (0.3 * (qt @ kt.transpose(1, 2))).masked_fill(~m, -math.inf)
        assert np.max(np.abs(o[r0:r1] - ref.transpose(0, 1).numpy())) < 1e-12
        assert np.max(np.abs(lse[r0:r1] - (torch.logsumexp(s, -1) / LN2).transpose(0, 1).numpy())) < 1e-12


def test_causal_and_full_masks_reduce_to_the_flags():
    rng = np.random.default_rng(4)
    qo_lens, kv_lens = [3, 5, 2], [3, 8, 6]
    qo, kv, q, k, v = _ragged_case(rng, qo_lens, kv_lens)
    causal_mask = np.concatenate([(np.arange(kl)[None, :] <= kl - ql + np.arange(ql)[:, None]).reshape(-1)
                                  for ql, kl in zip(qo_lens, kv_lens)])
    full = np.ones(sum(a * b for a, b in zip(qo_lens, kv_lens)), bool)
    kw = dict(qo_indptr=qo, kv_indptr=kv, num_kv_heads=2)
    for m, causal in ((causal_mask, True), (full, False)):
        o1, l1 = mk.ragged_attention(q, k, v, custom_mask=m, **kw)
        o2, l2 = mk.ragged_attention(q, k, v, causal=causal, **kw)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_fully_masked_row_is_the_empty_state():
    rng = np.random.default_rng(5)
    qo, kv, q, k, v = _ragged_case(rng, [2], [5])
    m = np.ones(10, bool)
    m[5:] = False                      # row 1 sees nothing
    o, lse = mk.ragged_attention(q, k, v, qo_indptr=qo, kv_indptr=kv, num_kv_heads=2, custom_mask=m)
    assert np.all(o[1] == 0.0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(lse[0]))


def test_mask_length_is_checked():
    rng = np.random.default_rng(6)
    qo, kv, q, k, v = _ragged_case(rng, [2, 1], [3, 4])
    with pytest.raises(md.MetadataError) as e:
        mk.ragged_attention(q, k, v, qo_indptr=qo, kv_indptr=kv, num_kv_heads=2, custom_mask=np.ones(9, bool))
    assert e.value.reason == "mask_length"


def _ragged_reason(**kw):
    with pytest.raises(md.MetadataError) as e:
        mk.validate_ragged(**kw)
    return e.value.reason


def test_validate_ragged_rules_by_hand():
    """Each rule of the ragged metadata ("FlashInfer 中的 KV-Cache 布局", "Ragged
    Tensor": num_requests + 1 entries, the first one zero, request i's length
    indptr[i+1] - indptr[i]) and the qo_len <= kv_len completion, with the
    expected reason written out by hand, and the rule order checked where two
    rules are broken at once."""
    # The pages' three-request batch as ragged tensors: qo 3/1/4, kv 6/2/9.
    assert mk.validate_ragged(qo_indptr=[0, 3, 4, 8], kv_indptr=[0, 6, 8, 17]) == [6, 2, 9]
    # A request with no keys and no rows is allowed; qo_len == kv_len is allowed.
    assert mk.validate_ragged(qo_indptr=[0, 2, 2, 7], kv_indptr=[0, 3, 3, 8], num_qo_heads=4,
                              num_kv_heads=2) == [3, 0, 5]
    assert mk.validate_ragged(qo_indptr=[0], kv_indptr=[0]) == []
    # Heads must group evenly (checked first, even when the indptrs are also bad).
    assert _ragged_reason(qo_indptr=[0, 1], kv_indptr=[0, 1], num_qo_heads=3, num_kv_heads=2) == "head_group"
    assert _ragged_reason(qo_indptr=[0, 1], kv_indptr=[0, 1], num_qo_heads=4, num_kv_heads=0) == "head_group"
    assert _ragged_reason(qo_indptr=[0, 1], kv_indptr=[0, 1], num_qo_heads=0, num_kv_heads=1) == "head_group"
    assert _ragged_reason(qo_indptr=[1, 2], kv_indptr=[0, 1], num_qo_heads=6, num_kv_heads=4) == "head_group"
    # Both indptrs cover the same requests; an empty kv_indptr is no batch at all.
    assert _ragged_reason(qo_indptr=[0, 1], kv_indptr=[0, 1, 2]) == "batch_size"
    assert _ragged_reason(qo_indptr=[], kv_indptr=[]) == "batch_size"
    # The first entry is zero, qo_indptr before kv_indptr.
    assert _ragged_reason(qo_indptr=[1, 2, 3], kv_indptr=[0, 2, 4]) == "indptr_start"
    assert _ragged_reason(qo_indptr=[0, 1, 2], kv_indptr=[2, 4, 6]) == "indptr_start"
    with pytest.raises(md.MetadataError, match="qo_indptr"):
        mk.validate_ragged(qo_indptr=[1, 2], kv_indptr=[1, 2])
    # Lengths are differences of consecutive entries, so an indptr never decreases.
    assert _ragged_reason(qo_indptr=[0, 2, 1], kv_indptr=[0, 2, 4]) == "indptr_order"
    assert _ragged_reason(qo_indptr=[0, 1, 1], kv_indptr=[0, 3, 2]) == "indptr_order"
    # Order before lengths: request 0 has qo 3 > kv 2, but kv_indptr decreases later.
    assert _ragged_reason(qo_indptr=[0, 3, 4], kv_indptr=[0, 2, 1]) == "indptr_order"
    # Completion: a request's keys include its new tokens, so qo_len <= kv_len.
    assert _ragged_reason(qo_indptr=[0, 3], kv_indptr=[0, 2]) == "qo_exceeds_kv"
    assert _ragged_reason(qo_indptr=[0, 1, 2], kv_indptr=[0, 5, 5]) == "qo_exceeds_kv"
    with pytest.raises(md.MetadataError, match="request 2"):
        mk.validate_ragged(qo_indptr=[0, 1, 2, 6], kv_indptr=[0, 1, 9, 12])
