"""Pins for oracle.attention: brute force, closed forms, an independent library
routine (torch SDPA in float64) on the cases that reduce to textbook attention,
and the invariances the pages state."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as at
from oracle import brute
from oracle import merge as mg
from oracle import metadata as md
from tests.conftest import load_golden


def _random_paged(rng, qo_lens, kv_lens, page_size, hq, hkv, d, layout="NHD", spare=3, dv=None):
    dv = d if dv is None else dv
    n_pages = [math.ceil(k / page_size) for k in kv_lens]
    pool = sum(n_pages) + spare
    perm = [int(x) for x in rng.permutation(pool)]
    kv_indptr = md.indptr_from_lengths(n_pages)
    kv_indices = perm[:sum(n_pages)]
    last = [k - (n - 1) * page_size for k, n in zip(kv_lens, n_pages)]
    qo_indptr = md.indptr_from_lengths(qo_lens)
    q = rng.standard_normal((qo_indptr[-1], hq, d))
    shape_k = (pool, page_size, hkv, d) if layout == "NHD" else (pool, hkv, page_size, d)
    shape_v = (pool, page_size, hkv, dv) if layout == "NHD" else (pool, hkv, page_size, dv)
    k = rng.standard_normal(shape_k)
    v = rng.standard_normal(shape_v)
    return dict(q=q, k=k, v=v, qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices,
                last=last, page_size=page_size, hkv=hkv, layout=layout)


def _oracle(c, causal=True, sm_scale=None, **kw):
    return at.paged_attention(c["q"], c["k"], c["v"], qo_indptr=c["qo_indptr"], kv_indptr=c["kv_indptr"],
                              kv_indices=c["kv_indices"], kv_last_page_len=c["last"],
                              page_size=c["page_size"], layout=c["layout"], num_kv_heads=c["hkv"],
                              causal=causal, sm_scale=sm_scale, **kw)


def _to_nhd(x, layout):
    return x if layout == "NHD" else x.transpose(0, 2, 1, 3)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [
    # (qo_lens, kv_lens, page_size, hq, hkv, d)
    ([3, 1, 4], [6, 2, 9], 4, 4, 2, 4),
    ([1, 1], [5, 3], 2, 2, 2, 3),
    ([2, 0, 5], [7, 3, 5], 3, 6, 2, 2),
    ([4], [4], 16, 3, 1, 5),
])
def test_numpy_oracle_matches_brute_force(layout, causal, shape):
    qo_lens, kv_lens, p, hq, hkv, d = shape
    rng = np.random.default_rng(5)
    c = _random_paged(rng, qo_lens, kv_lens, p, hq, hkv, d, layout)
    o, lse = _oracle(c, causal=causal, sm_scale=0.37)
    bo, bl = brute.attention(c["q"].tolist(), _to_nhd(c["k"], layout).tolist(),
                             _to_nhd(c["v"], layout).tolist(), qo_indptr=c["qo_indptr"],
                             kv_indptr=c["kv_indptr"], kv_indices=c["kv_indices"],
                             kv_last_page_len=c["last"], page_size=p, group=hq // hkv,
                             causal=causal, sm_scale=0.37)
    assert np.allclose(o, np.array(bo), rtol=0, atol=1e-12)
    assert np.allclose(lse, np.array(bl), rtol=0, atol=1e-12)


def test_single_request_full_prefill_is_causal_sdpa():
    """qo_len == kv_len on one page: the bottom-right mask is the ordinary
    causal triangle, so the result is textbook causal attention."""
    rng = np.random.default_rng(1)
    c = _random_paged(rng, [13], [13], 16, 8, 2, 16)
    o, lse = _oracle(c)
    k = torch.from_numpy(c["k"][c["kv_indices"][0]]).transpose(0, 1)[None]     # [1, Hkv, S, D]
    v = torch.from_numpy(c["v"][c["kv_indices"][0]]).transpose(0, 1)[None]
    k, v = k[:, :, :13], v[:, :, :13]
    q = torch.from_numpy(c["q"]).transpose(0, 1)[None]                           # [1, Hq, L, D]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
    assert np.allclose(o, ref[0].transpose(0, 1).numpy(), atol=1e-12)
    scores = (q @ k.repeat_interleave(4, dim=1).transpose(-1, -2)) / math.sqrt(16)
    scores = scores.masked_fill(torch.ones(13, 13, dtype=torch.bool).triu(1), -math.inf)
    ref_lse = torch.logsumexp(scores, dim=-1)[0].T.numpy() / math.log(2)
    assert np.allclose(lse, ref_lse, atol=1e-12)


def test_decode_rows_are_unmasked_sdpa():
    rng = np.random.default_rng(2)
    kv_lens = [9, 1, 20]
    c = _random_paged(rng, [1, 1, 1], kv_lens, 4, 4, 1, 8)
    o, lse = _oracle(c)
    for b, kl in enumerate(kv_lens):
        kb = at.gather_request(c["k"], "NHD", c["kv_indptr"], c["kv_indices"], 4, b, kl)
        vb = at.gather_request(c["v"], "NHD", c["kv_indptr"], c["kv_indices"], 4, b, kl)
        q = torch.from_numpy(c["q"][b:b + 1]).transpose(0, 1)[None]
        k = torch.from_numpy(kb).transpose(0, 1)[None]
        v = torch.from_numpy(vb).transpose(0, 1)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, enable_gqa=True)
        assert np.allclose(o[b], ref[0, :, 0].numpy(), atol=1e-12)


def test_bottom_right_mask_against_printed_rows():
    """R2 of the worked example (Q=4, K=9): SDPA with the printed mask rows."""
    g = load_golden("addresses_mask.json")
    mask = torch.tensor([[ch == "1" for ch in row] for row in g["printed_mask"]])
    rng = np.random.default_rng(4)
    c = _random_paged(rng, [4], [9], 4, 2, 2, 6)
    o, _ = _oracle(c)
    kb = at.gather_request(c["k"], "NHD", c["kv_indptr"], c["kv_indices"], 4, 0, 9)
    vb = at.gather_request(c["v"], "NHD", c["kv_indptr"], c["kv_indices"], 4, 0, 9)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(c["q"]).transpose(0, 1)[None], torch.from_numpy(kb).transpose(0, 1)[None],
        torch.from_numpy(vb).transpose(0, 1)[None], attn_mask=mask)
    assert np.allclose(o, ref[0].transpose(0, 1).numpy(), atol=1e-12)


def test_zero_query_closed_form():
    """With q = 0 every visible logit is 0: the output is the plain mean of the
    visible values and lse = log2(number of visible keys)."""
    rng = np.random.default_rng(6)
    c = _random_paged(rng, [3, 1, 4], [6, 2, 9], 4, 4, 2, 5)
    c["q"] = np.zeros_like(c["q"])
    o, lse = _oracle(c)
    for b, (ql, kl) in enumerate([(3, 6), (1, 2), (4, 9)]):
        kvb = at.gather_request(c["v"], "NHD", c["kv_indptr"], c["kv_indices"], 4, b, kl)
        for i in range(ql):
            n = kl - ql + i + 1
            row = c["qo_indptr"][b] + i
            for h in range(4):
                assert np.allclose(o[row, h], kvb[:n, h // 2].mean(axis=0), atol=1e-13)
                assert abs(lse[row, h] - math.log2(n)) < 1e-13


def test_invariances():
    """Page relabelling, page size, NHD/HND and split + merge leave the result
    unchanged (Deep Dive - FlashInfer, 'BSR as a memory-access contract' and
    'Core mechanism'; GPU attention backends, 'What it prints': page size 1
    and 4 give identical logits)."""
    rng = np.random.default_rng(8)
    qo_lens, kv_lens = [3, 1, 4, 2], [6, 2, 9, 31]
    base = _random_paged(rng, qo_lens, kv_lens, 4, 4, 2, 6)
    o0, l0 = _oracle(base)
    # logical sequences of each request, for rebuilding at other page sizes
    seq_k = [at.gather_request(base["k"], "NHD", base["kv_indptr"], base["kv_indices"], 4, b, kl)
             for b, kl in enumerate(kv_lens)]
    seq_v = [at.gather_request(base["v"], "NHD", base["kv_indptr"], base["kv_indices"], 4, b, kl)
             for b, kl in enumerate(kv_lens)]
    for p in (1, 3, 16):
        c = _random_paged(rng, qo_lens, kv_lens, p, 4, 2, 6)
        c["q"] = base["q"]
        for b, kl in enumerate(kv_lens):
            for j in range(kl):
                page, slot = md.token_address(c["kv_indptr"], c["kv_indices"], p, b, j)
                c["k"][page, slot] = seq_k[b][j]
                c["v"][page, slot] = seq_v[b][j]
        o, l = _oracle(c)
        assert np.allclose(o, o0, atol=1e-12) and np.allclose(l, l0, atol=1e-12)
    # HND storage of the same pages
    hnd = dict(base, k=base["k"].transpose(0, 2, 1, 3).copy(), v=base["v"].transpose(0, 2, 1, 3).copy(),
               layout="HND")
    o, l = _oracle(hnd)
    assert np.allclose(o, o0, atol=1e-13) and np.allclose(l, l0, atol=1e-13)
    # relabel physical pages by a permutation of the pool
    perm = rng.permutation(base["k"].shape[0])
    moved = dict(base, k=np.empty_like(base["k"]), v=np.empty_like(base["v"]),
                 kv_indices=[int(perm[x]) for x in base["kv_indices"]])
    moved["k"][perm] = base["k"]
    moved["v"][perm] = base["v"]
    o, l = _oracle(moved)
    assert np.allclose(o, o0, atol=1e-13) and np.allclose(l, l0, atol=1e-13)
    # any disjoint split of the keys, merged, equals the unsplit result
    for cuts in ([5], [2, 7], [1, 3, 8, 20]):
        bounds = [0] + cuts + [64]
        parts = [_oracle(base, key_range=(a, b)) for a, b in zip(bounds, bounds[1:])]
        v = np.stack([p[0] for p in parts], axis=1)
        s = np.stack([p[1] for p in parts], axis=1)
        mo, ml = mg.merge_states(v, s)
        assert np.allclose(mo, o0, atol=1e-12) and np.allclose(ml, l0, atol=1e-12)


def test_incremental_decode_equals_last_prefill_row():
    """Deep Dive - FlashInfer, 'A release checklist at the boundary': decode of
    the last token equals the last row of a full-prefix prefill."""
    rng = np.random.default_rng(9)
    c = _random_paged(rng, [7, 5], [7, 12], 4, 4, 2, 8)
    o, l = _oracle(c)
    last_rows = [c["qo_indptr"][1] - 1, c["qo_indptr"][2] - 1]
    dec = dict(c, q=c["q"][last_rows], qo_indptr=[0, 1, 2])
    od, ld = _oracle(dec)
    assert np.allclose(od, o[last_rows], atol=1e-13) and np.allclose(ld, l[last_rows], atol=1e-13)


def test_bf16_upcast_is_exact():
    x = np.array([1.0, -2.5, 3.140625, 0.0], dtype=np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(at.upcast(bits, "bf16"), x.astype(np.float64))


def test_mla_decode_is_sdpa_with_concatenated_keys():
    """MLA decode reduces to attention with key = [ckv, kpe] (576 wide), value =
    ckv (512 wide) and one shared kv head; checked with SDPA's GQA mode on a
    reduced width (24 + 8) so the check stays fast."""
    rng = np.random.default_rng(10)
    batch, heads, dc, dp, p = 3, 8, 24, 8, 4
    kv_lens = [5, 12, 1]
    n_pages = [math.ceil(k / p) for k in kv_lens]
    pool = sum(n_pages) + 2
    perm = [int(x) for x in rng.permutation(pool)]
    kv_indptr = md.indptr_from_lengths(n_pages)
    kv_indices = perm[:sum(n_pages)]
    last = [k - (n - 1) * p for k, n in zip(kv_lens, n_pages)]
    cache = rng.standard_normal((pool, p, dc + dp))
    q_ckv = rng.standard_normal((batch, heads, dc))
    q_kpe = rng.standard_normal((batch, heads, dp))
    scale = 0.11
    o, lse = at.mla_decode(q_ckv, q_kpe, cache[..., :dc], cache[..., dc:], kv_indptr=kv_indptr,
                           kv_indices=kv_indices, kv_last_page_len=last, page_size=p,
                           sm_scale=scale, dtype="f32")
    for b, kl in enumerate(kv_lens):
        rows = np.stack([cache[kv_indices[kv_indptr[b] + j // p], j % p] for j in range(kl)])
        q = torch.from_numpy(np.concatenate([q_ckv[b], q_kpe[b]], axis=1))[None, :, None]
        k = torch.from_numpy(rows)[None, None]
        v = torch.from_numpy(rows[:, :dc])[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale, enable_gqa=True)
        assert np.allclose(o[b], ref[0, :, 0].numpy(), atol=1e-12)
        s = (q[0, :, 0] @ k[0, 0].T) * scale
        assert np.allclose(lse[b], (torch.logsumexp(s, dim=-1) / math.log(2)).numpy(), atol=1e-12)


# ------------------------------------------------------------ fp8 storage --

def test_fp8_e4m3_decoding_matches_torch_for_every_code():
    """All 256 E4M3 codes against torch's float8_e4m3fn (an independent
    implementation of the same OCP format), NaN codes included."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = at.upcast(codes, "fp8")
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    # a few hand values: 1.0, -2.0, the largest finite, the smallest subnormal
    assert at.fp8_e4m3_value(0x38) == 1.0 and at.fp8_e4m3_value(0xC0) == -2.0
    assert at.fp8_e4m3_value(0x7E) == 448.0 and at.fp8_e4m3_value(0x01) == 2.0 ** -9


def test_fp8_scales_fold_into_scores_and_outputs():
    """k_scale multiplies every score (same as scaling sm_scale) and v_scale
    every output; the LSE shifts only through the scores."""
    rng = np.random.default_rng(9)
    c = _random_paged(rng, [2, 3], [9, 14], 4, 4, 2, 16)
    codes_k = rng.integers(0, 0x77, size=c["k"].shape).astype(np.uint8)
    codes_v = rng.integers(0, 0x77, size=c["v"].shape).astype(np.uint8)
    codes_k[rng.random(codes_k.shape) < 0.5] |= 0x80
    kw = dict(qo_indptr=c["qo_indptr"], kv_indptr=c["kv_indptr"], kv_indices=c["kv_indices"],
              kv_last_page_len=c["last"], page_size=4, layout="NHD", num_kv_heads=2, kv_dtype="fp8")
    o1, l1 = at.paged_attention(c["q"], codes_k, codes_v, sm_scale=0.1, k_scale=0.5, v_scale=3.0, **kw)
    o2, l2 = at.paged_attention(c["q"], codes_k, codes_v, sm_scale=0.05, **kw)
    assert np.max(np.abs(o1 - 3.0 * o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12
