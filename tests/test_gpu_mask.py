"""GPU parity of ragged-KV prefill and custom-masked attention (through the C
ABI) against the float64 oracle, plus the bit-packing kernel against
numpy's little-endian packbits."""

import math

import numpy as np
import pytest

import workloads as wl
from oracle import attention as oat
from oracle import mask as omask
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return gu.require_gpu()


@pytest.fixture(scope="module")
def pkv(torch):
    import paged_kv_cache_plan_amd as pkv
    return pkv


def _payload(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return wl.to_bf16_bits(x) if dtype == "bf16" else x


def _mask(rng, qo_lens, kv_lens, p=0.5, empty_rows=2):
    segs = []
    for q, k in zip(qo_lens, kv_lens):
        m = rng.random((q, k)) < p
        if q and empty_rows:
            m[rng.integers(0, q, size=min(q, empty_rows))] = False     # rows that see nothing
        segs.append(m.reshape(-1))
    return np.concatenate(segs) if segs else np.zeros(0, bool)


def _packed(torch, pkv, mask):
    packed = pkv.packbits(torch.from_numpy(mask.astype(np.uint8)).cuda())
    want = np.packbits(mask, bitorder="little")
    got = packed.cpu().numpy()
    assert np.array_equal(got[:len(want)], want) and not got[len(want):].any()
    return packed


@pytest.mark.parametrize("n", [1, 31, 32, 33, 1000, 65537])
def test_packbits_kernel(torch, pkv, n):
    rng = np.random.default_rng(n)
    _packed(torch, pkv, rng.random(n) < 0.5)


def _ragged_case(seed, dtype, hq, hkv, d, qo_lens, kv_extra):
    rng = np.random.default_rng(seed)
    kv_lens = [q + e for q, e in zip(qo_lens, kv_extra)]
    qo = np.array([0] + list(np.cumsum(qo_lens)), np.int32)
    kv = np.array([0] + list(np.cumsum(kv_lens)), np.int32)
    q = _payload(rng, (int(qo[-1]), hq, d), dtype)
    k = _payload(rng, (int(kv[-1]), hkv, d), dtype)
    v = _payload(rng, (int(kv[-1]), hkv, d), dtype)
    return rng, qo_lens, kv_lens, qo, kv, q, k, v


@pytest.mark.parametrize("dtype,hq,hkv,d,causal,masked,fixed", [
    ("bf16", 32, 8, 128, True, False, 0),     # MFMA tile kernel
    ("bf16", 32, 8, 128, False, False, 3),
    ("f32", 8, 2, 64, True, False, 0),        # row kernel
    ("bf16", 16, 4, 128, False, True, 0),     # custom mask on the MFMA kernel (group 4)
    ("bf16", 16, 8, 128, False, True, 2),     # group 2, forced splits
    ("bf16", 64, 8, 128, False, True, 0),     # group 8
    ("bf16", 8, 8, 128, False, True, 0),      # group 1: row kernel
    ("f32", 4, 4, 64, False, True, 1),
])
def test_ragged_prefill(torch, pkv, dtype, hq, hkv, d, causal, masked, fixed):
    print("case ragged", dtype, hq, hkv, d, causal, masked, fixed, flush=True)
    qo_lens = [37, 0, 300, 129, 64, 5]
    rng, qo_lens, kv_lens, qo, kv, q, k, v = _ragged_case(7, dtype, hq, hkv, d, qo_lens, [0, 9, 700, 0, 33, 1])
    mask = _mask(rng, qo_lens, kv_lens) if masked else None
    params = pkv.plan_params(mode="prefill", batch_size=len(qo_lens), num_qo_heads=hq, num_kv_heads=hkv,
                             head_dim_qk=d, page_size=16, causal=causal, dtype=dtype, ragged=True,
                             custom_mask=masked, fixed_split_pages=fixed, num_cus=16 if fixed else 0)
    plan = pkv.Plan(params, qo_indptr=qo, kv_indptr=kv, kv_last_page_len=None)
    if masked:
        assert plan.info["mask_bits"] == len(mask)
    qd = gu.to_dev(q, dtype)
    out = gu.empty_like_out(qd.shape, dtype)
    lse = torch.full((qd.shape[0], hq), float("nan"), dtype=torch.float32, device="cuda")
    plan.run_ragged(qd, gu.to_dev(k, dtype), gu.to_dev(v, dtype), gu.to_dev(kv, "i32"), out, lse,
                    mask_packed=_packed(torch, pkv, mask) if masked else None, sm_scale=1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    ro, rl = omask.ragged_attention(q, k, v, qo_indptr=list(qo), kv_indptr=list(kv), num_kv_heads=hkv,
                                    causal=causal, custom_mask=mask, sm_scale=1.0 / math.sqrt(d), q_dtype=dtype,
                                    kv_dtype=dtype)
    got = gu.as_f64(gu.to_host(out, dtype), dtype)
    gu.check_close(got, ro, dtype, "ragged o")
    gu.check_lse(lse.cpu().numpy(), rl, "ragged lse", atol=1e-5 if dtype == "f32" else 1e-3)


@pytest.mark.parametrize("hq,causal,fixed,masked", [(16, True, 0, False), (8, False, 3, False), (16, False, 0, True),
                                                    (32, False, 2, True), (8, False, 0, True)])
def test_ragged_prefill_fp8(torch, pkv, hq, causal, fixed, masked):
    """Ragged keys and values stored as E4M3 codes (bf16 queries and outputs):
    the MFMA tile kernel expands the tiles to bf16 in LDS, custom masks
    included (head groups 2 and 4); with one query head per kv head a masked
    plan runs the row kernel."""
    print("case ragged fp8", hq, causal, fixed, masked, flush=True)
    rng = np.random.default_rng(17)
    qo_lens, kv_extra = [37, 0, 300, 129, 64, 5], [0, 9, 700, 0, 33, 1]
    kv_lens = [q + e for q, e in zip(qo_lens, kv_extra)]
    qo = np.array([0] + list(np.cumsum(qo_lens)), np.int32)
    kv = np.array([0] + list(np.cumsum(kv_lens)), np.int32)
    q = _payload(rng, (int(qo[-1]), hq, 128), "bf16")
    k = wl.to_fp8_codes(rng.standard_normal((int(kv[-1]), 8, 128)).astype(np.float32))
    v = wl.to_fp8_codes(rng.standard_normal((int(kv[-1]), 8, 128)).astype(np.float32))
    mask = _mask(rng, qo_lens, kv_lens) if masked else None
    params = pkv.plan_params(mode="prefill", batch_size=len(qo_lens), num_qo_heads=hq, num_kv_heads=8,
                             head_dim_qk=128, page_size=16, causal=causal, dtype="bf16", kv_dtype="fp8",
                             ragged=True, custom_mask=masked, fixed_split_pages=fixed, num_cus=16 if fixed else 0)
    plan = pkv.Plan(params, qo_indptr=qo, kv_indptr=kv, kv_last_page_len=None)
    qd = gu.to_dev(q, "bf16")
    out = gu.empty_like_out(qd.shape, "bf16")
    lse = torch.full((qd.shape[0], hq), float("nan"), dtype=torch.float32, device="cuda")
    plan.run_ragged(qd, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), gu.to_dev(kv, "i32"), out, lse,
                    mask_packed=_packed(torch, pkv, mask) if masked else None, sm_scale=1.0 / math.sqrt(128))
    torch.cuda.synchronize()
    ro, rl = omask.ragged_attention(q, k, v, qo_indptr=list(qo), kv_indptr=list(kv), num_kv_heads=8, causal=causal,
                                    custom_mask=mask, sm_scale=1.0 / math.sqrt(128), q_dtype="bf16", kv_dtype="fp8")
    gu.check_close(gu.as_f64(gu.to_host(out, "bf16"), "bf16"), ro, "bf16", "ragged fp8 o")
    gu.check_lse(lse.cpu().numpy(), rl, "ragged fp8 lse")


@pytest.mark.parametrize("fixed", [0, 1, 2])
def test_paged_custom_mask(torch, pkv, fixed):
    """The pages' three-request batch shape on a paged cache (page 4) with a
    random custom mask, including rows that see no key; forced splits give
    chunks where a row sees nothing, which the merge must pass over."""
    print("case paged mask", fixed, flush=True)
    b = wl.make("worked", literal_pages=True)
    rng = np.random.default_rng(11)
    mask = _mask(rng, b.qo_lens, b.kv_lens, p=0.4, empty_rows=1)
    params = pkv.plan_params(mode="prefill", batch_size=3, num_qo_heads=4, num_kv_heads=2, head_dim_qk=64,
                             page_size=4, causal=False, dtype="f32", custom_mask=True, fixed_split_pages=fixed,
                             num_cus=4, max_num_pages=16)
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                    kv_last_page_len=b.kv_last_page_len)
    k_exp = b.k_cache.copy()
    v_exp = b.v_cache.copy()
    qd = gu.to_dev(b.q, "f32")
    out = gu.empty_like_out(qd.shape, "f32")
    lse = torch.full((qd.shape[0], 4), float("nan"), dtype=torch.float32, device="cuda")
    plan.run_masked(qd, gu.to_dev(k_exp, "f32"), gu.to_dev(v_exp, "f32"), gu.to_dev(b.kv_indices, "i32"),
                    _packed(torch, pkv, mask), out, lse, layout="NHD", sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oat.paged_attention(b.q, k_exp, v_exp, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                                 kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                                 page_size=4, layout="NHD", num_kv_heads=2, sm_scale=b.sm_scale, custom_mask=mask)
    gu.check_close(gu.to_host(out, "f32"), ro, "f32", "masked o")
    gu.check_lse(lse.cpu().numpy(), rl, "masked lse", atol=1e-5)
    assert np.isneginf(rl).any()


def test_paged_custom_mask_bf16_prefill_workload(torch, pkv):
    """The chunked-prefill workload (scaled to a quarter) with a random mask, HND, bf16."""
    b = wl.make("prefill", scale=0.25, batch=4, poison=False)
    rng = np.random.default_rng(13)
    mask = _mask(rng, b.qo_lens, b.kv_lens, p=0.7, empty_rows=3)
    params = pkv.plan_params(mode="prefill", batch_size=4, num_qo_heads=32, num_kv_heads=8, head_dim_qk=128,
                             page_size=16, causal=False, dtype="bf16", custom_mask=True,
                             max_num_pages=b.max_num_pages)
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                    kv_last_page_len=b.kv_last_page_len)
    qd = gu.to_dev(b.q, "bf16")
    out = gu.empty_like_out(qd.shape, "bf16")
    lse = torch.full((qd.shape[0], 32), float("nan"), dtype=torch.float32, device="cuda")
    plan.run_masked(qd, gu.to_dev(b.k_cache, "bf16"), gu.to_dev(b.v_cache, "bf16"), gu.to_dev(b.kv_indices, "i32"),
                    _packed(torch, pkv, mask), out, lse, layout="HND", sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oat.paged_attention(b.q, b.k_cache, b.v_cache, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                                 kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                                 page_size=16, layout="HND", num_kv_heads=8, sm_scale=b.sm_scale, q_dtype="bf16",
                                 kv_dtype="bf16", custom_mask=mask)
    gu.check_close(gu.as_f64(gu.to_host(out, "bf16"), "bf16"), ro, "bf16", "masked prefill o")
    gu.check_lse(lse.cpu().numpy(), rl, "masked prefill lse")


def test_paged_custom_mask_fp8_prefill_workload(torch, pkv):
    """The chunked-prefill workload (scaled to a quarter) over an E4M3 cache
    with a random mask, HND: the masked MFMA tile kernel on fp8 tiles, with
    non-unit K and V scales."""
    b = wl.make("prefill", scale=0.25, batch=4, poison=False, kv_dtype="fp8")
    rng = np.random.default_rng(19)
    mask = _mask(rng, b.qo_lens, b.kv_lens, p=0.7, empty_rows=3)
    params = pkv.plan_params(mode="prefill", batch_size=4, num_qo_heads=32, num_kv_heads=8, head_dim_qk=128,
                             page_size=16, causal=False, dtype="bf16", kv_dtype="fp8", custom_mask=True,
                             max_num_pages=b.max_num_pages)
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                    kv_last_page_len=b.kv_last_page_len)
    assert plan.info["rows_per_tile"] == 64
    qd = gu.to_dev(b.q, "bf16")
    out = gu.empty_like_out(qd.shape, "bf16")
    lse = torch.full((qd.shape[0], 32), float("nan"), dtype=torch.float32, device="cuda")
    plan.run_masked(qd, torch.from_numpy(b.k_cache).cuda(), torch.from_numpy(b.v_cache).cuda(),
                    gu.to_dev(b.kv_indices, "i32"), _packed(torch, pkv, mask), out, lse, layout="HND",
                    sm_scale=b.sm_scale, k_scale=0.5, v_scale=2.0)
    torch.cuda.synchronize()
    ro, rl = oat.paged_attention(b.q, b.k_cache, b.v_cache, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                                 kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                                 page_size=16, layout="HND", num_kv_heads=8, sm_scale=b.sm_scale, q_dtype="bf16",
                                 kv_dtype="fp8", custom_mask=mask, k_scale=0.5, v_scale=2.0)
    gu.check_close(gu.as_f64(gu.to_host(out, "bf16"), "bf16"), ro, "bf16", "masked fp8 prefill o")
    gu.check_lse(lse.cpu().numpy(), rl, "masked fp8 prefill lse")


def test_masked_and_ragged_plans_need_their_entry_points(torch, pkv):
    b = wl.make("worked", literal_pages=True)
    params = pkv.plan_params(mode="prefill", batch_size=3, num_qo_heads=4, num_kv_heads=2, head_dim_qk=64,
                             page_size=4, causal=False, dtype="f32", custom_mask=True, max_num_pages=16)
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                    kv_last_page_len=b.kv_last_page_len)
    qd = gu.to_dev(b.q, "f32")
    with pytest.raises(pkv.PkvError):
        plan.run(qd, gu.to_dev(b.k_cache, "f32"), gu.to_dev(b.v_cache, "f32"), gu.to_dev(b.kv_indices, "i32"),
                 torch.empty_like(qd), layout="NHD")
