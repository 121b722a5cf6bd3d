"""Work at the planner's limits.  Each kernel stages one chunk's page ids on
chip, at most 1024 of them, and the planner never makes a longer chunk.
With one key per page, requests of 2100-3100 keys split into chunks of
exactly 1024 pages, so the staged table is used to its last entry: the
decode row kernel, the MFMA prefill kernel and the MLA kernel each run such
a batch.  Batches of thousands of short requests give thousands of work
items and merge items.  Every case runs on a NaN-poisoned cache against the
float64 oracle."""

import pytest

import workloads as wl
from oracle import attention as oat
from oracle import metadata as omd
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

LIMIT = 1024   # page ids of one chunk (the planner's cap, the kernels' table size)


@pytest.fixture(scope="module")
def torch():
    return gu.require_gpu()


@pytest.fixture(scope="module")
def pkv(torch):
    import paged_kv_cache_plan_amd as pkv
    return pkv


def _plan(pkv, b, fixed, num_cus, max_num_pages, waves=0):
    mla = b.mode == "mla"
    params = pkv.plan_params(mode=b.mode, batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                             num_kv_heads=b.num_kv_heads, head_dim_qk=576 if mla else b.head_dim,
                             head_dim_vo=512 if mla else b.head_dim, page_size=b.page_size, causal=b.causal,
                             dtype=b.dtype, num_cus=num_cus, fixed_split_pages=fixed, max_num_pages=max_num_pages,
                             row_waves=waves)
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr if b.mode == "prefill" else None, kv_indptr=b.kv_indptr,
                    kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    info = plan.info
    assert info["chunk_pages"] == LIMIT and info["split"] == 1 and info["num_merges"] > 0, info
    return plan


def _check(o, lse, ro, rl, what):
    got = gu.as_f64(o, "bf16")
    gu.check_close(got, ro, "bf16", f"{what} o")
    gu.check_lse(lse, rl, f"{what} lse")
    print(what, gu.check_guard(got, ro, lse, rl, what), flush=True)


@pytest.mark.parametrize("fixed,num_cus,waves", [(LIMIT, 256, 0), (0, 1, 0), (LIMIT, 256, 1)])
def test_decode_chunks_at_the_limit(torch, pkv, fixed, num_cus, waves):
    """Forced 1024-page chunks (row kernel workgroups of 4 waves and of one),
    and the planner left to itself with one CU (it then makes the longest
    chunks it may)."""
    print("case decode chunk limit", fixed, num_cus, waves, flush=True)
    b = wl.make("decode", poison=True, page_size=1, batch=3, kv_range=(2100, 3100), seed=4101)
    k_dev, v_dev = gu.to_dev(b.k_cache, "bf16"), gu.to_dev(b.v_cache, "bf16")
    plan = _plan(pkv, b, fixed, num_cus, k_dev.shape[0], waves)
    q = gu.to_dev(b.q, "bf16")
    out = gu.empty_like_out(q.shape, "bf16")
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    plan.run(q, k_dev, v_dev, gu.to_dev(b.kv_indices, "i32"), out, lse, layout=b.layout, sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oat.paged_attention(b.q, b.k_cache, b.v_cache, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                                 kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                                 page_size=b.page_size, layout=b.layout, num_kv_heads=b.num_kv_heads, causal=True,
                                 sm_scale=b.sm_scale, q_dtype="bf16", kv_dtype="bf16")
    _check(gu.to_host(out, "bf16"), lse.cpu().numpy(), ro, rl, f"decode chunk limit {fixed}/{num_cus}")


def test_prefill_chunks_at_the_limit(torch, pkv):
    """Two requests of 100-160 new rows over 2000-2600-token prefixes (HND,
    32/8 heads, d 128): the MFMA tile kernel with 1024-page chunks."""
    print("case prefill chunk limit", flush=True)
    b = wl.make("prefill", poison=True, page_size=1, batch=2, qo_range=(100, 160), prefix_range=(2000, 2600),
                seed=4102)
    # The cache after the append of the new rows (their slots from the oracle's slot map).
    k_exp, v_exp = b.k_cache.copy(), b.v_cache.copy()
    targets = omd.append_targets(list(b.append_indptr), list(b.kv_indptr), list(b.kv_indices),
                                 list(b.kv_last_page_len), b.page_size)
    for t, (page, slot) in enumerate(targets):
        k_exp[page, :, slot], v_exp[page, :, slot] = b.k_new[t], b.v_new[t]
    k_dev, v_dev = gu.to_dev(k_exp, "bf16"), gu.to_dev(v_exp, "bf16")
    plan = _plan(pkv, b, LIMIT, 256, k_dev.shape[0])
    q = gu.to_dev(b.q, "bf16")
    out = gu.empty_like_out(q.shape, "bf16")
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    plan.run(q, k_dev, v_dev, gu.to_dev(b.kv_indices, "i32"), out, lse, layout=b.layout, sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oat.paged_attention(b.q, k_exp, v_exp, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                                 kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                                 page_size=b.page_size, layout=b.layout, num_kv_heads=b.num_kv_heads, causal=True,
                                 sm_scale=b.sm_scale, q_dtype="bf16", kv_dtype="bf16")
    _check(gu.to_host(out, "bf16"), lse.cpu().numpy(), ro, rl, "prefill chunk limit")


def test_mla_chunks_at_the_limit(torch, pkv):
    """Two MLA requests of 2100-2600 keys on one-key pages, 128 heads."""
    print("case mla chunk limit", flush=True)
    b = wl.make("mla", poison=True, page_size=1, batch=2, kv_range=(2100, 2600), seed=4103)
    cache = gu.to_dev(b.k_cache, "bf16")
    plan = _plan(pkv, b, LIMIT, 256, b.max_num_pages)
    out = gu.empty_like_out((b.batch_size, 128, 512), "bf16")
    lse = torch.full((b.batch_size, 128), float("nan"), dtype=torch.float32, device="cuda")
    plan.run_mla(gu.to_dev(b.q, "bf16"), gu.to_dev(b.q_kpe, "bf16"), cache[..., :512], cache[..., 512:],
                 gu.to_dev(b.kv_indices, "i32"), out, lse, sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oat.mla_decode(b.q, b.q_kpe, b.k_cache[..., :512], b.k_cache[..., 512:], kv_indptr=list(b.kv_indptr),
                            kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                            page_size=b.page_size, sm_scale=b.sm_scale, dtype="bf16")
    _check(gu.to_host(out, "bf16"), lse.cpu().numpy(), ro, rl, "mla chunk limit")


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_many_short_requests(torch, pkv, mode):
    """Thousands of work items: 2048 decode requests of 1-96 keys (page 16,
    64 workgroups per CU and a merge item for most requests), or 512 prefill
    requests of 1-12 new rows over prefixes of up to 80 keys."""
    print("case many requests", mode, flush=True)
    if mode == "decode":
        b = wl.make("decode", poison=True, batch=2048, kv_range=(1, 96), seed=4104)
        k_host, v_host = b.k_cache, b.v_cache
    else:
        b = wl.make("prefill", poison=True, batch=512, qo_range=(1, 12), prefix_range=(0, 80), seed=4105)
        k_host, v_host = b.k_cache.copy(), b.v_cache.copy()
        targets = omd.append_targets(list(b.append_indptr), list(b.kv_indptr), list(b.kv_indices),
                                     list(b.kv_last_page_len), b.page_size)
        for t, (page, slot) in enumerate(targets):
            k_host[page, :, slot], v_host[page, :, slot] = b.k_new[t], b.v_new[t]
    k_dev, v_dev = gu.to_dev(k_host, "bf16"), gu.to_dev(v_host, "bf16")
    params = pkv.plan_params(mode=mode, batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                             num_kv_heads=b.num_kv_heads, head_dim_qk=b.head_dim, page_size=b.page_size,
                             causal=True, dtype="bf16", max_num_pages=k_dev.shape[0])
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr if mode == "prefill" else None, kv_indptr=b.kv_indptr,
                    kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    assert plan.info["num_items"] >= 512, plan.info
    # 2048 short decode requests: the plan picks one-wave row workgroups
    assert plan.info["row_waves"] == (1 if mode == "decode" else 4), plan.info
    q = gu.to_dev(b.q, "bf16")
    out = gu.empty_like_out(q.shape, "bf16")
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    plan.run(q, k_dev, v_dev, gu.to_dev(b.kv_indices, "i32"), out, lse, layout=b.layout, sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oat.paged_attention(b.q, k_host, v_host, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                                 kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                                 page_size=b.page_size, layout=b.layout, num_kv_heads=b.num_kv_heads, causal=True,
                                 sm_scale=b.sm_scale, q_dtype="bf16", kv_dtype="bf16")
    _check(gu.to_host(out, "bf16"), lse.cpu().numpy(), ro, rl, f"many requests {mode} {plan.info['num_items']} items")
