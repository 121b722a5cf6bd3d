"""GPU parity of the fused append (pkv_run_append): one decode launch that
appends the batch's new K/V rows and attends over them must leave the cache
bit for bit as append_paged_kv does, and its outputs must match both the
float64 oracle over the post-append cache and append_paged_kv followed by
run (which sums the keys in another order: equal up to fp32 rounding).

The new rows are the last n_b keys of request b (kv_len counts them).  Their
cache slots are NaN before the call, so a kernel that read them from the
cache instead of from k_new / v_new would return non-finite outputs."""

import numpy as np
import pytest

import workloads as wl
from oracle import attention as oat
from oracle import metadata as omd
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return gu.require_gpu()


@pytest.fixture(scope="module")
def pkv(torch):
    import paged_kv_cache_plan_amd as pkv
    return pkv


def _batch(*, layout, page_size, dtype, kv_dtype, n_max, seed):
    """A small decode batch whose last n_b keys per request (n_b in [0, n_max],
    at most kv_len) are new rows, with their slots NaN in the cache."""
    b = wl.make("decode", scale=0.25, batch=12, layout=layout, page_size=page_size, dtype=dtype,
                kv_dtype=kv_dtype, poison=True)
    rng = np.random.default_rng(seed)
    n_new = np.minimum(rng.integers(0, n_max, size=b.batch_size, endpoint=True), b.kv_lens)
    append_indptr = np.zeros(b.batch_size + 1, dtype=np.int32)
    append_indptr[1:] = np.cumsum(n_new)
    nnz = int(append_indptr[-1])
    k_new = wl._payload(rng, (nnz, b.num_kv_heads, b.head_dim), kv_dtype)
    v_new = wl._payload(rng, (nnz, b.num_kv_heads, b.head_dim), kv_dtype)
    targets = omd.append_targets(list(append_indptr), list(b.kv_indptr), list(b.kv_indices),
                                 list(b.kv_last_page_len), b.page_size)
    nan = {"bf16": wl.BF16_NAN, "fp8": wl.FP8_NAN}.get(kv_dtype, np.float32(np.nan))
    k_pois, v_pois = b.k_cache.copy(), b.v_cache.copy()
    k_exp, v_exp = b.k_cache.copy(), b.v_cache.copy()
    for t, (page, slot) in enumerate(targets):
        if layout == "NHD":
            k_pois[page, slot] = nan
            v_pois[page, slot] = nan
            k_exp[page, slot], v_exp[page, slot] = k_new[t], v_new[t]
        else:
            k_pois[page, :, slot] = nan
            v_pois[page, :, slot] = nan
            k_exp[page, :, slot], v_exp[page, :, slot] = k_new[t], v_new[t]
    return b, append_indptr, k_new, v_new, (k_pois, v_pois), (k_exp, v_exp)


def _dev(torch, x, dtype):
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return gu.to_dev(x, dtype)


def _host(x, dtype):
    return x.cpu().numpy() if dtype == "fp8" else gu.to_host(x, dtype)


def _bits(x):
    """Storage bits, so that NaN slots compare equal."""
    x = np.ascontiguousarray(x)
    return x.view(np.uint32) if x.dtype == np.float32 else x


def _plan(pkv, b, kv_dtype, fixed, max_pages, waves=0):
    params = pkv.plan_params(mode="decode", batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                             num_kv_heads=b.num_kv_heads, head_dim_qk=b.head_dim, page_size=b.page_size,
                             causal=True, dtype=b.dtype, kv_dtype=kv_dtype, fixed_split_pages=fixed,
                             max_num_pages=max_pages, row_waves=waves)
    return pkv.Plan(params, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)


CASES = [
    # layout, page size, q dtype, cache dtype, largest n_b, forced chunk pages
    ("NHD", 16, "bf16", "bf16", 1, 0),
    ("NHD", 16, "bf16", "bf16", 40, 2),
    ("HND", 16, "bf16", "bf16", 21, 1),
    ("NHD", 3, "bf16", "bf16", 9, 2),
    ("HND", 1, "bf16", "bf16", 5, 7),
    ("NHD", 16, "bf16", "fp8", 17, 3),
    ("HND", 4, "f32", "f32", 6, 0),
]


@pytest.mark.parametrize("waves", [0, 1])
@pytest.mark.parametrize("layout,page_size,dtype,kv_dtype,n_max,fixed", CASES)
def test_fused_append_matches_append_then_run(torch, pkv, layout, page_size, dtype, kv_dtype, n_max, fixed, waves):
    """Row kernel workgroups as the plan picks them and forced to one wave."""
    print("case fused append", layout, page_size, dtype, kv_dtype, n_max, fixed, waves, flush=True)
    b, append_indptr, k_new, v_new, (k_pois, v_pois), (k_exp, v_exp) = _batch(
        layout=layout, page_size=page_size, dtype=dtype, kv_dtype=kv_dtype, n_max=n_max, seed=n_max + page_size)
    plan = _plan(pkv, b, kv_dtype, fixed, k_pois.shape[0], waves)
    assert plan.info["row_waves"] == waves if waves else plan.info["row_waves"] in (1, 4)
    if fixed:
        assert plan.info["split"] == 1
    q = gu.to_dev(b.q, dtype)
    idx = gu.to_dev(b.kv_indices, "i32")
    meta = dict(append_indptr=gu.to_dev(append_indptr, "i32"), kv_indptr=gu.to_dev(b.kv_indptr, "i32"),
                kv_last_page_len=gu.to_dev(b.kv_last_page_len, "i32"))
    kn, vn = _dev(torch, k_new, kv_dtype), _dev(torch, v_new, kv_dtype)
    scales = dict(k_scale=0.75, v_scale=1.25) if kv_dtype == "fp8" else {}

    # append_paged_kv, then run
    ka, va = _dev(torch, k_pois, kv_dtype), _dev(torch, v_pois, kv_dtype)
    pkv.append_paged_kv(kn, vn, meta["append_indptr"], meta["kv_indptr"], idx, meta["kv_last_page_len"], ka, va,
                        layout=layout, page_size=page_size)
    oa = gu.empty_like_out(q.shape, dtype)
    la = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    plan.run(q, ka, va, idx, oa, la, layout=layout, sm_scale=b.sm_scale, **scales)

    # the fused launch, with its merge and with a separate merge
    outs = []
    for with_merge in (True, False):
        kf, vf = _dev(torch, k_pois, kv_dtype), _dev(torch, v_pois, kv_dtype)
        of = gu.empty_like_out(q.shape, dtype)
        lf = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
        plan.run_append(q, kf, vf, idx, of, lf, k_new=kn, v_new=vn, layout=layout, sm_scale=b.sm_scale,
                        with_merge=with_merge, **meta, **scales)
        if not with_merge:
            plan.run_merge(of, lf)
        outs.append((kf, vf, of, lf))
    torch.cuda.synchronize()

    ka_h, va_h = _host(ka, kv_dtype), _host(va, kv_dtype)
    assert np.array_equal(_bits(ka_h), _bits(k_exp)) and np.array_equal(_bits(va_h), _bits(v_exp)), \
        "append_paged_kv cache"
    for kf, vf, of, lf in outs:
        assert np.array_equal(_bits(_host(kf, kv_dtype)), _bits(k_exp)), "fused append: K cache"
        assert np.array_equal(_bits(_host(vf, kv_dtype)), _bits(v_exp)), "fused append: V cache"
    # with its merge (inside the launch when the plan allows) and with a
    # separate merge: equal up to the merges' rounding (the separate merge
    # kernel sums rows of more than 64 chunks in another order)
    gu.check_close(gu.as_f64(gu.to_host(outs[0][2], dtype), dtype), gu.as_f64(gu.to_host(outs[1][2], dtype), dtype),
                   dtype, "merge inside vs separate merge o")
    gu.check_lse(outs[0][3].cpu().numpy(), outs[1][3].cpu().numpy(), "merge inside vs separate merge lse", atol=1e-5)
    # against append then run
    gu.check_close(gu.as_f64(gu.to_host(outs[0][2], dtype), dtype), gu.as_f64(gu.to_host(oa, dtype), dtype), dtype,
                   "fused vs separate append o")
    gu.check_lse(outs[0][3].cpu().numpy(), la.cpu().numpy(), "fused vs separate append lse", atol=1e-5)

    ro, rl = oat.paged_attention(b.q, k_exp, v_exp, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                                 kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                                 page_size=page_size, layout=layout, num_kv_heads=b.num_kv_heads, causal=True,
                                 sm_scale=b.sm_scale, q_dtype=dtype, kv_dtype=kv_dtype, **scales)
    o = gu.to_host(outs[0][2], dtype)
    gu.check_close(gu.as_f64(o, dtype), ro, dtype, "fused append o")
    gu.check_lse(outs[0][3].cpu().numpy(), rl, "fused append lse", atol=1e-5 if dtype == "f32" else gu.LSE_ATOL)


def test_fused_append_with_no_new_rows_is_a_plain_run(torch, pkv):
    print("case fused append nnz 0", flush=True)
    b = wl.make("decode", scale=0.25, batch=12, poison=True)
    plan = _plan(pkv, b, "bf16", 2, b.k_cache.shape[0])
    q, idx = gu.to_dev(b.q, "bf16"), gu.to_dev(b.kv_indices, "i32")
    k, v = gu.to_dev(b.k_cache, "bf16"), gu.to_dev(b.v_cache, "bf16")
    empty = torch.empty((0, b.num_kv_heads, b.head_dim), dtype=torch.bfloat16, device="cuda")
    meta = dict(append_indptr=gu.to_dev(np.zeros(b.batch_size + 1, np.int32), "i32"),
                kv_indptr=gu.to_dev(b.kv_indptr, "i32"), kv_last_page_len=gu.to_dev(b.kv_last_page_len, "i32"))
    o1, o2 = gu.empty_like_out(q.shape, "bf16"), gu.empty_like_out(q.shape, "bf16")
    l1 = torch.empty((q.shape[0], b.num_qo_heads), dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    plan.run(q, k, v, idx, o1, l1, layout=b.layout, sm_scale=b.sm_scale)
    plan.run_append(q, k, v, idx, o2, l2, k_new=empty, v_new=empty, layout=b.layout, sm_scale=b.sm_scale, **meta)
    torch.cuda.synchronize()
    assert np.array_equal(gu.to_host(o1, "bf16"), gu.to_host(o2, "bf16"))
    assert np.array_equal(l1.cpu().numpy().view(np.uint32), l2.cpu().numpy().view(np.uint32))
    assert np.array_equal(gu.to_host(k, "bf16"), b.k_cache)   # bf16 bit patterns


def test_fused_append_rejects_prefill_plans(torch, pkv):
    b = wl.make("worked", poison=False)
    params = pkv.plan_params(mode="prefill", batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                             num_kv_heads=b.num_kv_heads, head_dim_qk=b.head_dim, page_size=b.page_size,
                             causal=True, dtype="f32", max_num_pages=b.k_cache.shape[0])
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                    kv_last_page_len=b.kv_last_page_len)
    q = gu.to_dev(b.q, "f32")
    k, v = gu.to_dev(b.k_cache, "f32"), gu.to_dev(b.v_cache, "f32")
    out = gu.empty_like_out(q.shape, "f32")
    meta = dict(append_indptr=gu.to_dev(b.append_indptr, "i32"), kv_indptr=gu.to_dev(b.kv_indptr, "i32"),
                kv_last_page_len=gu.to_dev(b.kv_last_page_len, "i32"))
    with pytest.raises(pkv.PkvError) as e:
        plan.run_append(q, k, v, gu.to_dev(b.kv_indices, "i32"), out, None, k_new=gu.to_dev(b.k_new, "f32"),
                        v_new=gu.to_dev(b.v_new, "f32"), layout=b.layout, **meta)
    assert e.value.status == 3   # PKV_ERR_UNSUPPORTED
