"""GPU parity of the split merge folded into the decode launch (paged decode
plans made with merge_in_launch = 1 and a multiple of 8 kv heads): pkv_run
then makes one launch whose
last workgroup per (request, kv head) merges the chunks' partial states.
Its output must match the float64 oracle, equal the separate merge kernel's
bit for bit (up to 64 chunks a row, where both take the same steps), and stay
the same over repeated runs of one plan (the chunk counters return to zero).
Plans from pkv_plan_create fold the merge in only up to 16 chunks a row;
fixed-capacity plans always do, so they carry the long-row cases.
Outputs start as NaN, so a row nobody merged shows up as non-finite."""

import numpy as np
import pytest

import workloads as wl
from oracle import attention as oat
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return gu.require_gpu()


@pytest.fixture(scope="module")
def pkv(torch):
    import paged_kv_cache_plan_amd as pkv
    return pkv


def _dev(torch, x, dtype):
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return gu.to_dev(x, dtype)


def _setup(pkv, torch, b, fixed, kv_dtype):
    params = pkv.plan_params(mode="decode", batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                             num_kv_heads=b.num_kv_heads, head_dim_qk=b.head_dim, page_size=b.page_size,
                             causal=True, dtype=b.dtype, kv_dtype=kv_dtype, fixed_split_pages=fixed,
                             max_num_pages=b.k_cache.shape[0], merge_in_launch=True)
    plan = pkv.Plan(params, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    dev = dict(q=gu.to_dev(b.q, b.dtype), k=_dev(torch, b.k_cache, kv_dtype), v=_dev(torch, b.v_cache, kv_dtype),
               idx=gu.to_dev(b.kv_indices, "i32"))
    return plan, dev


def _run(pkv, torch, b, plan, dev, *, separate, scales):
    o = gu.empty_like_out(dev["q"].shape, b.dtype)
    lse = torch.full((dev["q"].shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    if separate:
        plan.run_attention(dev["q"], dev["k"], dev["v"], dev["idx"], o, lse, layout=b.layout, sm_scale=b.sm_scale,
                           **scales)
        plan.run_merge(o, lse)
    else:
        plan.run(dev["q"], dev["k"], dev["v"], dev["idx"], o, lse, layout=b.layout, sm_scale=b.sm_scale, **scales)
    torch.cuda.synchronize()
    return gu.to_host(o, b.dtype), lse.cpu().numpy()


def _bits(x):
    x = np.ascontiguousarray(x)
    return x.view(np.uint32) if x.dtype == np.float32 else x


CASES = [
    # name, overrides, cache dtype, forced chunk pages
    ("decode bf16 NHD p16", dict(), "bf16", 2),
    ("decode bf16 HND p16", dict(layout="HND"), "bf16", 1),
    ("decode bf16 p3", dict(page_size=3), "bf16", 5),
    ("decode bf16 p1", dict(page_size=1), "bf16", 40),
    ("decode bf16 G1", dict(hq=8), "bf16", 3),
    ("decode bf16 G8", dict(hq=64), "bf16", 3),
    ("decode bf16 d64", dict(dim=64), "bf16", 2),
    ("decode fp8", dict(kv_dtype="fp8"), "fp8", 2),
    ("decode f32", dict(dtype="f32", page_size=4), "f32", 4),
    ("decode planner split", dict(), "bf16", 0),
]


def _graph_plan(pkv, b, fixed, kv_dtype):
    """A fixed-capacity plan of the same batch: it keeps the merge inside the
    launch whatever the chunk count."""
    params = pkv.plan_params(mode="decode", batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                             num_kv_heads=b.num_kv_heads, head_dim_qk=b.head_dim, page_size=b.page_size,
                             causal=True, dtype=b.dtype, kv_dtype=kv_dtype, fixed_split_pages=fixed,
                             max_num_pages=b.k_cache.shape[0], merge_in_launch=True)
    plan = pkv.GraphPlan(params, pkv.graph_caps(max_total_rows=b.batch_size, max_total_pages=len(b.kv_indices)))
    plan.update(kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    return plan


@pytest.mark.parametrize("name,over,kv_dtype,fixed", CASES, ids=[c[0] for c in CASES])
def test_merge_in_launch_matches_oracle_and_separate_merge(torch, pkv, name, over, kv_dtype, fixed):
    print("case merge in launch", name, flush=True)
    b = wl.make("decode", scale=0.25, batch=12, poison=True, **over)
    plan, dev = _setup(pkv, torch, b, fixed, kv_dtype)
    assert plan.info["split"] == 1 and plan.info["num_merges"] > 0
    chunks = int(max(m[3] for m in pkv.plan_compute(plan.params, qo_indptr=None, kv_indptr=b.kv_indptr,
                                                    kv_indices=b.kv_indices,
                                                    kv_last_page_len=b.kv_last_page_len)[2]))
    # 8 kv heads on MI355X: the merge runs inside the launch up to 16 chunks a row
    assert plan.info["merge_in_launch"] == (1 if chunks <= 16 else 0), chunks
    gplan = _graph_plan(pkv, b, fixed, kv_dtype)
    assert gplan.info["merge_in_launch"] == 1
    scales = dict(k_scale=0.75, v_scale=1.25) if kv_dtype == "fp8" else {}
    o_sep, l_sep = _run(pkv, torch, b, plan, dev, separate=True, scales=scales)
    o_pl, l_pl = _run(pkv, torch, b, plan, dev, separate=False, scales=scales)
    o_in, l_in = _run(pkv, torch, b, gplan, dev, separate=False, scales=scales)
    # the same steps as the separate merge kernel up to 64 chunks a row
    for o, l, what in ((o_pl, l_pl, "plan"), (o_in, l_in, "fixed-capacity plan")):
        if chunks <= 64:
            assert np.array_equal(_bits(o), _bits(o_sep)), f"{name} {what}: o differs from the separate merge"
            assert np.array_equal(_bits(l), _bits(l_sep)), f"{name} {what}: lse differs from the separate merge"
        else:
            gu.check_close(gu.as_f64(o, b.dtype), gu.as_f64(o_sep, b.dtype), b.dtype, f"{name} {what} vs separate")
            gu.check_lse(l, l_sep, f"{name} {what} lse vs separate", atol=1e-5)
    for rep in range(2):   # the counters are back at zero: later runs merge again
        o2, l2 = _run(pkv, torch, b, gplan, dev, separate=False, scales=scales)
        assert np.array_equal(_bits(o2), _bits(o_in)) and np.array_equal(_bits(l2), _bits(l_in)), f"rerun {rep}"
    ro, rl = oat.paged_attention(b.q, b.k_cache, b.v_cache, qo_indptr=list(b.qo_indptr),
                                 kv_indptr=list(b.kv_indptr), kv_indices=list(b.kv_indices),
                                 kv_last_page_len=list(b.kv_last_page_len), page_size=b.page_size,
                                 layout=b.layout, num_kv_heads=b.num_kv_heads, causal=True, sm_scale=b.sm_scale,
                                 q_dtype=b.dtype, kv_dtype=kv_dtype, **scales)
    for o, l, what in ((o_pl, l_pl, "plan"), (o_in, l_in, "fixed-capacity plan")):
        gu.check_close(gu.as_f64(o, b.dtype), ro, b.dtype, f"{name} {what} o")
        gu.check_lse(l, rl, f"{name} {what} lse", atol=1e-5 if b.dtype == "f32" else gu.LSE_ATOL)


def test_merge_in_launch_long_row_past_64_chunks(torch, pkv):
    """The skewed batch (one 32768-key request split into 77 chunks, page 1).
    A plain plan merges rows of more than 16 chunks in their own launch; a
    fixed-capacity plan keeps the merge inside the launch for any chunk count,
    where the row with more than 64 chunks takes the wave's strided
    statistics."""
    print("case merge in launch skewed", flush=True)
    b = wl.make("skewed", poison=True)
    plan0, dev = _setup(pkv, torch, b, 0, "bf16")
    assert plan0.info["merge_in_launch"] == 0
    plan = _graph_plan(pkv, b, 0, "bf16")
    assert plan.info["merge_in_launch"] == 1 and plan.info["num_merges"] > 0
    o_in, l_in = _run(pkv, torch, b, plan, dev, separate=False, scales={})
    o_sep, l_sep = _run(pkv, torch, b, plan0, dev, separate=False, scales={})
    ro, rl = oat.paged_attention(b.q, b.k_cache, b.v_cache, qo_indptr=list(b.qo_indptr),
                                 kv_indptr=list(b.kv_indptr), kv_indices=list(b.kv_indices),
                                 kv_last_page_len=list(b.kv_last_page_len), page_size=b.page_size,
                                 layout=b.layout, num_kv_heads=b.num_kv_heads, causal=True, sm_scale=b.sm_scale,
                                 q_dtype="bf16", kv_dtype="bf16")
    gu.check_close(gu.as_f64(o_in, "bf16"), ro, "bf16", "skewed o")
    gu.check_lse(l_in, rl, "skewed lse")
    gu.check_guard(gu.as_f64(o_in, "bf16"), ro, l_in, rl, "skewed")
    gu.check_close(gu.as_f64(o_in, "bf16"), gu.as_f64(o_sep, "bf16"), "bf16", "skewed vs separate merge")
    gu.check_lse(l_in, l_sep, "skewed lse vs separate merge", atol=1e-5)


def test_merge_in_launch_needs_kv_heads_in_eights_and_the_request(torch, pkv):
    b = wl.make("decode", scale=0.25, batch=12, hq=8, hkv=2, poison=True)
    plan, dev = _setup(pkv, torch, b, 2, "bf16")
    assert plan.info["split"] == 1 and plan.info["merge_in_launch"] == 0
    b = wl.make("decode", scale=0.25, batch=12, poison=True)
    params = pkv.plan_params(mode="decode", batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                             num_kv_heads=b.num_kv_heads, head_dim_qk=b.head_dim, page_size=b.page_size,
                             dtype="bf16", fixed_split_pages=2, max_num_pages=b.k_cache.shape[0])
    plan = pkv.Plan(params, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    assert plan.info["split"] == 1 and plan.info["merge_in_launch"] == 0   # not asked for
